"""The C-ABI library loads, exports every symbol include/fa.h declares, and its
host-side validation rejects bad arguments before touching the GPU (these
calls return before any HIP call, so they run without a device)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

lib_mod = pytest.importorskip("io_aware_exact_tiled_amd._lib")


def _lib():
    if not os.path.exists(lib_mod.LIB_PATH):
        pytest.skip("libfa.so not built")
    return lib_mod.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(fa_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(lib_mod.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", lib_mod.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fa_\w+)", out))
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(L, s)


def test_scalars():
    L = _lib()
    assert L.fa_abi_version() == 7
    for code in list(lib_mod.STATUS) + [-99]:
        assert isinstance(L.fa_status_string(code), bytes)
    br, bc = ctypes.c_int32(), ctypes.c_int32()
    for d in (64, 128):
        for dt in (0, 1, 2):
            for p in (0, 1, 2):
                for N, causal in ((1, 0), (2048, 1), (2049, 1), (4096, 0)):
                    assert L.fa_tile_shape(d, dt, p, N, causal, ctypes.byref(br), ctypes.byref(bc)) == 0
                    assert 128 % br.value == 0 and 128 % bc.value == 0
    assert L.fa_tile_shape(96, 2, 0, 64, 0, ctypes.byref(br), ctypes.byref(bc)) == -3
    assert L.fa_tile_shape(64, 7, 0, 64, 0, ctypes.byref(br), ctypes.byref(bc)) == -4
    assert L.fa_tile_shape(64, 2, 0, 0, 0, ctypes.byref(br), ctypes.byref(bc)) == -2
    assert L.fa_bwd_workspace_bytes(1, 2, 256, 64) == 2048
    assert L.fa_bwd_workspace_bytes(1, 1, 3, 64) == 256
    assert L.fa_tile_shape(64, 2, 3, 64, 0, ctypes.byref(br), ctypes.byref(bc)) == -10
    assert L.fa_bwd_workspace_bytes(0, 1, 3, 64) == 0


@pytest.mark.parametrize("d,dt,N,causal,want", [
    # the four-wave dK/dV configuration: 16-bit inputs at d = 64 (any N, mask),
    # and causal d = 128 up to N = 2048
    (64, 2, 16384, 0, (32, 64)), (64, 1, 512, 1, (32, 64)), (128, 2, 2048, 1, (32, 64)),
    # the eight-wave one: 128 keys x 64 query rows (fp32: 32 rows)
    (128, 2, 2049, 1, (64, 128)), (128, 1, 1024, 0, (64, 128)), (128, 2, 16384, 1, (64, 128)),
    (64, 0, 256, 0, (32, 128)), (128, 0, 100, 1, (32, 128))])
def test_tile_shape_names_the_launched_dkdv_kernel(d, dt, N, causal, want):
    """fa_tile_shape(pass 1) is the tile of the dK/dV configuration fa_bwd
    launches for (d, dtype, N, causal); forward and dQ tiles do not depend on
    N or the mask."""
    L = _lib()
    br, bc = ctypes.c_int32(), ctypes.c_int32()
    assert L.fa_tile_shape(d, dt, 1, N, causal, ctypes.byref(br), ctypes.byref(bc)) == 0
    assert (br.value, bc.value) == want
    assert L.fa_tile_shape(d, dt, 0, N, causal, ctypes.byref(br), ctypes.byref(bc)) == 0
    assert (br.value, bc.value) == (128, 64)
    assert L.fa_tile_shape(d, dt, 2, N, causal, ctypes.byref(br), ctypes.byref(bc)) == 0
    assert (br.value, bc.value) == (128, 64)


P = 0x10000  # a 256-byte aligned fake device address: never dereferenced on these paths


def fwd(L, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=8, d=64, dt=2, scale=0.125, causal=0, p=0.0, seed=0,
        mask=None, opts=None, ws=P, ws_bytes=1 << 20):
    return L.fa_fwd(q, k, v, o, lse, B, H, N, d, dt, scale, causal, p, seed, mask, opts, ws, ws_bytes, None)


def bwd(L, B=1, H=1, N=8, d=64, dt=2, scale=0.125, p=0.0, opts=None, ws=P, ws_bytes=1 << 20, ptrs=None):
    ptrs = ptrs or [P] * 9
    return L.fa_bwd(*ptrs, B, H, N, d, dt, scale, 0, p, 0, None, opts, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(N=0), -2), (dict(H=70000), -2), (dict(N=1 << 26, d=64), -2),
    (dict(d=96), -3), (dict(d=0), -3),
    (dict(dt=5), -4),
    (dict(p=1.0), -5), (dict(p=-0.1), -5), (dict(p=float("nan")), -5),
    (dict(scale=0.0), -6), (dict(scale=-1.0), -6), (dict(scale=float("inf")), -6), (dict(scale=float("nan")), -6),
    (dict(o=P + 8), -7), (dict(k=P + 2), -7),
])
def test_fwd_validation(kw, code):
    assert fwd(_lib(), **kw) == code


def test_opts_validation():
    L = _lib()
    o = lib_mod.FaOpts()
    o.struct_size = 3
    assert fwd(L, opts=ctypes.byref(o)) == -10
    o.struct_size = ctypes.sizeof(lib_mod.FaOpts)
    o.flags = 1 << 7
    assert fwd(L, opts=ctypes.byref(o)) == -10
    o.flags = lib_mod.FA_FLAG_RECORD_TILES
    o.tile_visits = None
    assert fwd(L, opts=ctypes.byref(o)) == -1
    o.flags = lib_mod.FA_FLAG_REVERSE_KV
    assert bwd(L, opts=ctypes.byref(o)) == -10      # forward-only flag


def align256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("B,H,N,d", [(1, 2, 256, 64), (1, 1, 3, 64), (2, 3, 1000, 128), (1, 16, 16384, 128)])
def test_fwd_workspace_bytes(B, H, N, d):
    """bf16 needs the fp16 copy of V (B*H*N*d halves, rounded to 256 bytes)
    plus 4-byte per-head statistics (at most 64 chunk maxima and one exponent
    per head, each part rounded to 256); fp16 and fp32 need none."""
    L = _lib()
    n = L.fa_fwd_workspace_bytes(B, H, N, d, 2)
    v16 = align256(B * H * N * d * 2)
    assert v16 + 2 * 256 <= n <= v16 + align256(B * H * 64 * 4) + align256(B * H * 4)
    assert n % 256 == 0
    assert L.fa_fwd_workspace_bytes(B, H, N, d, 1) == 0
    assert L.fa_fwd_workspace_bytes(B, H, N, d, 0) == 0
    assert L.fa_fwd_workspace_bytes(B, H, N, 96, 2) == 0
    assert L.fa_fwd_workspace_bytes(0, H, N, d, 2) == 0
    assert L.fa_fwd_workspace_bytes(B, H, N, d, 9) == 0


def test_fwd_workspace_validation():
    L = _lib()
    need = L.fa_fwd_workspace_bytes(1, 1, 8, 64, 2)
    assert fwd(L, ws=None) == -8
    assert fwd(L, ws_bytes=need - 1) == -8
    assert fwd(L, ws=P + 16) == -8                  # not 256-byte aligned


def test_fwd_workspace_counts_kv_heads():
    """Grouped-query attention: the bf16 V copy covers the K/V heads only, so
    the sizer takes Hkv; fa_fwd checks against that size (one byte less is
    rejected before any launch), and the query-head value is an upper bound."""
    L = _lib()
    B, H, Hkv, N, d = 2, 8, 2, 1000, 128
    need_kv = L.fa_fwd_workspace_bytes(B, Hkv, N, d, 2)
    need_q = L.fa_fwd_workspace_bytes(B, H, N, d, 2)
    assert need_kv >= align256(B * Hkv * N * d * 2) and need_q >= 3 * need_kv
    o = lib_mod.FaOpts()
    o.struct_size = ctypes.sizeof(lib_mod.FaOpts)
    o.kv_heads = Hkv
    assert fwd(L, B=B, H=H, N=N, d=d, opts=ctypes.byref(o), ws_bytes=need_kv - 1) == -8


def test_kv_heads_validation():
    """Grouped-query attention: kv_heads must divide H; 0 means H; a struct
    from before the field (struct_size up to kv_heads) is still accepted."""
    L = _lib()
    o = lib_mod.FaOpts()
    o.struct_size = ctypes.sizeof(lib_mod.FaOpts)
    for bad in (3, 5, 8, -1):
        o.kv_heads = bad
        assert fwd(L, H=4, opts=ctypes.byref(o)) == -10, bad
        assert bwd(L, H=4, opts=ctypes.byref(o)) == -10, bad
    o.kv_heads = 2
    assert fwd(L, H=4, d=96, opts=ctypes.byref(o)) == -3     # past the options check
    o.struct_size = lib_mod.FaOpts.kv_heads.offset            # the previous layout
    o.kv_heads = 3                                            # not read
    assert fwd(L, H=4, d=96, opts=ctypes.byref(o)) == -3
    o.struct_size = lib_mod.FaOpts.kv_heads.offset - 8
    assert fwd(L, H=4, opts=ctypes.byref(o)) == -10


def test_bwd_validation():
    L = _lib()
    need = L.fa_bwd_workspace_bytes(1, 1, 8, 64)
    assert bwd(L, ws=None) == -8
    assert bwd(L, ws_bytes=need - 1) == -8
    assert bwd(L, ws=P + 16) == -8                  # not 256-byte aligned
    assert bwd(L, d=80) == -3
    assert bwd(L, p=2.0) == -5
    ptrs = [P] * 9
    ptrs[4] = None                                  # dO
    assert bwd(L, ptrs=ptrs) == -1
    ptrs = [P] * 9
    ptrs[6] = P + 4                                 # dQ misaligned
    assert bwd(L, ptrs=ptrs) == -7


def test_keep_mask_validation():
    L = _lib()
    assert L.fa_dropout_keep_mask(0, 0, 0.1, 1, 1, 8, None, None) == -1
    assert L.fa_dropout_keep_mask(0, 0, 1.5, 1, 1, 8, P, None) == -5
    assert L.fa_dropout_keep_mask(0, 0, 0.1, 0, 1, 8, P, None) == -2


def test_decode_validation_and_workspace():
    L = _lib()

    def dec(B=1, H=4, Hkv=2, Nq=1, Nk=100, d=64, dt=2, scale=0.125, ws=P, ws_bytes=1 << 24, ptrs=None):
        ptrs = ptrs or [P] * 5
        return L.fa_decode(*ptrs, B, H, Hkv, Nq, Nk, d, dt, scale, 0, None, None, ws, ws_bytes, None)

    assert dec(Hkv=3) == -2                  # must divide H
    assert dec(Hkv=0) == -2 and dec(Nq=0) == -2 and dec(Nk=0) == -2
    assert dec(d=80) == -3
    assert dec(dt=0) == -4                   # fp32 decode is not provided
    assert dec(scale=0.0) == -6
    assert dec(ptrs=[P, P, None, P, P]) == -1
    assert dec(ptrs=[P, P, P, P + 4, P]) == -7
    need = L.fa_decode_workspace_bytes(1, 4, 2, 1, 100, 64)
    assert need > 0 and need % 256 == 0
    assert dec(ws=None) == -8 and dec(ws_bytes=need - 1) == -8 and dec(ws=P + 16) == -8
    assert L.fa_decode_workspace_bytes(1, 4, 3, 1, 100, 64) == 0
    # per-split partials: O (fp32 x d) and one log-sum-exp per query row and split
    big = L.fa_decode_workspace_bytes(16, 32, 8, 1, 16384, 128)
    assert big >= 16 * 32 * 1 * (128 * 4 + 4)


def test_kv_outer_validation_and_workspace():
    L = _lib()

    def kvo(B=1, H=2, N=300, d=64, dt=2, scale=0.125, causal=0, bc=128, G=0, ws=P, ws_bytes=1 << 24,
            ptrs=None):
        ptrs = ptrs or [P] * 5
        return L.fa_fwd_kv_outer(*ptrs, B, H, N, d, dt, scale, causal, bc, G, None, ws, ws_bytes, None)

    assert kvo(N=0) == -2 and kvo(B=0) == -2
    assert kvo(d=96) == -3
    assert kvo(dt=0) == -4                   # fp32 is not provided in this order
    assert kvo(scale=float("nan")) == -6
    assert kvo(ptrs=[P, None, P, P, P]) == -1
    assert kvo(ptrs=[P, P, P, P, P + 8]) == -7
    assert kvo(bc=32) == -10 and kvo(bc=256) == -10
    assert kvo(G=4) == -2 and kvo(G=-1) == -2  # 300 rows: 3 query blocks
    need = L.fa_fwd_kv_outer_workspace_bytes(1, 2, 300, 64)
    # running O fp32 [B][H][N][d] then (m, l) per row, each part 256-byte aligned
    assert need == (1 * 2 * 300 * 64 * 4 + 255) // 256 * 256 + (1 * 2 * 300 * 8 + 255) // 256 * 256
    assert kvo(ws=None) == -8 and kvo(ws_bytes=need - 1) == -8 and kvo(ws=P + 64) == -8
    assert L.fa_fwd_kv_outer_workspace_bytes(1, 2, 300, 80) == 0


def test_header_compiles_as_c_and_links(tmp_path):
    """include/fa.h is a plain C99 header: a C program (tests/c_abi_check.c)
    compiles against it with gcc, links libfa.so and sees every entry point
    reject bad arguments on the host."""
    _lib()
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    libdir = os.path.dirname(lib_mod.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
           "-o", exe, os.path.join(here, "c_abi_check.c"), "-L", libdir, "-l:libfa.so",
           f"-Wl,-rpath,{libdir}"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c abi ok" in run.stdout


def test_bwd_noalloc_validation_on_the_host():
    """fa_bwd_noalloc validates like fa_bwd and rejects a problem whose D
    (4 bytes per query row) exceeds its static scratch with FA_ERR_SCRATCH,
    all before any device call."""
    L = _lib()
    rows = lib_mod.FA_BWD_SCRATCH_BYTES // 4
    args = [P] * 9
    assert L.fa_bwd_noalloc(*args, 1, 1, rows + 1, 64, 2, 0.125, 0, 0.0, 0, None, None, None) == -11
    assert L.fa_bwd_noalloc(*args, 2, 4, rows // 8 + 1, 128, 1, 0.125, 1, 0.0, 0, None, None, None) == -11
    assert L.fa_bwd_noalloc(None, *args[1:], 1, 1, 64, 64, 2, 0.125, 0, 0.0, 0, None, None, None) == -1
    assert L.fa_bwd_noalloc(*args, 1, 1, 64, 96, 2, 0.125, 0, 0.0, 0, None, None, None) == -3
    assert L.fa_bwd_noalloc(*args, 1, 1, 64, 64, 2, 0.125, 0, 1.5, 0, None, None, None) == -5
    assert b"static scratch" in L.fa_status_string(-11)
