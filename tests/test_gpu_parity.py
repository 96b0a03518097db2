"""GPU parity of the HIP forward and backward kernels against the fp64
oracle, through the C ABI, at sizes the oracle finishes in seconds: several
tiles plus a ragged tail, every mask kind, dropout, and the degenerate cases."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (check_grad, check_lse, check_o, cuda, f64, fa_kw, oracle_kw)

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("io_aware_exact_tiled_amd")

DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def run_and_check(x, bwd=True, label=""):
    print(f"[case] {label}", flush=True)
    q, k, v, do = (cuda(x[n]) for n in ("q", "k", "v", "do"))
    dtype = q.dtype
    okw = oracle_kw(x)
    O, L = oracle.attn_fwd(x["q"], x["k"], x["v"], x["scale"], **okw)
    o32, lse = fa.fwd(q, k, v, o_fp32=True, **fa_kw(x))
    o, lse2 = fa.fwd(q, k, v, **fa_kw(x))
    torch.cuda.synchronize()
    e_o = check_o(o32, O, dtype)
    check_o(o, O, dtype, "O(stored)", stored=True)
    e_l = check_lse(lse, L, dtype)
    assert torch.equal(lse, lse2)
    res = dict(o=e_o, lse=e_l)
    if bwd:
        dq, dk, dv = fa.bwd(q, k, v, o32 if dtype != torch.float32 else o, do, lse, **fa_kw(x))
        torch.cuda.synchronize()
        rq, rk, rv, _ = oracle.attn_bwd(x["q"], x["k"], x["v"], x["do"], x["scale"], **okw)
        res.update(dq=check_grad(dq, rq, dtype, "dQ"), dk=check_grad(dk, rk, dtype, "dK"),
                   dv=check_grad(dv, rv, dtype, "dV"))
    print(f"[ok] {label} {res}", flush=True)
    return res


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tiny_workload(dtype):
    w = W.WORKLOADS["tiny"]
    run_and_check(W.make_inputs(w, dtype=dtype), label=f"tiny {dtype}")


CASES = [
    # (N, d, dtype, causal, key_lens, sparse, dropout)
    (1, 64, "bf16", False, None, False, 0.0),
    (17, 64, "bf16", True, None, False, 0.0),
    (64, 128, "bf16", False, None, False, 0.0),
    (129, 128, "fp16", True, None, False, 0.0),
    (255, 64, "fp16", False, "mixed", False, 0.0),
    (300, 128, "bf16", True, "mixed", False, 0.0),
    (300, 64, "bf16", False, None, True, 0.0),
    (384, 128, "bf16", True, None, True, 0.0),
    (200, 64, "fp16", False, "mixed", False, 0.1),
    (257, 128, "bf16", True, None, False, 0.5),
    (300, 64, "bf16", True, "mixed", True, 0.2),
    (100, 64, "fp32", True, "mixed", False, 0.0),
    (130, 128, "fp32", False, None, False, 0.25),
    (513, 64, "bf16", True, None, False, 0.0),
    (640, 128, "fp16", False, None, False, 0.0),
    # d = 128 beyond the short-causal range: the eight-wave dK/dV kernel, whose
    # 16-bit hand-off of P (and of P o Z/(1-p)) is packed
    (200, 128, "bf16", False, "mixed", False, 0.15),
    (96, 128, "fp16", False, None, True, 0.3),
    (2100, 128, "bf16", True, None, False, 0.1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N%d-d%d-%s-c%d-kl%s-sp%d-p%g" % c)
def test_edge_matrix(case):
    N, d, dtype, causal, kl, sparse, p = case
    x = W.random_case(2, 2, N, d, dtype=dtype, seed=N * 7 + d, causal=causal,
                      dropout_p=p, dropout_seed=N + 11, rng_offset=3 if p else 0,
                      sparse_density=0.4 if sparse else None)
    if kl == "mixed":
        x["key_lens"] = torch.tensor([max(N // 3, 1), N], dtype=torch.int32)
    run_and_check(x, label=str(case))


GQA_CASES = [
    # (H, Hkv, N, d, dtype, causal, key_lens, sparse, dropout)
    (4, 2, 300, 64, "bf16", True, None, False, 0.0),
    (6, 1, 257, 128, "bf16", False, "mixed", False, 0.0),
    (4, 1, 200, 64, "fp16", False, "mixed", False, 0.1),
    (8, 2, 384, 128, "bf16", True, None, True, 0.0),
    (4, 2, 130, 128, "fp32", True, None, False, 0.0),
    (6, 3, 513, 64, "bf16", True, "mixed", False, 0.2),
    # eight-wave dK/dV kernel (d = 128, non-causal) with dropout and two query heads per K/V head
    (4, 2, 300, 128, "bf16", False, None, False, 0.2),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: "H%d-Hkv%d-N%d-d%d-%s-c%d-kl%s-sp%d-p%g" % c)
def test_grouped_query_matrix(case):
    """Grouped-query and multi-query attention: K, V (and dK, dV) have Hkv
    heads; dK, dV are the sums over each group's query heads."""
    H, hkv, N, d, dtype, causal, kl, sparse, p = case
    x = W.random_case(2, H, N, d, dtype=dtype, seed=N * 3 + hkv, causal=causal, dropout_p=p,
                      dropout_seed=N + 5, rng_offset=1 if p else 0,
                      sparse_density=0.4 if sparse else None, kv_heads=hkv)
    assert x["k"].shape[1] == hkv
    if kl == "mixed":
        x["key_lens"] = torch.tensor([max(N // 3, 1), N], dtype=torch.int32)
    run_and_check(x, label=str(case))


def test_grouped_query_tile_visits():
    """With grouped K/V heads the dK/dV kernel walks every query head of its
    group: each query head's visit map is still the exact tile set."""
    N = 700
    x = W.random_case(1, 4, N, 64, dtype="bf16", seed=31, causal=True, sparse_density=0.3, kv_heads=1)
    q, k, v, do = (cuda(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, **fa_kw(x))
    dq, dk, dv, tb = fa.bwd(q, k, v, o, do, lse, record_tiles=True, **fa_kw(x))
    okw = oracle_kw(x)
    for pass_, t in ((1, tb[0]), (2, tb[1])):
        br, bc = fa.tile_shape(64, 2, pass_, N, True)
        assert t.shape[2:] == (-(-N // br), -(-N // bc))
        want = oracle.expected_tiles(N, br, bc, 1, okw["causal"], okw["key_lens"], okw["block_mask"])
        got = t.cpu().numpy()
        for h in range(4):
            assert np.array_equal(got[:, h], want), f"pass {pass_} head {h}"


DECODE_CASES = [
    # (B, H, Hkv, Nq, Nk, d, dtype, causal, kv_lens)
    (2, 4, 4, 1, 1000, 128, "bf16", False, None),
    (3, 8, 2, 1, 3000, 128, "bf16", True, (3000, 1, 777)),
    (2, 8, 1, 4, 700, 64, "fp16", True, (700, 3)),
    (2, 6, 3, 16, 513, 64, "bf16", True, (513, 100)),
    (1, 16, 2, 8, 900, 128, "fp16", True, None),
    (2, 4, 1, 2, 4097, 64, "bf16", False, (4097, 2048)),
    (1, 2, 1, 1, 16384, 64, "bf16", True, (16000,)),      # 128 chunks: two batches in the merge
    (1, 4, 1, 3, 2600, 128, "fp16", True, (2599,)),       # 21 chunks
    (4, 8, 2, 2, 900, 128, "fp16", True, (500, 500, 200, 500)),   # equal lengths
    (70, 4, 2, 1, 300, 64, "bf16", True, tuple((i * 37) % 300 + 1 for i in range(70))),  # many short sequences
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B%d-H%d-Hkv%d-Nq%d-Nk%d-d%d-%s-c%d-%s" % (
    c[:8] + ("kl" if c[8] else "full",)))
def test_decode_matrix(case):
    """Decode over a key/value cache: split chunks merged on the device, against
    the fp64 oracle; rows with no valid key (cache shorter than Nq under the
    causal mask) give O = 0 and LSE = -inf."""
    B, H, hkv, nq, nk, d, dtype, causal, lens = case
    print(f"[case] decode {case}", flush=True)
    rng = np.random.default_rng(nk + nq + hkv)
    dt = DT[dtype]
    q = torch.from_numpy(rng.standard_normal((B, H, nq, d))).to(dt)
    k = torch.from_numpy(rng.standard_normal((B, hkv, nk, d))).to(dt)
    v = torch.from_numpy(rng.standard_normal((B, hkv, nk, d))).to(dt)
    kl = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    o, lse = fa.decode(cuda(q), cuda(k), cuda(v), kv_lens=cuda(kl), causal=causal)
    torch.cuda.synchronize()
    O, L = oracle.decode_fwd(q, k, v, 1.0 / np.sqrt(d), kv_lens=None if kl is None else kl.numpy(), causal=causal)
    res = dict(o=check_o(o, O, dt, "O(stored)", stored=True), lse=check_lse(lse, L, dt))
    print(f"[ok] decode {case} {res}", flush=True)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_decode_ignores_cache_past_valid_length(dtype, d):
    """Cache rows at or past kv_lens[b] are never read: filled with NaN they
    change nothing.  The expected values come from the oracle on the same cache
    with those rows zeroed (keys past the valid length take no part)."""
    B, H, hkv, nq, nk = 3, 8, 2, 2, 2048
    lens = (1500, 37, 2048)
    print(f"[case] decode NaN past length {dtype} d={d}", flush=True)
    rng = np.random.default_rng(91)
    dt = DT[dtype]
    q = torch.from_numpy(rng.standard_normal((B, H, nq, d))).to(dt)
    k = torch.from_numpy(rng.standard_normal((B, hkv, nk, d))).to(dt)
    v = torch.from_numpy(rng.standard_normal((B, hkv, nk, d))).to(dt)
    kn, vn = k.clone(), v.clone()
    for b, L in enumerate(lens):
        k[b, :, L:] = 0
        v[b, :, L:] = 0
        kn[b, :, L:] = float("nan")
        vn[b, :, L:] = float("nan")
    kl = torch.tensor(lens, dtype=torch.int32)
    o, lse = fa.decode(cuda(q), cuda(kn), cuda(vn), kv_lens=cuda(kl), causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    O, L = oracle.decode_fwd(q, k, v, 1.0 / np.sqrt(d), kv_lens=kl.numpy(), causal=True)
    res = dict(o=check_o(o, O, dt, "O(stored)", stored=True), lse=check_lse(lse, L, dt))
    print(f"[ok] decode NaN past length {res}", flush=True)


def test_fully_masked_rows_and_empty_keys():
    x = W.random_case(3, 2, 200, 64, dtype="bf16", seed=5)
    x["key_lens"] = torch.tensor([0, 1, 200], dtype=torch.int32)
    r = run_and_check(x, label="key_lens 0/1/N")
    o, lse = fa.fwd(cuda(x["q"]), cuda(x["k"]), cuda(x["v"]), key_lens=cuda(x["key_lens"]))
    assert (o[0] == 0).all() and torch.isneginf(lse[0]).all()


def test_block_mask_all_zero_rows():
    x = W.random_case(1, 2, 384, 64, dtype="bf16", seed=8)
    bm = torch.ones(3, 3, dtype=torch.uint8)
    bm[1] = 0                   # query rows 128..255 see nothing
    bm[2, 0] = 0
    x["block_mask"] = bm
    run_and_check(x, label="block mask with an empty row")


def test_dropout_keep_mask_bit_exact():
    B, H, N = 2, 3, 203
    for seed, off, p in ((3, 0, 0.1), (2 ** 40 + 5, 7, 0.5), (0, 0, 0.9)):
        keep = fa.dropout_keep_mask(seed, off, p, B, H, N).cpu().numpy()
        for b in range(B):
            for h in range(H):
                want = oracle.keep_mask(seed, off, p, b, h, H, np.arange(N), np.arange(N))
                assert np.array_equal(keep[b, h].astype(bool), want), (seed, off, p, b, h)


TILE_CASES = [
    # (N, d, dtype, causal, key_lens, sparse); the dK/dV kernel each one runs
    (1000, 64, "bf16", True, False, False),     # four-wave dK/dV (32 x 64 tiles)
    (1000, 64, "bf16", False, True, False),
    (700, 64, "bf16", True, False, True),
    (384, 64, "bf16", False, True, True),
    (777, 64, "fp16", True, True, True),
    (300, 64, "fp32", True, True, True),         # fp32: eight waves, 32 x 128
    (2048, 128, "bf16", True, False, True),      # causal d = 128 up to 2048: four waves
    (1100, 128, "fp16", True, True, False),
    (2300, 128, "bf16", True, False, True),      # causal d = 128 past 2048: eight waves, 64 x 128
    (640, 128, "bf16", False, True, True),
    (500, 128, "fp16", False, False, True),
    (257, 128, "fp32", False, True, True),
]


@pytest.mark.parametrize("case", TILE_CASES, ids=lambda c: "N%d-d%d-%s-c%d-kl%d-sp%d" % c)
def test_tile_visits_bit_exact(case):
    """Every kernel's set of visited tiles, at the tile shape fa_tile_shape
    names for this (d, dtype, N, causal), equals the exact set of tiles that
    hold a valid pair (summary, "Block-Sparse FlashAttention"; tutorial 10.2),
    for each kernel configuration fa_bwd can launch; the gradients recorded
    alongside still match the oracle (recording does not change the kernel)."""
    N, d, dtype, causal, kl, sparse = case
    print(f"[case] tile visits {case}", flush=True)
    x = W.random_case(2, 2, N, d, dtype=dtype, seed=N + d, causal=causal,
                      sparse_density=0.3 if sparse else None)
    if kl:
        x["key_lens"] = torch.tensor([N // 5, N - 1], dtype=torch.int32)
    q, k, v, do = (cuda(x[n]) for n in ("q", "k", "v", "do"))
    o, lse, tf = fa.fwd(q, k, v, record_tiles=True, **fa_kw(x))
    dq, dk, dv, tb = fa.bwd(q, k, v, o, do, lse, record_tiles=True, **fa_kw(x))
    ref = fa.bwd(q, k, v, o, do, lse, **fa_kw(x))
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)
    okw = oracle_kw(x)
    code = {"bf16": 2, "fp16": 1, "fp32": 0}[dtype]
    for pass_, t in ((0, tf), (1, tb[0]), (2, tb[1])):
        br, bc = fa.tile_shape(d, code, pass_, N, causal)
        assert t.shape[2:] == (-(-N // br), -(-N // bc))
        want = oracle.expected_tiles(N, br, bc, 2, okw["causal"], okw["key_lens"], okw["block_mask"])
        got = t.cpu().numpy()
        for h in range(2):
            assert np.array_equal(got[:, h], want), f"pass {pass_} head {h}"
    print(f"[ok] tile visits {case}", flush=True)


def test_grouped_query_exact_workspace():
    """The bf16 forward workspace covers the K/V heads only: a buffer of
    exactly fwd_workspace_bytes(B, Hkv, ...) bytes (Hkv = H / 4) gives the
    oracle's O."""
    B, H, hkv, N, d = 2, 8, 2, 300, 128
    x = W.random_case(B, H, N, d, dtype="bf16", seed=77, causal=True, kv_heads=hkv)
    q, k, v = (cuda(x[n]) for n in ("q", "k", "v"))
    need = fa.fwd_workspace_bytes(B, hkv, N, d, torch.bfloat16)
    assert need < fa.fwd_workspace_bytes(B, H, N, d, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(q, k, v, causal=True, o_fp32=True, workspace=ws)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal=True)
    check_o(o, O, torch.bfloat16)
    check_lse(lse, L, torch.bfloat16)


def test_forward_is_deterministic_and_order_free():
    x = W.random_case(2, 4, 777, 128, dtype="bf16", seed=9, causal=True)
    q, k, v = (cuda(x[n]) for n in ("q", "k", "v"))
    a = fa.fwd(q, k, v, causal=True, o_fp32=True)
    b = fa.fwd(q, k, v, causal=True, o_fp32=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    r = fa.fwd(q, k, v, causal=True, o_fp32=True, reverse_kv=True)
    assert (r[0] - a[0]).abs().max().item() < 1e-3
    assert (r[1] - a[1]).abs().max().item() < 1e-4


def test_backward_dk_dv_deterministic():
    x = W.random_case(1, 2, 500, 64, dtype="fp16", seed=10, causal=True)
    q, k, v, do = (cuda(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd(q, k, v, o, do, lse, causal=True)
    g2 = fa.bwd(q, k, v, o, do, lse, causal=True)
    assert torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])
    assert (g1[0].float() - g2[0].float()).abs().max().item() <= 1e-3 * g1[0].float().abs().max().item()


@pytest.mark.parametrize("vscale_log2", [0, 60, -60, 100])
def test_bf16_v_outside_fp16_range(vscale_log2):
    """bf16 forward: P*V runs in fp16 on a copy of V scaled by a power of two
    per (b, h).  Heads whose V lies far above fp16's range (2^60, 2^100), far
    below its normal range (2^-60), spans 2^20 within the head, or is all
    zero give O equal to the oracle's to the usual bound, relative to the
    head's own scale."""
    N = 300
    x = W.random_case(1, 4, N, 64, dtype="bf16", seed=21, causal=True)
    s = 2.0 ** vscale_log2
    v = x["v"].to(torch.float64)
    v[0, 0] *= s
    v[0, 1] = 0.0
    v[0, 2, ::7] *= 2.0 ** 20         # one key in seven is 2^20 times larger
    v[0, 2] *= s
    x["v"] = v.to(torch.bfloat16)     # exact: powers of two within bf16's range
    assert torch.equal(x["v"].to(torch.float64), v)
    print(f"[case] bf16 V scaled by 2^{vscale_log2}", flush=True)
    q, k, vv = (cuda(x[n]) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, vv, causal=True, o_fp32=True)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal=True)
    check_lse(lse, L, torch.bfloat16)
    got = f64(o)
    for h, unit in ((0, s), (2, s * 2.0 ** 20), (3, 1.0)):
        check_o(torch.from_numpy(got[:, h] / unit), O[:, h] / unit, torch.bfloat16, f"O head {h}")
    assert (got[:, 1] == 0).all()


def test_nan_propagates_without_hang():
    x = W.random_case(1, 1, 300, 64, dtype="bf16", seed=12)
    q = x["q"].clone()
    q[0, 0, 5, 3] = float("nan")
    o, lse = fa.fwd(cuda(q), cuda(x["k"]), cuda(x["v"]), o_fp32=True)
    torch.cuda.synchronize()
    o = o.cpu()
    assert torch.isnan(o[0, 0, 5]).all()
    rows = [i for i in range(300) if i != 5]
    assert torch.isfinite(o[0, 0, rows]).all()


def test_runs_on_a_non_default_stream():
    x = W.random_case(2, 2, 640, 64, dtype="bf16", seed=13, causal=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q, k, v = (x[n].to("cuda", non_blocking=False) for n in ("q", "k", "v"))
        q = q * 1.0          # producer work on the same stream
        o, lse = fa.fwd(q, k, v, causal=True, o_fp32=True)
        o2 = o * 2.0         # consumer on the same stream
    s.synchronize()
    O, L = oracle.attn_fwd(x["q"], x["k"], x["v"], x["scale"], causal=True)
    check_o(o2 / 2.0, O, torch.bfloat16)


def test_extra_memory_is_linear_in_n():
    N, d = 16384, 128
    q = torch.randn(1, 1, N, d, device="cuda", dtype=torch.bfloat16)
    k, v = torch.randn_like(q), torch.randn_like(q)
    do = torch.randn_like(q)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    # outputs (O, dQ, dK, dV in bf16, LSE) + the forward's fp16 copy of V + D:
    # all O(N d); a single N x N bf16 matrix would be 512 MiB
    linear = 4 * N * d * 2 + N * 4 + N * d * 4 + N * 4 + (1 << 20)
    assert peak <= linear, (peak, linear)


KVO_CASES = [
    # (B, H, N, d, dtype, causal, block_cols, groups_per_head)
    (1, 2, 1000, 64, "bf16", True, 64, 1),
    (2, 2, 777, 128, "bf16", False, 128, 0),
    (1, 3, 513, 128, "fp16", True, 128, 2),
    (2, 1, 300, 64, "fp16", False, 64, 3),
    (1, 2, 4096, 128, "bf16", True, 128, 4),
    (1, 1, 40, 64, "bf16", True, 128, 1),
]


@pytest.mark.parametrize("case", KVO_CASES, ids=lambda c: "B%d-H%d-N%d-d%d-%s-c%d-bc%d-G%d" % c)
def test_kv_outer_forward_matrix(case):
    """The key/value-outer forward (running O, m, l through device memory
    after every key tile) against the fp64 oracle."""
    B, H, N, d, dtype, causal, bc, G = case
    print(f"[case] kv-outer fwd {case}", flush=True)
    rng = np.random.default_rng(N + d + bc)
    dt = DT[dtype]
    q, k, v = (torch.from_numpy(rng.standard_normal((B, H, N, d))).to(dt) for _ in range(3))
    o, lse = fa.fwd_kv_outer(cuda(q), cuda(k), cuda(v), causal=causal, block_cols=bc, groups_per_head=G)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd(q, k, v, 1.0 / np.sqrt(d), causal=causal)
    res = dict(o=check_o(o, O, dt, "O(stored)", stored=True), lse=check_lse(lse, L, dt))
    print(f"[ok] kv-outer {case} {res}", flush=True)


@pytest.mark.parametrize("B,H,d", [(8, 2, 64), (4, 6, 128)])
def test_rank_order_dispatch_small_causal(B, H, d):
    """B*H a multiple of 8: causal launches walk each XCD's heads rank by rank
    (the heaviest tile of every head first); ragged N = 300 so tiles differ
    in cost and the last ones are partial."""
    x = W.random_case(B, H, 300, d, dtype="bf16", seed=B * 100 + H + d, causal=True)
    run_and_check(x, label=f"rank order B{B} H{H} d{d}")
