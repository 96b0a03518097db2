"""fa_bwd_noalloc (the backward for callers that cannot allocate: its D
scratch is the library's static device array) through the C ABI, against
fa_bwd with a caller workspace: the same kernels, so the gradients must be
bit-identical.  Two calls in a row, the second smaller, so the shared array
carries the first call's contents into the second."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from helpers import cuda, fa_kw

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("io_aware_exact_tiled_amd")
lib_mod = pytest.importorskip("io_aware_exact_tiled_amd._lib")


def _noalloc_call(x, o, lse, grads):
    """fa_bwd_noalloc straight through ctypes (no torch allocation)."""
    q, k, v, do = (cuda(x[n]) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    code = {torch.bfloat16: 2, torch.float16: 1, torch.float32: 0}[q.dtype]
    opts = lib_mod.FaOpts()
    opts.struct_size = ctypes.sizeof(lib_mod.FaOpts)
    opts.kv_heads = k.shape[1] if k.shape[1] != H else 0
    opts.o_fp32 = 1 if (o.dtype == torch.float32 and q.dtype != torch.float32) else 0
    kl = cuda(x["key_lens"])
    opts.key_lens = kl.data_ptr() if kl is not None else None
    opts.rng_offset = int(x["rng_offset"])
    bm = cuda(x["block_mask"])
    dq, dk, dv = grads
    st = lib_mod.lib().fa_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), B, H, N, d, code, float(x["scale"]), 1 if x["causal"] else 0,
        float(x["dropout_p"]), int(x["seed"]), bm.data_ptr() if bm is not None else None, ctypes.byref(opts),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st


CASES = [
    # larger first, then smaller: the second call reads a scratch the first left full
    dict(B=2, H=8, N=2100, d=128, dtype="bf16", causal=True, p=0.1, kv=2, kl=False),
    dict(B=1, H=2, N=300, d=64, dtype="fp16", causal=False, p=0.0, kv=None, kl=True),
]


def test_bwd_noalloc_matches_bwd_twice():
    for c in CASES:
        print(f"[case] fa_bwd_noalloc {c}", flush=True)
        x = W.random_case(c["B"], c["H"], c["N"], c["d"], dtype=c["dtype"], seed=c["N"], causal=c["causal"],
                          dropout_p=c["p"], dropout_seed=5, rng_offset=2 if c["p"] else 0, kv_heads=c["kv"])
        if c["kl"]:
            x["key_lens"] = torch.tensor([c["N"] // 3], dtype=torch.int32)
        q, k, v, do = (cuda(x[n]) for n in ("q", "k", "v", "do"))
        o, lse = fa.fwd(q, k, v, **fa_kw(x))
        ref = fa.bwd(q, k, v, o, do, lse, **fa_kw(x))
        grads = tuple(torch.full_like(t, float("nan")) for t in ref)
        assert _noalloc_call(x, o, lse, grads) == 0
        for a, b, name in zip(grads, ref, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), name
        # the binding's no_alloc path is the same entry point
        again = fa.bwd(q, k, v, o, do, lse, no_alloc=True, **fa_kw(x))
        for a, b in zip(again, ref):
            assert torch.equal(a, b)
        print(f"[ok] fa_bwd_noalloc {c['B']}x{c['H']}x{c['N']}", flush=True)


def test_bwd_noalloc_rejects_more_rows_than_the_scratch_holds():
    """B*H*N rows beyond FA_BWD_SCRATCH_BYTES / 4: FA_ERR_SCRATCH, before any
    launch (the pointers are never dereferenced)."""
    L = lib_mod.lib()
    P = 0x10000
    rows = lib_mod.FA_BWD_SCRATCH_BYTES // 4
    st = L.fa_bwd_noalloc(*([P] * 9), 1, 1, rows + 1, 64, 2, 0.125, 0, 0.0, 0, None, None, None)
    assert st == -11
    assert b"static scratch" in L.fa_status_string(-11)
