"""Shared pieces of the GPU parity tests: device transfer, tolerances and the
comparisons against the fp64 oracle.

Tolerances (inputs in bf16/fp16 unless stated):
  O  written as fp32 (o_fp32): max-abs <= 2e-3.  This checks the kernels'
     arithmetic; fp32 inputs: 1e-4.
  O  written in the input dtype: max-abs <= 2e-3 + half an ulp of the dtype at
     |O_ref| (storing O alone costs up to that half ulp).
  LSE: max-abs <= 1e-3 (fp32 inputs: 1e-4) where finite; -inf exactly where
     the oracle's row has no valid key.
  dQ, dK, dV: per tensor max|g - g_ref| <= 1e-2 * max|g_ref| (fp32: 1e-4);
     where the exact gradient is identically 0, max|g| <= 1e-5 (fp32 rounding
     of dP - D, two evaluations of one O(1) sum).
"""

import multiprocessing
import os

import numpy as np
import torch

import oracle
import workloads as W

O_TOL = {torch.bfloat16: 2e-3, torch.float16: 2e-3, torch.float32: 1e-4}
LSE_TOL = {torch.bfloat16: 1e-3, torch.float16: 1e-3, torch.float32: 1e-4}
G_TOL = {torch.bfloat16: 1e-2, torch.float16: 1e-2, torch.float32: 1e-4}
MANT = {torch.bfloat16: 7, torch.float16: 10, torch.float32: 23}


def cuda(x):
    return None if x is None else x.to("cuda")


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def half_ulp(x, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 0.5 * 2.0 ** (e - MANT[dtype])


def check_o(o_gpu, O_ref, dtype, what="O", stored=False):
    got = f64(o_gpu)
    err = np.abs(got - O_ref)
    bound = O_TOL[dtype] + (half_ulp(O_ref, dtype) if stored else 0.0)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: max err {np.nanmax(err):.3e} at {np.argwhere(bad)[:3].tolist()}"
    return float(np.nanmax(err)) if err.size else 0.0


def check_lse(lse_gpu, L_ref, dtype):
    got = f64(lse_gpu)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isneginf(got), ~fin), "LSE -inf pattern differs"
    err = np.abs(got[fin] - L_ref[fin]) if fin.any() else np.zeros(1)
    assert err.max() <= LSE_TOL[dtype], f"LSE max err {err.max():.3e}"
    return float(err.max())


def check_grad(g_gpu, g_ref, dtype, what):
    got = f64(g_gpu)
    scale = np.abs(g_ref).max()
    err = np.abs(got - g_ref).max()
    assert np.isfinite(got).all(), f"{what}: non-finite"
    if scale == 0:
        # exact gradient is 0 (e.g. a single valid key: dS = dP - D = 0); the
        # kernel's dP and D are two fp32 evaluations of the same O(1) sum
        assert err <= 1e-5, f"{what}: expected ~0, max {err}"
        return float(err)
    rel = err / scale
    assert rel <= G_TOL[dtype], f"{what}: max err / max|ref| = {rel:.3e}"
    return float(rel)


def oracle_kw(x):
    return dict(causal=x["causal"], key_lens=None if x["key_lens"] is None else x["key_lens"].numpy(),
                block_mask=None if x["block_mask"] is None else x["block_mask"].numpy(),
                dropout_p=x["dropout_p"], seed=x["seed"], rng_offset=x["rng_offset"])


def fa_kw(x):
    return dict(causal=x["causal"], key_lens=cuda(x["key_lens"]), block_mask=cuda(x["block_mask"]),
                dropout_p=x["dropout_p"], seed=x["seed"], rng_offset=x["rng_offset"], scale=x["scale"])


_WORKER_INPUTS = {}


def _kv_grads_worker(job):
    """dK, dV of the sampled key rows `cols` for the K/V heads in `kv` (each
    with all the query heads that read it), from a fresh draw of workload w's
    inputs: every row's LSE and D first (attn_stats), then the score columns."""
    import threadpoolctl
    w, kv, cols = job
    with threadpoolctl.threadpool_limits(2):
        if _WORKER_INPUTS.get("w") != w:          # one draw per worker process
            _WORKER_INPUTS.update(w=w, x=W.make_inputs(w))
        x = _WORKER_INPUTS["x"]
        okw = oracle_kw(x)
        G = w.H // w.Hkv
        heads = [(b, g * G + hh) for b, g in kv for hh in range(G)]
        Ls, Ds = oracle.attn_stats(x["q"], x["k"], x["v"], x["do"], x["scale"], heads=heads, **okw)
        _, rk, rv = oracle.attn_bwd_rows_cols(x["q"], x["k"], x["v"], x["do"], x["scale"], np.arange(1), cols,
                                              Ls, Ds, pairs=heads, **okw)
    return kv, rk[[b for b, _ in kv], [g for _, g in kv]], rv[[b for b, _ in kv], [g for _, g in kv]]


def oracle_kv_grads(w, cols, workers=None):
    """Oracle dK, dV [B, Hkv, len(cols), d] at the sampled key rows of every
    K/V head of workload w, one K/V head per task over a pool of fresh
    processes (spawned: they never touch the GPU)."""
    jobs = [(w, [(b, g)], cols) for b in range(w.B) for g in range(w.Hkv)]
    workers = workers or max(1, min(8, (os.cpu_count() or 2) // 2, len(jobs)))
    rk = np.zeros((w.B, w.Hkv, len(cols), w.d))
    rv = np.zeros_like(rk)
    ctx = multiprocessing.get_context("spawn")
    with ctx.Pool(workers) as pool:
        for n, (kv, k_, v_) in enumerate(pool.imap_unordered(_kv_grads_worker, jobs)):
            for t, (b, g) in enumerate(kv):
                rk[b, g], rv[b, g] = k_[t], v_[t]
            print(f"  oracle dK/dV: {n + 1}/{len(jobs)} K/V heads", flush=True)
    return rk, rv
