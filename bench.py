#!/usr/bin/env python3
"""Throughput of tiled exact attention (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]
    python bench.py --workload decode     # decode over a key/value cache, GB/s

A step is one full pass of the hot path on one batch: the forward (for bf16
the V pre-pass, then the forward kernel: O, LSE) followed by the backward
(D pre-pass, the dK/dV kernel, the dQ kernel), on inputs already resident
in device memory.  The default
workload is the long-context causal case (B=1, H=16, N=16384, d=128, bf16),
the d=128, N>=4K configuration the fraction-of-peak target is stated for.

Algorithmic work counts valid (query, key) pairs only: the forward does
4*d FLOP per pair (S = Q K^T and P V), the backward 10*d (S recomputed, dP,
dV, dK, dQ).  Peak: MI355X dense bf16/fp16 MFMA, 2.5 PFLOP/s.

Prints one JSON line (rank 0).  Timing uses HIP events on the stream the
kernels run on: fwd_ms and bwd_ms (and their TFLOP/s) are whole passes,
pre-passes included; fwd_kernel_ms, bwd_main_ms, bwd_kv_ms and bwd_dq_ms
come from events the library records around the main kernels.

roofline.traffic is the dominant kernel's HBM traffic per launch in bytes
(FETCH_SIZE + WRITE_SIZE counters, scaled by a plain copy of known size),
read from the counter summary under profiles/ when that summary was taken
on this workload from the kernel's current sources (else null).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
HBM_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "io_aware_exact_tiled_amd", "csrc")
KERNEL_SOURCES = {"fwd_kernel": "fa_fwd.hip", "bwd_kv_kernel": "fa_bwd.hip", "bwd_dq_kernel": "fa_bwd.hip",
                  "bwd_pre_kernel": "fa_bwd.hip", "v16_convert_kernel": "fa_fwd.hip",
                  "v16_rescale_kernel": "fa_fwd.hip", "decode_split_kernel": "fa_decode.hip",
                  "decode_merge_kernel": "fa_decode.hip", "fwd_kvo_kernel": "fa_kvouter.hip"}


def kernel_sources_sha256(kernel: str) -> str:
    """SHA-256 over the sources a kernel is compiled from (its file, then the
    two shared headers)."""
    import hashlib
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "fa_device.hpp", "fa_internal.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none for this workload and kernel or it predates the kernel's
    current sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            e = json.load(fh)["workloads"][workload][kernel]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    if e.get("sources_sha256") != kernel_sources_sha256(kernel):
        return None
    return int(e["fetch_bytes"] + e["write_bytes"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=6144,
                    help="leading causal rows per head the oracle baseline computes")
    ap.add_argument("--sweep", action="store_true", help="also time the N sweep (extra JSON lines)")
    ap.add_argument("--sweep-md", metavar="PATH", default=None,
                    help="with --sweep: also write the sweep as a markdown table to PATH")
    ap.add_argument("--power", metavar="SECONDS", type=float, default=0.0,
                    help="also run the workload's forward, then its backward, back to back for SECONDS each "
                         "while amd-smi samples socket power and the GFX clock (extra JSON lines)")
    ap.add_argument("--power-md", metavar="PATH", default=None,
                    help="with --power: also write the samples' medians as a markdown table to PATH")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (graph_ms_per_step; value stays eager)")
    ap.add_argument("--io-ablation", action="store_true",
                    help="also run the key/value-outer forward beside the query-outer one at N = 2K, 4K, 8K "
                         "(extra JSON lines with the HBM bytes each order implies)")
    ap.add_argument("--compare-standard", action="store_true",
                    help="also time standard attention (five separate ops on vendor GEMMs) against this "
                         "library at N = 1K, 2K, 4K (extra JSON lines)")
    ap.add_argument("--profile", metavar="DIR",
                    help="run rocprofv3 (kernel trace + four counter passes) on the workload as child processes, "
                         "writing raw output to DIR, then write the summaries under profiles/")
    ap.add_argument("--profile-report", metavar="DIR",
                    help="only reduce an existing --profile DIR into the summaries under profiles/")
    ap.add_argument("--profile-mode", default="workload", choices=("workload", "io-ablation", "compare-standard"),
                    help="what --profile runs: the workload (trace + counters), --io-ablation (trace + byte "
                         "counters) or --compare-standard (trace)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run one plain device-to-device copy of MIB MiB (a known-size kernel "
                         "that hardware byte counters can be scaled by)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(b) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def valid_pairs(x, w):
    """Number of valid (query, key) pairs over all heads: the unit of
    algorithmic work.  Valid: (not causal or j <= i) and j < len_b and the
    128 x 128 block of (i, j) is set in the block mask."""
    N, T = w.N, 128
    rows = np.arange(N, dtype=np.int64)
    bm = None if x["block_mask"] is None else x["block_mask"].numpy().astype(bool)
    total = 0
    for b in range(w.B):
        L = N if x["key_lens"] is None else int(min(max(int(x["key_lens"][b]), 0), N))
        if bm is None:
            lim = np.full(N, L, dtype=np.int64)
            if w.causal:
                lim = np.minimum(lim, rows + 1)
            total += int(lim.sum())
            continue
        for bi in range(bm.shape[0]):
            r = rows[bi * T:(bi + 1) * T]
            for bj in np.flatnonzero(bm[bi]):
                c0, c1 = bj * T, min((bj + 1) * T, L)
                if c1 <= c0:
                    continue
                hi = np.minimum(r + 1, c1) if w.causal else np.full(len(r), c1)
                total += int(np.clip(hi - c0, 0, None).sum())
    return total * w.H


def dominant_roofline(w, pairs, kernel_ms):
    """The roofline object for the kernel with the largest average launch
    time.  Algorithmic FLOPs per launch: fwd_kernel 4d per valid pair (S,
    PV); bwd_kv_kernel 8d (S, dP, dV, dK); bwd_dq_kernel 2d (dQ; its
    recomputed S and dP are extra work).  Minimum HBM bytes per launch (e =
    element bytes; K, V, dK, dV have Hkv heads): fwd_kernel reads Q, K, V and
    writes O, LSE; bwd_kv_kernel reads Q, K, V, dO, LSE, D and writes dK, dV;
    bwd_dq_kernel reads the same and writes dQ.  A kernel whose FLOP per
    minimum byte is below the ridge (peak FLOP/s / 8 TB/s) is rated against
    HBM bandwidth, otherwise against the MFMA peak.  Returns (roofline,
    {kernel: (ms, flop, bytes)})."""
    peak = PEAK_TFLOPS[w.dtype]
    e = {"bf16": 2, "fp16": 2, "fp32": 4}[w.dtype]
    q_b = w.B * w.H * w.N * w.d * e
    kv_b = w.B * w.Hkv * w.N * w.d * e
    row_b = w.B * w.H * w.N * 4
    kern = {"fwd_kernel": (kernel_ms["fwd_kernel"], 4.0 * w.d * pairs, 2 * q_b + 2 * kv_b + row_b),
            "bwd_kv_kernel": (kernel_ms["bwd_kv_kernel"], 8.0 * w.d * pairs, 2 * q_b + 4 * kv_b + 2 * row_b),
            "bwd_dq_kernel": (kernel_ms["bwd_dq_kernel"], 2.0 * w.d * pairs, 3 * q_b + 2 * kv_b + 2 * row_b)}
    dom = max(kern, key=lambda k: kern[k][0])
    dom_ms, dom_flop, dom_bytes = kern[dom]
    ridge = peak * 1e12 / (HBM_GBPS * 1e9)
    if dom_flop / dom_bytes >= ridge:
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(dom_flop / (dom_ms * 1e-3) / 1e12, 2),
                    "peak": peak, "unit": "TFLOP/s"}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dom_bytes / (dom_ms * 1e-3) / 1e9, 1),
                    "peak": HBM_GBPS, "unit": "GB/s"}
    roofline.update(frac=round(roofline["achieved"] / roofline["peak"], 4), traffic=measured_traffic(dom, w.name),
                    avg_launch_ms=round(dom_ms, 4), flop_per_launch=dom_flop, min_bytes_per_launch=dom_bytes,
                    flop_per_byte=round(dom_flop / dom_bytes, 1))
    return roofline, kern


def time_workload(w, steps, warmup, ev, graph=False):
    import torch
    import io_aware_exact_tiled_amd as fa
    import workloads as W

    x = W.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    kw = dict(causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed, rng_offset=w.rng_offset,
              key_lens=None if x["key_lens"] is None else x["key_lens"].to(dev),
              block_mask=None if x["block_mask"] is None else x["block_mask"].to(dev), scale=w.scale)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(1, fa.fwd_workspace_bytes(w.B, w.Hkv, w.N, w.d, q.dtype)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    n_ev = steps
    f0 = [ev.create() for _ in range(n_ev)]
    f1 = [ev.create() for _ in range(n_ev)]
    b0 = [ev.create() for _ in range(n_ev)]
    b1 = [ev.create() for _ in range(n_ev)]
    bm = [ev.create() for _ in range(n_ev)]
    s0 = [ev.create() for _ in range(n_ev)]
    sm = [ev.create() for _ in range(n_ev)]
    s1 = [ev.create() for _ in range(n_ev)]

    def step(i=None):
        if i is not None:
            ev.record(s0[i], stream)
        fa.fwd(q, k, v, out=o, lse=lse, workspace=fws, events=None if i is None else (f0[i], f1[i]), **kw)
        if i is not None:
            ev.record(sm[i], stream)
        fa.bwd(q, k, v, o, do, lse, grads=grads, workspace=ws,
               events=None if i is None else (b0[i], b1[i], bm[i]), **kw)
        if i is not None:
            ev.record(s1[i], stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [ev.ms(f0[i], f1[i]) for i in range(steps)]
    bwd_ms = [ev.ms(b0[i], b1[i]) for i in range(steps)]
    kv_ms = [ev.ms(b0[i], bm[i]) for i in range(steps)]
    dq_ms = [ev.ms(bm[i], b1[i]) for i in range(steps)]
    step_ms = [ev.ms(s0[i], s1[i]) for i in range(steps)]
    fwd_pass_ms = [ev.ms(s0[i], sm[i]) for i in range(steps)]
    bwd_pass_ms = [ev.ms(sm[i], s1[i]) for i in range(steps)]
    for e in f0 + f1 + b0 + b1 + bm + s0 + sm + s1:
        ev.destroy(e)
    graph_ms = None
    if graph:
        # the same step captured once in a HIP graph and replayed: what the step
        # costs without per-launch host overhead (the library calls only launch
        # kernels, so they are capturable)
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        e1.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
        del g
    pairs = valid_pairs(x, w)
    return dict(x=x, pairs=pairs, wall_s=wall, fwd_ms=fwd_ms, bwd_main_ms=bwd_ms, kv_ms=kv_ms, dq_ms=dq_ms,
                step_ms=step_ms, fwd_pass_ms=fwd_pass_ms, bwd_pass_ms=bwd_pass_ms, graph_ms=graph_ms)


def standard_attention(q, k, v, do, scale, causal, p, events=None):
    """Standard attention as the pages describe it, for comparison: five
    separate operations per forward, each reading and writing a full N x N
    matrix in HBM (FlashAttention explainer, "kernel fusion"; Self-Attention
    tutorial, section 4):
        S = scale * Q K^T  (vendor GEMM)   ->  masked_fill(-inf) (causal)
        P = softmax(S)     ->  dropout(P)  ->  O = P V  (vendor GEMM)
    and the matching backward (dV = P_d^T dO, dP_d = dO V^T, dropout
    backward, softmax backward dS = P o (dP - rowsum(dP o P)), dQ = dS K,
    dK = dS^T Q, scale folded).  The N x N matrices enter every GEMM in their
    natural layout (dV and dK are computed transposed, as dO^T P_d and Q^T dS,
    with the small left operands made contiguous), so no N x N transpose is
    materialised and no GEMM operand is a transposed view.  Returns (O, dQ, dK, dV, dropout keep mask or None).
    events: (e0, e1, e2) hipEvent_t handles recorded before the forward,
    between the passes and after the backward on the current stream."""
    import torch
    hip = HipEvents() if events is not None else None
    stream = torch.cuda.current_stream(q.device).cuda_stream if hip else None
    N = q.shape[2]
    if hip:
        hip.record(events[0], stream)
    s = torch.matmul(q * scale, k.transpose(-1, -2).contiguous())
    if causal:
        s.masked_fill_(torch.ones(N, N, dtype=torch.bool, device=q.device).triu_(1), float("-inf"))
    pm = torch.softmax(s, dim=-1)
    del s
    keep = None
    if p > 0:
        pd, keep = torch.ops.aten.native_dropout(pm, p, True)
    else:
        pd = pm
    o = torch.matmul(pd, v)
    if hip:
        hip.record(events[1], stream)
    dv = torch.matmul(do.transpose(-1, -2).contiguous(), pd).transpose(-1, -2)
    del pd
    dp = torch.matmul(do, v.transpose(-1, -2).contiguous())
    if keep is not None:
        dp = torch.ops.aten.native_dropout_backward(dp, keep, 1.0 / (1.0 - p))
    ds = torch.ops.aten._softmax_backward_data(dp, pm, -1, pm.dtype)
    del dp, pm
    dq = torch.matmul(ds, k) * scale
    dk = torch.matmul(q.transpose(-1, -2).contiguous(), ds).transpose(-1, -2) * scale
    if hip:
        hip.record(events[2], stream)
    return o, dq, dk, dv, keep


def compare_standard(ev, steps, warmup, d=64, heads=16, tokens=16384, p=0.1):
    """This library against standard attention on the same inputs: causal,
    dropout p, bf16, H heads, B*N = tokens, N = 1K, 2K, 4K.  Times fwd and
    bwd by HIP events (medians), and the peak device memory each step adds on
    top of the resident Q, K, V, dO (torch's allocator statistics)."""
    import torch
    import io_aware_exact_tiled_amd as fa
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    for N in (1024, 2048, 4096):
        B = tokens // N
        g = torch.Generator(device="cpu").manual_seed(N)
        q, k, v, do = (torch.randn(B, heads, N, d, generator=g).to(torch.bfloat16).to(dev) for _ in range(4))
        scale = 1.0 / np.sqrt(d)
        res = {}
        for name in ("ours", "standard"):
            e = [[ev.create() for _ in range(3)] for _ in range(steps)]

            def step(i=None):
                if name == "ours":
                    if i is not None:
                        ev.record(e[i][0], stream)
                    o, lse = fa.fwd(q, k, v, causal=True, dropout_p=p, seed=1, scale=scale)
                    if i is not None:
                        ev.record(e[i][1], stream)
                    out = fa.bwd(q, k, v, o, do, lse, causal=True, dropout_p=p, seed=1, scale=scale)
                    if i is not None:
                        ev.record(e[i][2], stream)
                    return out
                return standard_attention(q, k, v, do, scale, True, p, None if i is None else e[i])

            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            base = torch.cuda.memory_allocated(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            for i in range(steps):
                out = step(i)
                del out
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated(dev) - base
            fm = float(np.median([ev.ms(x[0], x[1]) for x in e]))
            bm = float(np.median([ev.ms(x[1], x[2]) for x in e]))
            for x in e:
                for h in x:
                    ev.destroy(h)
            res[name] = (fm, bm, peak)
        (of, ob, om), (sf, sb, sm) = res["ours"], res["standard"]
        print(json.dumps({"compare": "standard attention (5 separate ops, vendor GEMMs)", "B": B, "H": heads, "N": N,
                          "d": d, "causal": True, "dropout_p": p, "dtype": "bf16",
                          "ours_fwd_ms": round(of, 4), "ours_bwd_ms": round(ob, 4),
                          "std_fwd_ms": round(sf, 4), "std_bwd_ms": round(sb, 4),
                          "speedup_fwd": round(sf / of, 2), "speedup_bwd": round(sb / ob, 2),
                          "speedup_step": round((sf + sb) / (of + ob), 2),
                          "ours_peak_extra_MiB": round(om / 2**20, 1), "std_peak_extra_MiB": round(sm / 2**20, 1),
                          "memory_ratio": round(sm / om, 1)}), flush=True)
        del q, k, v, do
        torch.cuda.empty_cache()


def kv_outer_bytes(B, H, N, d, e, causal, bc, G):
    """Bytes the key/value-outer kernel moves by its own loop (fwd_kvo_kernel):
    each of the G workgroups of a head loads every key tile its query blocks
    need (K and V, e bytes per element); for each key tile, each 32-row wave
    whose rows see it loads its Q rows (e), and -- after the first tile --
    its running O (fp32) and (m, l); it stores them back (fp32), or, on its
    last tile, O (e) and LSE.  Also the pages' model of the same order
    (FlashAttention explainer, step-by-step algorithm): K, V once; Q, O, l, m
    loaded and O, l, m stored at every (query block, key block) step,
    elements in the same sizes."""
    Tr, Tc = -(-N // 128), -(-N // bc)
    rd = wr = 0
    for g in range(min(G, Tr)):
        its = list(range(g, Tr, G))
        j_end = min(Tc, (min(its[-1] * 128 + 128, N) - 1) // bc + 1) if causal else Tc
        for j in range(j_end):
            rows = min(bc, N - j * bc)
            rd += 2 * rows * d * e
            for it in its:
                for w in range(4):
                    q0 = it * 128 + w * 32
                    if q0 >= N or (causal and j * bc > q0 + 31):
                        continue
                    r = min(32, N - q0)
                    rd += r * d * e + (r * (d * 4 + 8) if j > 0 else 0)
                    last = (q0 // bc) if causal else Tc - 1
                    wr += r * d * e + r * 4 if j == last else r * (d * 4 + 8)
    # the pages' order with blocks of 128 query rows and bc keys, skipping
    # blocks above the diagonal: K, V once, then per step Q, O (e), l, m
    steps = 0
    for j in range(Tc):
        for i in range(Tr):
            if not causal or j * bc <= min(i * 128 + 127, N - 1):
                steps += min(128, N - i * 128)
    model_rd = 2 * N * d * e + steps * (2 * d * e + 8)
    model_wr = N * (d * e + 8) + steps * (d * e + 8)
    BH = B * H
    return rd * BH, wr * BH, model_rd * BH, model_wr * BH


def io_ablation(ev, steps, warmup):
    """Key/value-outer forward against the query-outer one: causal bf16,
    B=1, H=16, d=128, N = 2K/4K/8K, key tiles of 64 and 128, 1 and 4
    workgroups per head.  Times both by HIP events and prints the bytes each
    order implies; the HBM bytes measured for them are in profiles/."""
    import torch
    import io_aware_exact_tiled_amd as fa
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    B, H, d = 1, 16, 128
    for N in (2048, 4096, 8192):
        g = torch.Generator(device="cpu").manual_seed(N)
        q, k, v = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev) for _ in range(3))
        e = [ev.create(), ev.create()]
        ws = torch.empty(fa.fwd_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8, device=dev)
        ts = []
        for i in range(warmup + steps):
            fa.fwd(q, k, v, causal=True, workspace=ws, events=e if i >= warmup else None)
            if i >= warmup:
                ts.append(ev.ms(e[0], e[1]))
        qo_ms = float(np.median(ts))
        qo_bytes = B * H * (4 * N * d * 2 + 4 * N)
        for bc in (64, 128):
            for G in (1, 4):
                ts = []
                for i in range(warmup + steps):
                    fa.fwd_kv_outer(q, k, v, causal=True, block_cols=bc, groups_per_head=G,
                                    events=e if i >= warmup else None)
                    if i >= warmup:
                        ts.append(ev.ms(e[0], e[1]))
                rd, wr, mrd, mwr = kv_outer_bytes(B, H, N, d, 2, True, bc, G)
                print(json.dumps({"io_ablation": "key/value-outer forward", "B": B, "H": H, "N": N, "d": d,
                                  "causal": True, "block_cols": bc, "groups_per_head": G,
                                  "kv_outer_ms": round(float(np.median(ts)), 4), "q_outer_ms": round(qo_ms, 4),
                                  "kv_outer_read_MiB": round(rd / 2**20, 1), "kv_outer_write_MiB": round(wr / 2**20, 1),
                                  "model_read_MiB": round(mrd / 2**20, 1), "model_write_MiB": round(mwr / 2**20, 1),
                                  "q_outer_min_MiB": round(qo_bytes / 2**20, 1)}), flush=True)
        for h in e:
            ev.destroy(h)
        del q, k, v, ws
        torch.cuda.empty_cache()


def decode_bytes(x, w):
    """Algorithmic HBM bytes of one decode call, split by kernel: the chunk
    kernel must read Q and the valid cache rows of K and V (sum over b of
    kv_lens[b] rows per K/V head); the merge kernel must write O and LSE.  The
    chunk partials it also writes and the merge reads back are not counted."""
    el = 2
    L = np.full(w.B, w.N) if x["key_lens"] is None else np.clip(x["key_lens"].numpy().astype(np.int64), 0, w.N)
    kv = int(L.sum()) * w.Hkv * w.d * el * 2
    q = w.B * w.H * w.decode_q * w.d * el
    o = q + w.B * w.H * w.decode_q * 4
    return kv + q, o


def time_decode(w, steps, warmup, ev):
    import torch
    import io_aware_exact_tiled_amd as fa
    import workloads as W

    x = W.make_inputs(w, with_do=False)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kl = None if x["key_lens"] is None else x["key_lens"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.decode_q, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(w.B, w.H, w.Hkv, w.decode_q, w.N, w.d), dtype=torch.uint8,
                     device=dev)
    evs = [[ev.create() for _ in range(3)] for _ in range(steps)]

    def step(i=None):
        fa.decode(q, k, v, kv_lens=kl, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws,
                  events=None if i is None else evs[i])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    split_ms = [ev.ms(e[0], e[1]) for e in evs]
    merge_ms = [ev.ms(e[1], e[2]) for e in evs]
    call_ms = [ev.ms(e[0], e[2]) for e in evs]
    for e in evs:
        for h in e:
            ev.destroy(h)
    return dict(x=x, wall_s=wall, split_ms=split_ms, merge_ms=merge_ms, call_ms=call_ms)


def decode_report(w, args, ev):
    """One JSON line for a decode workload: memory-bound, so HBM GB/s of
    algorithmic bytes against the 8 TB/s peak."""
    r = time_decode(w, args.steps, args.warmup, ev)
    rd, wr = decode_bytes(r["x"], w)
    med = lambda a: float(np.median(a))
    call_ms = med(r["call_ms"])
    split_avg = float(np.mean(r["split_ms"]))
    gbps = (rd + wr) / (call_ms * 1e-3) / 1e9
    achieved = rd / (split_avg * 1e-3) / 1e9
    out = {
        "metric": "decode attention HBM GB/s (algorithmic bytes: valid K/V cache rows, Q, O, LSE)",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(call_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q and K/V cache, uniform valid lengths)",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} Hkv={w.Hkv} Nq={w.decode_q} Nk={w.N} d={w.d} "
                               f"{w.dtype}{' causal' if w.causal else ''} kv_lens U{list(w.key_len_range)}",
                   "B": w.B, "H": w.H, "Hkv": w.Hkv, "Nq": w.decode_q, "Nk": w.N, "d": w.d,
                   "bytes_per_call": rd + wr},
        "split_ms": round(med(r["split_ms"]), 5), "merge_ms": round(med(r["merge_ms"]), 5),
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_GBPS, 4),
                     "traffic": measured_traffic("decode_split_kernel", w.name),
                     "avg_launch_ms": round(split_avg, 5), "bytes_per_launch": rd},
        "wall_s": round(r["wall_s"], 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, rd + wr)
    print(json.dumps(out), flush=True)


def host_info():
    """Threads the oracle's BLAS uses, the CPU model and the BLAS library."""
    import numpy
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [0]) or None
    except Exception:  # pragma: no cover
        pass
    if threads is None:
        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:  # pragma: no cover
        pass
    blas = "unknown"
    try:
        cfg = numpy.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{cfg.get('name')} {cfg.get('version', '')}".strip()
    except Exception:  # pragma: no cover
        pass
    return int(threads), cpu, blas


def cpu_baseline_decode(w, bytes_per_call):
    """The fp64 oracle (untuned) on the whole decode workload, scaled to the
    same algorithmic bytes as the GPU figure."""
    import oracle
    import workloads as W
    threads, cpu, blas = host_info()
    x = W.make_inputs(w, with_do=False)
    kl = None if x["key_lens"] is None else x["key_lens"].numpy()
    runs, t0 = 0, time.perf_counter()
    while runs == 0 or time.perf_counter() - t0 < 10.0:      # whole calls, at least 10 s in all
        oracle.decode_fwd(x["q"], x["k"], x["v"], w.scale, kv_lens=kl, causal=w.causal)
        runs += 1
    dt = (time.perf_counter() - t0) / runs
    return {"value": round(bytes_per_call / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu": cpu, "blas": blas, "seconds": round(dt * runs, 2),
            "sample": f"fp64 numpy oracle decode over the whole workload ({w.B} sequences x {w.H} heads), "
                      f"{runs} calls, rated by the same bf16 algorithmic bytes"}


def cpu_baseline(w, rows):
    """The fp64 oracle (untuned) on a bounded sample of the same workload: the
    leading `rows` query rows of every head.  For causal attention those rows
    see only keys < rows, so the sample is an exact sub-problem: its forward
    (O, LSE) and backward (dQ, dK, dV restricted to those rows' pairs)."""
    import oracle
    import workloads as W
    threads, cpu, blas = host_info()
    x = W.make_inputs(w)
    R = min(rows, w.N)
    sub = {n: x[n][:, :, :R] for n in ("q", "k", "v", "do")}
    kl = None if x["key_lens"] is None else x["key_lens"].numpy()
    t0 = time.perf_counter()
    oracle.attn_fwd(sub["q"], sub["k"], sub["v"], w.scale, causal=w.causal, key_lens=kl)
    t1 = time.perf_counter()
    oracle.attn_bwd(sub["q"], sub["k"], sub["v"], sub["do"], w.scale, causal=w.causal, key_lens=kl)
    t2 = time.perf_counter()
    dt = t2 - t0
    pairs = oracle.valid_pair_count(R, w.B, w.H, w.causal, kl, None)
    flops = 14.0 * w.d * pairs
    # the oracle is dense per row chunk (S over all keys, then masked), so its
    # cost grows as rows x keys: the full problem is (N / R)^2 times the sample
    full = dt * (w.N / R) ** 2
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu": cpu, "blas": blas, "seconds": round(dt, 2),
            "fwd_s": round(t1 - t0, 2), "bwd_s": round(t2 - t1, 2),
            "fwd_gflops": round(4.0 * w.d * pairs / (t1 - t0) / 1e9, 2),
            "bwd_gflops": round(10.0 * w.d * pairs / (t2 - t1) / 1e9, 2),
            "extrapolated_full_s": round(full, 1),
            "sample": f"fp64 numpy oracle fwd+bwd on the leading {R} rows and keys of all {w.B * w.H} heads"
                      + (f" (an exact sub-problem: causal rows < {R} see only keys < {R})" if w.causal else
                         " (the same attention at N = R)")
                      + f"; {pairs} valid pairs, 14*d FLOP each; extrapolated_full_s scales the measured "
                        f"time by (N/R)^2 (not measured)"}


# ---------------------------------------------------------------------------
# rocprofv3 harness.  `bench.py --profile DIR --workload W` runs one kernel
# trace and four counter passes of the workload as child processes (this
# process never touches the GPU), then reduces their CSV output into the
# summaries under profiles/: per-kernel launch times, HBM bytes scaled by a
# plain device copy of known size, the clock, the MFMA busy fraction and the
# LDS / VALU instruction mix (the figures the IO model of the method is
# checked with: FlashAttention summary, "complexity"; Self-Attention tutorial
# section 12.4, HBM accesses).  `--profile-report DIR` redoes only the
# reduction from an existing DIR.

PROFILES = os.path.join(ROOT, "profiles")
PROFILE_TAGS = {"long": "long_causal_d128", "gpt2": "gpt2_causal_d64", "bert": "bert_fp16_padding_dropout",
                "sparse": "block_sparse_d64", "gqa": "gqa_causal_d128", "decode": "decode",
                "long_noncausal": "noncausal_d128_n8192", "tiny": "tiny_d64"}
PMC_PASSES = (
    ("fetch", ("FETCH_SIZE",)),
    ("write", ("WRITE_SIZE",)),
    ("sq1", ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
             "SQ_INSTS_VALU_TRANS_F32", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")),
    ("sq2", ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
             "SQ_ACTIVE_INST_VALU", "SQ_WAIT_ANY", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_DATA_FIFO_FULL")),
)
PROFILE_KERNELS = ("fwd_kvo_kernel", "fwd_kernel", "bwd_kv_kernel", "bwd_dq_kernel", "bwd_pre_kernel",
                   "v16_convert_kernel", "v16_rescale_kernel", "decode_split_kernel", "decode_merge_kernel",
                   "copyBuffer")
CALIBRATE_MIB = 256
XCDS = 8
SIMDS = 1024


def short_kernel(name: str) -> str:
    for k in PROFILE_KERNELS:
        if k in name:
            return k
    return name[:40]


PROFILE_MODES = ("workload", "io-ablation", "compare-standard")


def profile_commands(workload: str, steps: int, rocprof: str = "rocprofv3", python: str = sys.executable,
                     mode: str = "workload"):
    """(pass name, argv) of the trace pass and the counter passes, each
    running this script: on the workload (mode "workload"); with
    --io-ablation (the key/value-outer forward against the query-outer one:
    a trace and the two byte passes); or with --compare-standard (a trace of
    this library against the separate-op baseline)."""
    me = os.path.abspath(__file__)
    trace = [rocprof, "--kernel-trace", "--stats", "-f", "csv", "-d", "{DIR}/trace", "-o", "run", "--", python, me]
    if mode == "io-ablation":
        cmds = [("trace", trace + ["--steps", "8", "--warmup", "2", "--no-cpu-baseline", "--io-ablation"])]
        for name, counters in PMC_PASSES[:2]:
            cmds.append((name, [rocprof, "--pmc", *counters, "--kernel-include-regex",
                                "fwd_kvo_kernel|fwd_kernel|copyBuffer", "-f", "csv", "-d", "{DIR}/" + name, "-o",
                                "run", "--", python, me, "--steps", "4", "--warmup", "1", "--no-cpu-baseline",
                                "--io-ablation", "--calibrate-copy", str(CALIBRATE_MIB)]))
        return cmds
    if mode == "compare-standard":
        return [("trace", trace + ["--steps", "6", "--warmup", "2", "--no-cpu-baseline", "--compare-standard"])]
    cmds = [("trace", trace + ["--workload", workload, "--steps", str(steps), "--no-cpu-baseline"])]
    regex = "|".join(PROFILE_KERNELS)
    for name, counters in PMC_PASSES:
        cmds.append((name, [rocprof, "--pmc", *counters, "--kernel-include-regex", regex, "-f", "csv", "-d",
                            "{DIR}/" + name, "-o", "run", "--", python, me, "--workload", workload, "--steps", "2",
                            "--warmup", "1", "--no-cpu-baseline", "--calibrate-copy", str(CALIBRATE_MIB)]))
    return cmds


def run_profile(out_dir: str, workload: str, steps: int, timeout_s: int = 240, mode: str = "workload") -> None:
    """Run the passes one after another as child processes (each in its own
    process group, killed whole if it outlives timeout_s); stop at the first
    failure."""
    import signal
    import subprocess
    os.makedirs(out_dir, exist_ok=True)
    env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
    for name, argv in profile_commands(workload, steps, mode=mode):
        argv = [a.replace("{DIR}", out_dir) for a in argv]
        print(f"[profile] {name}: {' '.join(argv)}", flush=True)
        with open(os.path.join(out_dir, name + ".out"), "w") as fo, \
                open(os.path.join(out_dir, name + ".log"), "w") as fe:
            p = subprocess.Popen(argv, stdout=fo, stderr=fe, cwd="/tmp", env=env, start_new_session=True)
            try:
                rc = p.wait(timeout=timeout_s)
            except subprocess.TimeoutExpired:
                os.killpg(p.pid, signal.SIGKILL)
                p.wait()
                raise SystemExit(f"[profile] {name}: killed after {timeout_s} s")
        ok = _last_json(os.path.join(out_dir, name + ".out")) is not None
        # rocprofv3 may end with a fault of its own after the program finished
        # and its results are complete: accept that when the JSON line is there
        if rc != 0 and not ok:
            raise SystemExit(f"[profile] {name}: exit status {rc}; see {name}.log")
        print(f"[profile] {name}: done (exit {rc})", flush=True)


def _last_json(path):
    try:
        with open(path) as fh:
            lines = [l for l in fh.read().splitlines() if l.startswith("{")]
    except OSError:
        return None
    return json.loads(lines[-1]) if lines else None


def _find_csv(d: str, suffix: str):
    for root, _, files in os.walk(d):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def read_counters(path: str) -> dict:
    """{kernel: {counter: value per dispatch}} from a rocprofv3 counter CSV:
    the mean over the kernel's dispatches (for the calibration copy, the
    largest copy dispatch: input uploads are copies too), plus _dur_ns, the
    mean dispatch duration."""
    import collections
    import csv
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        k = short_kernel(r["Kernel_Name"])
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        vals[k]["_dur_ns_" + r["Counter_Name"]].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    out = {}
    for k, d in vals.items():
        red = max if k == "copyBuffer" else (lambda v: sum(v) / len(v))
        out[k] = {c: red(v) for c, v in d.items() if not c.startswith("_dur_ns_")}
        durs = [x for c, v in d.items() if c.startswith("_dur_ns_") for x in v]
        out[k]["_dur_ns"] = sum(durs) / len(durs)
    return out


def derived_metrics(C: dict, copy_mib: float = CALIBRATE_MIB) -> dict:
    """Per kernel: HBM read/write bytes per dispatch (FETCH_SIZE, WRITE_SIZE in
    KiB, each scaled so the calibration copy reads and writes copy_mib MiB),
    clock (GRBM_GUI_ACTIVE per XCD over the dispatch time), MFMA busy (busy
    cycles over the cycles all 1024 SIMDs had), VALU and LDS instructions per
    MFMA, LDS bank conflicts over LDS-active cycles, and the two scales."""
    cp = C.get("copyBuffer", {})
    fscale = copy_mib * 1024 / cp["FETCH_SIZE"] if cp.get("FETCH_SIZE") else None
    wscale = copy_mib * 1024 / cp["WRITE_SIZE"] if cp.get("WRITE_SIZE") else None
    out = {"_fetch_scale": fscale, "_write_scale": wscale}
    nan = float("nan")
    for k, d in C.items():
        if k == "copyBuffer":
            continue
        m = {}
        if fscale and "FETCH_SIZE" in d:
            m["read_bytes"] = d["FETCH_SIZE"] * fscale * 1024
        if wscale and "WRITE_SIZE" in d:
            m["write_bytes"] = d["WRITE_SIZE"] * wscale * 1024
        gui = d.get("GRBM_GUI_ACTIVE", 0) / XCDS
        mf = d.get("SQ_INSTS_MFMA", 0)
        m["clock_ghz"] = gui / d["_dur_ns"] if gui and d.get("_dur_ns") else nan
        m["mfma_busy_pct"] = (100 * d["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / gui
                              if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in d else nan)
        m["valu_per_mfma"] = (d["SQ_INSTS_VALU"] - mf) / mf if mf and "SQ_INSTS_VALU" in d else nan
        m["lds_per_mfma"] = d["SQ_INSTS_LDS"] / mf if mf and "SQ_INSTS_LDS" in d else nan
        m["lds_conflict_pct"] = (100 * d["SQ_LDS_BANK_CONFLICT"] / d["SQ_LDS_IDX_ACTIVE"]
                                 if d.get("SQ_LDS_IDX_ACTIVE") else nan)
        out[k] = m
    return out


def _dispatch_counters(path: str, kernel: str, counter: str) -> list:
    """The values of one counter for one kernel's dispatches, in dispatch order."""
    import csv
    rows = [r for r in csv.DictReader(open(path))
            if short_kernel(r["Kernel_Name"]) == kernel and r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [float(r["Counter_Value"]) for r in rows]


def io_ablation_report(out_dir: str, profiles_dir: str = PROFILES) -> str:
    """profiles_dir/kv_outer_io_ablation.md from an io-ablation profile: per
    configuration the times and byte models bench.py printed in the trace
    pass, and the HBM bytes the counter passes measured for fwd_kvo_kernel
    (copy-calibrated, the mean over the configuration's dispatches; the
    configurations run in the order bench.py prints them)."""
    import collections
    lines = []
    with open(os.path.join(out_dir, "trace.out")) as fh:
        for l in fh:
            if l.startswith("{") and '"io_ablation"' in l:
                lines.append(json.loads(l))
    f_csv = _find_csv(os.path.join(out_dir, "fetch"), "counter_collection.csv")
    w_csv = _find_csv(os.path.join(out_dir, "write"), "counter_collection.csv")
    C = {}
    for f in (f_csv, w_csv):
        for k, d in read_counters(f).items():
            C.setdefault(k, {}).update({c: v for c, v in d.items() if c != "_dur_ns"})
    M = derived_metrics(C)
    fs, wsc = M["_fetch_scale"], M["_write_scale"]
    fetch = _dispatch_counters(f_csv, "fwd_kvo_kernel", "FETCH_SIZE")
    write = _dispatch_counters(w_csv, "fwd_kvo_kernel", "WRITE_SIZE")
    n = len(lines)
    per = len(fetch) // n if n else 0
    assert n and per and len(fetch) == per * n and len(write) == per * n, (n, len(fetch), len(write))
    cmds = {k: " ".join(a).replace(sys.executable, "python").replace(os.path.abspath(__file__), "bench.py")
            .replace("{DIR}", "<dir>") for k, a in profile_commands("long", 8, mode="io-ablation")}
    t = ["# IO ablation: key/value-outer forward against the query-outer one", "",
         "Causal, bf16, B=1, H=16, d=128.  The key/value-outer kernel (fwd_kvo_kernel) keeps K_j, V_j in LDS and "
         "moves the running O (fp32), m, l of every query block through device memory at every key tile, as the "
         "explainer's step-by-step algorithm does; the query-outer fwd_kernel keeps them in registers.", "",
         "Made by `python bench.py --profile <dir> --profile-mode io-ablation`, whose passes are:", ""]
    t += ["    " + cmds[k] for k in ("trace", "fetch", "write")]
    t += ["", "Byte counters scaled by the %d MiB device copy of the same run: FETCH_SIZE x %.3f KiB, WRITE_SIZE x "
          "%.3f KiB.  Kernel bytes = what fwd_kvo_kernel's loop loads and stores (bench.py kv_outer_bytes); model = "
          "the pages' order with 128-row query blocks (pinned to the oracle's counts); measured = mean over the "
          "run's %d dispatches per configuration." % (CALIBRATE_MIB, fs, wsc, per), "",
          "| N | key tile | groups / head | kv-outer ms | q-outer ms | kernel read / write MiB | model read / write MiB "
          "| measured read / write MiB | measured / kernel |", "|---|---|---|---|---|---|---|---|---|"]
    for i, d in enumerate(lines):
        rd = sum(fetch[i * per:(i + 1) * per]) / per * fs / 1024
        wr = sum(write[i * per:(i + 1) * per]) / per * wsc / 1024
        own = d["kv_outer_read_MiB"] + d["kv_outer_write_MiB"]
        t.append("| %d | %d | %d | %.4f | %.4f | %.1f / %.1f | %.1f / %.1f | %.1f / %.1f | %.2f |" % (
            d["N"], d["block_cols"], d["groups_per_head"], d["kv_outer_ms"], d["q_outer_ms"],
            d["kv_outer_read_MiB"], d["kv_outer_write_MiB"], d["model_read_MiB"], d["model_write_MiB"], rd, wr,
            (rd + wr) / own))
    # the query-outer forward: per N, the same number of dispatches as each
    # configuration, the last fwd_kernel dispatches of the run (the timed
    # workload bench.py runs first comes before them)
    Ns = sorted({d["N"] for d in lines})
    qf = _dispatch_counters(f_csv, "fwd_kernel", "FETCH_SIZE")
    qw = _dispatch_counters(w_csv, "fwd_kernel", "WRITE_SIZE")
    if len(qf) >= per * len(Ns) and len(qw) >= per * len(Ns):
        qf, qw = qf[len(qf) - per * len(Ns):], qw[len(qw) - per * len(Ns):]
        t += ["", "The query-outer fwd_kernel on the same inputs (mean over its %d dispatches per N):" % per, "",
              "| N | q-outer ms | measured read / write MiB | Q, K, V in and O, LSE out, MiB |", "|---|---|---|---|"]
        for i, N in enumerate(Ns):
            d = next(x for x in lines if x["N"] == N)
            rd = sum(qf[i * per:(i + 1) * per]) / per * fs / 1024
            wr = sum(qw[i * per:(i + 1) * per]) / per * wsc / 1024
            least = d.get("q_outer_min_MiB")
            t.append("| %d | %.4f | %.1f / %.1f | %s |" % (N, d["q_outer_ms"], rd, wr,
                                                          "-" if least is None else "%.1f" % least))
    path = os.path.join(profiles_dir, "kv_outer_io_ablation.md")
    open(path, "w").write("\n".join(t) + "\n")
    return path


def compare_standard_report(out_dir: str, profiles_dir: str = PROFILES, top: int = 16) -> str:
    """profiles_dir/standard_attention_compare_kernel_trace.md from a
    compare-standard profile: the kernels with the most GPU time over the run
    and the comparison lines bench.py printed."""
    import csv
    rows = list(csv.DictReader(open(_find_csv(os.path.join(out_dir, "trace"), "kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    comp = []
    with open(os.path.join(out_dir, "trace.out")) as fh:
        for l in fh:
            if l.startswith("{") and '"compare"' in l:
                comp.append(json.loads(l))
    cmd = " ".join(profile_commands("long", 6, mode="compare-standard")[0][1]).replace(sys.executable, "python") \
        .replace(os.path.abspath(__file__), "bench.py").replace("{DIR}", "<dir>")
    t = ["# Kernel trace: this library against standard attention (five separate ops on vendor GEMMs)", "",
         "Causal, dropout 0.1, bf16, H=16, d=64, B*N = 16384 tokens at N = 1024, 2048, 4096 (plus the default long "
         "workload that bench.py times first).", "",
         "Made by `python bench.py --profile <dir> --profile-mode compare-standard`, whose trace pass is:", "",
         "    " + cmd, "", "Top kernels by total GPU time over the whole run:", "",
         "| kernel | calls | avg us | total ms | % of GPU time |", "|---|---|---|---|---|"]
    for r in rows[:top]:
        name = short_kernel(r["Name"]) if short_kernel(r["Name"]) in PROFILE_KERNELS else r["Name"][:90]
        t.append("| %s | %s | %.1f | %.2f | %.2f |" % (name, r["Calls"], float(r["AverageNs"]) / 1e3,
                                                     float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    t += ["", "bench.py's comparison lines from the same run (times by HIP events, medians; extra memory = the "
          "peak a step adds over the resident inputs):", "",
          "| N | B | this library fwd / bwd ms | standard fwd / bwd ms | speed-up fwd / bwd / step | extra MiB "
          "(ratio) |", "|---|---|---|---|---|---|"]
    for d in comp:
        t.append("| %d | %d | %.3f / %.3f | %.3f / %.3f | %.1f / %.1f / %.1f | %.0f vs %.0f (%.0fx) |" % (
            d["N"], d["B"], d["ours_fwd_ms"], d["ours_bwd_ms"], d["std_fwd_ms"], d["std_bwd_ms"], d["speedup_fwd"],
            d["speedup_bwd"], d["speedup_step"], d["ours_peak_extra_MiB"], d["std_peak_extra_MiB"],
            d["memory_ratio"]))
    path = os.path.join(profiles_dir, "standard_attention_compare_kernel_trace.md")
    open(path, "w").write("\n".join(t) + "\n")
    return path


def profile_report(out_dir: str, workload: str, tag=None, profiles_dir: str = PROFILES) -> dict:
    """Reduce the passes under out_dir into profiles_dir/<tag>_kernel_trace.md,
    profiles_dir/<tag>_counters.md and the workload's entry of
    profiles_dir/hbm_traffic.json (bytes per launch of each kernel, with the
    SHA-256 of its sources, so that bench.py reports them only while the
    kernel is unchanged).  Returns the derived metrics."""
    import csv
    tag = tag or PROFILE_TAGS.get(workload, workload)
    os.makedirs(profiles_dir, exist_ok=True)
    cmds = {n: " ".join(a).replace(sys.executable, "python").replace(os.path.abspath(__file__), "bench.py")
            for n, a in profile_commands(workload, 20)}
    written = []
    stats = _find_csv(os.path.join(out_dir, "trace"), "kernel_stats.csv")
    if stats:
        rows = list(csv.DictReader(open(stats)))
        bj = _last_json(os.path.join(out_dir, "trace.out"))
        t = [f"# Kernel trace: workload `{workload}`", "",
             "Made by `python bench.py --profile <dir> --workload " + workload + "` (run from the repository "
             "root; the passes run in /tmp with TMPDIR=/tmp), whose trace pass is:", "",
             "    " + cmds["trace"].replace("{DIR}", "<dir>"), "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
        for r in rows:
            t.append("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
                short_kernel(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        if bj:
            rf = bj.get("roofline", {})
            avg = {short_kernel(r["Name"]): float(r["AverageNs"]) / 1e6 for r in rows}
            t += ["", "bench.py's JSON line from the same run: value %s %s, %s ms per step." % (
                bj.get("value"), bj.get("unit"), bj.get("ms_per_step"))]
            if rf.get("kernel"):
                t.append("Dominant kernel %s: %.4f ms average launch by HIP events, trace average %.4f ms; "
                         "%s %s = %.1f %% of %s %s." % (
                             rf["kernel"], rf.get("avg_launch_ms", float("nan")),
                             avg.get(rf["kernel"], float("nan")), rf.get("achieved"), rf.get("unit"),
                             100 * rf.get("frac", float("nan")), rf.get("peak"), rf.get("unit")))
            if "fwd_ms" in bj:
                t.append("Event medians: forward pass %s ms, backward pass %s ms (dK/dV kernel %s ms, dQ kernel "
                         "%s ms)." % (bj["fwd_ms"], bj["bwd_ms"], bj.get("bwd_kv_ms"), bj.get("bwd_dq_ms")))
        path = os.path.join(profiles_dir, f"{tag}_kernel_trace.md")
        open(path, "w").write("\n".join(t) + "\n")
        written.append(path)
    C = {}
    for name, _ in PMC_PASSES:
        f = _find_csv(os.path.join(out_dir, name), "counter_collection.csv")
        if f:
            for k, d in read_counters(f).items():
                dur = d.pop("_dur_ns")
                C.setdefault(k, {}).update(d)
                if name == "sq1" or "_dur_ns" not in C[k]:
                    C[k]["_dur_ns"] = dur   # the clock uses the pass that read GRBM_GUI_ACTIVE
    if not C:
        return {}
    M = derived_metrics(C)
    ks = [k for k in PROFILE_KERNELS if k in C]
    names = sorted({c for k in ks for c in C[k] if not c.startswith("_")})
    o = [f"# Hardware counters: workload `{workload}`", "",
         "Made by `python bench.py --profile <dir> --workload " + workload + "`: one rocprofv3 run per counter "
         "group (each pass also runs a plain device copy of %d MiB, the calibration dispatch):" % CALIBRATE_MIB, ""]
    o += ["    " + cmds[n].replace("{DIR}", "<dir>") for n, _ in PMC_PASSES]
    o += ["", "Values per dispatch (mean over the run's dispatches of the kernel; for the copy, the "
          "calibration dispatch).", "", "| counter | " + " | ".join(ks) + " |", "|---|" + "---|" * len(ks)]
    for c in names:
        o.append(f"| {c} | " + " | ".join("%.4g" % C[k].get(c, float("nan")) for k in ks) + " |")
    fs, wsc = M["_fetch_scale"], M["_write_scale"]
    if fs and wsc:
        o += ["", "Byte calibration: the %d MiB copy reads FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB, so "
              "HBM bytes = FETCH_SIZE x %.3f KiB and WRITE_SIZE x %.3f KiB." % (
                  CALIBRATE_MIB, C["copyBuffer"]["FETCH_SIZE"], C["copyBuffer"]["WRITE_SIZE"], fs, wsc)]
    o += ["", "| kernel | HBM read MiB | HBM write MiB | clock GHz | MFMA busy % | MFMA % of 2.4 GHz peak | "
          "VALU instr / MFMA | LDS instr / MFMA | LDS bank conflicts % |", "|---|---|---|---|---|---|---|---|---|"]
    for k in ks:
        if k == "copyBuffer":
            continue
        m = M[k]
        o.append("| %s | %.1f | %.1f | %.2f | %.1f | %.1f | %.2f | %.2f | %.1f |" % (
            k, m.get("read_bytes", float("nan")) / 2**20, m.get("write_bytes", float("nan")) / 2**20,
            m["clock_ghz"], m["mfma_busy_pct"], m["mfma_busy_pct"] * m["clock_ghz"] / 2.4, m["valu_per_mfma"],
            m["lds_per_mfma"], m["lds_conflict_pct"]))
    o += ["", "clock = GRBM_GUI_ACTIVE / %d XCDs / dispatch time; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs "
          "x GRBM_GUI_ACTIVE / %d XCDs).  The 2.5 PFLOP/s dense bf16 peak assumes 2.4 GHz, so the fraction of that "
          "peak the matrix cores can reach at the measured clock is busy x clock / 2.4 GHz.  The clock is only "
          "meaningful for dispatches much longer than the profiler's per-dispatch overhead (tens of microseconds): "
          "for short ones GRBM_GUI_ACTIVE also counts cycles outside the dispatch." % (XCDS, SIMDS, XCDS)]
    path = os.path.join(profiles_dir, f"{tag}_counters.md")
    open(path, "w").write("\n".join(o) + "\n")
    written.append(path)
    traffic = {k: {"fetch_bytes": int(M[k]["read_bytes"]), "write_bytes": int(M[k]["write_bytes"]),
                   "sources_sha256": kernel_sources_sha256(k), "counters": os.path.basename(path)}
               for k in ks if k in KERNEL_SOURCES and "read_bytes" in M[k] and "write_bytes" in M[k]}
    if traffic:
        tf = os.path.join(profiles_dir, "hbm_traffic.json")
        try:
            old = json.load(open(tf))
            old.setdefault("workloads", {})
        except (OSError, ValueError):
            old = {"workloads": {}}
        old.pop("kernels", None)
        old["note"] = ("HBM bytes per launch by workload and kernel (FETCH_SIZE and WRITE_SIZE scaled by a plain "
                       "%d MiB device copy), made by bench.py --profile; sources_sha256 covers the kernel's source "
                       "file and the two shared headers when the counters were taken." % CALIBRATE_MIB)
        old["workloads"][workload] = traffic
        json.dump(old, open(tf, "w"), indent=1, sort_keys=True)
        written.append(tf)
    for p in written:
        print(f"[profile] wrote {os.path.relpath(p, ROOT) if p.startswith(ROOT) else p}", flush=True)
    return M


def main():
    args = parse()
    if args.profile or args.profile_report:
        # the passes run as child processes: this one never touches the GPU
        out = os.path.abspath(args.profile or args.profile_report)
        if args.profile:
            run_profile(out, args.workload, args.steps, mode=args.profile_mode)
        if args.profile_mode == "io-ablation":
            print("[profile] wrote", os.path.relpath(io_ablation_report(out), ROOT), flush=True)
        elif args.profile_mode == "compare-standard":
            print("[profile] wrote", os.path.relpath(compare_standard_report(out), ROOT), flush=True)
        else:
            profile_report(out, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each (b, h) head is "
              "independent, so a multi-GPU run would shard the heads with no communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ev = HipEvents()
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = W.WORKLOADS[args.workload]
    if w.decode_q is not None:
        decode_report(w, args, ev)
        return
    r = time_workload(w, args.steps, args.warmup, ev, graph=args.graph)
    fwd_flop = 4.0 * w.d * r["pairs"]
    bwd_flop = 10.0 * w.d * r["pairs"]
    med = lambda a: float(np.median(a))
    step_ms = med(r["step_ms"])
    fwd_ms, bwd_ms = med(r["fwd_pass_ms"]), med(r["bwd_pass_ms"])
    peak = PEAK_TFLOPS[w.dtype]
    total_tflops = (fwd_flop + bwd_flop) / (step_ms * 1e-3) / 1e12
    fwd_tf = fwd_flop / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_flop / (bwd_ms * 1e-3) / 1e12
    roofline, kern = dominant_roofline(w, r["pairs"], {"fwd_kernel": float(np.mean(r["fwd_ms"])),
                                                       "bwd_kv_kernel": float(np.mean(r["kv_ms"])),
                                                       "bwd_dq_kernel": float(np.mean(r["dq_ms"]))})
    out = {
        "metric": "attention fwd/bwd TFLOP/s (bf16, d=64/128, N 1K-16K), % of MFMA peak",
        "value": round(total_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q, K, V, dO)",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H}{f' Hkv={w.Hkv}' if w.Hkv != w.H else ''} N={w.N} "
                               f"d={w.d} {w.dtype}{' causal' if w.causal else ''}", "B": w.B, "H": w.H,
                   "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": w.causal, "valid_pairs": r["pairs"]},
        "pct_peak": round(100 * total_tflops / peak, 2),
        "fwd_tflops": round(fwd_tf, 2), "fwd_pct_peak": round(100 * fwd_tf / peak, 2), "fwd_ms": round(fwd_ms, 4),
        "bwd_tflops": round(bwd_tf, 2), "bwd_pct_peak": round(100 * bwd_tf / peak, 2), "bwd_ms": round(bwd_ms, 4),
        "fwd_kernel_ms": round(med(r["fwd_ms"]), 4), "bwd_main_ms": round(med(r["bwd_main_ms"]), 4),
        "bwd_kv_ms": round(med(r["kv_ms"]), 4), "bwd_dq_ms": round(med(r["dq_ms"]), 4),
        "fwd_hbm_gbps": round(kern["fwd_kernel"][2] / (fwd_ms * 1e-3) / 1e9, 1),
        "roofline": roofline,
        "wall_s": round(r["wall_s"], 3),
    }
    if r["graph_ms"] is not None:
        out["graph_ms_per_step"] = round(r["graph_ms"], 4)
        out["graph_tflops"] = round((fwd_flop + bwd_flop) / (r["graph_ms"] * 1e-3) / 1e12, 2)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)
    if args.compare_standard:
        compare_standard(ev, max(5, args.steps // 2), 2)
    if args.io_ablation:
        io_ablation(ev, max(2, args.steps // 4), 1)
    if args.power > 0:
        prow = power_run(w, args.power)
        if args.power_md:
            write_power_md(args.power_md, prow, out)
    if args.sweep:
        rows = []
        for d in (64, 128):
            for causal in (False, True):
                for N in (1024, 2048, 4096, 8192, 16384):
                    ws = W.Workload(f"sweep", 16384 // N, 16, N, d, "bf16", seed=7, causal=causal)
                    rr = time_workload(ws, max(3, args.steps // 2), 2, ev)
                    ff, bf = 4.0 * d * rr["pairs"], 10.0 * d * rr["pairs"]
                    fm, bm = med(rr["fwd_pass_ms"]), med(rr["bwd_pass_ms"])
                    rows.append({"sweep": True, "B": ws.B, "H": 16, "N": N, "d": d, "causal": causal,
                                 "fwd_ms": round(fm, 4), "bwd_ms": round(bm, 4),
                                 "fwd_tflops": round(ff / fm / 1e9, 1), "bwd_tflops": round(bf / bm / 1e9, 1),
                                 "fwd_pct": round(100 * ff / fm / 1e9 / peak, 2),
                                 "bwd_pct": round(100 * bf / bm / 1e9 / peak, 2)})
                    print(json.dumps(rows[-1]), flush=True)
        if args.sweep_md:
            write_sweep_md(args.sweep_md, rows, out)


def parse_amd_smi(text: str) -> tuple:
    """(socket power W, GFX_0 clock MHz) from `amd-smi metric -p -c` text, or
    None for a value it does not show."""
    power = clock = None
    in_gfx0 = False
    for raw in text.splitlines():
        l = raw.strip()
        if l.startswith("SOCKET_POWER:") and power is None:
            try:
                power = float(l.split(":", 1)[1].split()[0])
            except (ValueError, IndexError):
                pass
        elif l.startswith("GFX_"):
            in_gfx0 = l.rstrip(":") == "GFX_0"
        elif in_gfx0 and l.startswith("CLK:") and clock is None:
            try:
                clock = float(l.split(":", 1)[1].split()[0])
            except (ValueError, IndexError):
                pass
    return power, clock


def power_run(w, seconds: float) -> list:
    """Each pass of workload w back to back for `seconds` while a thread runs
    `amd-smi metric -p -c` every 0.5 s; medians over the samples after the
    first second (the clock ramps up first)."""
    import statistics
    import subprocess
    import threading
    import torch
    import io_aware_exact_tiled_amd as fa
    import workloads as W

    x = W.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    kw = dict(causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed, rng_offset=w.rng_offset,
              key_lens=None if x["key_lens"] is None else x["key_lens"].to(dev),
              block_mask=None if x["block_mask"] is None else x["block_mask"].to(dev), scale=w.scale)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(1, fa.fwd_workspace_bytes(w.B, w.Hkv, w.N, w.d, q.dtype)), dtype=torch.uint8, device=dev)
    fa.fwd(q, k, v, out=o, lse=lse, workspace=fws, **kw)
    passes = {"forward": lambda: fa.fwd(q, k, v, out=o, lse=lse, workspace=fws, **kw),
              "backward": lambda: fa.bwd(q, k, v, o, do, lse, grads=grads, workspace=ws, **kw)}
    out = []
    for name, run in passes.items():
        samples, stop = [], threading.Event()

        def sample():
            t0 = time.perf_counter()
            while not stop.is_set():
                try:
                    r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=10)
                    samples.append((time.perf_counter() - t0,) + parse_amd_smi(r.stdout))
                except (OSError, subprocess.SubprocessError):
                    return
                stop.wait(0.5)

        torch.cuda.synchronize()
        th = threading.Thread(target=sample)
        t0 = time.perf_counter()
        th.start()
        n = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                run()
            torch.cuda.synchronize()
            n += 10
        stop.set()
        th.join()
        late = [s for s in samples if s[0] >= 1.0 and s[1] is not None and s[2] is not None]
        out.append({"power": name, "calls": n, "seconds": round(time.perf_counter() - t0, 2),
                    "samples": len(late),
                    "socket_power_w": statistics.median(s[1] for s in late) if late else None,
                    "gfx_clock_mhz": statistics.median(s[2] for s in late) if late else None})
        print(json.dumps(out[-1]), flush=True)
    return out


def write_power_md(path: str, rows: list, line: dict) -> None:
    """The power lines as a markdown table, with the command and the main line
    of the same run."""
    t = ["# Socket power and GFX clock while each pass runs back to back", "",
         "Workload %s.  amd-smi (`metric -p -c`) sampled every 0.5 s; medians over the samples after the "
         "first second.  Made by:" % line["config"]["workload"], "",
         "    python bench.py " + " ".join(sys.argv[1:]), "",
         "The same run's main line: %.2f TFLOP/s per step, forward %.2f %%, backward %.2f %% of peak." % (
             line["value"], line["fwd_pct_peak"], line["bwd_pct_peak"]), "",
         "| pass | calls | seconds | samples | socket power W | GFX clock MHz |", "|---|---|---|---|---|---|"]
    for r in rows:
        t.append("| %s | %d | %.2f | %d | %s | %s |" % (
            r["power"], r["calls"], r["seconds"], r["samples"],
            "-" if r["socket_power_w"] is None else "%.0f" % r["socket_power_w"],
            "-" if r["gfx_clock_mhz"] is None else "%.0f" % r["gfx_clock_mhz"]))
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    open(path, "w").write("\n".join(t) + "\n")
    print("[power] wrote", path, flush=True)


def write_sweep_md(path: str, rows: list, line: dict) -> None:
    """The sweep's JSON lines as a markdown table, with the command and the
    main line of the same run."""
    argv = [a for a in sys.argv[1:]]
    t = ["# Sweep: fwd / bwd TFLOP/s and % of the 2.5 PFLOP/s bf16 peak", "",
         "B*N = 16384 tokens, H = 16, bf16, seeded Gaussian inputs (std 1); whole passes (pre-passes included), "
         "HIP events, medians.  Made by:", "", "    python bench.py " + " ".join(argv), "",
         "The same run's main line (workload %s): %.2f TFLOP/s per step, forward %.2f %%, backward %.2f %% of "
         "peak." % (line["config"]["workload"].split(":")[0], line["value"], line["fwd_pct_peak"],
                    line["bwd_pct_peak"]), "",
         "| N | B | d | causal | fwd ms | bwd ms | fwd TFLOP/s (%) | bwd TFLOP/s (%) |",
         "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        t.append("| %d | %d | %d | %s | %.4f | %.4f | %.1f (%.1f) | %.1f (%.1f) |" % (
            r["N"], r["B"], r["d"], "yes" if r["causal"] else "no", r["fwd_ms"], r["bwd_ms"], r["fwd_tflops"],
            r["fwd_pct"], r["bwd_tflops"], r["bwd_pct"]))
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    open(path, "w").write("\n".join(t) + "\n")
    print("[sweep] wrote", path, flush=True)


if __name__ == "__main__":
    main()
