"""Tiled exact attention (FlashAttention forward and backward) for MI355X.

Thin binding over the C ABI in include/fa.h: it checks tensor placement and
layout, allocates outputs with torch on the inputs' device and passes raw
device pointers plus torch's current HIP stream.  Every step of the
computation runs in the HIP kernels of libfa.so; when the library is missing
the calls raise.

    o, lse = fwd(q, k, v, causal=True)
    dq, dk, dv = bwd(q, k, v, o, do, lse, causal=True)
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib
from ._lib import FaOpts, check

__all__ = ["fwd", "bwd", "decode", "dropout_keep_mask", "tile_shape", "fwd_workspace_bytes",
           "bwd_workspace_bytes", "decode_workspace_bytes", "abi_version"]

_DT = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16, torch.bfloat16: _lib.FA_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _check_qkv(q, k, v, *more):
    """q (and dO, O): [B, H, N, d]; k, v: [B, Hkv, N, d] with Hkv dividing H
    (grouped-query attention; Hkv == H is plain multi-head).  Returns Hkv."""
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in (q, k, v) + more:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v (and dO) must share dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
    for t in more:
        if t.shape != q.shape:
            raise ValueError("dO must have q's shape")
    B, H, N, d = q.shape
    if k.shape != v.shape or k.dim() != 4 or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("k, v must be [B, Hkv, N, d] with q's B, N, d")
    hkv = k.shape[1]
    if hkv < 1 or H % hkv:
        raise ValueError("the number of K/V heads must divide the number of query heads")
    return hkv


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _opts(B, H, N, d, pass_, key_lens, rng_offset, o_fp32, record_tiles, reverse_kv, device, dtype_code,
          events=None, kv_heads=0, causal=False):
    opts = FaOpts()
    opts.kv_heads = 0 if kv_heads == H else int(kv_heads)
    if events is not None:
        opts.main_begin, opts.main_end = events[0], events[1]
        if len(events) > 2:
            opts.main_mid = events[2]
    opts.struct_size = ctypes.sizeof(FaOpts)
    opts.o_fp32 = 1 if o_fp32 else 0
    keep = []
    if key_lens is not None:
        kl = key_lens.to(device=device, dtype=torch.int32).contiguous()
        keep.append(kl)
        opts.key_lens = kl.data_ptr()
    opts.rng_offset = int(rng_offset)
    tiles = None
    if record_tiles:
        maps = []
        for p in ((0,) if pass_ == 0 else (1, 2)):
            br, bc = tile_shape(d, dtype_code, p, N, causal)
            maps.append(torch.full((B, H, -(-N // br), -(-N // bc)), 7, dtype=torch.uint8, device=device))
        opts.tile_visits = maps[0].data_ptr()
        if len(maps) > 1:
            opts.tile_visits2 = maps[1].data_ptr()
        tiles = maps[0] if pass_ == 0 else tuple(maps)
        opts.flags |= _lib.FA_FLAG_RECORD_TILES
    if reverse_kv:
        opts.flags |= _lib.FA_FLAG_REVERSE_KV
    return opts, keep, tiles


def _mask_ptr(block_mask, device, N):
    if block_mask is None:
        return None, None
    T = -(-N // 128)
    bm = block_mask.to(device=device, dtype=torch.uint8).contiguous()
    if bm.shape != (T, T):
        raise ValueError(f"block_mask must be [{T}, {T}]")
    return bm, bm.data_ptr()


def fwd_workspace_bytes(B, Hkv, N, d, dtype: torch.dtype) -> int:
    """Forward workspace bytes; Hkv = the K/V heads (H without grouped-query
    attention)."""
    return int(_lib.lib().fa_fwd_workspace_bytes(B, Hkv, N, d, _DT[dtype]))


def fwd(q, k, v, *, causal=False, dropout_p=0.0, seed=0, rng_offset=0, key_lens=None, block_mask=None,
        scale: Optional[float] = None, o_fp32=False, record_tiles=False, reverse_kv=False,
        out=None, lse=None, workspace=None, events=None):
    """Forward pass.  Returns (O, LSE) or (O, LSE, tile_visits) when
    record_tiles is set.  `events` = (hipEvent_t, hipEvent_t) raw handles
    recorded around the kernel (profiling).  O is fp32 when o_fp32, else q's dtype; LSE is fp32
    [B, H, N].  `workspace`: a uint8 device tensor of fwd_workspace_bytes
    (allocated here when None and needed)."""
    hkv = _check_qkv(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _dtype_code(q)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.float32 if o_fp32 else q.dtype,
                                                device=q.device)
    l = lse if lse is not None else torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    opts, keep, tiles = _opts(B, H, N, d, 0, key_lens, rng_offset, o_fp32, record_tiles, reverse_kv,
                              q.device, dt, events, hkv, causal)
    bm, bmp = _mask_ptr(block_mask, q.device, N)
    need = fwd_workspace_bytes(B, hkv, N, d, q.dtype)
    ws = workspace
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = _lib.lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                             B, H, N, d, dt, scale, 1 if causal else 0, float(dropout_p), int(seed),
                             bmp, ctypes.byref(opts), ws.data_ptr() if ws is not None else None,
                             ws.numel() if ws is not None else 0, _stream(q.device))
    check(code, "fa_fwd")
    del keep, bm, ws
    return (o, l, tiles) if record_tiles else (o, l)


def bwd_workspace_bytes(B, H, N, d) -> int:
    return int(_lib.lib().fa_bwd_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, do, lse, *, causal=False, dropout_p=0.0, seed=0, rng_offset=0, key_lens=None,
        block_mask=None, scale: Optional[float] = None, record_tiles=False, workspace=None, grads=None,
        events=None, no_alloc=False):
    """Backward pass.  Returns (dQ, dK, dV) in q's dtype (dK, dV with k's
    shape: summed over the query heads that share a K/V head), plus, when
    record_tiles is set, the (dK/dV kernel, dQ kernel) tile-visit maps.
    O may be fp32 (if the forward wrote it so) or q's dtype.  no_alloc: call
    fa_bwd_noalloc (the library's static scratch instead of a workspace;
    B*H*N up to FA_BWD_SCRATCH_BYTES / 4)."""
    hkv = _check_qkv(q, k, v, do)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dt = _dtype_code(q)
    if o.shape != q.shape or not o.is_contiguous() or o.dtype not in (q.dtype, torch.float32):
        raise ValueError("O must be contiguous [B, H, N, d] of q's dtype or fp32")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("LSE must be contiguous fp32 [B, H, N]")
    o_fp32 = o.dtype == torch.float32 and q.dtype != torch.float32
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
    opts, keep, tiles = _opts(B, H, N, d, 1, key_lens, rng_offset, o_fp32, record_tiles, False, q.device, dt,
                              events, hkv, causal)
    bm, bmp = _mask_ptr(block_mask, q.device, N)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), B, H, N, d, dt, scale, 1 if causal else 0, float(dropout_p), int(seed),
            bmp, ctypes.byref(opts))
    if no_alloc:
        check(_lib.lib().fa_bwd_noalloc(*ptrs, _stream(q.device)), "fa_bwd_noalloc")
    else:
        need = bwd_workspace_bytes(B, H, N, d)
        ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=q.device)
        check(_lib.lib().fa_bwd(*ptrs, ws.data_ptr(), ws.numel(), _stream(q.device)), "fa_bwd")
    del keep, bm
    return (dq, dk, dv, tiles) if record_tiles else (dq, dk, dv)


def decode_workspace_bytes(B, H, Hkv, Nq, Nk, d) -> int:
    return int(_lib.lib().fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d))


def decode(q, k, v, *, kv_lens=None, causal=False, scale: Optional[float] = None, out=None, lse=None,
           workspace=None, events=None):
    """Decode attention: q [B, H, Nq, d] (the newest Nq tokens) against a
    key/value cache k, v [B, Hkv, Nk, d] whose first kv_lens[b] rows are valid
    (all Nk when None).  Returns (O [B, H, Nq, d], LSE [B, H, Nq]).  events:
    None or three hipEvent_t handles recorded around the chunk and merge
    kernels."""
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q [B, H, Nq, d], k and v [B, Hkv, Nk, d]")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous GPU tensors of one dtype and device")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k, v must share q's B and d")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = out if out is not None else torch.empty_like(q)
    l = lse if lse is not None else torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H, Hkv, Nq, Nk, d)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    kl = None if kv_lens is None else kv_lens.to(device=q.device, dtype=torch.int32).contiguous()
    ev = None
    if events is not None:
        if len(events) != 3:
            raise ValueError("events: three hipEvent_t handles")
        ev = (ctypes.c_void_p * 3)(*events)
    code = _lib.lib().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, Hkv,
                                Nq, Nk, d, _dtype_code(q), scale, 1 if causal else 0,
                                None if kl is None else kl.data_ptr(), ev, ws.data_ptr(), ws.numel(),
                                _stream(q.device))
    check(code, "fa_decode")
    del kl, ws
    return o, l


def fwd_kv_outer_workspace_bytes(B, H, N, d) -> int:
    return int(_lib.lib().fa_fwd_kv_outer_workspace_bytes(B, H, N, d))


def fwd_kv_outer(q, k, v, *, causal=False, scale: Optional[float] = None, block_cols=128, groups_per_head=0,
                 out=None, lse=None, workspace=None, events=None):
    """Forward in the key/value-outer loop order (an IO ablation: the running
    O, m, l go through device memory after every key tile).  q, k, v: [B, H,
    N, d] bf16 or fp16.  Returns (O, LSE).  events: None or two hipEvent_t
    handles recorded around the kernel."""
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous GPU tensors of one dtype and device")
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = out if out is not None else torch.empty_like(q)
    l = lse if lse is not None else torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = fwd_kv_outer_workspace_bytes(B, H, N, d)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ev = None
    if events is not None:
        if len(events) != 2:
            raise ValueError("events: two hipEvent_t handles")
        ev = (ctypes.c_void_p * 2)(*events)
    code = _lib.lib().fa_fwd_kv_outer(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                                      B, H, N, d, _dtype_code(q), scale, 1 if causal else 0, int(block_cols),
                                      int(groups_per_head), ev, ws.data_ptr(), ws.numel(), _stream(q.device))
    check(code, "fa_fwd_kv_outer")
    del ws
    return o, l


def dropout_keep_mask(seed, rng_offset, p, B, H, N, device="cuda"):
    """uint8 [B, H, N, N] keep bits from the device generator (tests only)."""
    keep = torch.empty((B, H, N, N), dtype=torch.uint8, device=device)
    code = _lib.lib().fa_dropout_keep_mask(int(seed), int(rng_offset), float(p), B, H, N, keep.data_ptr(),
                                           _stream(keep.device))
    check(code, "fa_dropout_keep_mask")
    return keep


def tile_shape(d: int, dtype_code: int, pass_: int, N: int, causal: bool):
    """(Br, Bc) of the kernel fa_fwd (pass 0) or fa_bwd (1: dK/dV, 2: dQ)
    launches for this head dim, dtype, N and causal flag."""
    br, bc = ctypes.c_int32(), ctypes.c_int32()
    check(_lib.lib().fa_tile_shape(d, dtype_code, pass_, N, 1 if causal else 0, ctypes.byref(br),
                                   ctypes.byref(bc)), "fa_tile_shape")
    return br.value, bc.value


def abi_version() -> int:
    return int(_lib.lib().fa_abi_version())
