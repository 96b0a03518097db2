"""Seeded synthetic inputs for tiled exact attention.

This module is the only code shared by the fp64 oracle side (``oracle/`` and its
tests) and the GPU side (the HIP library's tests and ``bench.py``).  It holds
random draws, rounding to the storage dtype, per-sequence key lengths and the
block-sparsity pattern -- the *inputs* of the method -- and none of the
attention arithmetic.

Recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream per workload):

1. Q, K, V, dO are drawn in that order as fp64 ``standard_normal`` of shape
   [B, H, N, d] (K and V: [B, Hkv, N, d] for grouped-query workloads), each
   multiplied by ``std``, then rounded to the storage dtype with
   round-to-nearest-even (torch's CPU conversion).
2. Then, from the same stream, the key lengths (inclusive uniform integers,
   one per sequence, shared by all heads) if the workload pads keys.
3. Then the block mask if the workload is block-sparse: a band |i - j| <= 1 of
   128x128 tiles plus off-band tiles drawn uniformly without replacement until
   round(density * T^2) tiles are set.

The workload shapes follow the pages' own workloads (GPT-2 small and
BERT-large attention shapes, a 16K-token long-context case, the block-sparse
extension of the FlashAttention paper, and the grouped-query shape of the
Self-Attention tutorial's MHA / GQA / MQA comparison: 32 query heads, 8 K/V
heads, head_dim 128, 4096 tokens); the seeded Gaussian data stands in for the
text corpora those models were trained on.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

MASK_TILE = 128  # block-mask granularity in tokens (rows and columns)

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str               # storage dtype of Q, K, V, dO: fp32 | bf16 | fp16
    seed: int
    std: float = 1.0
    causal: bool = False
    key_len_range: Optional[tuple] = None   # inclusive (lo, hi) or None
    dropout_p: float = 0.0
    dropout_seed: int = 0
    rng_offset: int = 0
    sparse_density: Optional[float] = None  # block-sparse target density or None
    sample_rows: Optional[int] = None       # rows the oracle checks at full size
    kv_heads: Optional[int] = None          # K/V heads (grouped-query); None = H
    decode_q: Optional[int] = None          # decode: Nq new query rows against an N-row cache

    @property
    def Hkv(self) -> int:
        return self.H if self.kv_heads is None else self.kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny exact attention, oracle runs in seconds
    "tiny": Workload("tiny", 1, 2, 256, 64, "bf16", seed=0),
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 256, 64, "fp32", seed=0),
    # GPT-2 small attention shape, causal
    "gpt2": Workload("gpt2", 8, 12, 1024, 64, "bf16", seed=2, causal=True),
    # BERT-large attention shape, key padding + dropout 0.1
    "bert": Workload("bert", 16, 16, 512, 64, "fp16", seed=3,
                     key_len_range=(128, 512), dropout_p=0.1, dropout_seed=3,
                     rng_offset=0),
    # long-context causal, d = 128; "N(0, 0.5)" read as variance 0.5
    "long": Workload("long", 1, 16, 16384, 128, "bf16", seed=4,
                     std=math.sqrt(0.5), causal=True, sample_rows=256),
    # the d = 128, N >= 4K regime without the causal mask (every tile dense)
    "long_noncausal": Workload("long_noncausal", 1, 16, 8192, 128, "bf16", seed=8, sample_rows=256),
    # block-sparse, 128x128 tiles, band of 3 + random to density 0.1
    "sparse": Workload("sparse", 1, 8, 16384, 64, "bf16", seed=5,
                       sparse_density=0.1, sample_rows=256),
    # grouped-query attention: 32 query heads share 8 K/V heads, causal
    "gqa": Workload("gqa", 4, 32, 4096, 128, "bf16", seed=6, causal=True, kv_heads=8,
                    sample_rows=256),
    # decode: one new token per sequence against a 16K-row cache (valid
    # lengths 8K..16K), the same head shape
    "decode": Workload("decode", 16, 32, 16384, 128, "bf16", seed=7, causal=True, kv_heads=8,
                       key_len_range=(8192, 16384), decode_q=1),
}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def round_to(x: np.ndarray, dtype: str) -> torch.Tensor:
    """fp64 array -> CPU tensor of the storage dtype, round-to-nearest-even."""
    # Both sides consume the rounded tensor, so the exact rounding path of the
    # conversion does not affect parity; it only has to be deterministic.
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(_DTYPES[dtype])


def band_random_block_mask(T: int, density: float, rng: np.random.Generator,
                           band: int = 1) -> np.ndarray:
    """uint8 [T, T]: |i - j| <= band plus uniform off-band tiles to round(density*T^2)."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = (np.abs(i - j) <= band).astype(np.uint8)
    target = int(round(density * T * T))
    have = int(m.sum())
    if target > have:
        off = np.flatnonzero(m.reshape(-1) == 0)
        pick = rng.choice(off, size=target - have, replace=False)
        m.reshape(-1)[pick] = 1
    return m


def make_inputs(w: Workload, dtype: Optional[str] = None, with_do: bool = True) -> dict:
    """Draw one workload's tensors (CPU).  Returns a dict with q, k, v, do
    (storage dtype), key_lens (int32 [B] or None), block_mask (uint8 [T, T] or
    None) and the scalar settings."""
    dtype = dtype or w.dtype
    rng = np.random.default_rng(w.seed)
    out = {}
    for name in ("q", "k", "v", "do"):
        if name == "do" and w.decode_q is not None:
            continue                      # decode has no backward
        heads = w.Hkv if name in ("k", "v") else w.H
        rows = w.decode_q if (name == "q" and w.decode_q is not None) else w.N
        x = rng.standard_normal((w.B, heads, rows, w.d)) * w.std
        out[name] = round_to(x, dtype)
        del x
    key_lens = None
    if w.key_len_range is not None:
        lo, hi = w.key_len_range
        key_lens = torch.from_numpy(rng.integers(lo, hi, size=w.B, endpoint=True).astype(np.int32))
    block_mask = None
    if w.sparse_density is not None:
        T = -(-w.N // MASK_TILE)
        block_mask = torch.from_numpy(band_random_block_mask(T, w.sparse_density, rng))
    out.update(key_lens=key_lens, block_mask=block_mask, scale=w.scale,
               causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed,
               rng_offset=w.rng_offset, dtype=dtype)
    if not with_do:
        out.pop("do", None)
    return out


def random_case(B, H, N, d, dtype="bf16", seed=0, std=1.0, causal=False,
                key_len_range=None, dropout_p=0.0, dropout_seed=0, rng_offset=0,
                sparse_density=None, kv_heads=None) -> dict:
    """Ad-hoc shape with the same recipe (used for ragged / edge-case tests)."""
    w = Workload("case", B, H, N, d, dtype, seed=seed, std=std, causal=causal,
                 key_len_range=key_len_range, dropout_p=dropout_p,
                 dropout_seed=dropout_seed, rng_offset=rng_offset,
                 sparse_density=sparse_density, kv_heads=kv_heads)
    return make_inputs(w)


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Query (or key) rows the oracle checks at full size: the first 16 rows,
    where low-precision rounding concentrates on causal inputs, plus rows drawn
    uniformly without replacement from the rest."""
    first = np.arange(min(16, N))
    if count <= len(first) or N <= 16:
        return first[:count]
    rng = np.random.default_rng(seed + 1000)
    rest = rng.choice(np.arange(16, N), size=min(count - 16, N - 16), replace=False)
    return np.sort(np.concatenate([first, rest]))
