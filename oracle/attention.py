"""Exact attention forward and backward in fp64, materialising S and P.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP path.

What it computes is the plain definition that tiled exact attention reaches
(up to rounding order):

* scores  S = scale * Q K^T          -- scaled dot product (Self-Attention
  tutorial, infra-guide, section 3.2-3.3; FlashAttention explainer,
  azimuth.plus, "memory bandwidth, not compute" formula).
* validity A_ij = (not causal or j <= i) and (j < len_b) and M[i//128, j//128];
  invalid scores are set to -inf before the softmax (tutorial section 10.2,
  lower triangle kept including the diagonal; tutorial section 4.1 masked_fill
  with -inf; block mask M from the FlashAttention summary, xyznot.com,
  "Block-Sparse FlashAttention").
* safe softmax along each row: subtract the row max, exponentiate, normalise
  (tutorial section 7.2).  The saved statistic is LSE_i = m_i + ln l_i, the
  log of the softmax normaliser, which carries the pair (l, m) the
  FlashAttention summary says is stored for the backward pass (core ideas,
  recomputation).  A row with no valid key has P = 0, O = 0, LSE = -inf.
* dropout on P after the softmax and before the product with V (explainer,
  kernel fusion: matmul, mask, softmax, dropout, matmul), inverted scaling
  by s = 1 / P(keep) (`philox.keep_scale`: 2^16 / (2^16 - thr), the
  keep rule's exact probability); l and LSE use the undropped P.
* O = P_hat V.
* backward (the pages say only that S and P are recomputed; the gradients
  follow from the definition with the softmax Jacobian diag(p) - p p^T):
      dP_hat = dO V^T,  dV = P_hat^T dO,  dP = dP_hat * Z * s,
      D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
      dQ = scale dS K,  dK = scale dS^T Q.

* decode (tutorial section 11.2: one new query -- or a few -- against the
  whole key/value cache): Nq query rows per (b, h) against a cache of Nk
  rows of which the first len_b are valid; query row i sits at position
  len_b - Nq + i (the newest tokens), and with the causal mask sees keys
  j <= that position.  Same softmax, same LSE.
* the key/value-outer loop order of the original algorithm (explainer,
  step-by-step algorithm): the same O and LSE, reached block by block with
  the running statistics stored between steps; it also counts the HBM
  element traffic of that order for the IO model (`kv_outer_fwd`).
* grouped-query attention (tutorial section 9.2-9.3, MQA and GQA): K and V
  may have Hkv heads, Hkv dividing H; query head h uses K/V head
  h // (H / Hkv) (contiguous groups -- the pages do not fix the grouping),
  so dK, dV of a K/V head are the sums over its query heads.  Hkv = H is
  plain multi-head attention, Hkv = 1 multi-query.

Arrays are numpy float64 [B, H, N, d] (K, V: [B, Hkv, N, d]); the callers
convert the storage-dtype tensors exactly.  Long inputs are processed in chunks of query rows; every
row is always complete, so chunking changes nothing in the arithmetic.
"""

from __future__ import annotations

import numpy as np

from .philox import keep_mask, keep_scale

MASK_TILE = 128


def as_f64(t) -> np.ndarray:
    """torch tensor / array of any float dtype -> float64 numpy array (exact)."""
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        import torch
        return t.to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def scale_f32(scale: float) -> float:
    """The kernels receive scale as a float32; the oracle uses that value."""
    return float(np.float32(scale))


def validity(rows, N: int, causal: bool, key_len=None, block_mask=None) -> np.ndarray:
    """bool [len(rows), N]: A_ij for query rows i and all keys j."""
    rows = np.asarray(rows)
    j = np.arange(N)
    A = np.ones((len(rows), N), dtype=bool)
    if causal:
        A &= j[None, :] <= rows[:, None]
    if key_len is not None:
        A &= j[None, :] < min(max(int(key_len), 0), N)
    if block_mask is not None:
        bm = np.asarray(block_mask)
        A &= bm[rows[:, None] // MASK_TILE, j[None, :] // MASK_TILE] != 0
    return A


def safe_softmax(S: np.ndarray, A: np.ndarray):
    """Row softmax of S restricted to A.  Returns (P, LSE, m, l)."""
    S = np.where(A, S, -np.inf)
    m = S.max(axis=1)
    has = np.isfinite(m) | np.isnan(m)
    m_ref = np.where(has, m, 0.0)
    E = np.exp(S - m_ref[:, None])
    l = E.sum(axis=1)
    denom = np.where(has, l, 1.0)
    P = np.where(has[:, None], E / denom[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return P, lse, m, l


def _key_len(key_lens, b):
    return None if key_lens is None else int(np.asarray(key_lens)[b])


def _rows_scores(q, k, rows, scale):
    return scale * (q[rows] @ k.T)


def kv_head(h: int, H: int, Hkv: int) -> int:
    """K/V head that query head h reads (contiguous groups of H/Hkv)."""
    return h // (H // Hkv)


def _pairs(B, H, pairs):
    return pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]


def attn_fwd(q, k, v, scale, causal=False, key_lens=None, block_mask=None,
             dropout_p=0.0, seed=0, rng_offset=0, rows=None, chunk=512, pairs=None):
    """O [B,H,R,d] and LSE [B,H,R] for query rows `rows` (default: all).
    `pairs` restricts the work to a list of (b, h) (other heads stay 0)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    sc = scale_f32(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    O = np.zeros((B, H, len(rows), v.shape[-1]))
    LSE = np.zeros((B, H, len(rows)))
    for b, h in _pairs(B, H, pairs):
        kl = _key_len(key_lens, b)
        g = kv_head(h, H, Hkv)
        for s in range(0, len(rows), chunk):
            r = rows[s:s + chunk]
            S = _rows_scores(q[b, h], k[b, g], r, sc)
            A = validity(r, N, causal, kl, block_mask)
            P, lse, _, _ = safe_softmax(S, A)
            if dropout_p > 0.0:
                Z = keep_mask(seed, rng_offset, dropout_p, b, h, H, r, np.arange(N))
                P = P * Z * keep_scale(dropout_p)
            O[b, h, s:s + chunk] = P @ v[b, g]
            LSE[b, h, s:s + chunk] = lse
    return O, LSE


def attn_bwd(q, k, v, do, scale, causal=False, key_lens=None, block_mask=None,
             dropout_p=0.0, seed=0, rng_offset=0, chunk=512, pairs=None):
    """dQ, dK, dV [B,H,N,d] and D [B,H,N] over all rows (of the heads in
    `pairs`, default all)."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, H, N, d = q.shape
    sc = scale_f32(scale)
    ks = keep_scale(dropout_p)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    Dall = np.zeros((B, H, N))
    Hkv = k.shape[1]
    for b, h in _pairs(B, H, pairs):
        kl = _key_len(key_lens, b)
        g = kv_head(h, H, Hkv)
        for s in range(0, N, chunk):
            r = np.arange(s, min(s + chunk, N))
            S = _rows_scores(q[b, h], k[b, g], r, sc)
            A = validity(r, N, causal, kl, block_mask)
            P, _, _, _ = safe_softmax(S, A)
            if dropout_p > 0.0:
                Z = keep_mask(seed, rng_offset, dropout_p, b, h, H, r, np.arange(N))
            else:
                Z = np.ones_like(P, dtype=bool)
            P_hat = P * Z * ks
            dP_hat = do[b, h, r] @ v[b, g].T
            dv[b, g] += P_hat.T @ do[b, h, r]
            dP = dP_hat * Z * ks
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            dq[b, h, r] = sc * (dS @ k[b, g])
            dk[b, g] += sc * (dS.T @ q[b, h, r])
            Dall[b, h, r] = D
    return dq, dk, dv, Dall


def attn_bwd_rows_cols(q, k, v, do, scale, rows, cols, lse_all, D_all,
                       causal=False, key_lens=None, block_mask=None,
                       dropout_p=0.0, seed=0, rng_offset=0, chunk=1024, pairs=None):
    """Gradients at sampled positions of a large input.

    dQ for query rows `rows` needs only those rows' full score rows.
    dK, dV for key rows `cols` need the columns S[:, cols] over all query rows
    together with every row's LSE_i and D_i (passed in from a full pass,
    `attn_stats`).  P_ij = exp(S_ij - LSE_i) is the definition of the row
    softmax written with the log-normaliser.
    """
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, H, N, d = q.shape
    sc = scale_f32(scale)
    ks = keep_scale(dropout_p)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    Hkv = k.shape[1]
    dq = np.zeros((B, H, len(rows), d))
    dk = np.zeros((B, Hkv, len(cols), d))
    dv = np.zeros((B, Hkv, len(cols), d))
    for b, h in _pairs(B, H, pairs):
        kl = _key_len(key_lens, b)
        g = kv_head(h, H, Hkv)
        # dQ rows: full rows of S
        S = _rows_scores(q[b, h], k[b, g], rows, sc)
        A = validity(rows, N, causal, kl, block_mask)
        P, _, _, _ = safe_softmax(S, A)
        Z = (keep_mask(seed, rng_offset, dropout_p, b, h, H, rows, np.arange(N))
             if dropout_p > 0 else np.ones_like(P, dtype=bool))
        dP = (do[b, h, rows] @ v[b, g].T) * Z * ks
        D = (P * dP).sum(axis=1)
        dq[b, h] = sc * ((P * (dP - D[:, None])) @ k[b, g])
        # dK, dV columns: all query rows, selected keys (none: nothing to add)
        for s in range(0, N if len(cols) else 0, chunk):
            r = np.arange(s, min(s + chunk, N))
            Sc = sc * (q[b, h, r] @ k[b, g, cols].T)
            Ac = validity(r, N, causal, kl, block_mask)[:, cols]
            lse = lse_all[b, h, r]
            live = np.isfinite(lse)[:, None] & Ac
            Pc = np.where(live, np.exp(np.where(live, Sc - lse[:, None], -np.inf)), 0.0)
            Zc = (keep_mask(seed, rng_offset, dropout_p, b, h, H, r, cols)
                  if dropout_p > 0 else np.ones_like(Pc, dtype=bool))
            dv[b, g] += (Pc * Zc * ks).T @ do[b, h, r]
            dPc = (do[b, h, r] @ v[b, g, cols].T) * Zc * ks
            dSc = Pc * (dPc - D_all[b, h, r][:, None])
            dk[b, g] += sc * (dSc.T @ q[b, h, r])
    return dq, dk, dv


def attn_stats(q, k, v, do, scale, causal=False, key_lens=None, block_mask=None,
               dropout_p=0.0, seed=0, rng_offset=0, heads=None, chunk=512, rows=None):
    """LSE [B,H,N] and D [B,H,N] (D_i = sum_j P_ij dP_ij) over all rows, or
    over the query rows in `rows` (the others left 0).  `heads` restricts the
    work to a list of (b, h) pairs (others left 0)."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, H, N, d = q.shape
    sc = scale_f32(scale)
    ks = keep_scale(dropout_p)
    LSE = np.zeros((B, H, N))
    Dall = np.zeros((B, H, N))
    Hkv = k.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    for b, h in _pairs(B, H, heads):
        kl = _key_len(key_lens, b)
        g = kv_head(h, H, Hkv)
        for s in range(0, len(rows), chunk):
            r = rows[s:s + chunk]
            S = _rows_scores(q[b, h], k[b, g], r, sc)
            A = validity(r, N, causal, kl, block_mask)
            P, lse, _, _ = safe_softmax(S, A)
            Z = (keep_mask(seed, rng_offset, dropout_p, b, h, H, r, np.arange(N))
                 if dropout_p > 0 else np.ones_like(P, dtype=bool))
            dP = (do[b, h, r] @ v[b, g].T) * Z * ks
            LSE[b, h, r] = lse
            Dall[b, h, r] = (P * dP).sum(axis=1)
    return LSE, Dall


def tiled_fwd(q, k, v, scale, Br, Bc, causal=False, key_lens=None, block_mask=None):
    """The pages' tiled forward, blocks of Br query rows by Bc keys, written
    out step by step (FlashAttention summary, xyznot.com, "Method": block
    scores, block statistics, merged statistics, rescaled output; the
    incremental-softmax merge of two sub-vectors).  Kept separate from
    `attn_fwd` so the tests can check the block merge against the full-row
    softmax; it is a model of the method, not of any kernel's schedule.
    No dropout."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, H, N, d = q.shape
    sc = scale_f32(scale)
    O = np.zeros_like(q)
    LSE = np.zeros((B, H, N))
    for b in range(B):
        kl = _key_len(key_lens, b)
        for h in range(H):
            for i0 in range(0, N, Br):
                r = np.arange(i0, min(i0 + Br, N))
                m = np.full(len(r), -np.inf)
                l = np.zeros(len(r))
                Oi = np.zeros((len(r), d))
                for j0 in range(0, N, Bc):
                    c = np.arange(j0, min(j0 + Bc, N))
                    Sij = sc * (q[b, h, r] @ k[b, h, c].T)
                    Aij = validity(r, N, causal, kl, block_mask)[:, c]
                    Sij = np.where(Aij, Sij, -np.inf)
                    m, l, Oi = _merge_block(m, l, Oi, Sij, v[b, h, c])
                O[b, h, r] = Oi
                with np.errstate(divide="ignore"):
                    LSE[b, h, r] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, LSE


def kv_outer_fwd(q, k, v, scale, Br, Bc, causal=False):
    """The pages' forward in its original loop order, key/value blocks outer
    and query blocks inner (FlashAttention explainer, azimuth.plus,
    step-by-step algorithm; FlashAttention summary, xyznot.com, "Method"),
    with the running O, l, m kept in "HBM" arrays that every inner step
    loads, updates and stores back.  Blocks holding no valid pair (causal:
    above the diagonal) are skipped, as the block-sparse section of both
    pages skips zero blocks.  Returns (O, LSE, io), io = {"read": {...},
    "write": {...}} counting the elements each HBM array sees under the
    algorithm's loads and stores (summed over heads), for the IO model
    Theta(N^2 d^2 / M) of the summary's "complexity" section.  No dropout."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, H, N, d = q.shape
    sc = scale_f32(scale)
    rd = dict(Q=0, K=0, V=0, O=0, l=0, m=0)
    wr = dict(O=0, l=0, m=0)
    O = np.zeros_like(q)
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            # initialise O = 0, l = 0, m = -inf in HBM
            Oh = np.zeros((N, d))
            lh = np.zeros(N)
            mh = np.full(N, -np.inf)
            wr["O"] += N * d
            wr["l"] += N
            wr["m"] += N
            for j0 in range(0, N, Bc):
                c = np.arange(j0, min(j0 + Bc, N))
                rows = [np.arange(i0, min(i0 + Br, N)) for i0 in range(0, N, Br)]
                rows = [r for r in rows if validity(r, N, causal)[:, c].any()]
                if not rows:
                    continue
                Kj, Vj = k[b, h, c], v[b, h, c]                  # load K_j, V_j
                rd["K"] += Kj.size
                rd["V"] += Vj.size
                for r in rows:
                    Qi, Oi, li, mi = q[b, h, r], Oh[r], lh[r], mh[r]    # load Q_i, O_i, l_i, m_i
                    rd["Q"] += Qi.size
                    rd["O"] += Oi.size
                    rd["l"] += li.size
                    rd["m"] += mi.size
                    Sij = np.where(validity(r, N, causal)[:, c], sc * (Qi @ Kj.T), -np.inf)
                    mi_new, li_new, Oi_new = _merge_block(mi, li, Oi, Sij, Vj)
                    Oh[r], lh[r], mh[r] = Oi_new, li_new, mi_new     # write O_i, l_i, m_i
                    wr["O"] += Oi_new.size
                    wr["l"] += li_new.size
                    wr["m"] += mi_new.size
            O[b, h] = Oh
            with np.errstate(divide="ignore"):
                LSE[b, h] = np.where(lh > 0, mh + np.log(np.where(lh > 0, lh, 1.0)), -np.inf)
    return O, LSE, {"read": rd, "write": wr}


def _merge_block(m, l, Oi, Sij, Vj):
    """One block step of the summary's "Method" (block row max m~, block
    probabilities P~ = exp(S - m~), block row sum l~; m_new = max(m, m~),
    l_new = e^{m - m_new} l + e^{m~ - m_new} l~, O_new = diag(l_new)^-1
    (diag(l) e^{m - m_new} O + e^{m~ - m_new} P~ V)).  Rows with no valid key
    so far keep m = -inf, l = 0, O = 0."""
    m_t = Sij.max(axis=1)
    mt_ref = np.where(np.isfinite(m_t), m_t, 0.0)
    P_t = np.exp(Sij - mt_ref[:, None])
    l_t = P_t.sum(axis=1)
    m_new = np.maximum(m, m_t)
    mn_ref = np.where(np.isfinite(m_new), m_new, 0.0)
    a_old = np.exp(m - mn_ref)
    a_blk = np.exp(m_t - mn_ref)
    l_new = a_old * l + a_blk * l_t
    with np.errstate(invalid="ignore", divide="ignore"):
        O_new = np.where(l_new[:, None] > 0,
                         (l[:, None] * a_old[:, None] * Oi + a_blk[:, None] * (P_t @ Vj)) / l_new[:, None], 0.0)
    return m_new, l_new, O_new


def attn_bwd_jacobian(q, k, v, do, scale, causal=False, key_lens=None,
                      block_mask=None, Z=None, dropout_p=0.0):
    """Backward through the explicit per-row softmax Jacobian J = diag(p) - p p^T
    (small N only).  Z is an optional fixed bool keep mask [B,H,N,N]."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, H, N, d = q.shape
    sc = scale_f32(scale)
    ks = keep_scale(dropout_p)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        kl = _key_len(key_lens, b)
        for h in range(H):
            S = sc * (q[b, h] @ k[b, h].T)
            A = validity(np.arange(N), N, causal, kl, block_mask)
            P, _, _, _ = safe_softmax(S, A)
            z = np.ones((N, N)) if Z is None else Z[b, h].astype(np.float64) * ks
            for i in range(N):
                p = P[i]
                # O_i = sum_j p_j z_ij v_j
                dv[b, h] += np.outer(p * z[i], do[b, h, i])
                g = (v[b, h] @ do[b, h, i]) * z[i]          # dL/dp_j
                J = np.diag(p) - np.outer(p, p)
                ds = J @ g                                   # dL/dS_ij
                dq[b, h, i] += sc * (ds @ k[b, h])
                dk[b, h] += sc * np.outer(ds, q[b, h, i])
    return dq, dk, dv


def decode_fwd(q, k, v, scale, kv_lens=None, causal=False):
    """Decode attention.  q [B,H,Nq,d], k and v [B,Hkv,Nk,d] (a cache whose
    first kv_lens[b] rows are valid; None = Nk).  Returns O [B,H,Nq,d] and
    LSE [B,H,Nq]; query row i of sequence b is at position kv_lens[b]-Nq+i."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    sc = scale_f32(scale)
    O = np.zeros((B, H, Nq, v.shape[-1]))
    LSE = np.zeros((B, H, Nq))
    j = np.arange(Nk)
    for b in range(B):
        L = Nk if kv_lens is None else min(max(int(np.asarray(kv_lens)[b]), 0), Nk)
        pos = L - Nq + np.arange(Nq)
        A = np.broadcast_to(j[None, :] < L, (Nq, Nk)).copy()
        if causal:
            A &= j[None, :] <= pos[:, None]
        for h in range(H):
            g = kv_head(h, H, Hkv)
            S = sc * (q[b, h] @ k[b, g].T)
            P, lse, _, _ = safe_softmax(S, A)
            O[b, h] = P @ v[b, g]
            LSE[b, h] = lse
    return O, LSE
