"""Expected tile-visit sets (oracle side).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.

A kernel that splits the N x N score matrix into tiles of Br query rows by Bc
keys must visit exactly the tiles that hold at least one valid pair (i, j)
under A_ij = (not causal or j <= i) and (j < len_b) and M[i//128, j//128]:
tiles entirely above the diagonal are skipped for causal inputs (Self-Attention
tutorial, infra-guide, section 10.2 on skipping upper-triangle tiles) and zero
blocks of the mask are skipped outright (FlashAttention summary, xyznot.com,
"Block-Sparse FlashAttention"; explainer, azimuth.plus, block-sparse section).
Skipping fewer tiles is a failure as much as skipping more.
"""

from __future__ import annotations

import numpy as np

MASK_TILE = 128


def tile_has_valid(i0, i1, j0, j1, causal, key_len, block_mask):
    """True iff [i0, i1) x [j0, j1) holds a valid pair (closed form)."""
    if i1 <= i0 or j1 <= j0:
        return False
    if key_len is not None:
        j1 = min(j1, max(int(key_len), 0))
        if j1 <= j0:
            return False
    if block_mask is None:
        spans = [(i0, i1, j0, j1)]
    else:
        bm = np.asarray(block_mask)
        spans = []
        for bi in range(i0 // MASK_TILE, (i1 - 1) // MASK_TILE + 1):
            for bj in range(j0 // MASK_TILE, (j1 - 1) // MASK_TILE + 1):
                if bm[bi, bj]:
                    spans.append((max(i0, bi * MASK_TILE), min(i1, (bi + 1) * MASK_TILE),
                                  max(j0, bj * MASK_TILE), min(j1, (bj + 1) * MASK_TILE)))
    for a0, a1, c0, c1 in spans:
        # smallest key vs largest query of the sub-rectangle
        if not causal or c0 <= a1 - 1:
            return True
    return False


def expected_tiles(N, Br, Bc, B, causal=False, key_lens=None, block_mask=None):
    """uint8 [B, ceil(N/Br), ceil(N/Bc)]: 1 where the tile must be visited.
    The set does not depend on the head."""
    Tr, Tc = -(-N // Br), -(-N // Bc)
    out = np.zeros((B, Tr, Tc), dtype=np.uint8)
    for b in range(B):
        kl = None if key_lens is None else int(np.asarray(key_lens)[b])
        for i in range(Tr):
            for j in range(Tc):
                out[b, i, j] = tile_has_valid(i * Br, min((i + 1) * Br, N),
                                              j * Bc, min((j + 1) * Bc, N),
                                              causal, kl, block_mask)
    return out


def valid_pair_count(N, B, H, causal=False, key_lens=None, block_mask=None):
    """Number of valid (i, j) pairs over all heads: the algorithmic work unit."""
    total = 0
    rows = np.arange(N)
    for b in range(B):
        kl = N if key_lens is None else min(max(int(np.asarray(key_lens)[b]), 0), N)
        if block_mask is None:
            lim = np.full(N, kl)
            if causal:
                lim = np.minimum(lim, rows + 1)
            total += int(lim.sum())
        else:
            bm = np.asarray(block_mask)
            cnt = 0
            for bi in range(bm.shape[0]):
                r = rows[bi * MASK_TILE:(bi + 1) * MASK_TILE]
                for bj in np.flatnonzero(bm[bi]):
                    c0, c1 = bj * MASK_TILE, min((bj + 1) * MASK_TILE, kl)
                    if c1 <= c0:
                        continue
                    if causal:
                        cnt += int(np.clip(np.minimum(r + 1, c1) - c0, 0, None).sum())
                    else:
                        cnt += len(r) * (c1 - c0)
            total += cnt
    return total * H
