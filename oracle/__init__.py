"""fp64 CPU oracle for tiled exact attention.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call or link anything under oracle/.  The HIP
library and its Python binding never do, and the oracle never imports them;
the only module both sides share is ``workloads`` (seeded inputs, no
attention arithmetic).

Contents
  attention.py  plain materialising fwd/bwd, sampled-row variants, the pages'
                tiled forward as a model for the merge checks, the key/value-
                outer forward with its HBM access counts, and an explicit
                softmax-Jacobian backward for tiny inputs
  philox.py     Philox4x32-10 and the dropout keep rule
  tiles.py      expected tile-visit sets and valid-pair counts
  philox_ref.c  an independent C Philox4x32-10 used to cross-check philox.py

Every function is pinned by `-m "not gpu"` tests against closed forms,
invariants, brute force, finite differences or an independent library routine
(torch CPU fp64 scaled_dot_product_attention and autograd; numpy's Philox4x64).
One part is only partly pinned and says so: the Philox4x32 multipliers M0, M1
(the round structure and the Weyl constants are pinned, the two 32-bit
multipliers come from the SC'11 paper without a known-answer vector here).
"""

from .attention import (attn_fwd, attn_bwd, attn_bwd_rows_cols, attn_stats, kv_head, decode_fwd,  # noqa: F401
                        tiled_fwd, kv_outer_fwd, attn_bwd_jacobian, validity, safe_softmax,
                        as_f64, scale_f32)
from .philox import (philox4x32_10, philox4_scalar, keep_mask, keep_scale,  # noqa: F401
                     dropout_threshold)
from .tiles import expected_tiles, tile_has_valid, valid_pair_count  # noqa: F401
