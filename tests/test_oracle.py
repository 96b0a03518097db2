"""Pins for the fp64 oracle: closed forms, invariants, brute force, finite
differences and an independent library routine (torch CPU fp64 SDPA)."""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import safe_softmax, validity

RTOL = 1e-12


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def small_case(B=2, H=2, N=37, d=8, seed=0):
    return rnd((B, H, N, d), seed), rnd((B, H, N, d), seed + 1), rnd((B, H, N, d), seed + 2), \
        rnd((B, H, N, d), seed + 3)


def mask_variants(N, B):
    T = -(-N // 128)
    bm = np.ones((T, T), np.uint8)
    if T > 1:
        bm[0, T - 1] = 0
    return [dict(causal=False), dict(causal=True),
            dict(causal=False, key_lens=np.array([N // 2, N][:B])),
            dict(causal=True, key_lens=np.array([5, N - 3][:B])),
            dict(causal=False, block_mask=bm)]


# ---------------------------------------------------------------- golden fixtures

def test_golden_causal_mask(golden_dir):
    rows = [l.split() for l in open(f"{golden_dir}/causal_mask_4x4.txt") if not l.startswith("#")]
    want = np.array(rows, dtype=int).astype(bool)
    got = validity(np.arange(4), 4, causal=True)
    assert (got == want).all()


def test_golden_shape_trace(golden_dir):
    kv = {}
    for line in open(f"{golden_dir}/shape_trace.txt"):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        kv[k] = [int(x) for x in v]
    b, s, h, hd = kv["batch"][0], kv["seq_len"][0], kv["num_heads"][0], kv["head_dim"][0]
    q = rnd((b, h, s, hd), 1)
    k = rnd((b, h, s, hd), 2)
    v = rnd((b, h, s, hd), 3)
    scale = 1.0 / kv["scale_divisor"][0]
    assert scale == 1.0 / np.sqrt(hd)
    O, L = oracle.attn_fwd(q, k, v, scale)
    assert list(q.shape) == kv["q_shape"] and list(O.shape) == kv["out_shape"]
    # the score matrix is seq x seq per head: check by materialising one head
    S = scale * q[0, 0] @ k[0, 0].T
    assert [b, h, *S.shape] == kv["scores_shape"]


# ---------------------------------------------------------------- softmax / merge

def test_rows_sum_to_one():
    rng = np.random.default_rng(0)
    S = rng.standard_normal((50, 70)) * 30
    A = rng.random((50, 70)) < 0.3
    A[7] = False
    P, lse, m, l = safe_softmax(S, A)
    has = A.any(axis=1)
    assert np.allclose(P[has].sum(axis=1), 1.0, rtol=0, atol=RTOL)
    assert (P[~A] == 0).all()
    assert (P[7] == 0).all() and lse[7] == -np.inf
    # LSE is the log of the normaliser of the exponentials
    ref = np.array([np.log(np.exp(S[i][A[i]]).sum()) if A[i].any() else -np.inf for i in range(50)])
    assert np.allclose(lse[has], ref[has], rtol=1e-13, atol=0)


@pytest.mark.parametrize("seed", range(5))
def test_two_block_merge_formula(seed):
    """m(x) = max(m1, m2), l(x) = e^{m1-m} l1 + e^{m2-m} l2 equals the one-pass values,
    including a split where one part is entirely -inf."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(64) * 20
    if seed == 3:
        x[:20] = -np.inf
    cut = [1, 20, 33, 63, 40][seed]
    x1, x2 = x[:cut], x[cut:]

    def stats(z):
        m = z.max()
        return m, (np.exp(z - m).sum() if np.isfinite(m) else 0.0)
    m1, l1 = stats(x1)
    m2, l2 = stats(x2)
    m = max(m1, m2)
    l = (np.exp(m1 - m) * l1 if np.isfinite(m1) else 0.0) + (np.exp(m2 - m) * l2 if np.isfinite(m2) else 0.0)
    mf, lf = stats(x)
    assert m == mf
    assert abs(l - lf) <= 1e-12 * lf


@pytest.mark.parametrize("Br,Bc", [(1, 1), (7, 13), (16, 16), (64, 32), (37, 5)])
@pytest.mark.parametrize("variant", range(5))
def test_tiled_merge_equals_full_row_softmax(Br, Bc, variant):
    q, k, v, _ = small_case(B=2, H=1, N=37, d=8, seed=10 + variant)
    kw = mask_variants(37, 2)[variant]
    O, L = oracle.attn_fwd(q, k, v, 0.3, **kw)
    Ot, Lt = oracle.tiled_fwd(q, k, v, 0.3, Br, Bc, **kw)
    assert np.allclose(Ot, O, rtol=0, atol=1e-12)
    fin = np.isfinite(L)
    assert (np.isfinite(Lt) == fin).all()
    assert np.allclose(Lt[fin], L[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("variant", range(5))
def test_constant_v_gives_constant_output(variant):
    q, k, _, _ = small_case(B=2, H=2, N=300, d=8, seed=3)
    vrow = rnd((8,), 9)
    v = np.broadcast_to(vrow, q.shape).copy()
    kw = mask_variants(300, 2)[variant]
    O, L = oracle.attn_fwd(q, k, v, 0.5, **kw)
    assert np.allclose(O, vrow, rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant", range(5))
def test_zero_query_closed_form(variant):
    """Q = 0: P is uniform over the valid keys; O is their mean; LSE = ln(count)."""
    N = 300
    _, k, v, _ = small_case(B=2, H=1, N=N, d=8, seed=4)
    q = np.zeros_like(k)
    kw = mask_variants(N, 2)[variant]
    O, L = oracle.attn_fwd(q, k, v, 0.7, **kw)
    for b in range(2):
        kl = None if kw.get("key_lens") is None else kw["key_lens"][b]
        A = validity(np.arange(N), N, kw.get("causal", False), kl, kw.get("block_mask"))
        cnt = A.sum(axis=1)
        want = (A.astype(float) @ v[b, 0]) / cnt[:, None]
        assert np.allclose(O[b, 0], want, rtol=0, atol=1e-12)
        assert np.allclose(L[b, 0], np.log(cnt), rtol=0, atol=1e-12)


def test_causal_first_row():
    q, k, v, _ = small_case(B=1, H=3, N=50, d=16, seed=5)
    scale = 0.25
    O, L = oracle.attn_fwd(q, k, v, scale, causal=True)
    assert np.allclose(O[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    s32 = float(np.float32(scale))
    assert np.allclose(L[:, :, 0], s32 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-13)


def test_single_key():
    q, k, v, _ = small_case(B=1, H=1, N=1, d=8, seed=6)
    O, L = oracle.attn_fwd(q, k, v, 0.1)
    assert np.allclose(O, v) and np.allclose(L[0, 0, 0], float(np.float32(0.1)) * (q[0, 0, 0] @ k[0, 0, 0]))


# ---------------------------------------------------------------- invariants

def test_key_value_permutation_equivariance():
    q, k, v, _ = small_case(B=1, H=2, N=64, d=8, seed=7)
    perm = np.random.default_rng(1).permutation(64)
    O, L = oracle.attn_fwd(q, k, v, 0.4)
    Op, Lp = oracle.attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.4)
    assert np.allclose(O, Op, atol=1e-12) and np.allclose(L, Lp, atol=1e-12)
    # permuting query rows permutes the outputs
    Oq, Lq = oracle.attn_fwd(q[:, :, perm], k, v, 0.4)
    assert np.allclose(Oq, O[:, :, perm], atol=1e-12) and np.allclose(Lq, L[:, :, perm], atol=1e-12)


@pytest.mark.parametrize("mag", [1.0, 1e3])
def test_shift_invariance(mag):
    q, k, v, _ = small_case(B=1, H=2, N=40, d=8, seed=8)
    u = rnd((8,), 11) * mag
    scale = 0.5
    O, L = oracle.attn_fwd(q, k, v, scale, causal=True)
    Os, Ls = oracle.attn_fwd(q, k + u, v, scale, causal=True)
    s32 = float(np.float32(scale))
    assert np.all(np.isfinite(Os))
    assert np.allclose(Os, O, atol=1e-9 * mag)
    assert np.allclose(Ls, L + s32 * (q @ u), rtol=1e-12, atol=1e-9 * mag)


def test_fully_masked_rows():
    q, k, v, do = small_case(B=2, H=1, N=20, d=4, seed=9)
    kl = np.array([0, 20])
    O, L = oracle.attn_fwd(q, k, v, 0.5, key_lens=kl)
    assert (O[0] == 0).all() and (L[0] == -np.inf).all() and np.isfinite(L[1]).all()
    dq, dk, dv, D = oracle.attn_bwd(q, k, v, do, 0.5, key_lens=kl)
    assert (dq[0] == 0).all() and (dk[0] == 0).all() and (dv[0] == 0).all()


# ---------------------------------------------------------------- library routine

def _sdpa_ref(q, k, v, do, scale, causal, key_lens, block_mask):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    gqa = k.shape[1] != q.shape[1]
    B, H, N, d = q.shape
    mask = torch.ones(B, 1, N, N, dtype=torch.bool)
    if causal:
        mask &= torch.ones(N, N, dtype=torch.bool).tril()
    if key_lens is not None:
        mask &= (torch.arange(N)[None, :] < torch.tensor(key_lens)[:, None])[:, None, None, :]
    if block_mask is not None:
        idx = torch.arange(N) // 128
        mask &= torch.tensor(block_mask).bool()[idx[:, None], idx[None, :]]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=float(np.float32(scale)), enable_gqa=gqa)
    o.backward(torch.tensor(do))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("variant", range(5))
def test_against_torch_sdpa_fp64(variant):
    N = 300
    q, k, v, do = small_case(B=2, H=2, N=N, d=16, seed=20 + variant)
    kw = mask_variants(N, 2)[variant]
    if variant == 3:          # every row needs a valid key for SDPA (it NaNs empty rows)
        kw["key_lens"] = np.array([N - 100, N - 3])
    scale = 0.21
    O, L = oracle.attn_fwd(q, k, v, scale, **kw)
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, do, scale, **kw)
    Or, dqr, dkr, dvr = _sdpa_ref(q, k, v, do, scale, kw.get("causal", False),
                                  kw.get("key_lens"), kw.get("block_mask"))
    assert np.allclose(O, Or, rtol=0, atol=1e-12)
    for a, b in ((dq, dqr), (dk, dkr), (dv, dvr)):
        assert np.allclose(a, b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("hkv,variant", [(2, 0), (2, 1), (1, 3), (3, 4), (1, 2)])
def test_gqa_against_torch_sdpa_fp64(hkv, variant):
    """Grouped-query / multi-query attention (tutorial section 9.2-9.3): the
    oracle with Hkv < H K/V heads against torch's own GQA path
    (enable_gqa), forward and autograd gradients, dK and dV summed over each
    group of H / Hkv query heads."""
    N, H = 300, 6
    rng = np.random.default_rng(40 + hkv + variant)
    q, do = rng.standard_normal((2, H, N, 16)), rng.standard_normal((2, H, N, 16))
    k, v = rng.standard_normal((2, hkv, N, 16)), rng.standard_normal((2, hkv, N, 16))
    kw = mask_variants(N, 2)[variant]
    if variant == 3:
        kw["key_lens"] = np.array([N - 100, N - 3])
    O, L = oracle.attn_fwd(q, k, v, 0.3, **kw)
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, do, 0.3, **kw)
    assert dk.shape == k.shape and dv.shape == v.shape
    Or, dqr, dkr, dvr = _sdpa_ref(q, k, v, do, 0.3, kw.get("causal", False), kw.get("key_lens"),
                                  kw.get("block_mask"))
    assert np.allclose(O, Or, rtol=0, atol=1e-12)
    for a, b in ((dq, dqr), (dk, dkr), (dv, dvr)):
        assert np.allclose(a, b, rtol=0, atol=1e-11)


def test_gqa_grouping_and_sampled_variants():
    """Query head h reads K/V head h // (H / Hkv): moving K/V head 1 changes
    exactly the outputs of query heads 2 and 3 (H = 4, Hkv = 2); the sampled
    row/column backward and the statistics pass agree with the full pass."""
    N, H = 130, 4
    rng = np.random.default_rng(7)
    q, do = rng.standard_normal((1, H, N, 8)), rng.standard_normal((1, H, N, 8))
    k, v = rng.standard_normal((1, 2, N, 8)), rng.standard_normal((1, 2, N, 8))
    O, L = oracle.attn_fwd(q, k, v, 0.4, causal=True)
    k2 = k.copy()
    k2[0, 1] += 0.5 * rng.standard_normal((N, 8))   # (a constant shift would cancel in the softmax)
    O2, _ = oracle.attn_fwd(q, k2, v, 0.4, causal=True)
    changed = [not np.allclose(O[0, h], O2[0, h]) for h in range(H)]
    assert changed == [False, False, True, True]
    dq, dk, dv, D = oracle.attn_bwd(q, k, v, do, 0.4, causal=True)
    L2, D2 = oracle.attn_stats(q, k, v, do, 0.4, causal=True)
    assert np.allclose(L2, L) and np.allclose(D2, D)
    rows, cols = np.array([0, 7, 129]), np.array([3, 64, 128])
    sq, sk, sv = oracle.attn_bwd_rows_cols(q, k, v, do, 0.4, rows, cols, L2, D2, causal=True)
    assert np.allclose(sq, dq[:, :, rows]) and np.allclose(sk, dk[:, :, cols]) and np.allclose(sv, dv[:, :, cols])


@pytest.mark.parametrize("causal,hkv", [(False, 4), (True, 2), (True, 1)])
def test_decode_against_torch_sdpa_fp64(causal, hkv):
    """Decode: Nq newest query rows against a cache with per-sequence valid
    lengths, the causal mask aligned to the end of each sequence; against
    torch CPU fp64 SDPA with the same boolean mask and enable_gqa."""
    B, H, Nq, Nk, d = 3, 4, 5, 700, 16
    rng = np.random.default_rng(50 + hkv)
    q = rng.standard_normal((B, H, Nq, d))
    k, v = rng.standard_normal((B, hkv, Nk, d)), rng.standard_normal((B, hkv, Nk, d))
    lens = np.array([700, 3, 411])       # the second sequence is shorter than Nq
    O, L = oracle.decode_fwd(q, k, v, 0.25, kv_lens=lens, causal=causal)
    j = torch.arange(Nk)
    mask = torch.zeros(B, 1, Nq, Nk, dtype=torch.bool)
    for b in range(B):
        pos = lens[b] - Nq + torch.arange(Nq)
        m = (j[None, :] < lens[b]).expand(Nq, Nk)
        if causal:
            m = m & (j[None, :] <= pos[:, None])
        mask[b, 0] = m
    tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.25,
                                                           enable_gqa=hkv != H).numpy()
    rows = mask[:, 0].any(-1).numpy()                      # SDPA NaNs rows with no valid key
    for b in range(B):
        for h in range(H):
            assert np.allclose(O[b, h][rows[b]], ref[b, h][rows[b]], rtol=0, atol=1e-12)
            assert (O[b, h][~rows[b]] == 0).all() and np.isneginf(L[b, h][~rows[b]]).all()
    # empty rows exist only where causal and the sequence is shorter than Nq
    assert (~rows).any() == causal


def test_decode_reduces_to_square_attention():
    """Nq = Nk = len: the decode rows are all rows, aligned as in square
    causal attention; one query row with a one-key cache returns that V row."""
    q, k, v, _ = small_case(B=2, H=2, N=40, d=8, seed=60)
    for causal in (False, True):
        O, L = oracle.decode_fwd(q, k, v, 0.3, causal=causal)
        O2, L2 = oracle.attn_fwd(q, k, v, 0.3, causal=causal)
        assert np.allclose(O, O2, rtol=0, atol=1e-13) and np.allclose(L, L2, rtol=0, atol=1e-13)
    O, L = oracle.decode_fwd(q[:, :, :1], k, v, 0.3, kv_lens=np.array([1, 1]), causal=True)
    assert np.allclose(O[:, :, 0], v[:, :, 0])
    assert np.allclose(L[:, :, 0], float(np.float32(0.3)) * (q[:, :, 0] * k[:, :, 0]).sum(-1), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- gradients

def _loss(q, k, v, do, scale, kw):
    O, _ = oracle.attn_fwd(q, k, v, scale, **kw)
    return float((O * do).sum())


@pytest.mark.parametrize("variant", ["dense", "causal", "padding", "block", "dropout"])
def test_finite_differences(variant):
    N, d = 12, 4
    q, k, v, do = small_case(B=1, H=1, N=N, d=d, seed=31)
    kw = {}
    if variant == "causal":
        kw = dict(causal=True)
    elif variant == "padding":
        kw = dict(key_lens=np.array([7]))
    elif variant == "block":
        kw = dict(block_mask=np.array([[1]], np.uint8), causal=True)
    elif variant == "dropout":
        kw = dict(dropout_p=0.3, seed=123, rng_offset=5)
    scale = 0.37
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, do, scale, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = dict(q=q, k=k, v=v)
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, scale, kw)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, scale, kw)
            num[idx] = (fp - fm) / (2 * h)
        err = np.abs(num - g).max() / max(np.abs(g).max(), 1e-300)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("variant", range(5))
def test_dk_sums_to_zero_and_D_two_ways(variant):
    N = 200
    q, k, v, do = small_case(B=2, H=2, N=N, d=8, seed=40 + variant)
    kw = mask_variants(N, 2)[variant]
    kw.update(dropout_p=0.2, seed=7) if variant == 2 else None
    dq, dk, dv, D = oracle.attn_bwd(q, k, v, do, 0.3, **kw)
    assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-10)
    O, _ = oracle.attn_fwd(q, k, v, 0.3, **kw)
    assert np.allclose(D, (do * O).sum(axis=-1), atol=1e-12)


@pytest.mark.parametrize("dropout", [False, True])
def test_backward_matches_explicit_jacobian(dropout):
    N = 24
    q, k, v, do = small_case(B=1, H=2, N=N, d=4, seed=50)
    kw = dict(causal=True, key_lens=np.array([19]))
    Z = None
    if dropout:
        kw.update(dropout_p=0.25, seed=99, rng_offset=3)
        Z = np.stack([np.stack([oracle.keep_mask(99, 3, 0.25, 0, h, 2, np.arange(N), np.arange(N))
                                for h in range(2)])])
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, do, 0.6, **kw)
    jq, jk, jv = oracle.attn_bwd_jacobian(q, k, v, do, 0.6, causal=True, key_lens=np.array([19]),
                                          Z=Z, dropout_p=kw.get("dropout_p", 0.0))
    for a, b in ((dq, jq), (dk, jk), (dv, jv)):
        assert np.allclose(a, b, atol=1e-12)


def test_sampled_rows_and_columns_match_full_pass():
    N = 300
    q, k, v, do = small_case(B=2, H=2, N=N, d=8, seed=60)
    kw = dict(causal=True, key_lens=np.array([250, 300]), dropout_p=0.1, seed=4)
    O, L = oracle.attn_fwd(q, k, v, 0.3, **kw)
    dq, dk, dv, D = oracle.attn_bwd(q, k, v, do, 0.3, **kw)
    rows = np.array([0, 1, 5, 129, 299])
    cols = np.array([0, 3, 128, 249, 250, 299])
    Or, Lr = oracle.attn_fwd(q, k, v, 0.3, rows=rows, **kw)
    assert np.allclose(Or, O[:, :, rows], atol=1e-13) and np.allclose(Lr, L[:, :, rows], atol=1e-13)
    Ls, Ds = oracle.attn_stats(q, k, v, do, 0.3, **kw)
    assert np.allclose(Ls, L, atol=1e-13) and np.allclose(Ds, D, atol=1e-12)
    sub = np.array([3, 150, 298, 299])
    Lr2, Dr2 = oracle.attn_stats(q, k, v, do, 0.3, rows=sub, **kw)
    assert np.allclose(Lr2[:, :, sub], L[:, :, sub], atol=1e-13) and np.allclose(Dr2[:, :, sub], D[:, :, sub], atol=1e-12)
    assert not Lr2[:, :, 4].any() and not Dr2[:, :, 4].any()
    # causal: the last keys are seen only by the last rows, so those rows' stats suffice for them
    tail = np.arange(250, 300)
    Lt, Dt = oracle.attn_stats(q, k, v, do, 0.3, rows=tail, **kw)
    _, tk, tv = oracle.attn_bwd_rows_cols(q, k, v, do, 0.3, rows[:1], tail, Lt, Dt, **kw)
    assert np.allclose(tk, dk[:, :, tail], atol=1e-12) and np.allclose(tv, dv[:, :, tail], atol=1e-12)
    sq, sk, sv = oracle.attn_bwd_rows_cols(q, k, v, do, 0.3, rows, cols, Ls, Ds, **kw)
    assert np.allclose(sq, dq[:, :, rows], atol=1e-12)
    assert np.allclose(sk, dk[:, :, cols], atol=1e-12)
    assert np.allclose(sv, dv[:, :, cols], atol=1e-12)


# ---------------------------------------------------------------- dropout placement

def test_dropout_zero_is_dense():
    q, k, v, do = small_case(B=1, H=2, N=30, d=8, seed=70)
    a = oracle.attn_fwd(q, k, v, 0.3, dropout_p=0.0, seed=5)
    b = oracle.attn_fwd(q, k, v, 0.3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_dropout_scale_closed_form():
    """Q = 0 makes every valid weight 1/n; with V = I (N = d) the dropped
    forward is O_ij = s Z_ij / n exactly, s = 2^16 / (2^16 - thr) the keep
    scale: this pins dropout's placement after the softmax and before PV, its
    scale, and that the softmax normaliser ignores the mask (p = 0.1, where
    1/(1 - p) would differ)."""
    N = 16
    q = np.zeros((1, 2, N, N))
    k = np.random.default_rng(3).standard_normal((1, 2, N, N))
    v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
    O, L = oracle.attn_fwd(q, k, v, 0.5, dropout_p=0.1, seed=21, rng_offset=2)
    s = 65536 / (65536 - 6553)
    for h in range(2):
        Z = oracle.keep_mask(21, 2, 0.1, 0, h, 2, np.arange(N), np.arange(N))
        np.testing.assert_allclose(O[0, h], s * Z / N, rtol=0, atol=1e-15)
        np.testing.assert_allclose(L[0, h], np.log(N), rtol=0, atol=1e-14)


def test_dropout_is_unbiased_and_lse_undropped():
    """E_Z[O] = O at p = 0 (inverted dropout), statistically over seeds; LSE
    ignores the mask."""
    q, k, v, _ = small_case(B=1, H=1, N=6, d=3, seed=71)
    O0, L0 = oracle.attn_fwd(q, k, v, 0.5)
    outs = []
    for s in range(3000):
        O, L = oracle.attn_fwd(q, k, v, 0.5, dropout_p=0.5, seed=s)
        assert np.array_equal(L, L0)
        outs.append(O)
    outs = np.stack(outs)
    mean, se = outs.mean(0), outs.std(0) / np.sqrt(len(outs))
    assert (np.abs(mean - O0) <= 5 * se + 1e-12).all()


def test_standard_attention_baseline_matches_oracle():
    """The standard-attention comparison baseline (five separate ops and their
    backward, bench.py) computes the same function as the oracle: fp64 on the
    CPU, causal and not, without dropout; with dropout its keep mask applied
    to the oracle's P reproduces its O."""
    import bench
    rng = np.random.default_rng(12)
    B, H, N, d = 2, 3, 70, 16
    q, k, v, do = (torch.from_numpy(rng.standard_normal((B, H, N, d))) for _ in range(4))
    scale = float(np.float32(1 / np.sqrt(d)))         # the oracle takes the scale as float32
    for causal in (False, True):
        o, dq, dk, dv, _ = bench.standard_attention(q, k, v, do, scale, causal, 0.0)
        O, _ = oracle.attn_fwd(q, k, v, scale, causal=causal)
        dQ, dK, dV, _ = oracle.attn_bwd(q, k, v, do, scale, causal=causal)
        for got, want in ((o, O), (dq, dQ), (dk, dK), (dv, dV)):
            np.testing.assert_allclose(got.numpy(), want, atol=1e-12, rtol=1e-10)
    torch.manual_seed(0)
    o, *_, keep = bench.standard_attention(q, k, v, do, scale, True, 0.25)
    S = scale * np.einsum("bhid,bhjd->bhij", q.numpy(), k.numpy())
    S = np.where(np.tril(np.ones((N, N), dtype=bool)), S, -np.inf)
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    want = np.einsum("bhij,bhjd->bhid", P * keep.numpy() / 0.75, v.numpy())
    np.testing.assert_allclose(o.numpy(), want, atol=1e-12)


@pytest.mark.parametrize("N,Br,Bc,causal", [(70, 16, 8, False), (70, 8, 16, True), (64, 16, 16, True),
                                             (33, 32, 8, True), (5, 4, 4, False)])
def test_kv_outer_fwd_matches_definition(N, Br, Bc, causal):
    """The key/value-outer block order (running O, l, m stored between
    steps) reaches the plain definition's O and LSE."""
    rng = np.random.default_rng(N + Br + Bc)
    B, H, d = 2, 2, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) * 1.5 for _ in range(3))
    O, L, _ = oracle.kv_outer_fwd(q, k, v, 0.4, Br, Bc, causal=causal)
    O2, L2 = oracle.attn_fwd(q, k, v, 0.4, causal=causal)
    np.testing.assert_allclose(O, O2, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(L, L2, atol=1e-12, rtol=1e-12)


def test_kv_outer_io_counts_closed_form():
    """HBM element counts of the key/value-outer order (explainer,
    step-by-step algorithm): K and V once; every (query block, key block)
    step loads Q_i, O_i, l_i, m_i and stores O_i, l_i, m_i; plus the initial
    stores of O, l, m.  Non-causal: T_c steps per row, so Q and O traffic is
    T_c N d -- Theta(N^2 d / B_c), the summary's Theta(N^2 d^2 / M) with
    B_c ~ M / 4d.  Causal with B_r = B_c = b and N = T b: T (T + 1) / 2 steps."""
    B, H, d = 1, 3, 4
    for N, Br, Bc in ((48, 8, 16), (50, 16, 8), (7, 3, 2)):
        x = np.zeros((B, H, N, d))
        _, _, io = oracle.kv_outer_fwd(x, x, x, 1.0, Br, Bc, causal=False)
        Tc = -(-N // Bc)
        BH = B * H
        assert io["read"] == dict(Q=Tc * N * d * BH, K=N * d * BH, V=N * d * BH, O=Tc * N * d * BH,
                                  l=Tc * N * BH, m=Tc * N * BH)
        assert io["write"] == dict(O=(1 + Tc) * N * d * BH, l=(1 + Tc) * N * BH, m=(1 + Tc) * N * BH)
    T, b = 6, 8
    N = T * b
    x = np.zeros((B, H, N, d))
    _, _, io = oracle.kv_outer_fwd(x, x, x, 1.0, b, b, causal=True)
    steps = T * (T + 1) // 2
    assert io["read"]["Q"] == steps * b * d * H and io["read"]["O"] == steps * b * d * H
    assert io["read"]["K"] == N * d * H and io["write"]["l"] == (N + steps * b) * H


def test_kv_outer_byte_model_matches_oracle_counts():
    """bench.py's byte model of the key/value-outer order equals the oracle's
    element counts of that order (same blocks: 128 query rows by bc keys),
    weighted by the element sizes: e bytes for Q, K, V, O; 4 for l and m."""
    import bench
    d, e = 4, 2
    for N, bc, causal in ((300, 64, True), (300, 128, False), (129, 64, True)):
        x = np.zeros((1, 1, N, d))
        _, _, io = oracle.kv_outer_fwd(x, x, x, 1.0, 128, bc, causal=causal)
        _, _, mrd, mwr = bench.kv_outer_bytes(1, 1, N, d, e, causal, bc, 1)
        r, w = io["read"], io["write"]
        assert mrd == (r["Q"] + r["K"] + r["V"] + r["O"]) * e + (r["l"] + r["m"]) * 4
        assert mwr == w["O"] * e + (w["l"] + w["m"]) * 4
