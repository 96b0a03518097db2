"""Pins for the expected tile-visit sets and valid-pair counts (brute force)."""

import numpy as np
import pytest

import oracle
from oracle.attention import validity


def brute_tiles(N, Br, Bc, B, causal, key_lens, block_mask):
    Tr, Tc = -(-N // Br), -(-N // Bc)
    out = np.zeros((B, Tr, Tc), np.uint8)
    for b in range(B):
        kl = None if key_lens is None else key_lens[b]
        A = validity(np.arange(N), N, causal, kl, block_mask)
        for i in range(Tr):
            for j in range(Tc):
                out[b, i, j] = A[i * Br:(i + 1) * Br, j * Bc:(j + 1) * Bc].any()
    return out


@pytest.mark.parametrize("N", [1, 100, 257, 400])
@pytest.mark.parametrize("Br,Bc", [(128, 64), (32, 128), (64, 64), (48, 80)])
def test_expected_tiles_brute_force(N, Br, Bc):
    rng = np.random.default_rng(N + Br)
    T = -(-N // 128)
    bm = (rng.random((T, T)) < 0.5).astype(np.uint8)
    kls = np.array([0, max(N // 3, 1), N])
    for causal in (False, True):
        for key_lens in (None, kls):
            for block_mask in (None, bm):
                got = oracle.expected_tiles(N, Br, Bc, 3, causal, key_lens, block_mask)
                want = brute_tiles(N, Br, Bc, 3, causal, key_lens, block_mask)
                assert np.array_equal(got, want)


def test_causal_tile_count_and_ones_mask():
    T = 16
    t = oracle.expected_tiles(T * 64, 64, 64, 1, causal=True)
    assert t.sum() == T * (T + 1) // 2
    ones = np.ones((8, 8), np.uint8)
    assert np.array_equal(oracle.expected_tiles(1000, 128, 64, 2, block_mask=ones),
                          oracle.expected_tiles(1000, 128, 64, 2))


@pytest.mark.parametrize("N", [5, 130, 300])
def test_valid_pair_count_brute_force(N):
    rng = np.random.default_rng(N)
    T = -(-N // 128)
    bm = (rng.random((T, T)) < 0.6).astype(np.uint8)
    kls = np.array([N // 2, N])
    for causal in (False, True):
        for key_lens in (None, kls):
            for block_mask in (None, bm):
                want = sum(validity(np.arange(N), N, causal, None if key_lens is None else key_lens[b],
                                    block_mask).sum() for b in range(2)) * 3
                assert oracle.valid_pair_count(N, 2, 3, causal, key_lens, block_mask) == want


def test_valid_pairs_closed_forms():
    assert oracle.valid_pair_count(1024, 8, 12, causal=True) == 8 * 12 * 1024 * 1025 // 2
    assert oracle.valid_pair_count(16384, 1, 16, causal=True) == 2147614720


def test_bench_work_counts_match_oracle():
    """bench.py counts algorithmic work itself (its timed path does not
    import the oracle): its valid-pair count equals the oracle's on every
    workload's recipe at reduced size, and its decode byte count is the
    closed form (valid cache rows of K and V, Q, O, LSE)."""
    import bench
    import workloads as W
    for name in ("tiny", "gpt2", "bert", "long", "sparse", "gqa"):
        w = W.WORKLOADS[name]
        small = w.with_(B=min(w.B, 2), H=2, N=min(w.N, 640), d=8)
        if small.key_len_range is not None:
            small = small.with_(key_len_range=(100, 640))
        x = W.make_inputs(small, with_do=False)
        kl = None if x["key_lens"] is None else x["key_lens"].numpy()
        bm = None if x["block_mask"] is None else x["block_mask"].numpy()
        assert bench.valid_pairs(x, small) == oracle.valid_pair_count(small.N, small.B, small.H, small.causal,
                                                                      kl, bm), name
    w = W.WORKLOADS["decode"].with_(B=3, N=500, d=16, key_len_range=(10, 500))
    x = W.make_inputs(w, with_do=False)
    rd, wr = bench.decode_bytes(x, w)
    L = x["key_lens"].numpy().astype(np.int64)
    assert rd == int(L.sum()) * w.Hkv * w.d * 2 * 2 + w.B * w.H * 1 * w.d * 2
    assert wr == w.B * w.H * 1 * (w.d * 2 + 4)


def test_bench_roofline_bound_follows_intensity():
    """The dominant kernel is rated against HBM when its FLOP per minimum byte
    is below the ridge (2.5 PFLOP/s / 8 TB/s = 312.5), else against MFMA: the
    BERT-shaped workload (d = 64, N = 512, padded keys) is HBM-bound, the long
    causal one MFMA-bound (the pages' own classification of the configs)."""
    import bench
    import workloads as W
    ms = {"fwd_kernel": 1.0, "bwd_kv_kernel": 2.0, "bwd_dq_kernel": 1.5}
    long = W.WORKLOADS["long"]
    r, k = bench.dominant_roofline(long, oracle.valid_pair_count(long.N, long.B, long.H, True), ms)
    assert r["bound"] == "mfma" and r["kernel"] == "bwd_kv_kernel" and r["unit"] == "TFLOP/s"
    assert k["fwd_kernel"][2] == 4 * 16 * 16384 * 128 * 2 + 16 * 16384 * 4     # 4 BHNd e + 4 BHN
    bert = W.WORKLOADS["bert"]
    pairs = bert.H * 320 * bert.B * bert.N                                      # E[len] = 320
    r, _ = bench.dominant_roofline(bert, pairs, ms)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["flop_per_byte"] < 312.5
