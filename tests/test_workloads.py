"""The seeded input recipe: shapes, seeds, key lengths and the block mask."""

import numpy as np
import torch

import workloads as W


def test_block_mask_band_and_density():
    T = 128
    m = W.band_random_block_mask(T, 0.1, np.random.default_rng(5))
    i, j = np.indices((T, T))
    assert m[np.abs(i - j) <= 1].all()
    assert (np.abs(i - j) <= 1).sum() == 382
    assert m.sum() == round(0.1 * T * T) == 1638
    m2 = W.band_random_block_mask(T, 0.1, np.random.default_rng(5))
    assert np.array_equal(m, m2)


def test_inputs_are_reproducible_and_rounded():
    w = W.WORKLOADS["tiny"]
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for n in ("q", "k", "v", "do"):
        assert a[n].dtype == torch.bfloat16 and a[n].shape == (1, 2, 256, 64)
        assert torch.equal(a[n], b[n])
    f = W.make_inputs(w, dtype="fp32")
    # the bf16 tensor is the rounding of the same fp64 draw as the fp32 one
    rng = np.random.default_rng(0)
    q64 = rng.standard_normal((1, 2, 256, 64))
    assert torch.equal(f["q"], torch.from_numpy(q64).float())
    assert torch.equal(a["q"], torch.from_numpy(q64).to(torch.bfloat16))


def test_key_lengths_and_sparse_mask_recipe():
    w = W.WORKLOADS["bert"].with_(B=64, N=64, H=1, d=8)
    x = W.make_inputs(w)
    kl = x["key_lens"].numpy()
    assert kl.dtype == np.int32 and kl.min() >= 128 and kl.max() <= 512
    s = W.WORKLOADS["sparse"].with_(H=1, d=8)   # small head dim, same N and mask recipe
    y = W.make_inputs(s, with_do=False)
    assert y["block_mask"].shape == (128, 128) and int(y["block_mask"].sum()) == 1638


def test_sample_rows():
    r = W.sample_rows(16384, 256, 4)
    assert len(r) == 256 and (r[:16] == np.arange(16)).all() and (np.diff(r) > 0).all()


def test_grouped_query_shapes():
    w = W.WORKLOADS["gqa"].with_(B=1, N=64, d=8)
    x = W.make_inputs(w)
    assert x["q"].shape == x["do"].shape == (1, 32, 64, 8)
    assert x["k"].shape == x["v"].shape == (1, 8, 64, 8)
    # MHA workloads keep their draws: K/V heads default to H
    assert W.WORKLOADS["tiny"].Hkv == 2


def test_decode_workload_shapes():
    w = W.WORKLOADS["decode"].with_(B=3, N=300, d=8, key_len_range=(100, 300))
    x = W.make_inputs(w)
    assert x["q"].shape == (3, 32, 1, 8) and x["k"].shape == x["v"].shape == (3, 8, 300, 8)
    assert "do" not in x
    kl = x["key_lens"].numpy()
    assert kl.min() >= 100 and kl.max() <= 300
