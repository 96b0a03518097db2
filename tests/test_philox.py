"""Pins for the oracle's Philox4x32-10 and dropout keep rule."""

from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import philox, philox_ref


def test_round_structure_matches_numpy_philox4x64():
    """The generic Philox-4xW round, at W = 64, reproduces numpy's independent
    Philox4x64-10 (numpy advances the counter by one before its first block)."""
    rng = np.random.default_rng(0)
    for _ in range(20):
        ctr = [int(x) for x in rng.integers(0, 2 ** 63, size=4)]
        key = [int(x) for x in rng.integers(0, 2 ** 63, size=2)]
        g = np.random.Philox(counter=sum(c << (64 * i) for i, c in enumerate(ctr)),
                             key=key[0] | (key[1] << 64))
        want = [int(x) for x in g.random_raw(4)]
        ctr1 = list(ctr)
        ctr1[0] += 1   # no carry for these draws (< 2^63)
        assert list(philox.philox4_scalar(ctr1, key, width=64)) == want


@pytest.mark.parametrize("width", [32, 64])
def test_weyl_constants_from_closed_forms(width):
    """Key increments: the golden ratio and sqrt(3) - 1 as W-bit fractions."""
    getcontext().prec = 80
    phi_frac = (Decimal(5).sqrt() - 1) / 2
    s3 = Decimal(3).sqrt() - 1
    w0 = int(phi_frac * (Decimal(2) ** width))
    w1 = int(s3 * (Decimal(2) ** width))
    assert philox.PHILOX_W[width] == (w0, w1)


def test_multipliers_are_odd_and_distinct():
    # odd multipliers make each round a bijection of the counter block
    for w in (32, 64):
        m0, m1 = philox.PHILOX_M[w]
        assert m0 % 2 == 1 and m1 % 2 == 1 and m0 != m1 and m0 < 2 ** w and m1 < 2 ** w


def test_vectorised_matches_scalar():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2 ** 32, size=(4, 500), dtype=np.uint64)
    k = rng.integers(0, 2 ** 32, size=2, dtype=np.uint64)
    out = philox.philox4x32_10(c[0], c[1], c[2], c[3], k[0], k[1])
    for n in range(0, 500, 37):
        want = philox.philox4_scalar([int(c[i, n]) for i in range(4)], [int(k[0]), int(k[1])], 32)
        assert tuple(int(out[i][n]) for i in range(4)) == want


def test_numpy_matches_independent_c_implementation():
    rng = np.random.default_rng(2)
    ctr = rng.integers(0, 2 ** 32, size=(4096, 4), dtype=np.uint64).astype(np.uint32)
    for k0, k1 in ((0, 0), (0xFFFFFFFF, 0xFFFFFFFF), (123456789, 987654321)):
        c_out = philox_ref.batch(ctr, k0, k1)
        n_out = np.stack(philox.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], k0, k1), axis=1)
        assert np.array_equal(c_out, n_out)


def test_threshold_from_float32_p():
    assert philox.dropout_threshold(0.1) == 6553           # float32(0.1) * 2^16 = 6553.6..., floored
    assert philox.dropout_threshold(0.0) == 0
    assert philox.dropout_threshold(0.5) == 2 ** 15
    assert philox.dropout_threshold(0.25) == 2 ** 14
    assert philox.dropout_threshold(2.0 ** -17) == 0       # below one step of 2^-16
    assert philox.dropout_threshold(np.nextafter(np.float32(1), np.float32(0))) == 2 ** 16 - 1


def test_keep_mask_counter_layout_elementwise():
    """keep_mask equals the documented counter layout evaluated one element at a time."""
    seed, off, p, H = 0x1234_5678_9ABC_DEF0, 0x1_0000_0007, 0.3, 3
    rows, cols = np.array([0, 1, 2, 77, 510, 511]), np.arange(0, 23)
    thr = philox.dropout_threshold(p)
    for b, h in ((0, 0), (2, 1)):
        km = philox.keep_mask(seed, off, p, b, h, H, rows, cols)
        for a, i in enumerate(rows):
            for c, j in enumerate(cols):
                w = philox.philox4_scalar((j >> 2, i >> 1, b * H + h, off & 0xFFFFFFFF),
                                          (seed & 0xFFFFFFFF, seed >> 32), 32)
                u = (w[j & 3] >> 16) if i & 1 else (w[j & 3] & 0xFFFF)
                assert km[a, c] == (u >= thr)


def test_keep_rate_is_binomial():
    p = 0.1
    km = philox.keep_mask(3, 0, p, 0, 0, 1, np.arange(512), np.arange(512))
    n = km.size
    kept = km.sum()
    mean = n * (1 - p)
    sd = np.sqrt(n * p * (1 - p))
    assert abs(kept - mean) < 6 * sd


def test_streams_differ_across_heads_and_offsets():
    rows, cols = np.arange(64), np.arange(256)
    a = philox.keep_mask(3, 0, 0.5, 0, 0, 2, rows, cols)
    b = philox.keep_mask(3, 0, 0.5, 0, 1, 2, rows, cols)
    c = philox.keep_mask(3, 1, 0.5, 0, 0, 2, rows, cols)
    d = philox.keep_mask(4, 0, 0.5, 0, 0, 2, rows, cols)
    for x in (b, c, d):
        assert (a != x).mean() > 0.4
    # no two rows of one stream repeat
    assert len({r.tobytes() for r in a}) == len(a)


def test_row_pairs_use_independent_halves():
    """Rows 2m and 2m+1 share generator calls but read different 16-bit halves:
    at p = 1/2 their keep bits agree about half the time, as for independent
    rows, and neither row repeats its pair partner."""
    rows, cols = np.arange(256), np.arange(512)
    km = philox.keep_mask(11, 5, 0.5, 1, 2, 4, rows, cols)
    agree = (km[0::2] == km[1::2])
    n = agree.size
    assert abs(agree.sum() - n / 2) < 6 * np.sqrt(n / 4)
    assert not any(np.array_equal(km[2 * m], km[2 * m + 1]) for m in range(128))
    # and the halves are the only difference: the pair's counter is shared
    w = philox.philox4_scalar((3, 7, 1 * 4 + 2, 5), (11, 0), 32)
    assert [bool((x & 0xFFFF) >= 2 ** 15) for x in w] == list(km[14, 12:16])
    assert [bool((x >> 16) >= 2 ** 15) for x in w] == list(km[15, 12:16])
