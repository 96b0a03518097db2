"""Pins for the oracle's Philox4x32-10 and dropout keep rule."""

import os
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


# Known-answer vectors of Philox4x32-10 published with the generator's
# reference implementation (Salmon, Moraes, Dror, Shaw, "Parallel Random
# Numbers: As Easy as 1, 2, 3", SC'11, and its Random123 distribution):
# (counter words, key words) -> output words.
PHILOX4X32_10_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX4X32_10_KAT)
def test_known_answer_vectors(ctr, key, want):
    """All three oracle-side implementations (scalar, vectorised numpy, C)
    reproduce the published known answers: this pins the multipliers, the
    Weyl increments, the round structure and the word order."""
    assert philox.philox4_scalar(ctr, key, 32) == want
    vec = philox.philox4x32_10(*(np.array([c], dtype=np.uint64) for c in ctr), key[0], key[1])
    assert tuple(int(w[0]) for w in vec) == want
    c_out = philox_ref.batch(np.array([ctr], dtype=np.uint32), key[0], key[1])
    assert tuple(int(x) for x in c_out[0]) == want


_TRITON_PHILOX = r"""
import json, sys
import numpy as np, torch, triton, triton.language as tl

@triton.jit
def gen(c0, c1, c2, c3, o0, o1, o2, o3, seed, n: tl.constexpr):
    i = tl.arange(0, n)
    r0, r1, r2, r3 = tl.philox(seed, tl.load(c0 + i), tl.load(c1 + i), tl.load(c2 + i), tl.load(c3 + i), 10)
    tl.store(o0 + i, r0); tl.store(o1 + i, r1); tl.store(o2 + i, r2); tl.store(o3 + i, r3)

req = json.load(sys.stdin)
out = []
for seed, ctr in req:
    c = [torch.tensor(np.array(w, dtype=np.uint32)) for w in zip(*ctr)]
    o = [torch.zeros(len(ctr), dtype=torch.uint32) for _ in range(4)]
    gen[(1,)](*c, *o, seed, len(ctr))
    out.append([[int(o[w][i]) for w in range(4)] for i in range(len(ctr))])
json.dump(out, sys.stdout)
"""


def test_matches_triton_philox_on_cpu():
    """An independent Philox4x32-10: Triton's tl.philox (key = the seed's low
    and high 32-bit words), run on the CPU by Triton's interpreter, agrees
    word for word with the oracle over random counters and seeds."""
    import importlib.util
    import json
    import subprocess
    import sys
    if importlib.util.find_spec("triton") is None:
        pytest.skip("triton is not installed")
    rng = np.random.default_rng(17)
    req = []
    for _ in range(4):
        seed = int(rng.integers(0, 2 ** 63))
        ctr = rng.integers(0, 2 ** 32, size=(16, 4), dtype=np.uint64).tolist()
        req.append([seed, ctr])
    env = dict(os.environ, TRITON_INTERPRET="1")
    r = subprocess.run([sys.executable, "-c", _TRITON_PHILOX], input=json.dumps(req), capture_output=True,
                       text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    got = json.loads(r.stdout)
    for (seed, ctr), words in zip(req, got):
        for c, w in zip(ctr, words):
            assert tuple(w) == philox.philox4_scalar(c, (seed & 0xFFFFFFFF, seed >> 32), 32)


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


def test_keep_scale_is_the_inverse_keep_probability():
    """Inverted dropout: kept entries are scaled by 2^16 / (2^16 - thr), so over
    the 2^16 equally likely 16-bit uniforms the scaled keep bit averages
    exactly 1 (at p = 0.1: thr = 6553, scale 65536 / 58983, which 1 / (1 - p)
    misses by 1e-5)."""
    from fractions import Fraction
    for p in (0.1, 0.2, 0.25, 0.5, 0.9, 0.99999):
        thr = philox.dropout_threshold(p)
        s = philox.keep_scale(p)
        assert abs(s - 65536 / (65536 - thr)) <= 1e-15 * s
        u = np.arange(2 ** 16)
        mean = Fraction(int((u >= thr).sum()), 2 ** 16) * Fraction(s)
        assert abs(float(mean) - 1.0) < 1e-15
    assert philox.dropout_threshold(0.1) == 6553 and philox.keep_scale(0.1) == 65536 / 58983
    assert philox.keep_scale(0.0) == 1.0


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
