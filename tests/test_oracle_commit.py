"""Pins of the oracle's KV commit: the fp32 -> fp16 conversion, the Q4_0
quantiser reading and the row placement of the accepted path.

The pages keep the target's KV cache in Q4_0 or F16 and accept a root path
each step, but print no quantiser, so what pins the quantiser is: numpy's own
fp16 conversion (a library routine) for the scale, a block worked by hand
(tests/golden/q4_0_quantize_worked_block.txt), exact round trips of values
that lie on a block's code lattice, the error bound of rounding to the
nearest code, and the special blocks (zeros, one nonzero value).
"""

import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    vals = bts = None
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("values:"):
            vals = np.array([float(t) for t in line.split()[1:]], np.float32)
        elif line.startswith("bytes:"):
            bts = np.array([int(t, 16) for t in line.split()[1:]], np.uint8)
    return vals, bts


def test_float_to_half_matches_numpy():
    rng = np.random.default_rng(3)
    xs = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 18, 20000),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 70000.0, 2 ** -14, 2 ** -24, 2 ** -25,
                  3 * 2 ** -26, 2 ** -25 * 1.0000001, 6.1e-5, np.inf, -np.inf], np.float32),
        # exact ties between two fp16 neighbours, normal and subnormal
        ((np.arange(1, 2000, dtype=np.float64) + 0.5) * 2.0 ** -10).astype(np.float32),
        ((np.arange(1, 1000, dtype=np.float64) + 0.5) * 2.0 ** -24).astype(np.float32),
    ])
    got = np.array([oracle.float_to_half(x) for x in xs], np.uint16)
    with np.errstate(over="ignore"):  # values past 65520 become infinity on both sides
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.float_to_half(np.float32(np.nan)) & 0x7C00 == 0x7C00
    assert oracle.float_to_half(np.float32(np.nan)) & 0x03FF != 0


def test_hand_worked_block():
    vals, bts = _read("q4_0_quantize_worked_block.txt")
    assert np.array_equal(oracle.q4_0_quantize(vals), bts)
    # the same codes when the values are rounded to fp16 first
    assert np.array_equal(oracle.q4_0_quantize(vals.astype(np.float16).astype(np.float32)), bts)


def test_decode_block_round_trip():
    """The decode-side worked block re-quantises to its own bytes."""
    vals = bts = None
    for line in open(os.path.join(GOLDEN, "q4_0_worked_block.txt")):
        if line.startswith("values:"):
            vals = np.array([float(t) for t in line.split()[1:]], np.float32)
        elif line.startswith("bytes:"):
            bts = np.array([int(t, 16) for t in line.split()[1:]], np.uint8)
    assert np.array_equal(oracle.q4_0_quantize(vals), bts)


def test_lattice_round_trip():
    """Values s * (c - 8) with some code 0 (the unique largest magnitude)
    come back as exactly their own block, for any nonzero fp16 scale."""
    rng = np.random.default_rng(11)
    for _ in range(3000):
        s = np.float16(rng.choice([-1, 1]) * rng.uniform(1e-3, 50.0))
        if rng.random() < 0.1:
            s = np.float16(rng.choice([-1, 1]) * rng.integers(1, 1024)) * np.float16(2.0 ** -24)  # subnormal scale
        if s == 0:
            continue
        codes = rng.integers(0, 16, 32)
        codes[rng.integers(0, 32)] = 0
        x = (np.float32(s) * (codes - 8)).astype(np.float32)
        blk = np.zeros(18, np.uint8)
        blk[0:2] = np.array([s], np.float16).view(np.uint8)
        blk[2:] = (codes[:16] | (codes[16:] << 4)).astype(np.uint8)
        assert np.array_equal(oracle.q4_0_quantize(x), blk), (s, codes)
        assert np.array_equal(oracle.q4_0_dequant(blk, 32), x.astype(np.float64))


def test_error_bound_random_blocks():
    """Every value decodes within half a step of the block's scale, except
    values beyond 7.5 steps on the side opposite to m, which the top code 15
    caps (error t - 7 steps for t = -8x/m in (7.5, 8]); plus the fp16 rounding
    of the scale."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4000, 32)) * rng.uniform(0.01, 100, (4000, 1))).astype(np.float32)
    q = oracle.q4_0_quantize(x)
    dec = oracle.q4_0_dequant(q, 32)
    xd = x.astype(np.float64)
    m = xd[np.arange(len(x)), np.abs(xd).argmax(axis=1)]
    d = np.abs(m) / 8
    scale = np.abs(q[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64))
    assert np.all(np.abs(scale - d) <= d * 2.0 ** -11 + 1e-30)
    t = -8 * xd / m[:, None]
    steps = np.maximum(0.5, t - 7)
    lim = steps * d[:, None] * (1 + 1e-6) + 8 * np.abs(scale - d)[:, None]
    assert np.all(np.abs(dec - xd) <= lim + 1e-30)
    assert np.any(t > 7.5)  # the capped case occurs in this sample
    # the value of largest magnitude decodes to itself whenever m/8 is exact in fp16
    exact = scale == d
    assert np.all(dec[np.arange(len(x)), np.abs(xd).argmax(axis=1)][exact] == m[exact])


def test_special_blocks():
    z = np.zeros(32, np.float32)
    # a block of zeros stores the scale +0 (m / -8 alone would give -0) and
    # code 8 everywhere; it decodes to zeros
    assert np.array_equal(oracle.q4_0_quantize(z), np.array([0x00, 0x00] + [0x88] * 16, np.uint8))
    assert np.array_equal(oracle.q4_0_quantize(-z), np.array([0x00, 0x00] + [0x88] * 16, np.uint8))
    assert not oracle.q4_0_dequant(oracle.q4_0_quantize(z), 32).any()
    one = z.copy()
    one[5] = 3.0  # d = -0.375 (fp16 0xB600); element 5 gets code 0, all others code 8
    exp = np.array([0x00, 0xB6] + [0x88] * 16, np.uint8)
    exp[2 + 5] = 0x80
    assert np.array_equal(oracle.q4_0_quantize(one), exp)


def _tree_rows(rng, n, hkv, d):
    return (rng.standard_normal((n, hkv, d)) * 0.5).astype(np.float16)


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_commit_places_the_path(kv):
    rng = np.random.default_rng(21)
    n, hkv, D, cap, n_ctx = 9, 2, 64, 40, 17
    kt, vt = _tree_rows(rng, n, hkv, D), _tree_rows(rng, n, hkv, D)
    if kv == "q4_0":
        kc = rng.integers(0, 256, (hkv, cap, 36)).astype(np.uint8)
        vc = rng.integers(0, 256, (hkv, cap, 36)).astype(np.uint8)
    else:
        kc = rng.standard_normal((hkv, cap, D)).astype(np.float16)
        vc = rng.standard_normal((hkv, cap, D)).astype(np.float16)
    path = [0, 2, 5, 7]
    res = np.full(2 + 2 * n, -1, np.int32)
    res[0] = len(path) - 1
    res[1] = 42
    res[2:2 + len(path)] = path
    k2, v2 = oracle.commit(res, kt, vt, kc, vc, n_ctx)
    touched = np.zeros(cap, bool)
    touched[n_ctx:n_ctx + len(path)] = True
    assert np.array_equal(k2[:, ~touched], kc[:, ~touched]) and np.array_equal(v2[:, ~touched], vc[:, ~touched])
    for r, node in enumerate(path):
        for g in range(hkv):
            for src, dst in ((kt, k2), (vt, v2)):
                if kv == "f16":
                    assert np.array_equal(dst[g, n_ctx + r].view(np.uint16), src[node, g].view(np.uint16))
                else:
                    assert np.array_equal(dst[g, n_ctx + r], oracle.q4_0_quantize(src[node, g].astype(np.float32)))
                    dec = oracle.q4_0_dequant(dst[g, n_ctx + r], D)
                    step = np.repeat(np.abs(src[node, g].astype(np.float64).reshape(-1, 32)).max(1) / 8, 32)
                    assert np.all(np.abs(dec - src[node, g]) <= step * (1 + 2 ** -8) + 1e-30)


def test_commit_root_only_and_errors():
    rng = np.random.default_rng(2)
    n, hkv, D, cap = 4, 1, 32 * 2, 10
    kt, vt = _tree_rows(rng, n, hkv, D), _tree_rows(rng, n, hkv, D)
    kc = np.zeros((hkv, cap, D), np.float16)
    vc = np.zeros((hkv, cap, D), np.float16)
    res = np.array([0, 3, 0, -1, -1, -1, 3, -1, -1, -1], np.int32)
    k2, _ = oracle.commit(res, kt, vt, kc, vc, 6)
    assert np.array_equal(k2[0, 6], kt[0, 0]) and not k2[0, 7].any() and not k2[0, 5].any()
    with pytest.raises(ValueError):
        oracle.commit(res, kt, vt, kc, vc, 7)  # n_ctx + n > capacity
    bad = res.copy()
    bad[0] = 4  # n_acc must be < n
    with pytest.raises(ValueError):
        oracle.commit(bad, kt, vt, kc, vc, 0)
