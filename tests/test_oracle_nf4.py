"""Pins for the oracle's NF4 codebook, encoder, packing and dequantization."""
import math

import numpy as np
import pytest
from scipy.stats import norm

import oracle
from oracle.nf4 import DELTA
from conftest import golden_rows


def test_norm_ppf_textbook_values():
    for row in golden_rows("normal_quantiles.txt"):
        p, x = map(float, row.split())
        assert abs(oracle.norm_ppf(p) - x) <= 2e-15 * max(1.0, abs(x))
        if p != 0.5:
            assert abs(oracle.norm_ppf(1.0 - p) + x) <= 2e-15 * max(1.0, abs(x))


def test_norm_ppf_matches_independent_library():
    # error allowed: a few ulps of p divided by the density (the quantile's conditioning)
    for p in np.linspace(0.5005, 0.999, 37):
        x = norm.ppf(p)
        assert abs(oracle.norm_ppf(float(p)) - x) <= 1e-15 + 4e-16 / norm.pdf(x)


def test_codebook_printed_values():
    cb = oracle.nf4_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    for row in golden_rows("nf4_printed_levels.txt"):
        i, v = row.split()
        assert round(float(cb[int(i)]), 4) == float(v)
    assert cb[0] == -1.0 and cb[15] == 1.0


def test_codebook_shape_of_levels():
    cb = oracle.nf4_codebook()
    assert np.all(np.diff(cb) > 0)
    assert cb[7] == 0.0
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8


def test_codebook_is_normal_quantiles():
    """Each level times Phi^-1(delta) sits at the evenly spaced probabilities (scipy CDF)."""
    cb = oracle.nf4_codebook().astype(np.float64)
    zmax = norm.ppf(DELTA)
    pos = cb[8:] * zmax
    neg = -cb[:7] * zmax
    assert np.allclose(norm.cdf(pos[::-1]), np.linspace(DELTA, 0.5, 9)[:-1], atol=2e-8)
    assert np.allclose(norm.cdf(neg), np.linspace(DELTA, 0.5, 8)[:-1], atol=2e-8)


def test_delta_window_from_printed_values():
    """The two printed interior levels pin delta to a narrow window; the reading lies in it."""
    inside = []
    for d in np.linspace(0.96760, 0.96780, 401):
        cb = oracle.nf4_codebook(float(d))
        if round(float(cb[1]), 4) == -0.6962 and round(float(cb[2]), 4) == -0.5251:
            inside.append(d)
    assert inside, "no delta reproduces the printed levels"
    assert min(inside) <= DELTA <= max(inside)
    assert max(inside) - min(inside) < 1e-4


def test_encode_worked_block():
    rows = [r.split() for r in golden_rows("nf4_worked_block.txt")]
    vals = np.array([float(r[0]) for r in rows], dtype=np.float32)
    want = np.array([int(r[2]) for r in rows])
    codes, am = oracle.quantize_residual(vals, blocksize=len(vals))
    assert am[0] == 2.0
    assert np.array_equal(codes, want)


def test_encode_round_trip_of_levels():
    cb = oracle.nf4_codebook()
    for e in (-3, 0, 5):
        a = np.float32(2.0 ** e)
        R = (cb * a).astype(np.float32)   # exact: power-of-two scale
        codes, am = oracle.quantize_residual(R, blocksize=16)
        assert am[0] == a
        assert np.array_equal(codes, np.arange(16))
        deq = oracle.dequantize(codes, am, blocksize=16)
        assert np.array_equal(deq.view(np.uint32), R.view(np.uint32))


def _block_with_unit_absmax(xs):
    xs = np.asarray(xs, dtype=np.float32)
    out = np.concatenate([xs, np.ones(1, np.float32)])
    return out


def test_encode_transitions_at_midpoints():
    """Code changes exactly where x passes a midpoint of neighbouring fp32 levels."""
    m = oracle.nf4_midpoints()
    for j, mj in enumerate(m):
        below = np.float32(mj)
        if float(below) > mj:
            below = np.nextafter(below, np.float32(-2))
        above = np.nextafter(below, np.float32(2))
        assert float(below) <= mj < float(above)
        R = _block_with_unit_absmax([below, above])
        codes = oracle.nf4_encode(R, np.array([1.0], np.float32), blocksize=R.size)
        assert codes[0] == j and codes[1] == j + 1, (j, codes)


def test_encode_ties_go_to_lower_code():
    m = oracle.nf4_midpoints()
    exact = [j for j, mj in enumerate(m) if float(np.float32(mj)) == mj]
    assert len(exact) >= 1
    R = _block_with_unit_absmax([np.float32(m[j]) for j in exact])
    codes = oracle.nf4_encode(R, np.array([1.0], np.float32), blocksize=R.size)
    assert list(codes[:-1]) == exact


def test_encode_monotone_and_zero_block():
    x = np.sort(np.random.default_rng(1).uniform(-1, 1, 20000).astype(np.float32))
    R = _block_with_unit_absmax(x)
    codes = oracle.nf4_encode(R, np.array([1.0], np.float32), blocksize=R.size)
    assert np.all(np.diff(codes[:-1].astype(int)) >= 0)
    z = np.zeros(130, np.float32)
    c, am = oracle.quantize_residual(z)
    assert np.all(am == 0) and np.all(c == 7)
    assert np.all(oracle.dequantize(c, am) == 0)


def test_absmax_ragged_tail():
    r = np.arange(1, 151, dtype=np.float32) * np.where(np.arange(150) % 2, -1, 1)
    am = oracle.block_absmax(r, 64)
    assert am.tolist() == [64.0, 128.0, 150.0]


def test_nibble_order_fixture():
    for row in golden_rows("nibble_order.txt"):
        left, right = row.split("|")
        codes = np.array([int(v) for v in left.split()], np.uint8)
        want = bytes.fromhex(right.replace(" ", ""))
        packed = oracle.pack_nibbles(codes)
        assert packed.tobytes() == want
        assert np.array_equal(oracle.unpack_nibbles(packed, codes.size), codes)


def test_dequantize_residual_rounding():
    """E = fl32(W - fl32(c * a)) is one correctly rounded fp32 op per step."""
    rng = np.random.default_rng(3)
    W = rng.standard_normal(256).astype(np.float32)
    codes, am = oracle.quantize_residual(W)
    E = oracle.dequantize(codes, am, W=W)
    cb = oracle.nf4_codebook()
    deq32 = np.array([np.float32(cb[c]) * np.float32(am[i // 64]) for i, c in enumerate(codes)],
                     dtype=np.float32)
    assert np.array_equal(E, (W - deq32).astype(np.float32))


def test_nf4_relative_error_on_gaussian():
    """Plain NF4 (blockwise 64) on Gaussian data: relative error ~0.092 (level spacing / sqrt 12)."""
    W = (0.02 * np.random.default_rng(7).standard_normal(1 << 16)).astype(np.float32)
    codes, am = oracle.quantize_residual(W)
    E = oracle.dequantize(codes, am, W=W).astype(np.float64)
    rel = math.sqrt(np.sum(E * E) / np.sum(W.astype(np.float64) ** 2))
    assert 0.085 < rel < 0.10


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_non_finite_rejected(bad):
    with pytest.raises(ValueError):
        oracle.quantize_residual(np.array([1.0, bad], np.float32))


def test_lower_bit_codebooks_reduce_to_nf4_and_closed_forms():
    assert oracle.nf_delta(4) == DELTA
    assert np.array_equal(oracle.nf_codebook(4).view(np.uint32), oracle.nf4_codebook().view(np.uint32))
    # 2 bits: one negative level (-1), zero, and two positive quantiles of
    # {delta_2, (delta_2 + 1/2) / 2}, normalised by the larger one (library quantiles)
    d2 = 1.0 - 0.5 * (1.0 / 8.0 + 1.0 / 6.0)
    assert oracle.nf_delta(2) == d2
    hi, lo = norm.ppf(d2), norm.ppf(0.5 * (d2 + 0.5))
    assert np.allclose(oracle.nf_codebook(2), [-1.0, 0.0, lo / hi, 1.0], rtol=0, atol=1e-7)
    # 3 bits from the same definition written with library quantiles
    d3 = 1.0 - 0.5 * (1.0 / 16.0 + 1.0 / 14.0)
    pos = norm.ppf(np.linspace(d3, 0.5, 5)[:-1])
    neg = -norm.ppf(np.linspace(d3, 0.5, 4)[:-1])
    ref = np.sort(np.concatenate([pos, neg, [0.0]]))
    assert np.allclose(oracle.nf_codebook(3), ref / np.max(np.abs(ref)), rtol=0, atol=1e-7)


@pytest.mark.parametrize("bits", [2, 3])
def test_lower_bit_codebook_structure_and_round_trip(bits):
    cb = oracle.nf_codebook(bits)
    n = 2 ** bits
    assert cb.shape == (n,) and cb.dtype == np.float32
    assert np.all(np.diff(cb.astype(np.float64)) > 0)
    assert cb[0] == -1.0 and cb[-1] == 1.0 and cb[n // 2 - 1] == 0.0
    # every level quantizes to its own index (absmax 1 via the +1 level in each block)
    R = np.tile(np.concatenate([cb, np.ones(64 - n, np.float32)]), 3)
    codes, am = oracle.quantize_residual(R, 64, cb)
    assert np.all(am == 1.0)
    assert np.array_equal(codes.reshape(3, 64)[:, :n], np.tile(np.arange(n), (3, 1)))
    # a zero block encodes as the zero level
    z, za = oracle.quantize_residual(np.zeros(64, np.float32), 64, cb)
    assert np.all(z == n // 2 - 1) and za[0] == 0.0
