"""Pins for the oracle's double quantization (own invariants only) and sketch generator."""
import numpy as np

import oracle
from conftest import golden_rows


def test_double_quant_invariants():
    rng = np.random.default_rng(11)
    a = np.abs(rng.standard_normal(1000)).astype(np.float32) * 0.05
    q, s = oracle.double_quant(a, 256)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s.size == 4  # ragged last group of 232
    ap = oracle.dq_scales_expand(q, s, 256)
    for g in range(4):
        blk = slice(g * 256, min(1000, (g + 1) * 256))
        m = a[blk].max()
        assert s[g] == np.float32(np.float64(m) / 127.0)
        assert q[blk][np.argmax(a[blk])] == 127
        assert np.all(q[blk] >= 0)
        err = np.abs(a[blk].astype(np.float64) - ap[blk].astype(np.float64))
        assert np.all(err <= 0.5 * float(s[g]) * (1 + 1e-6) + 1e-12)


def test_double_quant_exact_multiples_round_trip():
    s = np.float32(0.25)
    a = (np.arange(0, 128, dtype=np.float32) * s).astype(np.float32)  # max = 127 * 0.25
    q, sc = oracle.double_quant(a, 256)
    assert sc[0] == s
    assert np.array_equal(q, np.arange(128).astype(np.int8))
    assert np.array_equal(oracle.dq_scales_expand(q, sc), a)


def test_double_quant_zero_group():
    q, s = oracle.double_quant(np.zeros(300, np.float32), 256)
    assert np.all(q == 0) and np.all(s == 0)
    assert np.all(oracle.dq_scales_expand(q, s) == 0)


def test_storage_bits_per_parameter():
    """4 + 32/64 = 4.5 bits without double quant; 4 + 8/64 + 32/(64*256) with it."""
    n = 64 * 256 * 8
    codes = n * 4
    single = (codes + (n // 64) * 32) / n
    dq = (codes + (n // 64) * 8 + (n // 64 // 256) * 32) / n
    assert single == 4.5
    assert abs(dq - (4 + 8 / 64 + 32 / (64 * 256))) < 1e-12


def test_splitmix64_published_outputs():
    want = [int(v, 16) for v in golden_rows("splitmix64_seed0.txt")]
    got = oracle.splitmix64_stream(0, np.arange(5))
    assert [int(v) for v in got] == want


def test_rademacher_sketch_layout():
    k, l = 300, 24
    om = oracle.rademacher_sketch(42, 2, k, l)
    assert om.shape == (k, l) and set(np.unique(om)) == {-1.0, 1.0}
    # entry (i, j) of alternation t is output number ((t-1)k + i) l + j
    z = oracle.splitmix64_stream(42, np.array([(1 * k + 5) * l + 7], dtype=np.uint64))[0]
    assert om[5, 7] == (1.0 if (int(z) >> 63) == 0 else -1.0)
    assert abs(om.mean()) < 0.05
    assert not np.array_equal(om, oracle.rademacher_sketch(42, 1, k, l))


def test_double_quant_tie_rule_golden():
    """Quotients exactly halfway between two codes go to the even code (hand-worked table)."""
    rows = [ln.split() for ln in golden_rows("dq_tie_rounding.txt")]
    a = np.array([float(r[0]) for r in rows], dtype=np.float32)
    want = np.array([int(r[1]) for r in rows], dtype=np.int8)
    q, s = oracle.double_quant(a, 256)
    assert s[0] == np.float32(1.0)
    assert np.array_equal(q, want)
