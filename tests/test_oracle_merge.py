"""Pins for the oracle's adapter merge / unmerge (PEFT guide, "量化": merging adapters
into quantized weights = dequantize, add the adapter, quantize again)."""
import numpy as np

import oracle
from conftest import golden_rows


def _base(rows, cols, seed):
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((rows, cols))).astype(np.float32)
    codes, am = oracle.quantize_residual(W.ravel())
    return codes, am


def test_worked_block():
    rows = [r.split() for r in golden_rows("merge_worked_block.txt")]
    codes = np.full(64, 7, np.uint8)
    A = np.zeros((1, 64))
    expect = np.full(64, 7, np.uint8)
    for col, cin, adapter, _, _, cout in rows:
        codes[int(col)] = int(cin)
        A[0, int(col)] = float(adapter)
        expect[int(col)] = int(cout)
    out = oracle.merge_adapter(codes, np.array([2.0], np.float32), np.array([[1.0]]), A, double_quant_on=False)
    assert np.array_equal(out["codes"], expect)
    assert out["absmax"][0] == np.float32(2.0)


def test_zero_adapter_requantizes_to_the_same_codes():
    # every block's largest element decodes to exactly +-a (code 0 or 15), and every
    # decoded c_j a re-encodes to level j (levels are >= 0.0796 apart; the round trip
    # moves x by at most two ulps), so Q is a fixed point of NF4(deq(.))
    codes, am = _base(48, 320, 1)
    for B, A in ((None, None), (np.zeros((48, 4)), np.zeros((4, 320)))):
        out = oracle.merge_adapter(codes, am, B, A, double_quant_on=False)
        assert np.array_equal(out["codes"], codes)
        assert np.array_equal(out["absmax"], am)


def test_doubling_adapter_doubles_the_scales():
    # B A = deq(Q) (a full-rank "adapter": B = deq(Q), A = I): the sum is 2 deq(Q)
    # exactly, so every absmax doubles and the codes stay
    rows, cols = 16, 192
    codes, am = _base(rows, cols, 2)
    D = oracle.dequantize(codes, am).reshape(rows, cols).astype(np.float64)
    out = oracle.merge_adapter(codes, am, D, np.eye(cols), double_quant_on=False)
    assert np.array_equal(out["codes"], codes)
    assert np.array_equal(out["absmax"], (2 * am.astype(np.float64)).astype(np.float32))


def test_cancelling_adapter_gives_zero_blocks():
    rows, cols = 16, 128
    codes, am = _base(rows, cols, 3)
    D = oracle.dequantize(codes, am).reshape(rows, cols).astype(np.float64)
    out = oracle.unmerge_adapter(codes, am, D, np.eye(cols), double_quant_on=True)
    assert np.all(out["codes"] == 7) and np.all(out["absmax"] == 0)
    assert np.all(out["qabsmax"] == 0) and np.all(out["dq_scale"] == 0)


def test_merge_then_unmerge_is_close_but_not_exact():
    # the pages: unmerge does not give back the original quantized weight (rounding
    # accumulates); an adapter of about one quantization step moves a third of the
    # codes on merge, and unmerge brings most but not all of them back
    rows, cols, r = 64, 256, 4
    codes, am = _base(rows, cols, 4)
    g = np.random.default_rng(5)
    B, A = 0.03 * g.standard_normal((rows, r)), 0.05 * g.standard_normal((r, cols))
    m = oracle.merge_adapter(codes, am, B, A, double_quant_on=False)
    assert 0.2 < float(np.mean(m["codes"] != codes)) < 0.5
    u = oracle.unmerge_adapter(m["codes"], m["absmax"], B, A, double_quant_on=False)
    same = float(np.mean(u["codes"] == codes))
    assert 0.8 < same < 1.0
    # the merged weight is closer to deq(Q) + B A than deq(Q) is
    D = oracle.dequantize(codes, am).astype(np.float64)
    Dm = oracle.dequantize(m["codes"], m["absmax"]).astype(np.float64)
    target = D + (B @ A).ravel()
    assert np.linalg.norm(Dm - target) < np.linalg.norm(D - target)


def test_double_quant_output_follows_the_new_absmax():
    codes, am = _base(32, 512, 6)
    g = np.random.default_rng(7)
    B, A = 0.01 * g.standard_normal((32, 8)), 0.01 * g.standard_normal((8, 512))
    out = oracle.merge_adapter(codes, am, B, A, alpha=2.0, double_quant_on=True)
    qa, s = oracle.double_quant(out["absmax"])
    assert np.array_equal(out["qabsmax"], qa) and np.array_equal(out["dq_scale"], s)
