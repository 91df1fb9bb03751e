"""The randomized SVD's products form the residual E = W - deq(Q) from the weight and the
codes as they stream them (loftq_config_t.materialize_residual = 0, the default) instead of
reading an E the dequant stored ("LoftQ…" §2.3: the low-rank step is the SVD of W - Q).
The element arithmetic is the dequant's own, fl32(w - fl32(level[code] a')), so both ways
give the same initialisation bit for bit: every output of loftq_init is compared exactly.
Cases: the 24-wide and 80-wide sketches, double quant on and off, bf16 and fp32 W, a
column count that is a multiple of 8 but not of 64 (blocks straddle rows), one that
falls back to the stored E, 2-bit codes, ragged row tiles with a split past the last
column and a wide matrix whose E P stages its panel in LDS (both with the full-line
loads E P uses when cols % 64 == 0), and the batched call.
"""
import numpy as np
import pytest
import torch

from loftq_qlora_initialization_amd import synth
from test_gpu_lowrank import dev_w, host

pytestmark = pytest.mark.gpu

KEYS = ("packed", "absmax", "qabsmax", "dq_scale", "B", "A", "sigma", "objective")


def _weight(rows, cols, dtype, seed):
    w = synth.Workload("t", rows, cols, dtype, 16, 1, True, 8, 2, False, seed, "gauss")
    bits, _ = synth.make_weight(w)
    return dev_w(bits, w)


def _same(a, b):
    for key in KEYS:
        if key in a:
            x, y = host(a[key]), host(b[key])
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), key


@pytest.mark.parametrize("rows,cols,dtype,r,p,q,dq,T,bits", [
    (1024, 768, "bf16", 16, 8, 2, 1, 3, 4),      # l = 24
    (1536, 1024, "bf16", 64, 16, 2, 1, 2, 4),    # l = 80
    (700, 516, "f32", 8, 8, 1, 0, 2, 4),         # fp32 W, no double quant, 516 = 8 * 64 + 4
    (640, 264, "bf16", 4, 4, 2, 1, 2, 4),        # 264 columns: 64-blocks straddle rows
    (640, 260, "bf16", 4, 4, 2, 1, 2, 4),        # 260 columns: E is stored either way (cols % 8 != 0)
    (512, 384, "bf16", 16, 8, 1, 1, 2, 2),       # 2-bit codes
    (1000, 704, "bf16", 16, 8, 2, 1, 2, 4),      # ragged row tiles; the last split runs past the last column
    (200, 8256, "bf16", 16, 8, 1, 1, 2, 4),      # l = 24 with a panel over 1 MiB (LDS-staged E P)
])
def test_formed_residual_matches_stored(lib, rows, cols, dtype, r, p, q, dq, T, bits):
    W = _weight(rows, cols, dtype, rows + cols)
    kw = dict(iterative_steps=T, rank=r, oversample=p, power_iters=q, double_quant=dq, bits=bits)
    formed = lib.loftq_init(W, lib.default_config(materialize_residual=0, **kw))
    stored = lib.loftq_init(W, lib.default_config(materialize_residual=1, **kw))
    _same(formed, stored)


def test_formed_residual_workspace_is_smaller(lib):
    kw = dict(iterative_steps=2, rank=16, oversample=8, power_iters=2)
    a = lib.workspace_bytes(4096, 4096, lib.default_config(materialize_residual=0, **kw))
    b = lib.workspace_bytes(4096, 4096, lib.default_config(materialize_residual=1, **kw))
    n = 4096 * 4096
    assert b - a >= n * 4 - (n // 64) * 4   # no E; one fp32 block scale per 64 elements instead


def test_formed_residual_batch_matches_stored(lib):
    Ws = [_weight(768, 512, "bf16", 11), _weight(512, 768, "bf16", 12), _weight(768, 512, "bf16", 13)]
    kw = dict(iterative_steps=2, rank=16, oversample=8, power_iters=2)
    formed = lib.loftq_init_batch(Ws, lib.default_config(materialize_residual=0, **kw), nstreams=2)
    stored = lib.loftq_init_batch(Ws, lib.default_config(materialize_residual=1, **kw), nstreams=2)
    for a, b in zip(formed, stored):
        _same({k: getattr(a, k) for k in KEYS}, {k: getattr(b, k) for k in KEYS})
