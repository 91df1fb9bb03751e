"""The allocation-free QLoRA forward (loftq_qlora_forward_noalloc) gives what
loftq_qlora_forward gives with a caller workspace, through the C ABI: two calls in a
row on the library's device scratch, the second with fewer tokens (its leftover
contents from the first call must not leak in), both bit for bit equal to the
workspace entry point on the same inputs, and within the forward's oracle bar
("参数高效微调：LoRA、Adapter 与 QLoRA" §2.2 and §4.3)."""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_forward import dev, host, make_case

pytestmark = pytest.mark.gpu


def _inputs(c, dq):
    X = torch.from_numpy(c["xbits"].view(np.int16).copy()).view(torch.bfloat16).cuda()
    kw = dict(qabsmax=dev(c["qabsmax"], np.int8), dq_scale=dev(c["dq_scale"])) if dq else \
        dict(absmax=dev(c["absmax"]))
    return X, dev(c["packed"], np.uint8), kw, dev(c["B"]), dev(c["A"])


@pytest.mark.parametrize("dq", [False, True])
def test_noalloc_forward_matches_workspace_call(lib, dq):
    rows, cols, r, alpha = 320, 1024, 16, 0.75
    assert lib.qlora_forward_noalloc_max_bytes() == 8 << 20
    for n_tok, seed in ((700, 3), (40, 4)):          # many tokens (tiled kernel), then few (few-token kernel)
        c = make_case(n_tok, rows, cols, r, 4, dq, seed)
        X, packed, kw, B, A = _inputs(c, dq)
        y_na = host(lib.loftq_qlora_forward_noalloc(X, packed, (rows, cols), **kw, B=B, A=A, alpha=alpha))
        y_ws = host(lib.loftq_qlora_forward(X, packed, (rows, cols), **kw, B=B, A=A, alpha=alpha))
        assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), n_tok
        ref = oracle.qlora_forward(c["X"], c["codes"], c["scale"], rows, cols, c["B"], c["A"], alpha)
        err = np.linalg.norm(y_na.astype(np.float64) - ref) / np.linalg.norm(ref)
        assert err <= 1e-5, (n_tok, err)


def test_noalloc_forward_rejects_beyond_scratch(lib):
    c = make_case(16, 64, 128, 16, 4, False, 5)
    X, packed, kw, B, A = _inputs(c, False)
    Xbig = torch.zeros((20000, 128), dtype=torch.bfloat16, device="cuda")   # 20000 x 16 x 8 x 4 B > 8 MiB
    with pytest.raises(lib.LoftqError) as e:
        lib.loftq_qlora_forward_noalloc(Xbig, packed, (64, 128), **kw, B=B, A=A)
    assert e.value.status == 3
