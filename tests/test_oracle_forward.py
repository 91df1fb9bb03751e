"""Pins for the oracle's bf16 rounding and QLoRA forward (PEFT course §2.2 h = Wx + BAx,
§4.3 bfloat16 compute)."""
import numpy as np
import torch

import oracle


def test_bf16_round_hand_values():
    one = 1.0
    cases = [(one, one), (one + 2.0 ** -8, one),                   # tie -> even (1.0)
             (one + 3 * 2.0 ** -8, one + 2.0 ** -6),                # tie -> even (mantissa 0b0000010)
             (one + 2.0 ** -8 + 2.0 ** -20, one + 2.0 ** -7),       # above the tie -> up
             (-0.1, -0.10009765625), (0.0, 0.0), (2.0 ** -130, 2.0 ** -130)]
    for x, want in cases:
        assert oracle.bf16_round(np.array([x], np.float32))[0] == np.float32(want), x


def test_bf16_round_matches_torch():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, 100000),
                        (1 + np.arange(-300, 300) * 2.0 ** -16).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.bf16_round(x).view(np.uint32), ref.view(np.uint32))


def _q(rows, cols, seed):
    g = np.random.default_rng(seed)
    W = (0.05 * g.standard_normal((rows, cols))).astype(np.float32)
    codes, am = oracle.quantize_residual(W.ravel())
    return codes, am


def test_forward_with_bf16_exact_weights_is_the_plain_product():
    # levels 0 and +-1 with power-of-two scales make deq(Q) exactly bf16; bf16-exact
    # A, B: then Y = X W^T + alpha (X A^T) B^T, computed here directly
    rows, cols, n, r = 8, 128, 5, 3
    g = np.random.default_rng(2)
    codes = g.choice([0, 7, 15], rows * cols).astype(np.uint8)
    scale = (2.0 ** g.integers(-4, 3, rows * cols // 64)).astype(np.float32)
    cb = oracle.nf_codebook(4).astype(np.float64)
    W = (cb[codes] * np.repeat(scale, 64)).reshape(rows, cols)
    X = oracle.bf16_round(g.standard_normal((n, cols)).astype(np.float32)).astype(np.float64)
    A = np.round(g.standard_normal((r, cols)) * 8) / 8
    B = np.round(g.standard_normal((rows, r)) * 8) / 8
    Y = oracle.qlora_forward(X, codes, scale, rows, cols, B, A, alpha=0.5)
    assert np.allclose(Y, X @ W.T + 0.5 * (X @ A.T) @ B.T, rtol=1e-13, atol=1e-13)


def test_forward_is_linear_in_x_and_adapter_free_without_b():
    rows, cols, n = 16, 192, 4
    codes, am = _q(rows, cols, 3)
    g = np.random.default_rng(4)
    X1 = oracle.bf16_round(g.standard_normal((n, cols)).astype(np.float32)).astype(np.float64)
    X2 = oracle.bf16_round(g.standard_normal((n, cols)).astype(np.float32)).astype(np.float64)
    B, A = g.standard_normal((rows, 2)), g.standard_normal((2, cols))
    f = lambda X: oracle.qlora_forward(X, codes, am, rows, cols, B, A, alpha=2.0)
    assert np.allclose(f(X1 + X2), f(X1) + f(X2), rtol=1e-12, atol=1e-12)
    base = oracle.qlora_forward(X1, codes, am, rows, cols)
    assert np.allclose(f(X1) - base, 2.0 * (X1 @ oracle.bf16_round(A.astype(np.float32)).T)
                       @ oracle.bf16_round(B.astype(np.float32)).T, rtol=1e-12, atol=1e-12)
