"""Pins of the oracle's QKV-block backward  y = RoPE(RMSNorm(hb) . W^T)  (CPU only):
the transposed rotation inverts the forward rotation of the C oracle, and the whole
backward equals float64 torch autograd of the forward definition on tiny inputs.  A
dropped RoPE sign, a swapped half, a missing RMSNorm term or a transposed weight fails
one of them."""
import numpy as np
import torch

import oracle

BASE, HD = 10000.0, 64


def _inputs(M, d, N, seed, pow2_gamma=True):
    rng = np.random.default_rng(seed)
    f32 = np.float32
    enc = lambda x: oracle.bf16_encode(np.asarray(x, dtype=np.float64))  # noqa: E731
    hb = enc(rng.standard_normal((M, d)))
    W = enc(rng.standard_normal((N, d)) / np.sqrt(d))
    dy = enc(rng.standard_normal((M, N)))
    # powers of two: gamma * W is exact in bf16, so the folded weight stands for W exactly
    gamma = (2.0 ** rng.integers(-1, 2, size=d)).astype(f32) if pow2_gamma else \
        (1 + 0.1 * rng.standard_normal(d)).astype(f32)
    pos = rng.integers(0, 300, size=M).astype(np.int32)
    return hb, W, dy, gamma, pos


def test_transpose_inverts_the_forward_rotation():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((9, 320))
    pos = rng.integers(0, 5000, size=9).astype(np.int32)
    for rot in (0, 64, 256):
        y = oracle.rope(v, pos, BASE, HD, rot)
        back = oracle.rope_transpose(y, pos, BASE, HD, rot)
        # the two sides evaluate base^(-2i/64) with different pow implementations (an ulp
        # apart), which positions up to 5000 turn into angle differences of ~5e-13 rad
        assert np.max(np.abs(back - v)) < 1e-11
        # an orthogonal map keeps each row's norm
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(v, axis=1), rtol=1e-13)
        if rot:
            assert np.max(np.abs(y[:, :rot] - v[:, :rot])) > 1e-3     # it did rotate


def _autograd(hb, W, dy, gamma, pos, rot, eps):
    t = lambda a: torch.tensor(oracle.bf16_decode(a), dtype=torch.float64)  # noqa: E731
    h = t(hb).requires_grad_(True)
    w = t(W).requires_grad_(True)
    g = torch.tensor(gamma, dtype=torch.float64).requires_grad_(True)
    d = h.shape[1]
    r = 1.0 / torch.sqrt((h * h).mean(dim=1, keepdim=True) + eps)
    z = (h * r * g) @ w.T
    half = HD // 2
    ang = torch.tensor(pos, dtype=torch.float64)[:, None] * \
        BASE ** (-2.0 * torch.arange(half, dtype=torch.float64) / HD)[None, :]
    c, s = torch.cos(ang), torch.sin(ang)
    parts = []
    for h0 in range(0, z.shape[1], HD):
        lo, hi = z[:, h0:h0 + half], z[:, h0 + half:h0 + HD]
        if h0 < rot:
            parts += [lo * c - hi * s, hi * c + lo * s]
        else:
            parts += [lo, hi]
    y = torch.cat(parts, dim=1)
    (y * t(dy)).sum().backward()
    assert d == hb.shape[1]
    return h.grad.numpy(), w.grad.numpy(), g.grad.numpy()


def test_backward_equals_autograd_of_the_forward():
    eps = 1e-5
    for (M, d, N, rot, seed) in ((5, 32, 192, 128, 1), (3, 48, 128, 0, 2), (4, 16, 64, 64, 3)):
        hb, W, dy, gamma, pos = _inputs(M, d, N, seed)
        Wp = oracle.fold_bf16(W, gamma)
        ref = oracle.qkv_rope_bwd(hb, gamma, Wp, 1.0, W, dy, pos, BASE, HD, rot, eps)
        gh, gw, gg = _autograd(hb, W, dy, gamma, pos, rot, eps)
        for a, b in ((ref["dh"], gh), (ref["dW"], gw), (ref["dgamma"], gg)):
            assert np.max(np.abs(a - b)) <= 1e-10 * (1 + np.max(np.abs(b)))


def test_row_and_column_samples_are_slices_of_the_full_result():
    hb, W, dy, gamma, pos = _inputs(7, 32, 192, 4, pow2_gamma=False)
    Wp = oracle.fold_bf16(W, gamma)
    full = oracle.qkv_rope_bwd(hb, gamma, Wp, 1.0, W, dy, pos, BASE, HD, 128, 1e-5, rss=True)
    rows, js, ks = [6, 0, 3], [191, 5, 64, 100], [31, 0, 7]
    part = oracle.qkv_rope_bwd(hb, gamma, Wp, 1.0, W, dy, pos, BASE, HD, 128, 1e-5, rows=rows, js=js, ks=ks,
                               rss=True)
    assert np.allclose(part["dh"], full["dh"][rows], rtol=1e-13, atol=1e-14)
    assert np.allclose(part["dz"], full["dz"][rows], rtol=1e-13, atol=1e-14)
    assert np.allclose(part["dW"], full["dW"][np.ix_(js, ks)], rtol=1e-13, atol=1e-14)
    assert np.allclose(part["rss"], full["rss"][np.ix_(js, ks)], rtol=1e-13, atol=1e-14)
    assert part["dgamma"] is None and full["dgamma"] is not None
    # each sum is bounded by its root-sum-square times the square root of its term count
    assert np.all(np.abs(full["dW"]) / np.abs(gamma)[None, :] <= full["rss"] * np.sqrt(7) * (1 + 1e-12))
    assert np.all(np.abs(full["dgamma"]) <= full["rss_gamma"] * np.sqrt(7 * 192) * (1 + 1e-12))
