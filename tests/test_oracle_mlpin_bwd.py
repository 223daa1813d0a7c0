"""Pins of the oracle's input gradient of the MLP-input block
y = SwiGLU(RMSNorm(h) . W^T) (the backward of the chain's second half).

The pages state that the reparameterisation carries over to the backward pass (kucoin
page, section "CODA: El epilogo esconde un tesoro") without formulas; the oracle is the
unfused chain rule.  It is pinned against torch's autograd (fp64, a library routine),
central finite differences of an independent fp64 forward, and the closed forms of a
scale-invariant map (at eps = 0: dh(2h) = dh(h)/2 and dh is orthogonal to h).
"""

import numpy as np
import torch

import oracle
import synth_inputs as si


def _case(M, d, F, seed, eps=1e-5):
    rng = np.random.default_rng(seed)
    hb = si.to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32))
    dy = si.to_bf16_bits(rng.standard_normal((M, F)).astype(np.float32))
    W = si.to_bf16_bits((rng.standard_normal((2 * F, d)) / np.sqrt(d)).astype(np.float32))
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    Wp = oracle.fold_bf16(W, g)
    W_or = oracle.bf16_decode(Wp) / g.astype(np.float64)[None, :]
    return hb, dy, g, Wp, W_or, eps


def _forward_np(h, g, W_or, eps):
    r = 1.0 / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
    z = (h * r * g[None, :]) @ W_or.T
    F = z.shape[1] // 2
    a, u = z[:, :F], z[:, F:]
    return a / (1.0 + np.exp(-a)) * u


def test_matches_torch_autograd():
    hb, dy, g, Wp, W_or, eps = _case(5, 48, 24, 1)
    o = oracle.mlpin_bwd(hb, g, Wp, oracle.BF16, 1.0, dy, eps)
    h = torch.from_numpy(oracle.bf16_decode(hb)).requires_grad_(True)
    gt = torch.from_numpy(g.astype(np.float64))
    r = torch.rsqrt((h * h).mean(1, keepdim=True) + eps)
    z = (h * r * gt) @ torch.from_numpy(W_or).T
    F = z.shape[1] // 2
    y = torch.nn.functional.silu(z[:, :F]) * z[:, F:]
    (y * torch.from_numpy(oracle.bf16_decode(dy))).sum().backward()
    assert np.allclose(o["dh"], h.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(o["r"], r.detach().numpy()[:, 0], rtol=1e-14)


def test_matches_central_differences():
    hb, dy, g, Wp, W_or, eps = _case(2, 16, 8, 2)
    o = oracle.mlpin_bwd(hb, g, Wp, oracle.BF16, 1.0, dy, eps)
    h0 = oracle.bf16_decode(hb)
    dyv = oracle.bf16_decode(dy)
    step = 1e-6
    num = np.zeros_like(h0)
    for m in range(h0.shape[0]):
        for k in range(h0.shape[1]):
            hp, hm = h0.copy(), h0.copy()
            hp[m, k] += step
            hm[m, k] -= step
            num[m, k] = (np.sum(_forward_np(hp, g, W_or, eps)[m] * dyv[m]) -
                         np.sum(_forward_np(hm, g, W_or, eps)[m] * dyv[m])) / (2 * step)
    assert np.allclose(o["dh"], num, rtol=1e-6, atol=1e-8)


def test_zero_upstream_gradient_gives_zero():
    hb, dy, g, Wp, W_or, eps = _case(3, 32, 16, 3)
    o = oracle.mlpin_bwd(hb, g, Wp, oracle.BF16, 1.0, np.zeros_like(dy), eps)
    assert np.all(o["dh"] == 0.0) and np.all(o["dz"] == 0.0)


def test_scale_invariance_at_zero_eps():
    # RMSNorm(2h) = RMSNorm(h) when eps = 0, so the gradient scales by 1/2 and is
    # orthogonal to h (the loss does not change along h)
    hb, dy, g, Wp, W_or, _ = _case(4, 64, 32, 4)
    o1 = oracle.mlpin_bwd(hb, g, Wp, oracle.BF16, 1.0, dy, 0.0)
    h2 = oracle.bf16_encode(2.0 * oracle.bf16_decode(hb))       # exact in bf16
    o2 = oracle.mlpin_bwd(h2, g, Wp, oracle.BF16, 1.0, dy, 0.0)
    assert np.allclose(o2["dh"], o1["dh"] / 2, rtol=1e-12, atol=1e-15)
    h = oracle.bf16_decode(hb)
    dots = np.sum(o1["dh"] * h, axis=1) / (np.linalg.norm(o1["dh"], axis=1) * np.linalg.norm(h, axis=1))
    assert np.all(np.abs(dots) < 1e-12)


def test_row_subset_equals_full():
    hb, dy, g, Wp, W_or, eps = _case(9, 32, 16, 5)
    full = oracle.mlpin_bwd(hb, g, Wp, oracle.BF16, 1.0, dy, eps)
    rows = np.array([8, 0, 4])
    part = oracle.mlpin_bwd(hb, g, Wp, oracle.BF16, 1.0, dy, eps, rows=rows)
    assert np.array_equal(part["dh"], full["dh"][rows])


def _pow2_case(M, d, F, seed, eps=1e-5):
    # gamma = powers of two makes the fold exact, so the raw weight and the unfused weight
    # W' / gamma coincide and the gamma gradient has one unambiguous reference
    rng = np.random.default_rng(seed)
    hb = si.to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32))
    dy = si.to_bf16_bits(rng.standard_normal((M, F)).astype(np.float32))
    W = si.to_bf16_bits((rng.standard_normal((2 * F, d)) / np.sqrt(d)).astype(np.float32))
    g = np.exp2(rng.integers(-2, 3, d)).astype(np.float32)
    Wp = oracle.fold_bf16(W, g)
    assert np.array_equal(oracle.bf16_decode(Wp) / g.astype(np.float64), oracle.bf16_decode(W))
    return hb, dy, g, Wp, W, eps


def test_weight_gradients_match_torch_autograd():
    hb, dy, g, Wp, W, eps = _pow2_case(6, 32, 16, 11)
    dW, dgam = oracle.mlpin_wgrad(hb, g, Wp, oracle.BF16, 1.0, W, dy, eps)
    h = torch.from_numpy(oracle.bf16_decode(hb))
    Wt = torch.from_numpy(oracle.bf16_decode(W)).requires_grad_(True)
    gt = torch.from_numpy(g.astype(np.float64)).requires_grad_(True)
    r = torch.rsqrt((h * h).mean(1, keepdim=True) + eps)
    z = (h * r * gt) @ Wt.T
    F = z.shape[1] // 2
    y = torch.nn.functional.silu(z[:, :F]) * z[:, F:]
    (y * torch.from_numpy(oracle.bf16_decode(dy))).sum().backward()
    assert np.allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dgam, gt.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_weight_gradient_samples_equal_the_full_result():
    hb, dy, g, Wp, W, eps = _pow2_case(9, 24, 8, 12)
    dW, dgam = oracle.mlpin_wgrad(hb, g, Wp, oracle.BF16, 1.0, W, dy, eps)
    js, ks = np.array([15, 0, 8, 3]), np.array([23, 1, 7])
    part, none = oracle.mlpin_wgrad(hb, g, Wp, oracle.BF16, 1.0, W, dy, eps, js=js, ks=ks)
    assert none is None
    assert np.array_equal(part, dW[np.ix_(js, ks)])


def test_weight_gradient_rss_is_the_root_sum_square_of_the_per_token_gradients():
    # the terms of the token sum are the one-token gradients: running the oracle on each
    # token alone gives them, so rss^2 = sum_m (dW_m / gamma)^2 and
    # rss_gamma^2 = sum_m sum_j (W dW_m / gamma)^2
    hb, dy, g, Wp, W, eps = _pow2_case(5, 16, 8, 13)
    dW, dgam, rss, rssg = oracle.mlpin_wgrad(hb, g, Wp, oracle.BF16, 1.0, W, dy, eps, rss=True)
    Wr = oracle.bf16_decode(W)
    sq, sqg = np.zeros_like(rss), np.zeros_like(rssg)
    for m in range(hb.shape[0]):
        dWm, _ = oracle.mlpin_wgrad(hb[m:m + 1], g, Wp, oracle.BF16, 1.0, W, dy[m:m + 1], eps)
        t = dWm / g.astype(np.float64)[None, :]
        sq += t * t
        sqg += np.sum((Wr * t) ** 2, axis=0)
    assert np.allclose(rss, np.sqrt(sq), rtol=1e-12, atol=0)
    assert np.allclose(rssg, np.sqrt(sqg), rtol=1e-12, atol=0)
    # Cauchy-Schwarz over the M terms
    assert np.all(np.abs(dW) / g.astype(np.float64)[None, :] <= np.sqrt(hb.shape[0]) * rss * (1 + 1e-12))
    # sampled rss equals the full one
    js, ks = np.array([3, 12]), np.array([15, 0])
    _, _, part, none = oracle.mlpin_wgrad(hb, g, Wp, oracle.BF16, 1.0, W, dy, eps, js=js, ks=ks, rss=True)
    assert none is None and np.array_equal(part, rss[np.ix_(js, ks)])
