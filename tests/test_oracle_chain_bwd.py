"""Pins of the oracle's backward of the whole chain h = x_res + A . Wo^T,
y = SwiGLU(RMSNorm(h) . W^T): torch autograd in fp64 on inputs that make every stored
rounding exact (small integers for A, Wo, x_res so that h is exact in bf16; powers of two
for gamma so that the fold is exact), linearity in the residual gradient, row subsets,
and the root-sum-square helpers against per-term decompositions run through the oracle
itself (per token for dWo, per hidden column of the residual gradient for dA).
"""

import numpy as np
import torch

import oracle
import synth_inputs as si


def _case(M, K1, d, F, seed, eps=1e-5):
    rng = np.random.default_rng(seed)
    bits = lambda a: si.to_bf16_bits(np.asarray(a, dtype=np.float32))  # noqa: E731
    inp = {
        "A": bits(rng.integers(-2, 3, (M, K1))),
        "Wo_t": bits(rng.integers(-2, 3, (d, K1))),
        "W_t": bits(rng.standard_normal((2 * F, d)) / np.sqrt(d)),
        "gamma": np.exp2(rng.integers(-2, 3, d)).astype(np.float32),
    }
    x_res = bits(rng.integers(-3, 4, (M, d)))
    dy = bits(rng.standard_normal((M, F)))
    dres = bits(rng.standard_normal((M, d)))
    prep = oracle.prepare(inp, "bf16")
    return inp, prep, x_res, dy, dres, eps


def test_chain_backward_matches_torch_autograd():
    inp, prep, x_res, dy, dres, eps = _case(5, 8, 16, 8, 1)
    o = oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], dy, eps, dres=dres)
    t = lambda c: torch.from_numpy(oracle.bf16_decode(c))  # noqa: E731
    A, Wo, W = t(inp["A"]).requires_grad_(True), t(inp["Wo_t"]).requires_grad_(True), t(inp["W_t"]).requires_grad_(True)
    xr = t(x_res).requires_grad_(True)
    g = torch.from_numpy(inp["gamma"].astype(np.float64)).requires_grad_(True)
    h = xr + A @ Wo.T
    assert np.array_equal(h.detach().numpy(), oracle.bf16_decode(oracle.bf16_encode(h.detach().numpy())))
    r = torch.rsqrt((h * h).mean(1, keepdim=True) + eps)
    z = (h * r * g) @ W.T
    F = z.shape[1] // 2
    y = torch.nn.functional.silu(z[:, :F]) * z[:, F:]
    loss = (y * t(dy)).sum() + (h * t(dres)).sum()
    loss.backward()
    close = lambda a, b: np.allclose(a, b.numpy(), rtol=1e-11, atol=1e-12)  # noqa: E731
    assert close(o["dh"], xr.grad) and close(o["dA"], A.grad) and close(o["dWo"], Wo.grad)
    assert close(o["dW"], W.grad) and close(o["dgamma"], g.grad)


def test_residual_gradient_enters_linearly():
    inp, prep, x_res, dy, dres, eps = _case(4, 16, 24, 8, 2)
    a = oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], dy, eps, dres=dres)
    b = oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], dy, eps)
    e = oracle.bf16_decode(dres)
    assert np.allclose(a["dh"] - b["dh"], e, rtol=0, atol=1e-12)
    assert np.allclose(a["dA"] - b["dA"], e @ oracle.bf16_decode(inp["Wo_t"]), atol=1e-11)
    assert np.allclose(a["dWo"] - b["dWo"], e.T @ oracle.bf16_decode(inp["A"]), atol=1e-11)
    assert np.array_equal(a["dW"], b["dW"]) and np.array_equal(a["dgamma"], b["dgamma"])


def test_row_subset_equals_full():
    inp, prep, x_res, dy, dres, eps = _case(9, 8, 16, 8, 3)
    full = oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], dy, eps, dres=dres)
    rows = np.array([8, 0, 5])
    part = oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], dy, eps, dres=dres, rows=rows)
    assert np.array_equal(part["dh"], full["dh"][rows]) and np.allclose(part["dA"], full["dA"][rows], rtol=1e-14)
    assert "dWo" not in part


def test_rss_of_dWo_is_over_the_per_token_gradients():
    inp, prep, x_res, dy, dres, eps = _case(4, 8, 16, 8, 4)
    o = oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], dy, eps, dres=dres, rss=True)
    sq = np.zeros_like(o["dWo"])
    for m in range(4):
        one = dict(inp, A=inp["A"][m:m + 1])
        pm = oracle.prepare(one, "bf16")
        om = oracle.chain_bwd(pm, x_res[m:m + 1], inp["gamma"], inp["W_t"], dy[m:m + 1], eps, dres=dres[m:m + 1])
        sq += om["dWo"] ** 2
    assert np.allclose(o["rss_dWo"], np.sqrt(sq), rtol=1e-12, atol=0)


def test_rss_of_dA_is_over_the_hidden_columns():
    # with dy = 0 the block gradient vanishes and dh = dres; a residual gradient with one
    # nonzero column n gives dA's n-th term alone
    inp, prep, x_res, dy, dres, eps = _case(3, 8, 16, 8, 5)
    zero = np.zeros_like(dy)
    o = oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], zero, eps, dres=dres, rss=True)
    sq = np.zeros_like(o["dA"])
    for n in range(dres.shape[1]):
        col = np.zeros_like(dres)
        col[:, n] = dres[:, n]
        sq += oracle.chain_bwd(prep, x_res, inp["gamma"], inp["W_t"], zero, eps, dres=col)["dA"] ** 2
    assert np.allclose(o["rss_dA"], np.sqrt(sq), rtol=1e-12, atol=0)


def test_whole_chain_backward_inputs_extend_the_forward_draws():
    # the backward workload draws the forward's inputs first, in the same order, then the
    # upstream and residual-stream gradients: its forward is the forward workload's
    fwd = si.generate(si.custom(24, 16, 32, 48, si.ACT_SWIGLU, seed=7))
    bwd = si.generate(si.custom(24, 16, 32, 48, si.ACT_CHAIN_BWD, seed=7))
    for k in ("A", "Wo_t", "x_res", "gamma", "W_t"):
        assert np.array_equal(fwd[k], bwd[k])
    assert bwd["dy"].shape == (24, 24) and bwd["dres"].shape == (24, 32)
    w2, w9 = si.WORKLOADS[2], si.WORKLOADS[9]
    assert (w9.M, w9.K1, w9.d, w9.N2w, w9.seed) == (w2.M, w2.K1, w2.d, w2.N2w, w2.seed)
