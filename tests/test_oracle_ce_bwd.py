"""Pins of the oracle's LM-head backward  sum_m g_m CE(RMSNorm(hb) . W^T, t_m)  (CPU
only): float64 torch autograd of torch's own cross_entropy on tiny inputs (ignored
targets included), a one-class vocabulary (zero gradient), the softmax rows summing to
zero against the one-hot, and samples as slices of the full result.  A sign flip of the
one-hot, a dropped g, a missing RMSNorm term or a gradient left on ignored rows fails
one of them."""
import numpy as np
import torch

import oracle


def _inputs(M, d, V, seed):
    rng = np.random.default_rng(seed)
    enc = lambda x: oracle.bf16_encode(np.asarray(x, dtype=np.float64))  # noqa: E731
    hb = enc(rng.standard_normal((M, d)))
    W = enc(2.0 * rng.standard_normal((V, d)) / np.sqrt(d))
    # powers of two: gamma * W is exact in bf16, so the folded weight stands for W exactly
    gamma = (2.0 ** rng.integers(-1, 2, size=d)).astype(np.float32)
    t = rng.integers(0, V, size=M).astype(np.int32)
    t[1] = -100                                   # an ignored row
    g = rng.uniform(0.5, 2.0, size=M)
    return hb, W, gamma, t, g


def _autograd(hb, W, gamma, t, g, eps):
    T = lambda a: torch.tensor(oracle.bf16_decode(a), dtype=torch.float64)  # noqa: E731
    h = T(hb).requires_grad_(True)
    w = T(W).requires_grad_(True)
    gm = torch.tensor(gamma, dtype=torch.float64).requires_grad_(True)
    r = 1.0 / torch.sqrt((h * h).mean(dim=1, keepdim=True) + eps)
    z = (h * r * gm) @ w.T
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(t, dtype=torch.int64), reduction="none",
                                             ignore_index=-100)
    (loss * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return h.grad.numpy(), w.grad.numpy(), gm.grad.numpy(), torch.logsumexp(z, dim=1).detach().numpy()


def test_backward_equals_autograd_of_cross_entropy():
    eps = 1e-5
    for (M, d, V, seed) in ((6, 32, 40, 1), (5, 16, 300, 2), (3, 48, 7, 3)):
        hb, W, gamma, t, g = _inputs(M, d, V, seed)
        Wp = oracle.fold_bf16(W, gamma)
        ref = oracle.lmhead_ce_bwd(hb, gamma, Wp, 1.0, W, t, g, eps, js="all")
        gh, gw, gg, lse = _autograd(hb, W, gamma, t, g, eps)
        for a, b in ((ref["dh"], gh), (ref["dW"], gw), (ref["dgamma"], gg), (ref["lse"], lse)):
            assert np.max(np.abs(a - b)) <= 1e-10 * (1 + np.max(np.abs(b)))
        assert np.all(ref["dz"][1] == 0.0)                     # the ignored row


def test_one_class_vocabulary_has_no_gradient():
    hb, W, gamma, t, g = _inputs(4, 16, 1, 5)
    t[:] = 0
    ref = oracle.lmhead_ce_bwd(hb, gamma, oracle.fold_bf16(W, gamma), 1.0, W, t, g, 1e-5, js="all")
    for k in ("dh", "dz", "dW", "dgamma"):
        assert np.all(np.abs(ref[k]) < 1e-15), k


def test_logit_gradient_rows_sum_to_zero_and_samples_are_slices():
    hb, W, gamma, t, g = _inputs(9, 32, 200, 7)
    Wp = oracle.fold_bf16(W, gamma)
    full = oracle.lmhead_ce_bwd(hb, gamma, Wp, 1.0, W, t, g, 1e-5, js="all", rss=True)
    # softmax sums to 1 and the one-hot removes 1: each counted row's gradient sums to 0,
    # with -g (1 - p_t) at the target
    assert np.allclose(full["dz"].sum(axis=1), 0.0, atol=1e-13)
    i = 0
    assert full["dz"][i, t[i]] < 0 and np.all(np.delete(full["dz"][i], t[i]) > 0)
    rows, js, ks = [8, 0, 4], [199, 3, 50], [31, 2]
    part = oracle.lmhead_ce_bwd(hb, gamma, Wp, 1.0, W, t, g, 1e-5, rows=rows, js=js, ks=ks, rss=True)
    assert np.allclose(part["dh"], full["dh"][rows], rtol=1e-12, atol=1e-15)
    assert np.allclose(part["dW"], full["dW"][np.ix_(js, ks)], rtol=1e-12, atol=1e-15)
    assert np.allclose(part["rss"], full["rss"][np.ix_(js, ks)], rtol=1e-12, atol=1e-15)
    assert part["dgamma"] is None
    assert np.all(np.abs(full["dW"]) / np.abs(gamma)[None, :] <= full["rss"] * np.sqrt(9) * (1 + 1e-12))
