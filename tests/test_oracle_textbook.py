"""Pins of ``oracle.chain_textbook``, the chain as a model defines it (raw second weight,
gamma inside RMSNorm, unrounded residual stream) -- the reference of the numerics
diagnostic that compares the fused chain and the unfused PyTorch chain with it.

- Where the definitions coincide it equals the C oracle's chain (a separate
  implementation): integer-valued A, Wo and x_res keep h exact in bf16, and power-of-two
  gamma keeps the gamma fold exact, so the folded weight divided by gamma is the raw one.
- It equals PyTorch's own float64 RMSNorm (``torch.nn.functional.rms_norm``), linear
  layers and SiLU on random inputs, for SwiGLU and no activation.
- A row sample is the corresponding slice of the full result.
"""

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si


def _exact_case(M, K1, d, N2w, act, seed):
    rng = np.random.default_rng(seed)
    w = si.custom(M, K1, d, N2w, act, seed=seed)
    inp = si.generate(w)
    # small integers: every h = x_res + A . Wo^T is an integer below 2^8 in magnitude
    inp["A"] = si.to_bf16_bits(rng.integers(-2, 3, (M, K1)).astype(np.float32))
    inp["Wo_t"] = si.to_bf16_bits(rng.integers(-1, 2, (d, K1)).astype(np.float32))
    inp["x_res"] = si.to_bf16_bits(rng.integers(-8, 9, (M, d)).astype(np.float32))
    inp["gamma"] = np.exp2(rng.integers(-3, 4, d)).astype(np.float32) * rng.choice([-1.0, 1.0], d).astype(np.float32)
    return w, inp


@pytest.mark.parametrize("act", [si.ACT_SWIGLU, si.ACT_NONE])
def test_equals_the_c_oracle_where_the_definitions_coincide(act):
    w, inp = _exact_case(37, 24, 40, 64, act, seed=3 + act)
    ref = oracle.chain(oracle.prepare(inp, "bf16"), inp["x_res"], inp["gamma"], act, w.eps)
    assert np.max(np.abs(ref["h"])) < 256
    for round_h in (False, True):
        tb = oracle.chain_textbook(inp, act, w.eps, round_h=round_h)
        assert np.array_equal(tb["h"], ref["h"])
        np.testing.assert_allclose(tb["r"], ref["r"], rtol=1e-14, atol=0)
        np.testing.assert_allclose(tb["y"], ref["y"], rtol=1e-12, atol=1e-13 * np.abs(ref["y"]).max())


@pytest.mark.parametrize("act", [si.ACT_SWIGLU, si.ACT_NONE])
def test_equals_torch_float64(act):
    w = si.custom(29, 40, 72, 2 * 48 if act == si.ACT_SWIGLU else 56, act, seed=17)
    inp = si.generate(w)
    tb = oracle.chain_textbook(inp, act, w.eps)
    t = lambda b: torch.from_numpy(oracle.bf16_decode(b))  # noqa: E731
    h = t(inp["x_res"]) + torch.nn.functional.linear(t(inp["A"]), t(inp["Wo_t"]))
    n = torch.nn.functional.rms_norm(h, (w.d,), weight=torch.from_numpy(inp["gamma"].astype(np.float64)),
                                     eps=w.eps)
    z = torch.nn.functional.linear(n, t(inp["W_t"]))
    if act == si.ACT_SWIGLU:
        y = torch.nn.functional.silu(z[:, : w.n_out]) * z[:, w.n_out:]
    else:
        y = z
    np.testing.assert_allclose(tb["h"], h.numpy(), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(tb["y"], y.numpy(), rtol=1e-10, atol=1e-12)
    hr = oracle.chain_textbook(inp, act, w.eps, round_h=True)
    assert np.array_equal(oracle.bf16_encode(tb["h"]), oracle.bf16_encode(hr["h"]))
    assert np.array_equal(hr["h"], oracle.bf16_decode(oracle.bf16_encode(tb["h"])))


def test_row_sample_is_a_slice():
    w = si.custom(50, 16, 24, 2 * 16, si.ACT_SWIGLU, seed=5)
    inp = si.generate(w)
    full = oracle.chain_textbook(inp, w.act, w.eps)
    rows = np.array([0, 7, 49], np.int64)
    part = oracle.chain_textbook(inp, w.act, w.eps, rows=rows)
    for k in ("h", "r", "y"):
        assert np.array_equal(part[k], full[k][rows])
