"""Pins for the oracle's chain (CPU only).

The oracle computes the unfused chain GEMM -> residual -> RMSNorm -> GEMM(+SwiGLU) in
fp64.  Here it is pinned to things other than itself:
  * exact rational brute force (``Fraction``) for the linear parts and 60-digit
    ``Decimal`` arithmetic for sqrt / exp on tiny shapes;
  * numpy's BLAS matmul for the first product (a library routine the oracle does not use);
  * the reparameterisation invariant: the row scale commutes with the next GEMM
    (kucoin "CODA: new research optimizes Transformer training..." section
    "CODA: El epilogo esconde un tesoro"), so act(r * (hb @ W'^T)) must equal the
    oracle's unfused result;
  * closed forms: constant rows, an identity second weight, zero weights, eps = 0
    scale invariance, SiLU(0) = 0.
"""

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth_inputs as si

getcontext().prec = 60


def _run(w, inp=None, rows=None, eps=None):
    inp = si.generate(w) if inp is None else inp
    prep = oracle.prepare(inp, w.dtype)
    out = oracle.chain(prep, inp["x_res"], inp["gamma"], w.act, w.eps if eps is None else eps,
                       rows=rows)
    return inp, prep, out


def _bf16_nearest(x: Fraction) -> int:
    """Nearest bf16 code to an exact rational (ties to even), brute force over the two
    bf16 values that bracket it (found through fp32 truncation, then checked exactly)."""
    f = np.float32(float(x))
    b = int(np.array([f], np.float32).view(np.uint32)[0]) & 0xFFFF0000
    cands = []
    for bb in (b - 0x10000, b, b + 0x10000):
        if bb < 0:
            continue
        code = bb >> 16
        v = Fraction(float(np.array([bb], np.uint32).view(np.float32)[0]))
        if v != v:  # nan guard
            continue
        cands.append((abs(v - x), code % 2, code))
    # sign handling: the truncation keeps the sign bit, so cands share x's sign
    return min(cands)[2]


def _dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


@pytest.mark.parametrize("act", [si.ACT_NONE, si.ACT_SWIGLU])
def test_chain_exact_brute_force_tiny(act):
    M, K1, d, N2w = 3, 5, 4, 6
    w = si.custom(M, K1, d, N2w, act, seed=77)
    inp, prep, out = _run(w)
    F = lambda b: Fraction(float(oracle.bf16_decode(np.array([b], np.uint16))[0]))  # noqa: E731
    A = [[F(inp["A"][m, k]) for k in range(K1)] for m in range(M)]
    Wo = [[F(inp["Wo_t"][n, k]) for k in range(K1)] for n in range(d)]
    X = [[F(inp["x_res"][m, n]) for n in range(d)] for m in range(M)]
    g = [Fraction(float(v)) for v in inp["gamma"]]
    Wp = [[F(prep["Wp"][n, k]) for k in range(d)] for n in range(N2w)]
    eps = Fraction(w.eps)
    n_out = N2w // 2 if act == si.ACT_SWIGLU else N2w
    for m in range(M):
        h = [X[m][n] + sum(A[m][k] * Wo[n][k] for k in range(K1)) for n in range(d)]
        for n in range(d):
            assert abs(Fraction(out["h"][m, n]) - h[n]) <= abs(h[n]) * Fraction(1, 10 ** 15)
        hb_codes = [_bf16_nearest(v) if v >= 0 else (_bf16_nearest(-v) | 0x8000) for v in h]
        assert [int(c) for c in out["hb"][m]] == hb_codes
        hb = [F(c) for c in hb_codes]
        S = sum(v * v for v in hb)
        assert Fraction(out["S"][m]) == S                       # exact: few 8-bit squares
        r = 1 / (_dec(S / d + eps)).sqrt()
        assert abs(Decimal(out["r"][m]) - r) <= r * Decimal("1e-15")
        nrm = [_dec(hb[k]) * r * _dec(g[k]) for k in range(d)]
        z = [sum(nrm[k] * _dec(Wp[n][k] / g[k]) for k in range(d)) for n in range(N2w)]
        for j in range(n_out):
            if act == si.ACT_SWIGLU:
                gate, up = z[j], z[n_out + j]
                yv = gate / (1 + (-gate).exp()) * up
            else:
                yv = z[j]
            assert abs(Decimal(out["y"][m, j]) - yv) <= Decimal("1e-14") * (1 + abs(yv)), (m, j)


def test_first_gemm_matches_blas():
    w = si.custom(40, 96, 64, 32, si.ACT_NONE, seed=5)
    inp, prep, out = _run(w)
    A = oracle.bf16_decode(inp["A"])
    Wo = oracle.bf16_decode(inp["Wo_t"])
    X = oracle.bf16_decode(inp["x_res"])
    ref = X + A @ Wo.T
    assert np.max(np.abs(out["h"] - ref)) <= 1e-13 * (1 + np.abs(ref).max())
    assert np.array_equal(out["hb"], oracle.bf16_encode(out["h"]))


@pytest.mark.parametrize("act", [si.ACT_NONE, si.ACT_SWIGLU])
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_row_scale_commutes_with_second_gemm(act, dtype):
    """act(r * (hb @ W'^T)) == the unfused oracle output (reparameterisation identity)."""
    w = si.custom(48, 80, 128, 2 * 72, act, seed=21, dtype=dtype)
    inp, prep, out = _run(w)
    hb = oracle.bf16_decode(out["hb"])
    dec = oracle.bf16_decode if prep["wp_dt"] == oracle.BF16 else oracle.e4m3_decode
    Wp = dec(prep["Wp"]) * prep["wp_scale"]
    z = out["r"][:, None] * (hb @ Wp.T)
    if act == si.ACT_SWIGLU:
        F = Wp.shape[0] // 2
        y = z[:, :F] / (1 + np.exp(-z[:, :F])) * z[:, F:]
    else:
        y = z
    assert np.max(np.abs(out["y"] - y) / (1 + np.abs(y))) <= 1e-12
    # and S/r follow the bf16 hb, row by row
    assert np.allclose(out["S"], (hb * hb).sum(1), rtol=1e-15, atol=0)
    d = hb.shape[1]
    assert np.allclose(out["r"], 1 / np.sqrt(out["S"] / d + w.eps), rtol=1e-15, atol=0)


def test_constant_row_closed_form():
    # A = 0 makes h = x_res; a constant row c gives r = 1/sqrt(c^2 + eps) exactly.
    w = si.custom(4, 16, 32, 64, si.ACT_NONE, seed=3)
    inp = si.generate(w)
    inp["A"][:] = 0
    cs = [1.0, -0.5, 3.0, 0.0078125]
    for m, c in enumerate(cs):
        inp["x_res"][m, :] = si.to_bf16_bits(np.full(w.d, c, np.float32))
    _, _, out = _run(w, inp)
    for m, c in enumerate(cs):
        assert np.all(out["h"][m] == c)
        assert out["S"][m] == w.d * c * c
        assert abs(out["r"][m] - 1 / np.sqrt(c * c + w.eps)) <= 1e-16 / np.sqrt(c * c + w.eps) * 4


def test_identity_second_weight_closed_form():
    # act NONE, W = I and gamma exactly bf16-representable: W' = diag(gamma) exactly and
    # y[m,n] = hb[m,n] * r[m] * gamma[n].
    d = 64
    w = si.custom(6, 32, d, d, si.ACT_NONE, seed=8)
    inp = si.generate(w)
    inp["W_t"] = si.to_bf16_bits(np.eye(d, dtype=np.float32))
    g = oracle.bf16_decode(si.to_bf16_bits(inp["gamma"])).astype(np.float32)
    inp["gamma"] = g
    _, prep, out = _run(w, inp)
    assert np.array_equal(oracle.bf16_decode(prep["Wp"]), np.diag(g.astype(np.float64)))
    hb = oracle.bf16_decode(out["hb"])
    ref = hb * out["r"][:, None] * g[None, :].astype(np.float64)
    assert np.max(np.abs(out["y"] - ref)) <= 1e-15 * (1 + np.abs(ref).max())
    # mean((y/gamma)^2) = ms/(ms+eps)
    ms = out["S"] / d
    lhs = np.mean((out["y"] / g[None, :]) ** 2, axis=1)
    assert np.allclose(lhs, ms / (ms + w.eps), rtol=1e-13)


def test_zero_first_weight_and_no_residual():
    w = si.custom(5, 24, 32, 40, si.ACT_NONE, seed=4)
    inp = si.generate(w)
    inp0 = dict(inp, Wo_t=np.zeros_like(inp["Wo_t"]))
    _, _, out = _run(w, inp0)
    assert np.array_equal(out["h"], oracle.bf16_decode(inp["x_res"]))
    prep = oracle.prepare(inp, "bf16")
    out2 = oracle.chain(prep, None, inp["gamma"], w.act, w.eps)
    A = oracle.bf16_decode(inp["A"])
    Wo = oracle.bf16_decode(inp["Wo_t"])
    assert np.allclose(out2["h"], A @ Wo.T, rtol=1e-13, atol=1e-13)


def test_zero_gate_gives_zero_output():
    w = si.custom(8, 32, 48, 2 * 40, si.ACT_SWIGLU, seed=6)
    inp = si.generate(w)
    inp["W_t"][:40] = 0                              # gate rows (first half)
    _, _, out = _run(w, inp)
    assert np.all(out["y"] == 0.0)
    inp = si.generate(w)
    inp["W_t"][40:] = 0                              # up rows (second half)
    _, _, out = _run(w, inp)
    assert np.all(out["y"] == 0.0)


def test_scale_invariance_at_zero_eps():
    # Scaling A and x_res by 2 doubles h and hb exactly and halves r exactly at eps = 0.
    w = si.custom(16, 32, 64, 2 * 48, si.ACT_SWIGLU, seed=12)
    inp = si.generate(w)
    _, _, o1 = _run(w, inp, eps=0.0)
    inp2 = dict(inp, A=(inp["A"] + np.uint16(0x80)), x_res=(inp["x_res"] + np.uint16(0x80)))
    assert np.array_equal(oracle.bf16_decode(inp2["A"]), 2 * oracle.bf16_decode(inp["A"]))
    _, _, o2 = _run(w, inp2, eps=0.0)
    assert np.array_equal(oracle.bf16_decode(o2["hb"]), 2 * oracle.bf16_decode(o1["hb"]))
    assert np.allclose(o2["r"], o1["r"] / 2, rtol=1e-15, atol=0)
    assert np.allclose(o2["y"], o1["y"], rtol=1e-14, atol=1e-14)


def test_gate_up_order_and_silu_closed_form():
    # d = F, W = [I; 2I]: gate = n, up = 2n, y = silu(n) * 2n with n = hb*r*gamma (W'=diag).
    d = 32
    w = si.custom(4, 16, d, 2 * d, si.ACT_SWIGLU, seed=10)
    inp = si.generate(w)
    inp["gamma"] = np.ones(d, np.float32)
    inp["W_t"] = si.to_bf16_bits(np.concatenate([np.eye(d), 2 * np.eye(d)]).astype(np.float32))
    _, _, out = _run(w, inp)
    n = oracle.bf16_decode(out["hb"]) * out["r"][:, None]
    ref = n / (1 + np.exp(-n)) * 2 * n
    assert np.max(np.abs(out["y"] - ref)) <= 1e-15 * (1 + np.abs(ref).max())


def test_row_subset_matches_full():
    w = si.custom(37, 64, 96, 2 * 64, si.ACT_SWIGLU, seed=14)
    inp, prep, full = _run(w)
    rows = np.array([36, 0, 17, 5])
    sub = oracle.chain(prep, inp["x_res"], inp["gamma"], w.act, w.eps, rows=rows)
    for key in ("h", "hb", "S", "r", "y"):
        assert np.array_equal(sub[key], full[key][rows])
