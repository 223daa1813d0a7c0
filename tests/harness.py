"""Shared helpers of the GPU parity tests: run the HIP chain through the binding (which
calls the C ABI) and the fp64 oracle on the same seeded inputs, and compare.

Tolerances (elementwise): |gpu - ref| <= tol * (1 + |ref|) with tol = 2e-2 for the bf16
chain and 6e-2 for the 8-bit chain, for h and y.  Tighter diagnostics on the
intermediates: h is within the fp32 summation bound of the oracle's rounded hb (bf16
path); the partials sum to sum_n h_gpu^2 within the fp32 summation bound; r follows the
GPU's own partials within 2 fp32 ulp, and the oracle's r within 1e-4 (bf16) / 2e-3
(8-bit) relative.
"""

from __future__ import annotations

import numpy as np
import torch

import gemm_epilogue_transformer_amd as coda
import oracle
import synth_inputs as si

TOL = {"bf16": 2e-2, "e4m3": 6e-2}


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def upload(inp: dict) -> dict:
    return {
        "A": dev_bf16(inp["A"]),
        "Wo_t": dev_bf16(inp["Wo_t"]),
        "x_res": dev_bf16(inp["x_res"]),
        "gamma": torch.from_numpy(inp["gamma"]).cuda(),
        "W_t": dev_bf16(inp["W_t"]),
    }


def gpu_prepare(w: si.Workload, d: dict) -> dict:
    """Weight/activation preparation through the library (fold, or quantise)."""
    if w.dtype == "bf16":
        return dict(A=d["A"], Wo=d["Wo_t"], Wp=coda.prepare_weight_bf16(d["W_t"], d["gamma"]),
                    a_scale=None, wo_scale=None, wp_scale=None)
    qa, sa = coda.quantize_e4m3(d["A"])
    qo, so = coda.quantize_e4m3(d["Wo_t"])
    qw, sw = coda.quantize_e4m3(d["W_t"], d["gamma"])
    return dict(A=qa, Wo=qo, Wp=qw, a_scale=sa[1:], wo_scale=so[1:], wp_scale=sw[1:],
                amax_scale=(sa, so, sw))


def gpu_chain_gfold(w: si.Workload, d: dict, gamma=None):
    """The bf16 chain with the second GEMM on the raw weight, gamma folded in on chip."""
    g = d["gamma"] if gamma is None else gamma
    h, P = coda.gemm_resid_partialrms(d["A"], d["Wo_t"], d["x_res"])
    r = coda.rowscale_reduce(P, d["Wo_t"].shape[0], w.eps)
    y = coda.gemm_rowscale_gfold(h, d["W_t"], g, r, act=w.act)
    return h, P, r, y


def gpu_chain(w: si.Workload, d: dict, prep: dict, x_res="x_res", h_out=None):
    xr = d[x_res] if isinstance(x_res, str) else x_res
    h, P, r, y = coda.chain(prep["A"], prep["Wo"], xr, prep["Wp"], w.eps, act=w.act,
                            a_scale=prep["a_scale"], wo_scale=prep["wo_scale"],
                            wp_scale=prep["wp_scale"],
                            out=None if h_out is None else {"h": h_out})
    return h, P, r, y


def sample_rows(M: int, n_random: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 127, 128, 129, 255, 256, M // 2, M - 129, M - 128, M - 33, M - 1]
    rows = set(r for r in fixed if 0 <= r < M)
    rows |= set(int(x) for x in rng.choice(M, size=min(n_random, M), replace=False))
    return np.array(sorted(rows), np.int64)


def check_chain(w: si.Workload, inp: dict, h, P, r, y, rows=None, ref=None, prep_ref=None):
    """Compare the GPU chain outputs (device tensors) with the oracle on `rows`."""
    tol = TOL[w.dtype]
    if prep_ref is None:
        prep_ref = oracle.prepare(inp, w.dtype)
    if ref is None:
        ref = oracle.chain(prep_ref, inp["x_res"], inp["gamma"], w.act, w.eps, rows=rows)
    sel = slice(None) if rows is None else torch.from_numpy(rows).to(h.device)
    hg = oracle.bf16_decode(host_bits(h[sel]))
    yg = oracle.bf16_decode(host_bits(y[sel]))
    Pg = P[sel].cpu().numpy().astype(np.float64)
    rg = r[sel].cpu().numpy().astype(np.float64)

    # gate: h and y within tol*(1+|ref|), elementwise
    eh = np.abs(hg - ref["h"]) / (1 + np.abs(ref["h"]))
    ey = np.abs(yg - ref["y"]) / (1 + np.abs(ref["y"]))
    assert np.all(np.isfinite(yg)), "non-finite y"
    assert eh.max() <= tol, f"h error {eh.max():.3e} > {tol}"
    assert ey.max() <= tol, f"y error {ey.max():.3e} > {tol} at {np.unravel_index(ey.argmax(), ey.shape)}"

    # diagnostics on the intermediates
    #  h: the GPU sums exact products in fp32 (any order), adds x_res in fp32 and rounds
    #  once to bf16, so |h_gpu - hb_ref| <= gamma_K * sum_k |a_k w_k| + 2^-24 |v|
    #  + half a bf16 ulp of each side (gamma_K = K u / (1 - K u), u = 2^-24).  The 8-bit
    #  MFMA sums its 64 products per instruction at a precision the ISA does not pin to
    #  IEEE fp32, so for e4m3 the bound is reported (ratio) and only checked loosely.
    hb_ref = oracle.bf16_decode(ref["hb"])
    K = prep_ref["A"].shape[1]
    dec = oracle.bf16_decode if prep_ref["a_dt"] == oracle.BF16 else oracle.e4m3_decode
    rows_sel = slice(None) if rows is None else rows
    a_abs = np.abs(dec(prep_ref["A"][rows_sel]) * prep_ref["a_scale"])
    w_abs = np.abs((oracle.bf16_decode if prep_ref["wo_dt"] == oracle.BF16 else oracle.e4m3_decode)(
        prep_ref["Wo"]) * prep_ref["wo_scale"])
    s_abs = a_abs @ w_abs.T
    u = 2.0 ** -24
    gamma_k = K * u / (1 - K * u)
    bound = gamma_k * s_abs + u * np.abs(ref["h"]) + 2.0 ** -8 * (np.abs(hg) + np.abs(hb_ref)) + 2.0 ** -133
    dev = np.abs(hg - hb_ref)
    ratio = dev / bound
    print(f"h vs oracle hb: max {ratio.max():.3f} of the fp32-summation bound; "
          f"max |h-hb_ref|/sum|a w| {np.max(dev / (s_abs + 1e-30)):.3e}", flush=True)
    if w.dtype == "bf16":
        assert np.all(ratio <= 1.0), "h outside the fp32 summation bound"
    else:
        assert np.all(dev <= 2.0 ** -10 * s_abs + 2.0 ** -8 * (np.abs(hg) + np.abs(hb_ref)) + 1e-30), \
            "8-bit h deviates by more than 2^-10 of sum|a w|"
    d = hg.shape[1]
    s_gpu = (hg * hg).sum(1)
    assert np.allclose(Pg.sum(1), s_gpu, rtol=d * 2.0 ** -24, atol=0), "partials disagree with h"
    r64 = 1.0 / np.sqrt(Pg.sum(1) / d + np.float64(np.float32(w.eps)))
    assert np.all(np.abs(rg - r64) <= 2 * np.spacing(np.float32(r64)).astype(np.float64)), "r not fp32-rounded"
    r_rel = float(np.max(np.abs(rg - ref["r"]) / ref["r"]))
    print(f"r vs oracle: max rel {r_rel:.3e}", flush=True)
    assert r_rel <= (1e-4 if w.dtype == "bf16" else 2e-3), "r disagrees with the oracle"
    return dict(h_err=float(eh.max()), y_err=float(ey.max()),
                y_err_rms=float(np.sqrt(np.mean((yg - ref["y"]) ** 2))))
