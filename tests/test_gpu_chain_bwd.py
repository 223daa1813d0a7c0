"""GPU parity of the whole chain's backward (h = x_res + A . Wo^T -> RMSNorm -> gate/up
GEMM -> SwiGLU): dh (= the gradient of x_res), dA, dWo, dW and dgamma from the
forward's saved h and r, against the oracle's unfused chain rule on ragged shapes (every
entry), and at the LLaMA-3-1B shape on sampled rows of dh and dA plus the definition of
dWo over the GPU's own dh.

Bounds.  dh: 2e-2 * (1 + |ref|).  The other gradients are sums of products of stored
bf16 values (dh and dz rounded by the path, h possibly one bf16 step from the oracle's
rounding of the same fp64 value): each summed term carries a relative error of at most
about 2^-7, independent between terms, so the elementwise bound adds 8 * 2^-7 times the
root-sum-square of the terms (the oracle's rss; by Hoeffding's inequality exceeded with
probability below 3e-14), and the Frobenius-relative error must stay below 1e-2.
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import oracle
import synth_inputs as si
from harness import TOL, dev_bf16, host_bits

pytestmark = pytest.mark.gpu

U = 2.0 ** -7
C = 8.0


def _log(msg):
    print(msg, flush=True)


def _gpu(w, inp, saved=False):
    """The forward chain, then its backward: recomputing the gate/up product, or (saved)
    from the pre-activation the forward kept."""
    A, Wo, xr = dev_bf16(inp["A"]), dev_bf16(inp["Wo_t"]), dev_bf16(inp["x_res"])
    W, dy, dres = dev_bf16(inp["W_t"]), dev_bf16(inp["dy"]), dev_bf16(inp["dres"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    Wp = coda.prepare_weight_bf16(W, gamma)
    Wpt, WoT = coda.transpose_bf16(Wp), coda.transpose_bf16(Wo)
    if saved:
        h, _, r, y, z = coda.chain(A, Wo, xr, Wp, w.eps, save_z=True)
        y_plain = coda.gemm_rowscale_swiglu(h, Wp, r)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))
    else:
        h, _, r, _ = coda.chain(A, Wo, xr, Wp, w.eps)
        z = None
    g = coda.chain_bwd(A, WoT, h, r, Wp, Wpt, W, gamma, dy, dres, z=z)
    torch.cuda.synchronize()
    dec = lambda t: oracle.bf16_decode(host_bits(t))  # noqa: E731
    return {"dh": dec(g["dh"]), "dA": dec(g["dA"]), "dWo": g["dWo"].cpu().numpy().astype(np.float64),
            "dW": g["dW"].cpu().numpy().astype(np.float64), "dgamma": g["dgamma"].cpu().numpy().astype(np.float64),
            "A": inp["A"]}


def _bounded(name, gpu, ref, rss):
    e = np.abs(gpu - ref) / (TOL["bf16"] * (1 + np.abs(ref)) + C * U * rss)
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)
    _log(f"  {name}: err/bound max {e.max():.2e}, rel fro {rel:.2e}")
    assert np.all(np.isfinite(gpu)) and e.max() <= 1 and rel <= 1e-2


SMALL = [
    # M tokens, K1, d, F: ragged against every tile (several tiles), tokens a multiple of 8
    (296, 136, 200, 104),
    (264, 72, 264, 200),
    (520, 264, 128, 256),
    (8, 8, 8, 8),
]


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved_z"])
@pytest.mark.parametrize("M,K1,d,F", SMALL)
def test_chain_bwd_small_all_entries(M, K1, d, F, saved):
    w = si.custom(M, K1, d, 2 * F, si.ACT_CHAIN_BWD, seed=5 * M + K1 + d + F)
    _log(f"chain bwd small {w.name} saved={saved}")
    inp = si.generate(w)
    got = _gpu(w, inp, saved)
    o = oracle.chain_bwd(oracle.prepare(inp, "bf16"), inp["x_res"], inp["gamma"], inp["W_t"], inp["dy"], w.eps,
                         dres=inp["dres"], rss=True)
    e_dh = np.abs(got["dh"] - o["dh"]) / (1 + np.abs(o["dh"]))
    _log(f"  dh: err max {e_dh.max():.2e}")
    assert np.all(np.isfinite(got["dh"])) and e_dh.max() <= TOL["bf16"]
    _bounded("dA", got["dA"], o["dA"], o["rss_dA"])
    _bounded("dWo", got["dWo"], o["dWo"], o["rss_dWo"])
    _bounded("dW", got["dW"], o["dW"], np.abs(inp["gamma"].astype(np.float64))[None, :] * o["rss_dW"])
    _bounded("dgamma", got["dgamma"], o["dgamma"], o["rss_dgamma"])


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved_z"])
def test_chain_bwd_workload_sampled(saved):
    w = si.WORKLOADS[9]
    _log(f"chain bwd workload {w.name} saved={saved}")
    inp = si.generate(w)
    got = _gpu(w, inp, saved)
    rows = np.array(sorted({0, 1, 255, 256, w.M // 2, w.M - 1} |
                           set(np.random.default_rng(9).choice(w.M, 10, replace=False).tolist())))
    o = oracle.chain_bwd(oracle.prepare(inp, "bf16"), inp["x_res"], inp["gamma"], inp["W_t"], inp["dy"], w.eps,
                         dres=inp["dres"], rows=rows, rss=True)
    e_dh = np.abs(got["dh"][rows] - o["dh"]) / (1 + np.abs(o["dh"]))
    _log(f"  dh sampled rows: err max {e_dh.max():.2e}")
    assert e_dh.max() <= TOL["bf16"]
    _bounded("dA sampled rows", got["dA"][rows], o["dA"], o["rss_dA"])
    # dWo is the token sum of the GPU's own dh against A: fp32 sums of exact bf16
    # products, |err| <= M * 2^-24 * sum_m |dh A| on sampled entries
    rng = np.random.default_rng(10)
    ns, ks = rng.choice(w.d, 12, replace=False), rng.choice(w.K1, 12, replace=False)
    Ad = oracle.bf16_decode(inp["A"])
    ref = got["dh"][:, ns].T @ Ad[:, ks]
    bound = w.M * 2.0 ** -24 * (np.abs(got["dh"][:, ns]).T @ np.abs(Ad[:, ks]))
    err = np.abs(got["dWo"][np.ix_(ns, ks)] - ref)
    _log(f"  dWo vs its definition over the GPU's dh: err max {err.max():.2e}, bound min {bound.min():.2e}")
    assert np.all(err <= bound)
    assert np.all(np.isfinite(got["dW"])) and np.all(np.isfinite(got["dgamma"]))


def test_plain_gemm_matches_its_definition_and_adds_the_residual():
    rng = np.random.default_rng(19)
    M, N, K = 300, 136, 200
    a = si.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    b = si.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    c = si.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    Cg = coda.gemm_bf16(dev_bf16(a), dev_bf16(b))
    cres = dev_bf16(c)
    Cr = coda.gemm_bf16(dev_bf16(a), dev_bf16(b), c_res=cres)
    coda.gemm_bf16(dev_bf16(a), dev_bf16(b), c_res=cres, C=cres)          # in place
    torch.cuda.synchronize()
    assert torch.equal(Cr.view(torch.int16), cres.view(torch.int16))
    ad, bd, cd = oracle.bf16_decode(a), oracle.bf16_decode(b), oracle.bf16_decode(c)
    for got, ref, res in ((Cg, ad @ bd.T, 0.0), (Cr, ad @ bd.T + cd, np.abs(cd))):
        g = oracle.bf16_decode(host_bits(got))
        # one bf16 rounding of the fp32 sum: |err| <= 2^-8 |ref| + (K + 2) 2^-24 sum|terms|
        bound = 2.0 ** -8 * np.abs(ref) + (K + 2) * 2.0 ** -24 * (np.abs(ad) @ np.abs(bd).T + res)
        assert np.all(np.abs(g - ref) <= bound * 1.01)


@pytest.mark.parametrize("K", [2056, 8200])
def test_plain_gemm_long_contraction_matches_its_definition(K):
    # K from 2048 up: the stage-ring mainloop (33 or 129 k-tiles, the last one ragged)
    rng = np.random.default_rng(20 + K)
    M, N = 300, 136
    a = si.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    b = si.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    Cg = coda.gemm_bf16(dev_bf16(a), dev_bf16(b))
    torch.cuda.synchronize()
    ad, bd = oracle.bf16_decode(a), oracle.bf16_decode(b)
    ref = ad @ bd.T
    g = oracle.bf16_decode(host_bits(Cg))
    bound = 2.0 ** -8 * np.abs(ref) + (K + 2) * 2.0 ** -24 * (np.abs(ad) @ np.abs(bd).T)
    assert np.all(np.abs(g - ref) <= bound * 1.01)


def test_saved_pre_activation_and_its_backward():
    # z = bf16(r * (h . W'^T)) against its definition over the GPU's own h and r; the
    # saved backward's transposed copy is the exact transpose of its dz; ragged rows
    rng = np.random.default_rng(23)
    M, K, F = 200, 136, 104
    hb = si.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    Wb = si.to_bf16_bits((rng.standard_normal((2 * F, K)) / np.sqrt(K)).astype(np.float32))
    dyb = si.to_bf16_bits(rng.standard_normal((M, F)).astype(np.float32))
    h, W, dy = dev_bf16(hb), dev_bf16(Wb), dev_bf16(dyb)
    r = coda.rowscale_from_h(h, 1e-5)
    y, z = coda.gemm_rowscale_swiglu_save(h, W, r)
    dz, dzt, P = coda.swiglu_bwd_saved(z, dy, r)
    dz2, none, P2 = coda.swiglu_bwd_saved(z, dy, r, transpose=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(dz.view(torch.int16), dz2.view(torch.int16)) and torch.equal(P, P2)
    assert torch.equal(dzt.view(torch.int16), dz.view(torch.int16).t().contiguous())
    H, Wd = oracle.bf16_decode(hb), oracle.bf16_decode(Wb)
    rr = r.cpu().numpy().astype(np.float64)[:, None]
    ref = rr * (H @ Wd.T)
    bound = 2.0 ** -8 * np.abs(ref) + (K + 2) * 2.0 ** -24 * rr * (np.abs(H) @ np.abs(Wd).T)
    zg = oracle.bf16_decode(host_bits(z))
    assert np.all(np.abs(zg - ref) <= bound * 1.01)
    # the backward of the saved z, in fp64 from the same bf16 z: dz and the partials
    g, u = zg[:, :F], zg[:, F:]
    d = oracle.bf16_decode(dyb)
    s = 1.0 / (1.0 + np.exp(-g))
    dg, du = d * u * s * (1 + g * (1 - s)), d * g * s
    ref_dz = rr * np.concatenate([dg, du], axis=1)
    e = np.abs(oracle.bf16_decode(host_bits(dz)) - ref_dz) / (1e-3 + np.abs(ref_dz))
    _log(f"  saved backward dz rel err max {e.max():.2e}")
    assert e.max() <= 2.0 ** -7
    T = P.shape[1]
    assert T == -(-F // 128)
    terms = (dg * g + du * u) / rr
    ref_P = np.stack([terms[:, 128 * t:128 * (t + 1)].sum(1) for t in range(T)], axis=1)
    scale = np.stack([np.abs(terms[:, 128 * t:128 * (t + 1)]).sum(1) for t in range(T)], axis=1)
    assert np.all(np.abs(P.cpu().numpy() - ref_P) <= 1e-5 * scale + 1e-30)


@pytest.mark.parametrize("M", [13, 1, 70])
def test_saved_backward_without_transpose_takes_any_row_count(M):
    # without the transposed copy the row count is free (no 16-byte token runs); dz and the
    # partials against the fp64 formulas from the same bf16 z, rows past the tile masked
    rng = np.random.default_rng(24 + M)
    F = 136
    zb = si.to_bf16_bits(rng.standard_normal((M, 2 * F)).astype(np.float32))
    dyb = si.to_bf16_bits(rng.standard_normal((M, F)).astype(np.float32))
    rr = (0.5 + rng.random(M)).astype(np.float32)
    dz, none, P = coda.swiglu_bwd_saved(dev_bf16(zb), dev_bf16(dyb), torch.from_numpy(rr).cuda(), transpose=False)
    torch.cuda.synchronize()
    assert none is None
    zg, d, r = oracle.bf16_decode(zb), oracle.bf16_decode(dyb), rr.astype(np.float64)[:, None]
    g, u = zg[:, :F], zg[:, F:]
    s = 1.0 / (1.0 + np.exp(-g))
    dg, du = d * u * s * (1 + g * (1 - s)), d * g * s
    ref_dz = r * np.concatenate([dg, du], axis=1)
    e = np.abs(oracle.bf16_decode(host_bits(dz)) - ref_dz) / (1e-3 + np.abs(ref_dz))
    assert e.max() <= 2.0 ** -7
    terms = (dg * g + du * u) / r
    T = P.shape[1]
    ref_P = np.stack([terms[:, 128 * t:128 * (t + 1)].sum(1) for t in range(T)], axis=1)
    scale = np.stack([np.abs(terms[:, 128 * t:128 * (t + 1)]).sum(1) for t in range(T)], axis=1)
    assert np.all(np.abs(P.cpu().numpy() - ref_P) <= 1e-5 * scale + 1e-30)
