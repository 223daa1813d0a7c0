"""GPU parity of the LM-head block's backward, loss_m = CE(RMSNorm(h) . W^T, t_m): the
recomputed logits with the loss backward in the epilogue (r * g * (softmax - onehot)
and the row-scale partials, from the forward's lse), then the row coefficient, the
input-gradient GEMM and the weight / gamma gradients on dz and h as stored, against the
oracle's unfused chain rule on ragged shapes (every entry; vocabulary tails, ignored
targets), at the LLaMA-3-1B LM-head shape on sampled rows (dz, dh) and against the
definitions of dW and dgamma over the GPU's own dz, plus exact zeros for ignored rows.

The loss weights g are drawn in [16, 64] in the parity cases so that the gradients are
of order one and the bound 2e-2 * (1 + |ref|) is meaningful (the path is linear in g).
dz: most logit gradients are tiny (softmax probabilities), so its bound is relative,
2^-7 |ref| (the bf16 rounding, 2^-9, and the fp32 logits' error in exp) plus 1e-4 of
the row's largest entry.  dh, dW and dgamma are sums over the vocabulary or the tokens
of terms with the bf16-rounded dz as an operand: reading 18's bound (u = 2^-8, the
root-sum-square of the terms from the oracle) and a Frobenius-relative error below
1e-2.
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import oracle
import synth_inputs as si
from harness import TOL, dev_bf16, host_bits

pytestmark = pytest.mark.gpu

U = 2.0 ** -8
C = 8.0


def _log(msg):
    print(msg, flush=True)


def _run(w, inp, g):
    h, W = dev_bf16(inp["h"]), dev_bf16(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    t = torch.from_numpy(inp["targets"]).cuda()
    gd = torch.from_numpy(np.asarray(g, dtype=np.float32)).cuda()
    Wp = coda.prepare_weight_bf16(W, gamma)
    Wpt = coda.transpose_bf16(Wp)
    r = coda.rowscale_from_h(h, w.eps)
    partials, tl = coda.gemm_rowscale_ce(h, Wp, r, t)
    lse, _ = coda.ce_reduce(partials, t, tl, w.N2w)
    out = coda.lmhead_ce_bwd(h, r, Wp, Wpt, W, gamma, t, lse, gd)
    torch.cuda.synchronize()
    return out, dict(h=h, W=W, Wp=Wp, r=r, t=t, lse=lse, g=gd, gamma=gamma)


def _np(x):
    return x.cpu().numpy().astype(np.float64)


def _check_dz(gpu, ref, name="dz"):
    bound = 2.0 ** -7 * np.abs(ref) + 1e-4 * np.max(np.abs(ref), axis=1, keepdims=True)
    e = np.abs(gpu - ref) / np.maximum(bound, 1e-300)
    _log(f"  {name}: err/bound max {e.max():.2e}")
    assert np.all(np.isfinite(gpu)) and e.max() <= 1


def _dh_rss(inp, o):
    """Root-sum-square of dh's product terms, r * gamma_k * sqrt(sum_v (dL/dz_v W_vk)^2): dh
    sums them over the vocabulary with the bf16-rounded dz as operand (reading 18)."""
    Wr = oracle.bf16_decode(inp["W_t"])
    gam = np.abs(inp["gamma"].astype(np.float64))
    return o["r"][:, None] * gam[None, :] * np.sqrt((o["dz"] ** 2) @ (Wr ** 2))


def _bounded(name, gpu, ref, rss):
    e = np.abs(gpu - ref) / (TOL["bf16"] * (1 + np.abs(ref)) + C * U * rss)
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)
    _log(f"  {name}: err/bound max {e.max():.2e}, rel fro {rel:.2e}")
    assert np.all(np.isfinite(gpu)) and e.max() <= 1 and rel <= 1e-2


SMALL = [
    # M tokens, d, V: ragged against the 256 x 256 tiles; V = 296: the last tile's second
    # wave lies wholly past V (3 partial columns per row, not 4)
    (300, 136, 296),
    (264, 200, 1000),
    (130, 64, 2056),
    (8, 8, 8),
]


@pytest.mark.parametrize("M,d,V", SMALL)
def test_ce_bwd_small_all_entries(M, d, V):
    w = si.custom(M, 0, d, V, si.ACT_CE_BWD, seed=11 * M + d + V)
    _log(f"ce bwd small {w.name}")
    inp = si.generate(w)
    inp["targets"][::7] = -100                   # ignored rows
    inp["targets"][1] = V - 1
    g = np.random.default_rng(M + V).uniform(16, 64, size=M)
    got, _ = _run(w, inp, g)
    o = oracle.lmhead_ce_bwd(inp["h"], inp["gamma"], oracle.fold_bf16(inp["W_t"], inp["gamma"]), 1.0, inp["W_t"],
                             inp["targets"], g, w.eps, js="all", rss=True)
    dz = oracle.bf16_decode(host_bits(got["dz"]))
    _check_dz(dz, o["r"][:, None] * o["dz"])
    assert np.all(dz[::7] == 0.0)
    _bounded("dh", oracle.bf16_decode(host_bits(got["dh"])), o["dh"], _dh_rss(inp, o))
    _bounded("dW", _np(got["dW"]), o["dW"], np.abs(inp["gamma"].astype(np.float64))[None, :] * o["rss"])
    _bounded("dgamma", _np(got["dgamma"]), o["dgamma"], o["rss_gamma"])


def test_ce_bwd_workload_sampled():
    w = si.WORKLOADS[11]
    _log(f"ce bwd workload {w.name}")
    inp = si.generate(w)
    g = np.full(w.M, 32.0)
    got, st = _run(w, inp, g)
    rng = np.random.default_rng(12)
    rows = np.array(sorted({0, 255, 256, w.M - 1} | set(rng.choice(w.M, 6, replace=False).tolist())))
    o = oracle.lmhead_ce_bwd(inp["h"], inp["gamma"], oracle.fold_bf16(inp["W_t"], inp["gamma"]), 1.0, inp["W_t"],
                             inp["targets"], g, w.eps, rows=rows)
    dz = oracle.bf16_decode(host_bits(got["dz"][torch.from_numpy(rows).cuda()]))
    _check_dz(dz, o["r"][:, None] * o["dz"], "dz sampled rows")
    lse = _np(st["lse"])[rows]
    _log(f"  lse (forward) vs oracle: err max {np.abs(lse - o['lse']).max():.2e}")
    assert np.max(np.abs(lse - o["lse"])) <= 1e-3
    _bounded("dh sampled rows", oracle.bf16_decode(host_bits(got["dh"]))[rows], o["dh"], _dh_rss(inp, o))
    # dW against its definition over the GPU's own dz: fp32 sums of exact bf16 products
    js = np.array(sorted({0, 1, w.N2w - 1} | set(rng.choice(w.N2w, 7, replace=False).tolist())))
    ks = rng.choice(w.d, 8, replace=False)
    dzj = oracle.bf16_decode(host_bits(got["dz"][:, torch.from_numpy(js).cuda()].contiguous()))
    hk = oracle.bf16_decode(inp["h"])[:, ks]
    gam = inp["gamma"].astype(np.float64)[ks]
    ref = (dzj.T @ hk) * gam[None, :]
    bound = (w.M + 256) * 2.0 ** -24 * (np.abs(dzj).T @ np.abs(hk)) * np.abs(gam)[None, :]
    err = np.abs(_np(got["dW"])[np.ix_(js, ks)] - ref)
    _log(f"  dW vs its definition over the GPU's dz: err max {err.max():.2e}, bound min {bound.min():.2e}")
    assert np.all(err <= bound)
    # dgamma = sum_j W[j, k] G[j, k], G = dW / gamma: from the GPU's own dW columns
    dW, dgam = _np(got["dW"]), _np(got["dgamma"])
    Wr = oracle.bf16_decode(inp["W_t"])
    ref_g = (Wr[:, ks] * dW[:, ks]).sum(axis=0) / gam
    scale = (np.abs(Wr[:, ks] * dW[:, ks])).sum(axis=0) / np.abs(gam)
    assert np.all(np.abs(dgam[ks] - ref_g) <= 1e-4 * scale)


def test_ce_bwd_deterministic_bitwise():
    w = si.custom(264, 0, 136, 1000, si.ACT_CE_BWD, seed=51)
    inp = si.generate(w)
    g = np.full(w.M, 1.0 / w.M)
    a, _ = _run(w, inp, g)
    b, _ = _run(w, inp, g)
    for k in ("dz", "dh", "dW", "dgamma", "q"):
        x, y = a[k], b[k]
        vt = torch.int32 if x.dtype == torch.float32 else torch.int16
        assert torch.equal(x.view(vt), y.view(vt)), k
