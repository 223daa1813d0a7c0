"""GPU parity of the MLP-input block's weight gradients (dL/dW = gamma * G and
dL/dgamma = sum_j W * G with G = (r * dL/dz)^T h over the tokens) against the oracle's
unfused chain rule: every entry on ragged shapes, sampled entries of dW and the
dW / dgamma consistency at the LLaMA-3-1B shape; the plain token-contracting GEMM
(gamma = NULL, W = NULL) against its fp64 definition; the empty token batch; bitwise
determinism.

The GPU gradient starts from the backward's own bf16 dz (r * dL/dz rounded once, a
relative error of at most 2^-8 per term), the oracle from fp64 throughout.  Summed over
M tokens these roundings add like independent zero-mean errors, so the elementwise
bound is 2e-2 * (1 + |ref|) plus 8 * 2^-8 times the root-sum-square of the summed terms
(the oracle's rss): by Hoeffding's inequality a sum of independent terms bounded by
2^-8 |a_m| exceeds c * 2^-8 * sqrt(sum a_m^2) with probability below 2 exp(-c^2 / 2),
about 3e-14 at c = 8 (the probabilistic rounding analysis of Higham and Mary).  A
dropped gamma, r or W factor moves entries by whole multiples of the entry itself and
still fails.
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import oracle
import synth_inputs as si
from harness import TOL, dev_bf16

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _run(w):
    inp = si.generate(w)
    h = dev_bf16(inp["h"])
    W = dev_bf16(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    Wp = coda.prepare_weight_bf16(W, gamma)
    r = coda.rowscale_from_h(h, w.eps)
    dy = dev_bf16(inp["dy"])
    dz, _ = coda.gemm_swiglu_bwd(h, Wp, r, dy)
    dW, dgam = coda.mlpin_wgrad(dz, h, gamma, W)
    torch.cuda.synchronize()
    return inp, dW.cpu().numpy().astype(np.float64), dgam.cpu().numpy().astype(np.float64)


C_HOEFFDING = 8.0
U_BF16 = 2.0 ** -8


def _err(gpu, ref, rss):
    """|gpu - ref| in units of the bound 2e-2 (1 + |ref|) + 8 * 2^-8 * rss (pass: <= 1)."""
    return np.abs(gpu - ref) / (TOL["bf16"] * (1 + np.abs(ref)) + C_HOEFFDING * U_BF16 * rss)


SMALL = [
    # tokens M (the contraction: a multiple of 8, ragged against the 64-token step),
    # hidden d and gate width F (ragged against the 256-wide tiles, several tiles)
    (296, 200, 104),
    (264, 264, 200),
    (520, 128, 256),
    (8, 8, 8),
]


@pytest.mark.parametrize("M,d,F", SMALL)
def test_wgrad_small_all_entries(M, d, F):
    w = si.custom(M, 0, d, 2 * F, si.ACT_SWIGLU_BWD, seed=3 * M + d + F)
    _log(f"wgrad small {w.name}")
    inp, dW, dgam = _run(w)
    Wp_ref = oracle.fold_bf16(inp["W_t"], inp["gamma"])
    ref_dW, ref_dg, rss, rss_g = oracle.mlpin_wgrad(inp["h"], inp["gamma"], Wp_ref, oracle.BF16, 1.0,
                                                    inp["W_t"], inp["dy"], w.eps, rss=True)
    g = np.abs(inp["gamma"].astype(np.float64))[None, :]
    e_w, e_g = _err(dW, ref_dW, g * rss), _err(dgam, ref_dg, rss_g)
    rel = np.linalg.norm(dW - ref_dW) / np.linalg.norm(ref_dW)
    _log(f"  dW err/bound max {e_w.max():.2e} (rel fro {rel:.2e}), dgamma err/bound max {e_g.max():.2e}")
    assert np.all(np.isfinite(dW)) and np.all(np.isfinite(dgam))
    assert e_w.max() <= 1 and e_g.max() <= 1
    assert rel <= 1e-2


def test_wgrad_workload_sampled():
    w = si.WORKLOADS[8]
    _log(f"wgrad workload {w.name}")
    inp, dW, dgam = _run(w)
    F2, d = inp["W_t"].shape
    rng = np.random.default_rng(81)
    js = np.array(sorted({0, 255, 256, F2 // 2 - 1, F2 // 2, F2 - 1} |
                         set(rng.choice(F2, 10, replace=False).tolist())))
    ks = np.array(sorted({0, 7, 255, 256, d - 1} | set(rng.choice(d, 11, replace=False).tolist())))
    Wp_ref = oracle.fold_bf16(inp["W_t"], inp["gamma"])
    ref, none, rss, _ = oracle.mlpin_wgrad(inp["h"], inp["gamma"], Wp_ref, oracle.BF16, 1.0, inp["W_t"],
                                           inp["dy"], w.eps, js=js, ks=ks, rss=True)
    assert none is None
    e = _err(dW[np.ix_(js, ks)], ref, np.abs(inp["gamma"][ks].astype(np.float64))[None, :] * rss)
    rel = np.linalg.norm(dW[np.ix_(js, ks)] - ref) / np.linalg.norm(ref)
    _log(f"  dW sampled err/bound max {e.max():.2e} (rel fro {rel:.2e})")
    assert e.max() <= 1 and rel <= 1e-2
    # dgamma[k] = sum_j W[j,k] G[j,k] with G = dW / gamma: the partial reduction, the
    # column sum and the fold agree with the GPU's own dW (fp64 on the host).  Each
    # per-tile fp32 partial is a chain of at most 8 * 4 + 2 + 1 additions (a lane's rows,
    # the 4 lanes sharing its columns, the 2 waves), so |err| <= 64 * 2^-24 * sum |W G|.
    Wr = oracle.bf16_decode(inp["W_t"])
    terms = Wr * (dW / inp["gamma"].astype(np.float64)[None, :])
    own, scale = terms.sum(0), np.abs(terms).sum(0)
    e_g = np.abs(dgam - own) / (1e-30 + scale)
    _log(f"  dgamma vs own dW: err / sum|W G| max {e_g.max():.2e}")
    assert np.all(np.isfinite(dgam)) and e_g.max() <= 64 * 2.0 ** -24


def test_plain_token_gemm_matches_its_definition():
    # gamma = NULL and W = NULL: dW = At . Bt^T over the tokens (a linear layer's weight
    # gradient), checked against the fp64 sum of the same bf16 operands
    rng = np.random.default_rng(17)
    NR, NC, K = 300, 136, 712
    a = si.to_bf16_bits(rng.standard_normal((NR, K)).astype(np.float32))
    b = si.to_bf16_bits(rng.standard_normal((NC, K)).astype(np.float32))
    dW, P = coda.gemm_wgrad(dev_bf16(a), dev_bf16(b))
    torch.cuda.synchronize()
    assert P is None
    ref = oracle.bf16_decode(a) @ oracle.bf16_decode(b).T
    # fp32 accumulation over K = 712 products of unit normals: |err| <~ K * 2^-24 * sum|ab|
    bound = K * 2.0 ** -24 * (np.abs(oracle.bf16_decode(a)) @ np.abs(oracle.bf16_decode(b)).T)
    err = np.abs(dW.cpu().numpy().astype(np.float64) - ref)
    _log(f"  plain token GEMM err max {err.max():.2e}, bound min {bound.min():.2e}")
    assert np.all(err <= bound)


def test_gamma_scales_columns_and_partials_sum_to_dgamma():
    rng = np.random.default_rng(18)
    NR, NC, K = 520, 72, 256
    a = dev_bf16(si.to_bf16_bits(rng.standard_normal((NR, K)).astype(np.float32)))
    b = dev_bf16(si.to_bf16_bits(rng.standard_normal((NC, K)).astype(np.float32)))
    W = dev_bf16(si.to_bf16_bits(rng.standard_normal((NR, NC)).astype(np.float32)))
    g = torch.from_numpy(np.exp2(rng.integers(-3, 4, NC)).astype(np.float32)).cuda()
    G, _ = coda.gemm_wgrad(a, b)
    dW, P = coda.gemm_wgrad(a, b, g, W)
    dg = coda.colsum_reduce(P)
    torch.cuda.synchronize()
    assert P.shape == (coda.wgrad_partials_rows(NR), NC) == (3, NC)
    # powers of two: the column scale is exact
    assert torch.equal(dW, G * g[None, :])
    ref = (W.double() * G.double()).sum(0)
    scale = (W.double() * G.double()).abs().sum(0)
    assert torch.all((dg.double() - ref).abs() <= 64 * 2.0 ** -24 * scale)


def test_empty_token_batch_writes_zeros():
    NR, NC = 96, 64
    a = torch.empty((NR, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((NC, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((NR, NC), dtype=torch.bfloat16, device="cuda")
    dW = torch.full((NR, NC), 7.0, device="cuda")
    P = torch.full((1, NC), 7.0, device="cuda")
    coda.gemm_wgrad(a, b, None, W, dW=dW, partials=P)
    dg = coda.colsum_reduce(P)
    torch.cuda.synchronize()
    assert torch.all(dW == 0) and torch.all(P == 0) and torch.all(dg == 0)


def test_wgrad_deterministic_bitwise():
    w = si.custom(264, 0, 200, 208, si.ACT_SWIGLU_BWD, seed=31)
    _, dW1, dg1 = _run(w)
    _, dW2, dg2 = _run(w)
    assert np.array_equal(dW1, dW2) and np.array_equal(dg1, dg2)


def test_token_split_matches_the_definition_and_is_reproducible():
    # 3 output tiles over 8200 tokens: the workspace lets 4 blocks share each tile (the
    # last split ragged), their sums added in a fixed order, then gamma
    rng = np.random.default_rng(20)
    NR, NC, K = 520, 136, 8200
    assert coda.wgrad_workspace_bytes(NR, NC, K) == 4 * (NR + 3) * NC * 4    # dW slices + 3 row tiles' partials
    a = si.to_bf16_bits(rng.standard_normal((NR, K)).astype(np.float32))
    b = si.to_bf16_bits(rng.standard_normal((NC, K)).astype(np.float32))
    g = np.exp2(rng.integers(-3, 4, NC)).astype(np.float32)
    ad, bd = dev_bf16(a), dev_bf16(b)
    gd = torch.from_numpy(g).cuda()
    ws = torch.empty(coda.wgrad_workspace_bytes(NR, NC, K), dtype=torch.uint8, device="cuda")
    s1, _ = coda.gemm_wgrad(ad, bd, gd, workspace=ws)
    s2, _ = coda.gemm_wgrad(ad, bd, gd, workspace=ws)
    one, _ = coda.gemm_wgrad(ad, bd, gd)                       # no workspace: one block per tile
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    A, B = oracle.bf16_decode(a), oracle.bf16_decode(b)
    ref = (A @ B.T) * g.astype(np.float64)[None, :]
    bound = K * 2.0 ** -24 * (np.abs(A) @ np.abs(B).T) * g.astype(np.float64)[None, :]
    for got in (s1, one):
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
        _log(f"  token split err max {err.max():.2e}, bound min {bound.min():.2e}")
        assert np.all(err <= bound)


@pytest.mark.parametrize("tok", [False, True], ids=["transposed", "token_major"])
def test_token_split_with_gamma_partials(tok):
    # few output tiles and a raw weight: each split writes its dW slice and the partial
    # rows sum_j W[j,k] G_s[j,k] of its tokens; both are added in a fixed order.  Against
    # the fp64 definitions (fp32 sums: |err| <= (K + 256) 2^-24 sum |terms|), reproducible
    rng = np.random.default_rng(21)
    NR, NC, K = 520, 136, 8200
    a = si.to_bf16_bits(rng.standard_normal((K, NR)).astype(np.float32))      # token-major
    b = si.to_bf16_bits(rng.standard_normal((K, NC)).astype(np.float32))
    w = si.to_bf16_bits(rng.standard_normal((NR, NC)).astype(np.float32))
    g = np.exp2(rng.integers(-3, 4, NC)).astype(np.float32)
    ad, bd, wd = dev_bf16(a), dev_bf16(b), dev_bf16(w)
    gd = torch.from_numpy(g).cuda()
    if tok:
        run = lambda ws: coda.gemm_wgrad_tok(ad, bd, gd, wd, workspace=ws)  # noqa: E731
    else:
        at, bt = ad.t().contiguous(), bd.t().contiguous()
        run = lambda ws: coda.gemm_wgrad(at, bt, gd, wd, workspace=ws)  # noqa: E731
    ws = torch.empty(coda.wgrad_workspace_bytes(NR, NC, K), dtype=torch.uint8, device="cuda")
    d1, p1 = run(ws)
    d2, p2 = run(ws)
    d0, p0 = run(None)                                              # one block per tile
    torch.cuda.synchronize()
    assert torch.equal(d1, d2) and torch.equal(p1, p2)
    A, B, W = oracle.bf16_decode(a), oracle.bf16_decode(b), oracle.bf16_decode(w)
    G, Ga = A.T @ B, np.abs(A).T @ np.abs(B)
    u = (K + 256) * 2.0 ** -24
    gg = g.astype(np.float64)[None, :]
    for dW, P in ((d1, p1), (d0, p0)):
        err = np.abs(dW.cpu().numpy().astype(np.float64) - G * gg)
        assert np.all(err <= u * Ga * gg)
        Pn = P.cpu().numpy().astype(np.float64)
        assert Pn.shape == (3, NC)
        for t in range(3):
            rows = slice(256 * t, min(256 * (t + 1), NR))
            ref = (W[rows] * G[rows]).sum(axis=0)
            bound = u * (np.abs(W[rows]) * Ga[rows]).sum(axis=0)
            _log(f"  partials tile {t}: err max {np.abs(Pn[t] - ref).max():.2e}, bound min {bound.min():.2e}")
            assert np.all(np.abs(Pn[t] - ref) <= bound)


@pytest.mark.parametrize("K,NR,NC,lda,ldb", [(712, 300, 136, 304, 136), (520, 264, 72, 264, 80), (8200, 520, 136, 520, 136),
                                             (64, 8, 8, 8, 8)])
def test_token_major_operands_match_the_transposed_path(K, NR, NC, lda, ldb):
    # the same MFMA k order: bit-identical to the GEMM on the transposed copies, with and
    # without the raw weight's partials and the token split
    print(f"wgrad tok K={K} NR={NR} NC={NC} lda={lda} ldb={ldb}", flush=True)
    rng = np.random.default_rng(K + NR + NC)
    X = dev_bf16(si.to_bf16_bits(rng.standard_normal((K, lda)).astype(np.float32)))
    Y = dev_bf16(si.to_bf16_bits(rng.standard_normal((K, ldb)).astype(np.float32)))
    W = dev_bf16(si.to_bf16_bits(rng.standard_normal((NR, NC)).astype(np.float32)))
    g = torch.from_numpy((1 + 0.1 * rng.standard_normal(NC)).astype(np.float32)).cuda()
    Xt = X[:, :NR].t().contiguous()
    Yt = Y[:, :NC].t().contiguous()
    t_dW, t_P = coda.gemm_wgrad_tok(X, Y, g, W, NR=NR, NC=NC)
    r_dW, r_P = coda.gemm_wgrad(Xt, Yt, g, W)
    t_s, _ = coda.gemm_wgrad_tok(X, Y, g, None, NR=NR, NC=NC, workspace="auto")
    r_s, _ = coda.gemm_wgrad(Xt, Yt, g, None, workspace="auto")
    torch.cuda.synchronize()
    assert torch.equal(t_dW, r_dW) and torch.equal(t_P, r_P) and torch.equal(t_s, r_s)


@pytest.mark.parametrize("K", [1, 13, 77, 200, 8221])
def test_token_major_any_token_count(K):
    # no granule on the tokens: against the fp64 definition, |err| <= (K + 2) 2^-24 sum|terms|
    # (8221 tokens in one block: the stage-ring mainloop with a ragged last k-tile)
    rng = np.random.default_rng(50 + K)
    NR, NC = 136, 72
    xb = si.to_bf16_bits(rng.standard_normal((K, NR)).astype(np.float32))
    yb = si.to_bf16_bits(rng.standard_normal((K, NC)).astype(np.float32))
    dW, _ = coda.gemm_wgrad_tok(dev_bf16(xb), dev_bf16(yb))
    torch.cuda.synchronize()
    Xd, Yd = oracle.bf16_decode(xb), oracle.bf16_decode(yb)
    ref = Xd.T @ Yd
    bound = (K + 2) * 2.0 ** -24 * (np.abs(Xd).T @ np.abs(Yd))
    assert np.all(np.abs(dW.cpu().numpy().astype(np.float64) - ref) <= bound)
