"""GPU parity of the MLP-input block's input gradient (recompute + SwiGLU backward, the
row-coefficient reduction, the input-gradient GEMM with the RMSNorm backward) against
the oracle's unfused chain rule, on ragged shapes (all rows) and on sampled rows of the
LLaMA-3-1B shape; plus the building blocks (transpose, row scale of a stored h) and the
properties that pin the wiring (dy = 0 leaves the residual gradient, in-place residual
gradient, bitwise determinism).
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import oracle
import synth_inputs as si
from harness import TOL, dev_bf16, host_bits

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _setup(w):
    inp = si.generate(w)
    h = dev_bf16(inp["h"])
    W = dev_bf16(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    Wp = coda.prepare_weight_bf16(W, gamma)
    Wpt = coda.transpose_bf16(Wp)
    r = coda.rowscale_from_h(h, w.eps)
    dy = dev_bf16(inp["dy"])
    return inp, h, Wp, Wpt, r, dy


def _check(w, inp, dh, dz, r, rows=None, dh_res=None):
    Wp_ref = oracle.fold_bf16(inp["W_t"], inp["gamma"])
    o = oracle.mlpin_bwd(inp["h"], inp["gamma"], Wp_ref, oracle.BF16, 1.0, inp["dy"], w.eps, rows=rows)
    sel = slice(None) if rows is None else rows
    ref_dh = o["dh"] + (0.0 if dh_res is None else oracle.bf16_decode(dh_res)[sel])
    dhg = oracle.bf16_decode(host_bits(dh))[sel]
    dzg = oracle.bf16_decode(host_bits(dz))[sel]
    rg = r.cpu().numpy().astype(np.float64)[sel]
    ref_dz = o["r"][:, None] * o["dz"]
    tol = TOL["bf16"]
    # dh sums 2F products whose dz operand the path rounds to bf16: its error grows with
    # the root-sum-square of the terms (reading 18: 2e-2 (1 + |ref|) + 8 * 2^-8 * rss)
    Wd = oracle.bf16_decode(Wp_ref)
    rss = np.sqrt((ref_dz ** 2) @ (Wd ** 2))
    e_dh = np.abs(dhg - ref_dh) / (tol * (1 + np.abs(ref_dh)) + 8 * 2.0 ** -8 * rss)
    e_dz = np.abs(dzg - ref_dz) / (1 + np.abs(ref_dz))
    rel_dh = np.linalg.norm(dhg - ref_dh) / np.linalg.norm(ref_dh)
    _log(f"  dh err/bound max {e_dh.max():.2e} (rel fro {rel_dh:.2e}), dz err max {e_dz.max():.2e}, "
         f"r rel {np.max(np.abs(rg - o['r']) / o['r']):.2e}")
    assert np.all(np.isfinite(dhg))
    assert e_dh.max() <= 1 and rel_dh <= 1e-2 and e_dz.max() <= tol
    assert np.all(np.abs(rg - o["r"]) <= 2 * np.spacing(np.float32(o["r"])).astype(np.float64))


@pytest.mark.parametrize("R,C", [(333, 130), (328, 136), (8, 8), (136, 328), (1, 5)])
def test_transpose_is_exact(R, C):
    # general shapes and the 16-byte path (both sides multiples of 8, ragged against the
    # 128 x 64 tile)
    x = torch.randint(-30000, 30000, (R, C), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    y = coda.transpose_bf16(x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), x.view(torch.int16).t().contiguous())


SMALL = [
    # M, d, F: ragged rows, hidden and gate widths (several tiles in each)
    (300, 200, 104),
    (257, 264, 200),
    (64, 128, 256),
    (1, 8, 8),
    # a contraction of 2F = 8208 (a ragged k-tile): the input-gradient GEMM on its stage rings
    (130, 136, 4104),
]


@pytest.mark.parametrize("M,d,F", SMALL)
def test_bwd_small_all_rows(M, d, F):
    w = si.custom(M, 0, d, 2 * F, si.ACT_SWIGLU_BWD, seed=M + d + F)
    _log(f"bwd small {w.name}")
    inp, h, Wp, Wpt, r, dy = _setup(w)
    dh, dz, P, q = coda.mlpin_bwd(h, Wp, Wpt, r, dy)
    torch.cuda.synchronize()
    _check(w, inp, dh, dz, r)


def test_bwd_workload_sampled_rows():
    w = si.WORKLOADS[8]
    _log(f"bwd workload {w.name}")
    inp, h, Wp, Wpt, r, dy = _setup(w)
    dh, dz, P, q = coda.mlpin_bwd(h, Wp, Wpt, r, dy)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 255, 256, w.M // 2, w.M - 1} |
                           set(np.random.default_rng(8).choice(w.M, 26, replace=False).tolist())))
    _check(w, inp, dh, dz, r, rows=rows)
    assert torch.isfinite(dh.float()).all()


def test_residual_gradient_is_added_and_may_be_in_place():
    w = si.custom(300, 0, 200, 208, si.ACT_SWIGLU_BWD, seed=21)
    inp, h, Wp, Wpt, r, dy = _setup(w)
    res = np.random.default_rng(3).standard_normal((w.M, w.d)).astype(np.float32)
    res_bits = si.to_bf16_bits(res)
    g = dev_bf16(res_bits)
    dz, P = coda.gemm_swiglu_bwd(h, Wp, r, dy)
    q = coda.rmsnorm_bwd_reduce(P, r, w.d, w.N2w // 2)
    dh = coda.gemm_rmsnorm_bwd(dz, Wpt, h, q, dh_res=g)
    coda.gemm_rmsnorm_bwd(dz, Wpt, h, q, dh_res=g, dh=g)          # in place
    torch.cuda.synchronize()
    assert torch.equal(dh.view(torch.int16), g.view(torch.int16))
    _check(w, inp, dh, dz, r, dh_res=res_bits)


def test_zero_upstream_gradient_leaves_the_residual_gradient():
    w = si.custom(130, 0, 136, 112, si.ACT_SWIGLU_BWD, seed=22)
    inp, h, Wp, Wpt, r, dy = _setup(w)
    res = dev_bf16(si.to_bf16_bits(np.random.default_rng(4).standard_normal((w.M, w.d)).astype(np.float32)))
    dh, dz, P, q = coda.mlpin_bwd(h, Wp, Wpt, r, torch.zeros_like(dy), dh_res=res)
    torch.cuda.synchronize()
    assert torch.all(dz.float() == 0) and torch.all(q == 0)
    assert torch.equal(dh.float(), res.float())


def test_bwd_deterministic_bitwise():
    w = si.custom(300, 0, 200, 208, si.ACT_SWIGLU_BWD, seed=23)
    inp, h, Wp, Wpt, r, dy = _setup(w)
    a = coda.mlpin_bwd(h, Wp, Wpt, r, dy)
    b = coda.mlpin_bwd(h, Wp, Wpt, r, dy)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
