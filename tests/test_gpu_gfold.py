"""The second GEMM with the RMSNorm weight folded in on chip (raw bf16 weight + gamma).

Against the fp64 oracle: the chain with this GEMM as its second step matches the
oracle's unfused chain on ragged shapes and on the LLaMA-3-1B MLP-in shape (sampled
rows), for gamma drawn as the workloads draw it and over a wide range of signs and
magnitudes.

Against the library's other path: bit-identical to the same GEMM on the separately
prepared W' = bf16(gamma * W), for the SwiGLU and plain epilogues, on ragged shapes
(rows, columns and K not multiples of the tiles; gamma of mixed signs and magnitudes)
and on the LLaMA-3-1B MLP-in shape.  The on-chip fold uses the preparation's arithmetic
and the same MFMA order, so any difference is a mistake (a gamma of the wrong k, a
stale per-tile gamma, a rounding that differs).
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import synth_inputs as si
from harness import check_chain, dev_bf16, gpu_chain_gfold, sample_rows, upload

pytestmark = pytest.mark.gpu


def _case(M, K, n_w, seed):
    rng = np.random.default_rng(seed)
    h = dev_bf16(si.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    W = dev_bf16(si.to_bf16_bits((rng.standard_normal((n_w, K)) / np.sqrt(K)).astype(np.float32)))
    g = rng.standard_normal(K).astype(np.float32) * np.exp2(rng.integers(-4, 5, K)).astype(np.float32)
    gamma = torch.from_numpy(g).cuda()
    r = torch.from_numpy((0.5 + rng.random(M)).astype(np.float32)).cuda()
    return h, W, gamma, r


# K = 8: the first persistent kernel; the others the overlapped one (K > 128), with one row
# (1 x 136: the fewest k-tiles it takes), tiles per workgroup from one to three, ragged
# edges in every dimension and a K tail inside a k-tile
@pytest.mark.parametrize("act", [coda.SWIGLU, coda.NONE], ids=["swiglu", "none"])
@pytest.mark.parametrize("M,K,n_w", [(300, 200, 208), (257, 264, 528), (64, 8, 16), (513, 1032, 272),
                                     (1, 136, 16), (2049, 192, 1040), (4100, 328, 2000)])
def test_on_chip_fold_is_bit_identical(M, K, n_w, act):
    print(f"gfold M={M} K={K} n_w={n_w} act={act}", flush=True)
    h, W, gamma, r = _case(M, K, n_w, M + K + n_w)
    Wp = coda.prepare_weight_bf16(W, gamma)
    ref = coda.gemm_rowscale_swiglu(h, Wp, r, act)
    got = coda.gemm_rowscale_gfold(h, W, gamma, r, act)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M,K,n_w", [(257, 264, 528), (10241, 264, 2048)])
def test_persistent_ragged_row_tiles_repeat_bit_identical(M, K, n_w):
    """The persistent SwiGLU GEMM on row tiles whose last one holds a single row (so some
    waves' rows all lie past M), once with one tile per workgroup and once with more tiles
    than compute units: ten calls in a row, each bit-identical to the on-chip-fold path
    (a separate kernel with its own mainloop).  A row-scale load skipped by such waves let
    the mainloop's first wait pass before its DMA had landed."""
    print(f"persistent ragged rows M={M} K={K} n_w={n_w}", flush=True)
    h, W, gamma, r = _case(M, K, n_w, M + 3 * K + n_w)
    Wp = coda.prepare_weight_bf16(W, gamma)
    ref = coda.gemm_rowscale_gfold(h, W, gamma, r, coda.SWIGLU)
    for i in range(10):
        got = coda.gemm_rowscale_swiglu(h, Wp, r, coda.SWIGLU)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"call {i}"


def test_on_chip_fold_workload_shape():
    w = si.WORKLOADS[2]
    print(f"gfold {w.name}", flush=True)
    h, W, gamma, r = _case(w.M, w.d, w.N2w, 2)
    Wp = coda.prepare_weight_bf16(W, gamma)
    ref = coda.gemm_rowscale_swiglu(h, Wp, r)
    got = coda.gemm_rowscale_gfold(h, W, gamma, r)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


# ---------------------------------------------------------------- against the oracle ----
# The whole chain with the on-chip fold as its second GEMM, compared element by element
# with the fp64 oracle's unfused chain (its own fold of the raw weight, the weight that
# fold stands for = W' / gamma) at the bf16 tolerance 2e-2 (1 + |ref|).  gamma is drawn as
# the workloads draw it (1 + 0.1 N(0, 1)) or over a wide range (mixed signs, magnitudes
# 2^-4 .. 2^4 times N(0, 1)), where a gamma applied to the wrong k would show at once.

def _wide_gamma(d: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(d) * np.exp2(rng.integers(-4, 5, d))).astype(np.float32)


@pytest.mark.parametrize("gamma_kind", ["workload", "wide"])
@pytest.mark.parametrize("M,K1,d,N2w,act", [(300, 136, 200, 2 * 104, si.ACT_SWIGLU),
                                            (257, 72, 264, 392, si.ACT_NONE),
                                            (513, 64, 1032, 2 * 136, si.ACT_SWIGLU),
                                            (64, 16, 8, 16, si.ACT_NONE)])
def test_on_chip_fold_chain_matches_oracle(M, K1, d, N2w, act, gamma_kind):
    w = si.custom(M, K1, d, N2w, act, seed=M + d + N2w)
    print(f"gfold chain vs oracle {w.name} gamma={gamma_kind}", flush=True)
    inp = si.generate(w)
    if gamma_kind == "wide":
        inp["gamma"] = _wide_gamma(d, M + d)
    dd = upload(inp)
    h, P, r, y = gpu_chain_gfold(w, dd)
    torch.cuda.synchronize()
    stats = check_chain(w, inp, h, P, r, y)
    print(f"  {stats}", flush=True)


@pytest.mark.parametrize("gamma_kind", ["workload", "wide"])
def test_on_chip_fold_workload_shape_matches_oracle(gamma_kind):
    w = si.WORKLOADS[2]
    print(f"gfold chain vs oracle {w.name} gamma={gamma_kind}: generating", flush=True)
    inp = si.generate(w)
    if gamma_kind == "wide":
        inp["gamma"] = _wide_gamma(w.d, 2)
    dd = upload(inp)
    h, P, r, y = gpu_chain_gfold(w, dd)
    torch.cuda.synchronize()
    rows = sample_rows(w.M, 48, seed=7)
    print(f"  gpu done; oracle on {rows.size} sampled rows", flush=True)
    stats = check_chain(w, inp, h, P, r, y, rows=rows)
    print(f"  {stats}", flush=True)
