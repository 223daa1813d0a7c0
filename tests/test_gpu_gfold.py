"""The second GEMM with the RMSNorm weight folded in on chip (raw bf16 weight + gamma):
bit-identical to the same GEMM on the separately prepared W' = bf16(gamma * W), for the
SwiGLU and plain epilogues, on ragged shapes (rows, columns and K not multiples of the
tiles; gamma of mixed signs and magnitudes) and on the LLaMA-3-1B MLP-in shape.  The
on-chip fold uses the preparation's arithmetic and the same MFMA order, so any
difference is a mistake (a gamma of the wrong k, a stale per-tile gamma, a rounding
that differs).
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import synth_inputs as si
from harness import dev_bf16

pytestmark = pytest.mark.gpu


def _case(M, K, n_w, seed):
    rng = np.random.default_rng(seed)
    h = dev_bf16(si.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    W = dev_bf16(si.to_bf16_bits((rng.standard_normal((n_w, K)) / np.sqrt(K)).astype(np.float32)))
    g = rng.standard_normal(K).astype(np.float32) * np.exp2(rng.integers(-4, 5, K)).astype(np.float32)
    gamma = torch.from_numpy(g).cuda()
    r = torch.from_numpy((0.5 + rng.random(M)).astype(np.float32)).cuda()
    return h, W, gamma, r


@pytest.mark.parametrize("act", [coda.SWIGLU, coda.NONE], ids=["swiglu", "none"])
@pytest.mark.parametrize("M,K,n_w", [(300, 200, 208), (257, 264, 528), (64, 8, 16), (513, 1032, 272)])
def test_on_chip_fold_is_bit_identical(M, K, n_w, act):
    print(f"gfold M={M} K={K} n_w={n_w} act={act}", flush=True)
    h, W, gamma, r = _case(M, K, n_w, M + K + n_w)
    Wp = coda.prepare_weight_bf16(W, gamma)
    ref = coda.gemm_rowscale_swiglu(h, Wp, r, act)
    got = coda.gemm_rowscale_gfold(h, W, gamma, r, act)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_on_chip_fold_workload_shape():
    w = si.WORKLOADS[2]
    print(f"gfold {w.name}", flush=True)
    h, W, gamma, r = _case(w.M, w.d, w.N2w, 2)
    Wp = coda.prepare_weight_bf16(W, gamma)
    ref = coda.gemm_rowscale_swiglu(h, Wp, r)
    got = coda.gemm_rowscale_gfold(h, W, gamma, r)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
