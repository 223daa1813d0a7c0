"""The allocation-free weight-gradient entry point (coda_gemm_wgrad_tok_noalloc), called
through the C ABI: bit-identical to coda_gemm_wgrad_tok with a caller workspace, on two
calls in a row (the second smaller, so it runs on what the first left in the library's
scratch), with and without the gamma-gradient partials; and its size check rejects a
split the scratch cannot hold before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import synth_inputs as si
from gemm_epilogue_transformer_amd import _lib
from harness import dev_bf16

SCRATCH = 128 << 20          # CODA_NOALLOC_SCRATCH_BYTES


def _operands(K, NR, NC, seed):
    rng = np.random.default_rng(seed)
    X = dev_bf16(si.to_bf16_bits(rng.standard_normal((K, NR)).astype(np.float32)))
    Y = dev_bf16(si.to_bf16_bits(rng.standard_normal((K, NC)).astype(np.float32)))
    W = dev_bf16(si.to_bf16_bits(rng.standard_normal((NR, NC)).astype(np.float32)))
    g = torch.from_numpy((1 + 0.1 * rng.standard_normal(NC)).astype(np.float32)).cuda()
    return X, Y, W, g


@pytest.mark.gpu
@pytest.mark.parametrize("with_w", [True, False], ids=["with_partials", "plain"])
def test_noalloc_matches_workspace_entry_point_twice(with_w):
    # (tokens, NR, NC): both take a token split (4, then 2 ranges), the second smaller
    shapes = [(8200, 520, 136), (4200, 264, 72)]
    for i, (K, NR, NC) in enumerate(shapes):
        ws_bytes = coda.wgrad_workspace_bytes(NR, NC, K)
        assert 0 < ws_bytes <= SCRATCH, "the case must take a split that fits the scratch"
        print(f"noalloc call {i}: K={K} NR={NR} NC={NC} split workspace {ws_bytes} B", flush=True)
        X, Y, W, g = _operands(K, NR, NC, seed=40 + i)
        Wr = W if with_w else None
        ref_dW, ref_P = coda.gemm_wgrad_tok(X, Y, g, Wr, workspace="auto")
        dW = torch.full((NR, NC), float("nan"), device="cuda")
        P = torch.full((coda.wgrad_partials_rows(NR), NC), float("nan"), device="cuda") if with_w else None
        L = _lib.load()
        st = L.coda_gemm_wgrad_tok_noalloc(NR, NC, K, X.data_ptr(), NR, Y.data_ptr(), NC, g.data_ptr(),
                                           Wr.data_ptr() if with_w else None, dW.data_ptr(),
                                           P.data_ptr() if with_w else None,
                                           torch.cuda.current_stream().cuda_stream)
        assert st == 0, L.coda_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(dW, ref_dW), f"call {i}: dW differs"
        if with_w:
            assert torch.equal(P, ref_P), f"call {i}: partials differ"
        # the binding's call of the same entry point
        dW2, P2 = coda.gemm_wgrad_tok_noalloc(X, Y, g, Wr)
        torch.cuda.synchronize()
        assert torch.equal(dW2, ref_dW)
        if with_w:
            assert torch.equal(P2, ref_P)


def _too_big():
    """Sizes whose planned split needs more than the scratch holds."""
    for n in range(1024, 8192 + 1, 256):
        for K in (1 << 15, 1 << 16, 1 << 17):
            if coda.wgrad_workspace_bytes(n, n, K) > SCRATCH:
                return n, n, K
    raise AssertionError("no size found whose split exceeds the scratch")


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer validation runs on GPU-less hosts only")
def test_noalloc_rejects_a_split_larger_than_the_scratch():
    # validation only: fake (aligned) addresses, rejected before anything is enqueued
    NR, NC, K = _too_big()
    L = _lib.load()
    st = L.coda_gemm_wgrad_tok_noalloc(NR, NC, K, 0x10000000, NR, 0x20000000, NC, None, None,
                                       0x30000000, None, None)
    assert st == 2                    # CODA_ERR_SHAPE
    assert coda.wgrad_workspace_bytes(NR, NC, K) > SCRATCH
