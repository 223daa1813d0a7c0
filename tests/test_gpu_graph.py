"""The chain's calls under HIP graph capture: the forward chain and the whole-chain
backward (saved pre-activation) captured once on a side stream, replayed several times
with eager work and synchronisations in between, every replay bit-identical to the eager
result.  The library allocates nothing and issues no memset, so every node is one of its
own kernels.
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import synth_inputs as si
from harness import dev_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_forward_chain_graph_replays_match_eager():
    w = si.custom(520, 264, 200, 2 * 104, si.ACT_SWIGLU, seed=41)
    inp = si.generate(w)
    A, Wo, xr, W = dev_bf16(inp["A"]), dev_bf16(inp["Wo_t"]), dev_bf16(inp["x_res"]), dev_bf16(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    Wp = coda.prepare_weight_bf16(W, gamma)
    ref = [t.clone() for t in coda.chain(A, Wo, xr, Wp, w.eps)]
    out = {"h": torch.empty_like(ref[0]), "partials": torch.empty_like(ref[1]), "r": torch.empty_like(ref[2]),
           "y": torch.empty_like(ref[3])}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            coda.chain(A, Wo, xr, Wp, w.eps, out=out)
    torch.cuda.synchronize()
    for i in range(4):
        for t in out.values():
            t.fill_(0)                                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (out["h"], out["partials"], out["r"], out["y"])):
            assert torch.equal(_bits(a), _bits(b)), f"replay {i}"


def test_backward_graph_replays_match_eager():
    w = si.custom(264, 136, 200, 2 * 104, si.ACT_CHAIN_BWD, seed=42)
    inp = si.generate(w)
    A, Wo, xr, W = dev_bf16(inp["A"]), dev_bf16(inp["Wo_t"]), dev_bf16(inp["x_res"]), dev_bf16(inp["W_t"])
    dy, dres = dev_bf16(inp["dy"]), dev_bf16(inp["dres"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    Wp = coda.prepare_weight_bf16(W, gamma)
    Wpt, WoT = coda.transpose_bf16(Wp), coda.transpose_bf16(Wo)
    h, _, r, _, z = coda.chain(A, Wo, xr, Wp, w.eps, save_z=True)
    ref = coda.chain_bwd(A, WoT, h, r, Wp, Wpt, W, gamma, dy, dres, z=z)
    ref = {k: v.clone() for k, v in ref.items()}
    # every intermediate preallocated, so the captured calls allocate nothing
    F, M, d, K1 = w.N2w // 2, w.M, w.d, w.K1
    b16, f32 = dict(dtype=torch.bfloat16, device="cuda"), dict(dtype=torch.float32, device="cuda")
    nws = coda.wgrad_workspace_bytes(d, K1, M)
    out = {"dz": torch.empty((M, 2 * F), **b16), "dzt": torch.empty((2 * F, M), **b16),
           "partials": torch.empty((M, -(-F // 128)), **f32), "q": torch.empty(M, **f32),
           "dh": torch.empty((M, d), **b16), "ht": torch.empty((d, M), **b16),
           "dW": torch.empty((2 * F, d), **f32), "wpartials": torch.empty((coda.wgrad_partials_rows(2 * F), d), **f32),
           "dgamma": torch.empty(d, **f32), "dA": torch.empty((M, K1), **b16), "dht": torch.empty((d, M), **b16),
           "At": torch.empty((K1, M), **b16), "dWo": torch.empty((d, K1), **f32),
           "ws": torch.empty(nws, dtype=torch.uint8, device="cuda") if nws > 0 else None}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            got = coda.chain_bwd(A, WoT, h, r, Wp, Wpt, W, gamma, dy, dres, z=z, out=out)
    torch.cuda.synchronize()
    for i in range(4):
        for k in ("dh", "dA", "dWo", "dW", "dgamma"):
            got[k].fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("dh", "dA", "dWo", "dW", "dgamma"):
            assert torch.equal(_bits(ref[k]), _bits(got[k])), f"replay {i}: {k}"
