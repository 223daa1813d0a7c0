"""GPU parity of the QKV block's backward, y = RoPE(RMSNorm(h) . W^T): the RoPE backward
(r * RoPE^T(dy) and the row-scale partials from the saved output), then the row
coefficient, the input-gradient GEMM and the weight / gamma gradients on dz and h as
stored, against the oracle's unfused chain rule (fp64 angles) on ragged shapes (every
entry), at the LLaMA-3-1B QKV shape on sampled entries, and in the special cases that
have exact answers (no rotation; positions outside the table).

Bounds as for the other backward tests: dz and dh 2e-2 * (1 + |ref|); the token sums dW
and dgamma 2e-2 * (1 + |ref|) plus 8 * 2^-8 times the root-sum-square of their terms
(each term carries the bf16 rounding of dz, independent between tokens: Hoeffding),
with the Frobenius-relative error below 1e-2.
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


def _forward(w, inp):
    h, W = dev_bf16(inp["h"]), dev_bf16(inp["W_t"])
    gamma = torch.from_numpy(inp["gamma"]).cuda()
    pos = torch.from_numpy(inp["pos"]).cuda()
    Wp = coda.prepare_weight_bf16(W, gamma)
    r = coda.rowscale_from_h(h, w.eps)
    cos, sin = coda.rope_table(w.seq_len, w.rope_base)
    y = coda.gemm_rowscale_rope(h, Wp, r, pos, cos, sin, w.rot_cols)
    return dict(h=h, W=W, gamma=gamma, pos=pos, Wp=Wp, Wpt=coda.transpose_bf16(Wp), r=r, cos=cos, sin=sin, y=y,
                dy=dev_bf16(inp["dy"]))


def _backward(w, f):
    g = coda.qkv_rope_bwd(f["h"], f["r"], f["Wpt"], f["W"], f["gamma"], f["dy"], f["y"], f["pos"], f["cos"],
                          f["sin"], w.rot_cols)
    torch.cuda.synchronize()
    return g


def _np(t):
    return t.cpu().numpy().astype(np.float64)


def _bounded(name, gpu, ref, rss):
    e = np.abs(gpu - ref) / (TOL["bf16"] * (1 + np.abs(ref)) + C * U * rss)
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)
    _log(f"  {name}: err/bound max {e.max():.2e}, rel fro {rel:.2e}")
    assert np.all(np.isfinite(gpu)) and e.max() <= 1 and rel <= 1e-2


def _near(name, gpu, ref):
    e = np.abs(gpu - ref) / (1 + np.abs(ref))
    _log(f"  {name}: err max {e.max():.2e}")
    assert np.all(np.isfinite(gpu)) and e.max() <= TOL["bf16"]


def _oracle(w, inp, **kw):
    return oracle.qkv_rope_bwd(inp["h"], inp["gamma"], oracle.fold_bf16(inp["W_t"], inp["gamma"]), 1.0, inp["W_t"],
                               inp["dy"], inp["pos"], w.rope_base, w.head_dim, w.rot_cols, w.eps, rss=True, **kw)


SMALL = [
    # M tokens, d, N columns, rotated columns, sequence length: ragged against the 64-row
    # and 128-column tiles of the RoPE backward and the GEMM tiles
    (296, 200, 320, 256, 37),
    (264, 136, 192, 192, 5),      # every column rotated
    (130, 64, 136, 64, 300),      # a last tile of 8 columns, one rotated head
    (8, 8, 64, 0, 1),             # no rotation
]


@pytest.mark.parametrize("M,d,N,rot,seq", SMALL)
def test_rope_bwd_small_all_entries(M, d, N, rot, seq):
    w = si.custom(M, 0, d, N, si.ACT_ROPE_BWD, seed=7 * M + d + N, rot_cols=rot, seq_len=seq)
    _log(f"rope bwd small {w.name} rot={rot} seq={seq}")
    inp = si.generate(w)
    f = _forward(w, inp)
    g = _backward(w, f)
    o = _oracle(w, inp)
    dz = oracle.bf16_decode(host_bits(g["dz"]))
    _near("dz", dz, o["r"][:, None] * o["dz"])
    _near("dh", oracle.bf16_decode(host_bits(g["dh"])), o["dh"])
    _bounded("dW", _np(g["dW"]), o["dW"], np.abs(inp["gamma"].astype(np.float64))[None, :] * o["rss"])
    _bounded("dgamma", _np(g["dgamma"]), o["dgamma"], o["rss_gamma"])


def test_rope_bwd_workload_sampled():
    w = si.WORKLOADS[10]
    _log(f"rope bwd workload {w.name}")
    inp = si.generate(w)
    f = _forward(w, inp)
    g = _backward(w, f)
    rng = np.random.default_rng(11)
    rows = np.array(sorted({0, 1, 63, 64, w.M // 2, w.M - 1} | set(rng.choice(w.M, 10, replace=False).tolist())))
    js = np.array(sorted({0, 31, 32, w.rot_cols - 1, w.rot_cols, w.N2w - 1} |
                         set(rng.choice(w.N2w, 6, replace=False).tolist())))
    ks = rng.choice(w.d, 10, replace=False)
    o = _oracle(w, inp, rows=rows, js=js, ks=ks)
    _near("dz sampled rows", oracle.bf16_decode(host_bits(g["dz"]))[rows], o["r"][:, None] * o["dz"])
    _near("dh sampled rows", oracle.bf16_decode(host_bits(g["dh"]))[rows], o["dh"])
    _bounded("dW sampled", _np(g["dW"])[np.ix_(js, ks)], o["dW"],
             np.abs(inp["gamma"].astype(np.float64))[ks][None, :] * o["rss"])
    # dgamma = sum_j W[j, k] G[j, k] (G = dW / gamma): the GPU's own dW columns give it
    # back up to fp32 rounding of the fixed-order sums
    dW, dgam = _np(g["dW"]), _np(g["dgamma"])
    Wr = oracle.bf16_decode(inp["W_t"])
    gam = inp["gamma"].astype(np.float64)
    ref = (Wr[:, ks] * dW[:, ks]).sum(axis=0) / gam[ks]
    scale = (np.abs(Wr[:, ks] * dW[:, ks])).sum(axis=0) / np.abs(gam[ks])
    err = np.abs(dgam[ks] - ref)
    _log(f"  dgamma vs the GPU's dW: err max {err.max():.2e}, scale min {scale.min():.2e}")
    assert np.all(err <= 1e-4 * scale)


def test_no_rotation_gives_the_scaled_gradient_exactly():
    w = si.custom(200, 0, 64, 192, si.ACT_ROPE_BWD, seed=41, rot_cols=0, seq_len=1)
    inp = si.generate(w)
    f = _forward(w, inp)
    dz, P = coda.rope_bwd(f["dy"], f["y"], f["r"], None, None, None, 0)
    torch.cuda.synchronize()
    ref = (f["dy"].float() * f["r"][:, None]).to(torch.bfloat16)
    assert torch.equal(dz.view(torch.int16), ref.view(torch.int16))
    # the partials: (1/r) sum over each 128-column tile of dy * y
    prod = (f["dy"].float() * f["y"].float()).cpu().numpy().astype(np.float64)
    r = _np(f["r"])
    ref_p = np.stack([prod[:, 0:128].sum(1), prod[:, 128:192].sum(1)], 1) / r[:, None]
    got_p = _np(P)
    assert np.max(np.abs(got_p - ref_p) / (1e-3 + np.abs(ref_p))) < 1e-4


def test_positions_outside_the_table_have_no_rotated_gradient():
    w = si.custom(96, 0, 64, 256, si.ACT_ROPE_BWD, seed=43, rot_cols=128, seq_len=16)
    inp = si.generate(w)
    f = _forward(w, inp)
    pos = f["pos"].clone()
    pos[::3] = 16 + 5            # past the 16-row table: the forward read zero angles there
    pos[1::7] = -1
    dz, _ = coda.rope_bwd(f["dy"], f["y"], f["r"], pos, f["cos"], f["sin"], w.rot_cols)
    torch.cuda.synchronize()
    out = (pos < 0) | (pos >= 16)
    assert torch.all(dz[out][:, :128].float() == 0)
    ref_v = (f["dy"].float() * f["r"][:, None]).to(torch.bfloat16)
    assert torch.equal(dz[:, 128:].contiguous().view(torch.int16), ref_v[:, 128:].contiguous().view(torch.int16))


def test_rope_bwd_deterministic_bitwise():
    w = si.custom(264, 0, 136, 192, si.ACT_ROPE_BWD, seed=47, rot_cols=128, seq_len=9)
    inp = si.generate(w)
    f = _forward(w, inp)
    a, b = _backward(w, f), _backward(w, f)
    for k in ("dz", "dh", "dW", "dgamma", "q"):
        assert torch.equal(a[k].view(torch.int32) if a[k].dtype == torch.float32 else a[k].view(torch.int16),
                           b[k].view(torch.int32) if b[k].dtype == torch.float32 else b[k].view(torch.int16)), k
