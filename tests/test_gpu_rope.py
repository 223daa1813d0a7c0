"""GPU parity of the RoPE epilogue of the second GEMM (the QKV product of workload 3)
against the oracle: the act-NONE chain followed by the oracle's RoPE, on every row of
small ragged shapes and on sampled rows of the full workload, plus the properties that
pin the rotation itself (no rotation = the plain path, position 0 = identity, positions
outside the table read zero angles' cos and sin).
"""

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import oracle
import synth_inputs as si
from harness import check_chain, gpu_prepare, host_bits, sample_rows, upload

pytestmark = pytest.mark.gpu

BASE = 500000.0


def _log(msg):
    print(msg, flush=True)


def _gpu_rope_chain(w, d, prep, pos, cos, sin):
    h, P = coda.gemm_resid_partialrms(prep["A"], prep["Wo"], d["x_res"], prep["a_scale"], prep["wo_scale"])
    r = coda.rowscale_reduce(P, prep["Wo"].shape[0], w.eps)
    y = coda.gemm_rowscale_rope(h, prep["Wp"], r, pos, cos, sin, w.rot_cols, prep["wp_scale"])
    return h, P, r, y


def _oracle_rope_chain(w, inp, prep_ref, rows=None):
    ref = oracle.chain(prep_ref, inp["x_res"], inp["gamma"], si.ACT_NONE, w.eps, rows=rows)
    pos = inp["pos"] if rows is None else inp["pos"][rows]
    ref["y"] = oracle.rope(ref["y"], pos, w.rope_base, w.head_dim, w.rot_cols)
    return ref


def test_rope_table_within_an_ulp_of_the_fp64_angles():
    rows = 8192
    cos, sin = coda.rope_table(rows, BASE)
    torch.cuda.synchronize()
    p = np.arange(rows, dtype=np.float64)[:, None]
    theta = np.power(BASE, -2.0 * np.arange(32) / 64.0)[None, :]
    ang = p * theta
    for got, ref in ((cos.cpu().numpy(), np.cos(ang)), (sin.cpu().numpy(), np.sin(ang))):
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp), "table off by more than an fp32 ulp"
    c, s = cos.cpu().numpy(), sin.cpu().numpy()
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)


SMALL = [
    # M, K1, d, N2w, rot_cols, seq_len, dtype: ragged M and d, V columns in a partial tile
    (300, 136, 200, 384, 256, 64, "bf16"),
    (257, 72, 264, 392, 320, 100, "bf16"),      # 392 = 6 heads + 8 V columns
    (130, 64, 144, 512, 512, 7, "bf16"),        # every column rotated
    (64, 48, 128, 256, 0, 16, "bf16"),          # nothing rotated
    (130, 64, 144, 320, 192, 33, "e4m3"),
]


@pytest.mark.parametrize("M,K1,d,N2w,rot,seq,dtype", SMALL)
def test_rope_chain_small_all_rows(M, K1, d, N2w, rot, seq, dtype):
    w = si.custom(M, K1, d, N2w, si.ACT_ROPE, seed=M + N2w, dtype=dtype, rot_cols=rot, seq_len=seq)
    _log(f"rope small {w.name} rot={rot} seq={seq} {dtype}")
    inp = si.generate(w)
    d_ = upload(inp)
    prep = gpu_prepare(w, d_)
    cos, sin = coda.rope_table(seq, w.rope_base)
    pos = torch.from_numpy(inp["pos"]).cuda()
    h, P, r, y = _gpu_rope_chain(w, d_, prep, pos, cos, sin)
    torch.cuda.synchronize()
    prep_ref = oracle.prepare(inp, dtype)
    st = check_chain(w, inp, h, P, r, y, ref=_oracle_rope_chain(w, inp, prep_ref), prep_ref=prep_ref)
    _log(f"  errors {st}")


def test_rope_workload_sampled_rows():
    w = si.WORKLOADS[6]
    _log(f"rope workload {w.name}")
    inp = si.generate(w)
    d_ = upload(inp)
    prep = gpu_prepare(w, d_)
    cos, sin = coda.rope_table(w.seq_len, w.rope_base)
    pos = torch.from_numpy(inp["pos"]).cuda()
    h, P, r, y = _gpu_rope_chain(w, d_, prep, pos, cos, sin)
    torch.cuda.synchronize()
    rows = sample_rows(w.M, 48, seed=6)
    prep_ref = oracle.prepare(inp, w.dtype)
    st = check_chain(w, inp, h, P, r, y, rows=rows, ref=_oracle_rope_chain(w, inp, prep_ref, rows),
                     prep_ref=prep_ref)
    _log(f"  errors {st}")
    assert torch.isfinite(y.float()).all()


def _small_case(seed=11):
    w = si.custom(200, 64, 128, 384, si.ACT_ROPE, seed=seed, rot_cols=256, seq_len=50)
    inp = si.generate(w)
    d_ = upload(inp)
    prep = gpu_prepare(w, d_)
    h, P = coda.gemm_resid_partialrms(prep["A"], prep["Wo"], d_["x_res"])
    r = coda.rowscale_reduce(P, 128, w.eps)
    plain = coda.gemm_rowscale_swiglu(h, prep["Wp"], r, coda.NONE)
    return w, inp, prep, h, r, plain


def test_no_rotation_and_position_zero_equal_the_plain_path():
    w, inp, prep, h, r, plain = _small_case()
    cos, sin = coda.rope_table(w.seq_len, w.rope_base)
    y0 = coda.gemm_rowscale_rope(h, prep["Wp"], r, None, None, None, 0)
    zeros = torch.zeros(w.M, dtype=torch.int32, device="cuda")
    yz = coda.gemm_rowscale_rope(h, prep["Wp"], r, zeros, cos, sin, w.rot_cols)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y0), host_bits(plain))
    assert np.array_equal(host_bits(yz), host_bits(plain))     # cos 1, sin 0: x*1 - x'*0 = x


def test_positions_outside_the_table_read_zero_angles():
    w, inp, prep, h, r, plain = _small_case(seed=12)
    cos, sin = coda.rope_table(w.seq_len, w.rope_base)
    pos_np = inp["pos"].copy()
    bad = np.array([0, 5, 77, 199])
    pos_np[bad[:2]] = w.seq_len             # one past the table
    pos_np[bad[2:]] = -3                    # negative
    y = coda.gemm_rowscale_rope(h, prep["Wp"], r, torch.from_numpy(pos_np).cuda(), cos, sin, w.rot_cols)
    torch.cuda.synchronize()
    yv = oracle.bf16_decode(host_bits(y))
    pv = oracle.bf16_decode(host_bits(plain))
    assert np.all(yv[bad, : w.rot_cols] == 0.0)
    assert np.array_equal(yv[bad, w.rot_cols:], pv[bad, w.rot_cols:])
    good = np.setdiff1d(np.arange(w.M), bad)
    assert not np.all(yv[good, : w.rot_cols] == 0.0)
