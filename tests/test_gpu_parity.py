"""GPU parity of the HIP chain against the fp64 oracle (through the C ABI).

Every element of h and y is compared with the oracle, on small ragged shapes and on the
full-size 16K-token workloads alike.
"""

import time

import numpy as np
import pytest
import torch

import gemm_epilogue_transformer_amd as coda
import oracle
import synth_inputs as si
from harness import (check_chain, dev_bf16, gpu_chain, gpu_prepare, host_bits,
                     upload)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------- weight preparation ----

@pytest.mark.parametrize("N,K", [(8, 8), (3, 64), (200, 136), (1024, 2048)])
def test_fold_bf16_bit_exact(N, K):
    w = si.custom(4, 16, K, N, si.ACT_NONE, seed=N + K)
    inp = si.generate(w)
    d = upload(inp)
    Wp = coda.prepare_weight_bf16(d["W_t"], d["gamma"])
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Wp), oracle.fold_bf16(inp["W_t"], inp["gamma"]))
    Wc = coda.prepare_weight_bf16(d["W_t"], None)
    assert np.array_equal(host_bits(Wc), inp["W_t"])


@pytest.mark.parametrize("N,K,fold", [(1, 16, False), (37, 48, True), (256, 1024, True),
                                      (16384, 2048, True), (2048, 2048, False)])
def test_quantize_e4m3_bit_exact(N, K, fold):
    w = si.custom(4, 16, K, N, si.ACT_NONE, seed=3 * N + K)
    inp = si.generate(w)
    d = upload(inp)
    q, sc = coda.quantize_e4m3(d["W_t"], d["gamma"] if fold else None)
    torch.cuda.synchronize()
    qo, amax, scale = oracle.quant_e4m3(inp["W_t"], inp["gamma"] if fold else None)
    sc = sc.cpu().numpy()
    assert sc[0] == amax and sc[1] == scale
    assert np.array_equal(q.cpu().numpy(), qo)


def test_quantize_e4m3_every_code_and_tie():
    # amax = 448 makes the scale exactly 1, so every e4m3 value, every midpoint between
    # neighbours and the bf16 values one ulp either side of it reach the GPU encoder
    # unchanged; its codes must equal the oracle's.
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    mids = oracle.bf16_encode((vals[:-1] + vals[1:]) / 2)
    near = np.concatenate([mids[mids > 0] + np.uint16(1), mids[mids > 0] - np.uint16(1)])
    pos = np.concatenate([oracle.bf16_encode(vals), mids, near])
    bits = np.concatenate([pos, pos | np.uint16(0x8000)])
    K = ((bits.size + 15) // 16) * 16
    row = np.zeros(K, np.uint16)
    row[: bits.size] = bits
    X = np.stack([row, row[::-1].copy()])
    q, sc = coda.quantize_e4m3(dev_bf16(X))
    torch.cuda.synchronize()
    qo, amax, scale = oracle.quant_e4m3(X, None)
    assert amax == 448.0 and scale == 1.0
    assert sc.cpu().numpy()[1] == scale
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("act", [coda.NONE, coda.SWIGLU])
def test_weight_only_e4m3_gemm_reproduces_every_code(act):
    # One-hot rows of h pick single weights: with r = sw = 1 the NONE output y[m, n] is the
    # one exact product 1 * decode(W[n, m]), so every finite e4m3 code must come back as
    # its exact bf16 value (the oracle's decoder).  -0 comes back as +0 (the zero products
    # of the other k are +0).  With SwiGLU the up rows are all 0x38 (= 1.0), so y is
    # SiLU(decode(gate)), compared at the bf16 tolerance.
    K = 256
    N = K if act == coda.NONE else 2 * K
    codes = ((np.arange(N)[:, None] + 7 * np.arange(K)[None, :]) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                       # the two NaN codes
    if act == coda.SWIGLU:
        codes[K:] = 0x38                                    # up rows: 1.0
    h = np.zeros((K, K), np.uint16)
    h[np.arange(K), np.arange(K)] = 0x3F80                 # bf16 1.0
    y = coda.gemm_rowscale_swiglu(dev_bf16(h), torch.from_numpy(codes).cuda(),
                                  torch.ones(K, device="cuda"), act,
                                  w_scale=torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    if act == coda.NONE:
        expect = oracle.bf16_encode(oracle.e4m3_decode(codes.T) + 0.0)
        assert np.array_equal(host_bits(y), expect)
    else:
        g = oracle.e4m3_decode(codes[:K].T)
        ref = g / (1.0 + np.exp(-g))
        got = oracle.bf16_decode(host_bits(y))
        assert np.all(np.abs(got - ref) <= 2e-2 * (1.0 + np.abs(ref)))


# ---------------------------------------------------------------------- the chain ----

SMALL = [
    # M, K1, d, N2w, act, dtype: several tiles and ragged tails in every dimension
    (128, 256, 256, 512, si.ACT_NONE, "bf16"),
    (300, 136, 200, 2 * 104, si.ACT_SWIGLU, "bf16"),
    (257, 72, 264, 392, si.ACT_NONE, "bf16"),
    (1, 8, 8, 16, si.ACT_SWIGLU, "bf16"),
    (130, 64, 144, 2 * 72, si.ACT_SWIGLU, "e4m3"),
    (333, 272, 528, 2 * 200, si.ACT_SWIGLU, "e4m3"),
    (64, 48, 128, 136, si.ACT_NONE, "e4m3"),
    # six k-tiles with a ragged last one: every combination of the first GEMM's three A
    # stages and two B stages, and the residual prefetch on a short loop
    (200, 328, 256, 2 * 128, si.ACT_SWIGLU, "bf16"),
    (200, 704, 256, 2 * 128, si.ACT_NONE, "e4m3"),
    # two and five k-tiles (the rings' other phases)
    (130, 256, 144, 2 * 64, si.ACT_SWIGLU, "e4m3"),
    (260, 320, 264, 136, si.ACT_NONE, "bf16"),
]


@pytest.mark.parametrize("M,K1,d,N2w,act,dtype", SMALL)
def test_chain_small_all_rows(M, K1, d, N2w, act, dtype):
    w = si.custom(M, K1, d, N2w, act, seed=M * 7 + d, dtype=dtype)
    _log(f"chain small {w.name} {dtype}")
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    h, P, r, y = gpu_chain(w, dd, prep)
    torch.cuda.synchronize()
    assert P.shape == (M, coda.partials_per_row(d))
    check_chain(w, inp, h, P, r, y)


@pytest.mark.parametrize("d", [128, 192, 328])
def test_many_tiles_per_workgroup_all_rows(d):
    """More output tiles than CUs, not a multiple of them (17 x 31 = 527 tiles of 256 x 128
    outputs): the forward SwiGLU GEMM's persistent workgroups take two or three tiles each,
    the last pass over the CUs filling them partly; every row is checked, so a tile skipped
    or written twice by the tile loop fails.  d = 128 (2 k-tiles) runs the persistent
    kernel, d = 192 (3 k-tiles, the fewest it takes) and d = 328 (6 k-tiles, the last one
    ragged) the one whose epilogues overlap the next tile's first k-tile."""
    w = si.custom(4196, 72, d, 2 * 3880, si.ACT_SWIGLU, seed=4196 + d)
    _log(f"chain many tiles {w.name}")
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    h, P, r, y = gpu_chain(w, dd, prep)
    torch.cuda.synchronize()
    stats = check_chain(w, inp, h, P, r, y)
    _log(f"  {stats}")


def test_tiny_workload_all_rows():
    w = si.WORKLOADS[1]
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    h, P, r, y = gpu_chain(w, dd, prep)
    torch.cuda.synchronize()
    stats = check_chain(w, inp, h, P, r, y)
    _log(f"tiny workload: {stats}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_workload_all_rows(cfg):
    """The full-size workloads, every element of h and y against the oracle (which runs
    every row: about 10^12 fp64 multiply-adds on workload 4), in the launch
    configuration the bench times."""
    w = si.WORKLOADS[cfg]
    _log(f"full workload {cfg} {w.name}: generating")
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    h, P, r, y = gpu_chain(w, dd, prep)
    torch.cuda.synchronize()
    _log(f"full workload {cfg}: gpu done; oracle on all {w.M} rows ({oracle.max_threads()} threads)")
    t0 = time.perf_counter()
    stats = check_chain(w, inp, h, P, r, y)
    _log(f"full workload {cfg}: {stats} ({time.perf_counter() - t0:.1f} s)")
    assert torch.isfinite(y.float()).all()


# ------------------------------------------------------------- metamorphic / edges ----

def _small(act=si.ACT_SWIGLU, dtype="bf16", M=200, seed=1):
    return si.custom(M, 96, 136, 2 * 88 if act == si.ACT_SWIGLU else 176, act, seed=seed, dtype=dtype)


def test_deterministic_bitwise():
    w = _small()
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    o1 = [t.clone() for t in gpu_chain(w, dd, prep)]
    o2 = gpu_chain(w, dd, prep)
    torch.cuda.synchronize()
    for a, b in zip(o1, o2):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_zero_first_weight_gives_residual_exactly():
    w = _small()
    inp = si.generate(w)
    inp["Wo_t"][:] = 0
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    h, P, r, y = gpu_chain(w, dd, prep)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(h), inp["x_res"])
    check_chain(w, inp, h, P, r, y)


def test_zero_gate_gives_zero_output():
    w = _small()
    inp = si.generate(w)
    inp["W_t"][: w.n_out] = 0
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    h, P, r, y = gpu_chain(w, dd, prep)
    torch.cuda.synchronize()
    assert torch.all(y.float() == 0)


def test_no_residual_and_in_place_residual():
    w = _small(act=si.ACT_NONE)
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    # x_res = NULL: h = A.W^T
    h, P, r, y = gpu_chain(w, dd, prep, x_res=None)
    torch.cuda.synchronize()
    inp0 = dict(inp, x_res=np.zeros_like(inp["x_res"]))
    check_chain(w, inp0, h, P, r, y)
    # h written over x_res (the one alias the ABI allows)
    buf = dd["x_res"].clone()
    h2, P2, r2, y2 = gpu_chain(w, dd, prep, x_res=buf, h_out=buf)
    torch.cuda.synchronize()
    assert h2.data_ptr() == buf.data_ptr()
    check_chain(w, inp, h2, P2, r2, y2)


def test_scale_invariance_at_zero_eps():
    # inputs x2 (exact in bf16) and eps = 0: hb doubles exactly, r halves, y is unchanged
    w = si.custom(160, 64, 128, 2 * 64, si.ACT_SWIGLU, seed=5, eps=0.0)
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    h1, P1, r1, y1 = [t.clone() for t in gpu_chain(w, dd, prep)]
    inp2 = dict(inp, A=inp["A"] + np.uint16(0x80), x_res=inp["x_res"] + np.uint16(0x80))
    dd2 = upload(inp2)
    prep2 = gpu_prepare(w, dd2)
    h2, P2, r2, y2 = gpu_chain(w, dd2, prep2)
    torch.cuda.synchronize()
    assert torch.equal(h2.float(), 2 * h1.float())
    assert torch.equal(P2, 4 * P1)
    assert torch.equal(r2, r1 / 2)
    assert torch.equal(y2.view(torch.int16), y1.view(torch.int16))


def test_empty_m_is_a_no_op():
    w = _small(M=1)
    inp = si.generate(w)
    dd = upload(inp)
    prep = gpu_prepare(w, dd)
    A0 = prep["A"][:0]
    h, P = coda.gemm_resid_partialrms(A0, prep["Wo"], dd["x_res"][:0])
    r = coda.rowscale_reduce(P, w.d, w.eps)
    y = coda.gemm_rowscale_swiglu(h, prep["Wp"], r, act=w.act)
    torch.cuda.synchronize()
    assert h.shape[0] == 0 and y.shape[0] == 0


def test_binding_rejects_bad_arguments_on_device():
    w = _small()
    inp = si.generate(w)
    dd = upload(inp)
    # h overlapping x_res without being exactly x_res (the one alias allowed): the
    # library's overlap check, after the binding's shape checks passed
    M, d = w.M, w.d
    buf = torch.empty(M * d + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(coda.CodaError) as e:
        coda.gemm_resid_partialrms(dd["A"], dd["Wo_t"], buf[:M * d].view(M, d), h=buf[8:].view(M, d))
    assert e.value.status == 5
    # a caller's output of the wrong shape never reaches the library
    with pytest.raises(ValueError, match="partials"):
        coda.gemm_resid_partialrms(dd["A"], dd["Wo_t"], dd["x_res"],
                                   partials=torch.empty((M, coda.partials_per_row(d) + 1), device="cuda"))
    with pytest.raises(coda.CodaError) as e:
        coda.rowscale_reduce(torch.zeros((4, coda.partials_per_row(w.d)), device="cuda"), w.d, -1.0)
    assert e.value.status == 4
