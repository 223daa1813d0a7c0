"""Pins for the oracle's number formats and weight preparation (CPU only).

The oracle's bf16 / e4m3 codecs are written from the formats' definitions; here they
are pinned to things other than themselves:
  * torch's dtype casts (library routines) where those are single roundings,
  * exact rational brute force (``fractions.Fraction``) for nearest-value rounding,
  * the format constants printed in the OCP 8-bit floating point specification
    (``tests/golden/e4m3_ocp_points.txt``).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _all_bf16_values():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return codes, oracle.bf16_decode(codes)


def test_bf16_decode_all_codes_match_torch():
    codes, vals = _all_bf16_values()
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(vals), nan)
    assert np.array_equal(vals[~nan], ref[~nan])


def test_bf16_encode_matches_torch_on_fp32_inputs():
    # fp32 -> bf16 in torch is a single RNE rounding; the oracle rounds the same value.
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),     # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38], np.float32),
    ])
    # exact ties: bf16 value + half an ulp (exactly representable in fp32)
    base = rng.standard_normal(20000).astype(np.float32)
    bits = base.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ours = oracle.bf16_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _nearest_even(x: Fraction, cands):
    """Brute-force round-to-nearest, ties to the even code, over (code, value) pairs."""
    best = None
    for code, v in cands:
        dist = abs(Fraction(v) - x)
        key = (dist, code % 2)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def test_bf16_encode_brute_force_on_fp64_inputs():
    # fp64 inputs (more bits than fp32): the oracle must round ONCE.  Brute force: the
    # nearest of all bf16 values bracketing x, with exact rational distances.
    codes, vals = _all_bf16_values()
    pos = [(int(c), float(v)) for c, v in zip(codes[:0x7F80], vals[:0x7F80])]
    pos_vals = np.array([v for _, v in pos])
    rng = np.random.default_rng(11)
    xs = list(rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000)))
    # fp64 values just off a bf16 tie (a double rounding through fp32 would tie them)
    for v in rng.standard_normal(300):
        b = np.float32(v).view(np.uint32) & np.uint32(0xFFFF0000)
        lo = float(b.view(np.float32))
        hi = float((b + np.uint32(0x10000)).view(np.float32))
        mid = (lo + hi) / 2
        xs += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    xs = np.array(xs, np.float64)
    ours = oracle.bf16_encode(xs)
    for x, o in zip(xs, ours):
        a = abs(x)
        i = int(np.searchsorted(pos_vals, a))
        cands = pos[max(0, i - 1): i + 1]
        c = _nearest_even(Fraction(a), cands)
        if x < 0 or (x == 0 and np.signbit(x)):
            c |= 0x8000
        assert int(o) == c, (x, hex(o), hex(c))


def test_e4m3_decode_all_codes_match_torch_and_ocp_points():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(vals), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(vals[~nan], ref[~nan])
    # points printed in the OCP 8-bit FP specification (E4M3 column)
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        v = oracle.e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(v)
        else:
            assert v == float(Fraction(val)), (code, val, v)
        n += 1
    assert n >= 8


def test_e4m3_encode_matches_torch_in_range_and_saturates():
    rng = np.random.default_rng(3)
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    mids = (vals[:-1] + vals[1:]) / 2                     # exact ties
    x = np.concatenate([rng.uniform(-448, 448, 100000),
                        rng.standard_normal(100000) * 0.01,
                        mids, -mids, vals, -vals,
                        np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    x32 = x.astype(np.float32)                            # torch rounds from fp32 once
    ours = oracle.e4m3_encode(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # saturation (torch gives NaN above 464; the saturating conversion gives +-448)
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf])
    assert list(oracle.e4m3_encode(big)) == [0x7E] * 6 + [0xFE, 0xFE]
    assert oracle.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_e4m3_encode_brute_force_ties_to_even():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    cands = [(int(c), float(v)) for c, v in zip(codes, vals)]
    rng = np.random.default_rng(5)
    xs = np.concatenate([(vals[:-1] + vals[1:]) / 2, rng.uniform(0, 448, 2000),
                         rng.uniform(0, 2 ** -6, 500)])
    ours = oracle.e4m3_encode(xs)
    for x, o in zip(xs, ours):
        assert int(o) == _nearest_even(Fraction(float(x)), cands), x


def test_fold_bf16_definition():
    # W'[n,k] = bf16_rne(fl32(gamma[k] * W[n,k])): fp32 product by numpy (IEEE), then the
    # nearest bf16 by brute force.
    rng = np.random.default_rng(9)
    N, K = 7, 33
    W = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32)).to(torch.bfloat16)
    Wb = W.view(torch.int16).numpy().view(np.uint16)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    out = oracle.fold_bf16(Wb, g)
    codes, vals = _all_bf16_values()
    pos = [(int(c), float(v)) for c, v in zip(codes[:0x7F80], vals[:0x7F80])]
    pos_vals = np.array([v for _, v in pos])
    Wf = W.to(torch.float32).numpy()
    for n in range(N):
        for k in range(K):
            p = np.float32(g[k]) * np.float32(Wf[n, k])
            a = abs(float(p))
            i = int(np.searchsorted(pos_vals, a))
            c = _nearest_even(Fraction(a), pos[max(0, i - 1): i + 1])
            if p < 0:
                c |= 0x8000
            assert int(out[n, k]) == c
    # gamma None = plain copy
    assert np.array_equal(oracle.fold_bf16(Wb, None), Wb)


def test_quant_e4m3_definition():
    rng = np.random.default_rng(13)
    N, K = 9, 40
    W = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32)).to(torch.bfloat16)
    Wb = W.view(torch.int16).numpy().view(np.uint16)
    Wf = W.to(torch.float32).numpy()
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    q, amax, scale = oracle.quant_e4m3(Wb, g)
    x = (g[None, :] * Wf).astype(np.float32)              # IEEE fp32 products
    assert amax == np.abs(x).max()
    assert scale == np.float32(amax) / np.float32(448.0)
    codes = np.arange(0x7F, dtype=np.uint8)
    cands = [(int(c), float(v)) for c, v in zip(codes, oracle.e4m3_decode(codes))]
    for n in range(N):
        for k in range(K):
            v = np.float32(x[n, k]) / np.float32(scale)
            a = min(abs(float(v)), 448.0)
            c = _nearest_even(Fraction(a), cands)
            if v < 0:
                c |= 0x80
            assert int(q[n, k]) == c
    # the largest element maps to +-448 exactly (amax / (amax/448) rounds to 448)
    assert np.abs(oracle.e4m3_decode(q)).max() == 448.0
    # amax = 0: scale 1, all-zero codes
    z, a0, s0 = oracle.quant_e4m3(np.zeros((3, 4), np.uint16), None)
    assert a0 == 0 and s0 == 1 and not z.any()


def test_quant_error_bound():
    # |deq(q)/gamma - W| <= 2^-4 |W| + s*2^-10/|gamma| (e4m3 RNE bound incl. subnormals)
    rng = np.random.default_rng(17)
    W = torch.from_numpy(rng.standard_normal((64, 128)).astype(np.float32) / 11).to(torch.bfloat16)
    Wb = W.view(torch.int16).numpy().view(np.uint16)
    Wf = W.to(torch.float64).numpy()
    g = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    q, amax, s = oracle.quant_e4m3(Wb, g)
    back = oracle.e4m3_decode(q) * float(s) / g.astype(np.float64)[None, :]
    bound = 2.0 ** -4 * np.abs(Wf) + float(s) * 2.0 ** -10 / np.abs(g)[None, :] + 1e-12
    assert np.all(np.abs(back - Wf) <= bound)


@pytest.mark.parametrize("code", [0x00, 0x80])
def test_e4m3_zero_codes(code):
    assert oracle.e4m3_decode(np.array([code], np.uint8))[0] == 0.0
