"""The parity checker itself, on the CPU: ``harness.check_chain`` accepts outputs that
equal the oracle's (the bf16 codes of its h and y, fp32 partials and row scales formed
from its h) and rejects each planted mistake -- one wrong element of y or h, a NaN, an
Inf, two rows of y swapped, a wrong partial, a row scale off by more than its rounding.

The "device outputs" here are CPU tensors built from the oracle's own results, so the
checker's gate and every diagnostic run exactly as in the GPU tests without a GPU.
"""

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from harness import TOL, check_chain

import gemm_epilogue_transformer_amd as coda


def _bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _outputs_from_oracle(w, inp):
    """CPU tensors (h, P, r, y) as a correct chain would return them."""
    prep = oracle.prepare(inp, w.dtype)
    ref = oracle.chain(prep, inp["x_res"], inp["gamma"], w.act, w.eps)
    hb = ref["hb"]
    T = coda.partials_per_row(w.d)
    tile = -(-w.d // T)
    hv = oracle.bf16_decode(hb).astype(np.float32)          # exact: bf16 values in fp32
    P = np.stack([(hv[:, t * tile:(t + 1) * tile] ** 2).sum(1, dtype=np.float32) for t in range(T)], 1)
    r = (1.0 / np.sqrt(P.astype(np.float64).sum(1) / w.d + np.float64(np.float32(w.eps)))).astype(np.float32)
    y = oracle.bf16_encode(ref["y"])
    return (_bf16_tensor(hb.copy()), torch.from_numpy(P), torch.from_numpy(r), _bf16_tensor(y)), prep, ref


CASES = [si.custom(70, 48, 264, 2 * 72, si.ACT_SWIGLU, seed=11),
         si.custom(33, 40, 136, 96, si.ACT_NONE, seed=12),
         si.custom(40, 64, 144, 2 * 40, si.ACT_SWIGLU, seed=13, dtype="e4m3")]


@pytest.fixture(scope="module", params=CASES, ids=lambda w: f"{w.name}_{w.dtype}")
def clean(request):
    w = request.param
    inp = si.generate(w)
    outs, prep, ref = _outputs_from_oracle(w, inp)
    return w, inp, outs, prep, ref


def _check(clean, outs, rows=None):
    w, inp, _, prep, ref = clean
    if rows is not None:
        ref = {k: v[rows] for k, v in ref.items()}
    return check_chain(w, inp, *outs, rows=rows, ref=ref, prep_ref=prep)


def test_exact_outputs_pass(clean):
    stats = _check(clean, clean[2])
    # h and y carry one bf16 rounding each (relative error at most 2^-8)
    assert stats["y_err"] <= 2.0 ** -8 and stats["h_err"] <= 2.0 ** -8


def test_exact_outputs_pass_on_sampled_rows(clean):
    w = clean[0]
    rows = np.array([0, w.M // 2, w.M - 1], np.int64)
    _check(clean, clean[2], rows=rows)


def _planted(clean, which, fn):
    h, P, r, y = (t.clone() for t in clean[2])
    outs = {"h": h, "P": P, "r": r, "y": y}
    fn(outs[which])
    with pytest.raises(AssertionError):
        _check(clean, (outs["h"], outs["P"], outs["r"], outs["y"]))


def _set(t, i, j, v):
    t[i, j] = torch.tensor(v, dtype=t.dtype)


def test_one_wrong_output_element_fails(clean):
    w = clean[0]
    i, j = w.M // 3, w.n_out - 1
    tol = TOL[w.dtype]

    def bump(y):
        v = float(y[i, j])
        _set(y, i, j, v + 3 * tol * (1 + abs(v)))
    _planted(clean, "y", bump)


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")], ids=["nan", "inf", "-inf"])
def test_non_finite_output_fails(clean, bad):
    _planted(clean, "y", lambda y: _set(y, 1, 2, bad))


@pytest.mark.parametrize("bad", [float("nan"), float("inf")], ids=["nan", "inf"])
def test_non_finite_h_fails(clean, bad):
    _planted(clean, "h", lambda h: _set(h, 0, 3, bad))


def test_one_wrong_h_element_fails(clean):
    w = clean[0]

    def bump(h):
        v = float(h[w.M - 1, w.d // 2])
        _set(h, w.M - 1, w.d // 2, v + 3 * TOL[w.dtype] * (1 + abs(v)))
    _planted(clean, "h", bump)


def test_swapped_rows_fail(clean):
    def swap(y):
        a = y[0].clone()
        y[0] = y[1]
        y[1] = a
    _planted(clean, "y", swap)


def test_wrong_partial_fails(clean):
    def bump(P):
        P[2, 0] *= 1.001
    _planted(clean, "P", bump)


def test_row_scale_off_by_more_than_its_rounding_fails(clean):
    def bump(r):
        r[4] = float(np.nextafter(np.nextafter(np.nextafter(np.float32(r[4]), np.float32(2)),
                                               np.float32(2)), np.float32(2)))
    _planted(clean, "r", bump)
