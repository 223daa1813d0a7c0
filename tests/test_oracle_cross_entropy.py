"""Pins of the oracle's cross-entropy (the LM-head product's loss).

The pages name the cross-entropy loss among the operations the reparameterisation
covers and name its pieces (kucoin page, sections "CODA: El epilogo esconde un tesoro"
and "Cinco bloques y un lenguaje LEGO": block log-sum-exp, the max / sum-exp statistics
of online normalisation) without a formula; the standard definition is used:
lse = log sum_v exp(z_v), loss = lse - z_target, 0 for an ignored target.  The pins
check it by exact arithmetic, closed forms and torch's library routine.
"""

from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle


def test_uniform_logits_give_log_v():
    for V in (1, 2, 10, 128256):
        z = np.full((3, V), 1.75)
        lse, loss = oracle.cross_entropy(z, [0, V - 1, V // 2])
        assert np.allclose(lse, 1.75 + np.log(V), rtol=1e-15, atol=1e-12)
        assert np.allclose(loss, np.log(V), rtol=1e-15, atol=1e-12)


def test_two_classes_is_softplus_of_the_margin():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((50, 2)) * 5
    t = rng.integers(0, 2, 50)
    _, loss = oracle.cross_entropy(z, t)
    margin = z[np.arange(50), 1 - t] - z[np.arange(50), t]
    assert np.allclose(loss, np.logaddexp(0.0, margin), rtol=1e-14, atol=1e-14)


def test_exact_against_decimal_arithmetic():
    getcontext().prec = 60
    rng = np.random.default_rng(2)
    z = rng.standard_normal((4, 7)) * 3
    t = np.array([0, 3, 6, 2])
    lse, loss = oracle.cross_entropy(z, t)
    for i in range(4):
        s = sum(Decimal(float(v)).exp() for v in z[i])
        ref = s.ln()
        assert abs(Decimal(float(lse[i])) - ref) <= Decimal("1e-14") * abs(ref)
        assert abs(Decimal(float(loss[i])) - (ref - Decimal(float(z[i, t[i]])))) <= Decimal("1e-13")


def test_shift_invariance_and_no_overflow():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((5, 300))
    t = rng.integers(0, 300, 5)
    _, l0 = oracle.cross_entropy(z, t)
    _, l1 = oracle.cross_entropy(z + 1000.0, t)          # exp(1000) would overflow
    assert np.all(np.isfinite(l1))
    assert np.allclose(l0, l1, rtol=1e-12, atol=1e-12)


def test_matches_torch_cross_entropy():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((64, 1000)) * 2
    t = rng.integers(0, 1000, 64).astype(np.int64)
    t[5] = -100                                           # ignored row
    _, loss = oracle.cross_entropy(z, t)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z), torch.from_numpy(t),
                                            reduction="none", ignore_index=-100).numpy()
    assert np.allclose(loss, ref, rtol=1e-13, atol=1e-13)


def test_ignored_targets_give_zero_loss():
    z = np.random.default_rng(5).standard_normal((4, 9))
    lse, loss = oracle.cross_entropy(z, [-1, 9, 100, 4])
    assert np.all(loss[:3] == 0.0) and loss[3] > 0.0
    assert np.all(np.isfinite(lse))


def test_layout_errors_are_rejected():
    with pytest.raises(ValueError):
        oracle.cross_entropy(np.zeros((2, 3)), [0])
