"""Pins for the oracle's input transforms (oracle/prologue.py), and mutants they must catch.

The transforms are L2 normalisation of q and k over the key dimension (Hermitian
for complex rows),
beta = beta_scale * sigmoid(b) and alpha = exp(-softplus(a)).  The pins check
them against closed forms (special values, an exact hand-worked token),
invariants (per-row rescaling of the raw q and k) and an identity
(exp(-softplus(a)) = 1 / (1 + e^a)) that rebuilds logits from given gates and
must reproduce the plain oracle; complex rows are pinned by unit phasors (norm
sqrt(d)), by the real vector a complex row stands for, and by the phase a
rescaled complex query puts on the output.  Each mutant plants one plausible mistake in a
copy of the transforms; some pin must reject it.  CPU only.
"""
import types
import warnings

import numpy as np
import pytest

import oracle
from oracle import prologue as pro


def _impl(prologue_fn):
    """A transforms implementation (prologue, prologue_fwd) built on `prologue_fn`."""
    def prologue_fwd(q, k, v, a, b, beta_scale=1.0, S0=None):
        qh, kh, alpha, beta = prologue_fn(q, k, a, b, beta_scale)
        v = np.asarray(v, np.complex128 if np.iscomplexobj(v) else np.float64)
        o, S, _ = oracle.recurrent_fwd(qh, kh, v, alpha, beta, S0, threads=1)
        return o, S
    return types.SimpleNamespace(prologue=prologue_fn, prologue_fwd=prologue_fwd)


REAL = _impl(pro.prologue)


def _raw(rng, B, T, H, d):
    q = rng.normal(size=(B, T, H, d)) * rng.uniform(0.2, 5.0, size=(B, T, H, 1))
    k = rng.normal(size=(B, T, H, d)) * rng.uniform(0.2, 5.0, size=(B, T, H, 1))
    v = rng.normal(size=(B, T, H, d))
    a = rng.normal(-2.0, 2.0, size=(B, T, H))
    b = rng.normal(0.0, 2.0, size=(B, T, H))
    S0 = rng.normal(size=(B, H, d, d))
    return q, k, v, a, b, S0


def pin_special_values(impl):
    """alpha(0) = 1/2, alpha -> 1 as a -> -inf, alpha ~ e^{-a} for large a; beta(0) = scale / 2, beta -> scale."""
    z = np.zeros((1, 5, 1, 2))
    a = np.array([0.0, -60.0, 40.0, 0.0, 0.0]).reshape(1, 5, 1)
    b = np.array([0.0, 0.0, 0.0, 60.0, -60.0]).reshape(1, 5, 1)
    for scale in (1.0, 2.0):
        _, _, alpha, beta = impl.prologue(z + 1.0, z + 1.0, a, b, scale)
        alpha, beta = alpha.ravel(), beta.ravel()
        assert abs(alpha[0] - 0.5) < 1e-15
        assert abs(alpha[1] - 1.0) < 1e-15
        assert abs(alpha[2] / np.exp(-40.0) - 1.0) < 1e-12
        assert abs(beta[0] - scale / 2) < 1e-15
        assert abs(beta[3] - scale) < 1e-15 and abs(beta[4]) < 1e-15


def pin_unit_rows(impl):
    """Every (b, t, h) row of q_hat and k_hat has unit norm and the raw row's direction; zero rows stay zero."""
    rng = np.random.default_rng(3)
    q, k, _, a, b, _ = _raw(rng, 2, 7, 3, 6)
    q[1, 2, 0] = 0.0
    qh, kh, _, _ = impl.prologue(q, k, a, b, 1.0)
    assert np.all(qh[1, 2, 0] == 0.0)
    nq = np.linalg.norm(qh, axis=-1)
    nq[1, 2, 0] = 1.0
    assert np.allclose(nq, 1.0, atol=1e-14) and np.allclose(np.linalg.norm(kh, axis=-1), 1.0, atol=1e-14)
    cos = np.sum(kh * k, axis=-1) / np.linalg.norm(k, axis=-1)
    assert np.allclose(cos, 1.0, atol=1e-14)


def pin_handworked_token(impl):
    """One token, S0 = 0: q = (3, 4) -> (0.6, 0.8); k = (0, 2) -> (0, 1); a = 0 -> alpha = 1/2;
    b = 0 with scale 2 -> beta = 1.  Then S_1 = beta k v^T = [[0], [5]] and o = S_1^T q_hat = 4."""
    q = np.array([3.0, 4.0]).reshape(1, 1, 1, 2)
    k = np.array([0.0, 2.0]).reshape(1, 1, 1, 2)
    v = np.array([5.0]).reshape(1, 1, 1, 1)
    zero = np.zeros((1, 1, 1))
    o, S = impl.prologue_fwd(q, k, v, zero, zero, 2.0)
    assert abs(o.ravel()[0] - 4.0) < 1e-14
    assert np.allclose(S.ravel(), [0.0, 5.0], atol=1e-14)


def pin_row_rescaling_invariance(impl):
    """Scaling each raw (b, t, h) row of q and k by its own positive factor changes nothing."""
    rng = np.random.default_rng(5)
    q, k, v, a, b, S0 = _raw(rng, 2, 9, 2, 5)
    o1, S1 = impl.prologue_fwd(q, k, v, a, b, 2.0, S0)
    o2, S2 = impl.prologue_fwd(q * rng.uniform(0.1, 10.0, size=(2, 9, 2, 1)),
                               k * rng.uniform(0.1, 10.0, size=(2, 9, 2, 1)), v, a, b, 2.0, S0)
    assert np.linalg.norm(o1 - o2) <= 1e-12 * np.linalg.norm(o1)
    assert np.linalg.norm(S1 - S2) <= 1e-12 * np.linalg.norm(S1)


def pin_logits_from_gates(impl):
    """exp(-softplus(a)) = 1 / (1 + e^a), so a = ln(1/alpha - 1) and b = ln(beta / (scale - beta)) turn
    given gates into logits; the layer forward on unit rows must then equal the plain oracle."""
    rng = np.random.default_rng(9)
    for scale in (1.0, 2.0):
        q, k, v, _, _, S0 = _raw(rng, 1, 12, 2, 4)
        qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
        kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
        alpha = rng.uniform(0.05, 0.95, size=(1, 12, 2))
        beta = rng.uniform(0.05, 0.95, size=(1, 12, 2)) * scale
        a = np.log(1.0 / alpha - 1.0)
        b = np.log(beta / (scale - beta))
        o1, S1 = impl.prologue_fwd(qn, kn, v, a, b, scale, S0)
        o2, S2, _ = oracle.recurrent_fwd(qn, kn, v, alpha, beta, S0, threads=1)
        assert np.linalg.norm(o1 - o2) <= 1e-12 * np.linalg.norm(o2)
        assert np.linalg.norm(S1 - S2) <= 1e-12 * np.linalg.norm(S2)


def _craw(rng, B, T, H, d):
    q = (rng.normal(size=(B, T, H, d)) + 1j * rng.normal(size=(B, T, H, d))) * rng.uniform(0.2, 5.0, (B, T, H, 1))
    k = (rng.normal(size=(B, T, H, d)) + 1j * rng.normal(size=(B, T, H, d))) * rng.uniform(0.2, 5.0, (B, T, H, 1))
    v = rng.normal(size=(B, T, H, d)) + 1j * rng.normal(size=(B, T, H, d))
    return q, k, v


def pin_complex_phasor_rows(impl):
    """Rows of d unit phasors e^{i theta} (the DeltaPhase keys) have Hermitian norm sqrt(d), so they normalise to
    e^{i theta} / sqrt(d) exactly; a general complex row normalises to the same unit vector as the real vector
    (Re x, Im x) it stands for."""
    rng = np.random.default_rng(21)
    d = 8
    th = rng.uniform(-np.pi, np.pi, size=(1, 3, 2, d))
    ph = np.exp(1j * th)
    _, kh, _, _ = impl.prologue(ph, ph, np.zeros((1, 3, 2)), np.zeros((1, 3, 2)), 2.0)
    assert np.allclose(kh, ph / np.sqrt(d), atol=1e-15, rtol=0)
    q, k, _ = _craw(rng, 1, 4, 2, 5)
    qh, _, _, _ = impl.prologue(q, k, np.zeros((1, 4, 2)), np.zeros((1, 4, 2)), 1.0)
    r = np.concatenate([q.real, q.imag], axis=-1)
    rh = r / np.linalg.norm(r, axis=-1, keepdims=True)
    assert np.allclose(np.concatenate([qh.real, qh.imag], axis=-1), rh, atol=1e-14, rtol=0)


def pin_complex_query_phase(impl):
    """Multiplying each raw complex query row by its own nonzero complex factor c rescales the output row by
    conj(c / |c|) (the readout uses the conjugated query) and leaves the final state unchanged."""
    rng = np.random.default_rng(23)
    q, k, v = _craw(rng, 1, 10, 2, 4)
    a = rng.normal(-2.0, 1.0, size=(1, 10, 2))
    b = rng.normal(0.0, 1.0, size=(1, 10, 2))
    c = rng.normal(size=(1, 10, 2, 1)) + 1j * rng.normal(size=(1, 10, 2, 1))
    o1, S1 = impl.prologue_fwd(q, k, v, a, b, 2.0)
    o2, S2 = impl.prologue_fwd(q * c, k, v, a, b, 2.0)
    assert np.linalg.norm(o2 - np.conj(c / np.abs(c)) * o1) <= 1e-12 * np.linalg.norm(o1)
    assert np.linalg.norm(S2 - S1) <= 1e-12 * np.linalg.norm(S1)


PINS = [pin_special_values, pin_unit_rows, pin_handworked_token, pin_row_rescaling_invariance,
        pin_logits_from_gates, pin_complex_phasor_rows, pin_complex_query_phase]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_prologue_pin(pin):
    pin(REAL)


def _norm_axis(x, axis):
    x = np.asarray(x, np.float64)
    return x / np.maximum(np.sqrt(np.sum(x * x, axis=axis, keepdims=True)), pro.EPS)


def _square_norm(x):
    """x / sqrt(sum x_i^2) without the modulus (the real formula applied to complex rows)."""
    x = np.asarray(x)
    return x / np.maximum(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)), pro.EPS)


def _real_part_norm(x):
    """Complex rows divided by the norm of their real parts only."""
    x = np.asarray(x)
    return x / np.maximum(np.sqrt(np.sum(np.real(x) ** 2, axis=-1, keepdims=True)), pro.EPS)


def _mut(**over):
    """The real transforms with one piece replaced."""
    def fn(q, k, a, b, scale):
        qh = over["q"](q) if "q" in over else pro.l2_normalise(q)
        kh = over["k"](k) if "k" in over else pro.l2_normalise(k)
        alpha = over["alpha"](a) if "alpha" in over else np.exp(-pro.softplus(a))
        beta = over["beta"](b, scale) if "beta" in over else scale * pro.sigmoid(b)
        return qh, kh, alpha, beta
    return _impl(fn)


MUTANTS = {
    "q_not_normalised": _mut(q=lambda q: np.asarray(q, np.float64)),
    "k_not_normalised": _mut(k=lambda k: np.asarray(k, np.float64)),
    "normalised_over_tokens": _mut(q=lambda q: _norm_axis(q, 1), k=lambda k: _norm_axis(k, 1)),
    "normalised_over_heads": _mut(k=lambda k: _norm_axis(k, 2)),
    "zero_row_divides_by_zero": _mut(q=lambda q: np.asarray(q, np.float64)
                                     / np.sqrt(np.sum(np.asarray(q, np.float64) ** 2, axis=-1, keepdims=True))),
    "alpha_exp_plus_softplus": _mut(alpha=lambda a: np.minimum(np.exp(pro.softplus(a)), 1.0)),
    "alpha_exp_minus_logit": _mut(alpha=lambda a: np.minimum(np.exp(-np.asarray(a)), 1.0)),
    "alpha_sigmoid_of_logit": _mut(alpha=lambda a: pro.sigmoid(a)),
    "beta_sigmoid_negated": _mut(beta=lambda b, s: s * pro.sigmoid(-np.asarray(b))),
    "beta_scale_dropped": _mut(beta=lambda b, s: pro.sigmoid(b)),
    "beta_scale_squared": _mut(beta=lambda b, s: s * s * pro.sigmoid(b)),
    "complex_norm_without_modulus": _mut(q=lambda q: _square_norm(q), k=lambda k: _square_norm(k)),
    "complex_norm_real_part_only": _mut(q=lambda q: _real_part_norm(q), k=lambda k: _real_part_norm(k)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prologue_mutant_caught(name):
    impl = MUTANTS[name]
    with np.errstate(all="ignore"), warnings.catch_warnings():
        warnings.simplefilter("ignore", np.exceptions.ComplexWarning)
        caught = []
        for pin in PINS:
            try:
                pin(impl)
            except (AssertionError, FloatingPointError, ValueError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every prologue pin"
