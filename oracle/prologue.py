"""Input transforms of a gated delta-rule layer, in plain NumPy fp64.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring): only tests,
the smoke check and the benchmark's CPU baseline use it, and it shares nothing
with the HIP path.

Per token t and head h the layer forms, from raw projections:

* q_t / max(||q_t||, eps) and k_t / max(||k_t||, eps): L2 normalisation over
  the key dimension (the unit-norm keys and queries of the input recipe; a
  zero row stays zero).  For complex rows the norm is the Hermitian one,
  ||x||^2 = sum |x_i|^2, the length of x read as a real vector of twice the
  size (DeltaPhase README, section 2: the keys are unit phasors, so a key
  of d phasors has norm sqrt(d));
* beta_t = beta_scale * sigmoid(b_t): DeltaPhase README, section 1 "Extended
  Householder Beta Range" (beta_scale = 2 there; 1 gives the (0, 1) range);
* alpha_t = exp(-softplus(a_t)): the data-dependent forget gate of the Sykra
  README, "Architectural Highlights", read as the logistic map of a logit into
  (0, 1] (the pages name the gate but give no formula).

``prologue_fwd`` applies them and then runs the token-by-token definition
(``oracle.recurrent_fwd``).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-12


def _widen(x) -> np.ndarray:
    """fp64, or complex128 for complex input."""
    x = np.asarray(x)
    return x.astype(np.complex128 if np.iscomplexobj(x) else np.float64)


def l2_normalise(x, eps: float = EPS) -> np.ndarray:
    """Rows of the last axis scaled to unit L2 norm (Hermitian for complex rows); rows with norm below eps are
    divided by eps."""
    x = _widen(x)
    n = np.sqrt(np.sum(np.abs(x) ** 2, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def softplus(a) -> np.ndarray:
    """log(1 + e^a), evaluated as max(a, 0) + log1p(e^{-|a|}) so that no exponent overflows."""
    a = np.asarray(a, dtype=np.float64)
    return np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a)))


def sigmoid(b) -> np.ndarray:
    """1 / (1 + e^{-b}), split by sign so that no exponent overflows."""
    b = np.asarray(b, dtype=np.float64)
    e = np.exp(-np.abs(b))
    return np.where(b >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def prologue(q, k, a_logit, b_logit, beta_scale: float = 1.0):
    """(q_hat, k_hat, alpha, beta) from raw q, k [B, T, H, dk] and logits a, b [B, T, H]."""
    return (l2_normalise(q), l2_normalise(k), np.exp(-softplus(a_logit)),
            float(beta_scale) * sigmoid(b_logit))


def prologue_fwd(q, k, v, a_logit, b_logit, beta_scale: float = 1.0, S0=None, threads: int = 0):
    """The layer forward from raw inputs: the transforms above, then the recurrence.

    Real or complex q, k, v (the gates are real either way).  Returns (o, S_final) in fp64 or complex128, as
    ``oracle.recurrent_fwd`` does.
    """
    from . import recurrent_fwd
    qh, kh, alpha, beta = prologue(q, k, a_logit, b_logit, beta_scale)
    o, S, _ = recurrent_fwd(qh, kh, _widen(v), alpha, beta, S0, threads=threads)
    return o, S
