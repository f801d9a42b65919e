"""The delta rule with a per-output-channel decay, in plain NumPy fp64.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring): only tests,
the smoke check and the benchmark's CPU baseline use it, and it shares nothing
with the HIP path.

DeltaPhase README, section 5 (LaplacePhaseCore): the decay is a diagonal
diag(r_t) acting on the value channels of the memory, one factor per channel
and token, in (0, 1].  With the state S [dk, dv] (row = key dimension), that
scales the columns of S.  The decay is applied to the Householder-updated
state, the ordering taken for the scalar gate:

    S_t = (I - beta_t k_t k_t^T) S_{t-1} diag(r_t) + beta_t k_t v_t^T,
    o_t = S_t^T q_t.

With r_t = alpha_t (1, ..., 1) this is the scalar-gated rule of
oracle.recurrent_fwd.  Each column of S evolves on its own.
"""
from __future__ import annotations

import numpy as np


def channel_decay_fwd(q, k, v, r, beta, S0=None):
    """q, k [B, T, H, dk]; v, r [B, T, H, dv]; beta [B, T, H]; S0 [B, H, dk, dv] or None.

    Returns (o [B, T, H, dv], S_final [B, H, dk, dv]) in fp64.
    """
    q, k, v, r = (np.asarray(x, dtype=np.float64) for x in (q, k, v, r))
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((B, T, H, dv))
    for t in range(T):
        kt, b = k[:, t], beta[:, t, :, None, None]
        u = np.einsum("bhij,bhi->bhj", S, kt)  # k^T S
        S = (S - b * kt[..., :, None] * u[..., None, :]) * r[:, t][..., None, :] \
            + b * kt[..., :, None] * v[:, t][..., None, :]
        o[:, t] = np.einsum("bhij,bhi->bhj", S, q[:, t])
    return o, S
