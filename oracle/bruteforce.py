"""Brute-force gated delta rule through explicit dense transition products.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see ``oracle/__init__.py``).

For short sequences the state is written in closed form as a sum over writes,
each carried forward by the ordered product of the per-token transition
matrices (the unrolled recurrence of the gated delta rule: a rank-one delta
write along the key, decay by the forget gate alpha, Householder-type erase
I - beta k kread^T; DeltaPhase README section 2, Sykra README "Architectural
Highlights"):

    Phi(t, s) = M_t M_{t-1} ... M_{s+1},   M_r = alpha_r (I - beta_r k_r kread_r^T)
    S_t       = Phi(t, -1) S_0 + sum_{s <= t} Phi(t, s) beta_s k_s v_s^T
    o_t       = S_t^T qread_t

Every M_r is formed as a dense dk x dk matrix, so this shares no structure with
either the token loop or the chunked form.  Cost is O(T^2 dk^3); use T <= 16.
"""
from __future__ import annotations

import numpy as np


def bruteforce_fwd(q, k, v, alpha, beta, S0=None):
    """Same contract as ``recurrent_fwd`` for one batch of short sequences."""
    q, k, v = (np.asarray(x) for x in (q, k, v))
    cplx = any(np.iscomplexobj(x) for x in (q, k, v)) or (S0 is not None and np.iscomplexobj(S0))
    dt = np.complex128 if cplx else np.float64
    q, k, v = (x.astype(dt) for x in (q, k, v))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv), dtype=dt)
    S_fin = np.zeros((B, H, dk, dv), dtype=dt)
    I = np.eye(dk, dtype=dt)
    for b in range(B):
        for h in range(H):
            kk = k[b, :, h]
            kread = np.conj(kk) if cplx else kk
            qread = np.conj(q[b, :, h]) if cplx else q[b, :, h]
            M = [alpha[b, t, h] * (I - beta[b, t, h] * np.outer(kk[t], kread[t])) for t in range(T)]
            S_init = np.zeros((dk, dv), dtype=dt) if S0 is None else np.asarray(S0[b, h], dtype=dt)
            for t in range(T):
                # Phi(t, s) for s = t-1, ..., -1, built by right-multiplying with M_{s+1}
                Phi = I.copy()
                St = beta[b, t, h] * np.outer(kk[t], v[b, t, h])  # s = t term, Phi(t, t) = I
                for s in range(t - 1, -2, -1):
                    Phi = Phi @ M[s + 1]
                    if s >= 0:
                        St = St + Phi @ (beta[b, s, h] * np.outer(kk[s], v[b, s, h]))
                St = St + Phi @ S_init
                o[b, t, h] = St.T @ qread[t]
                if t == T - 1:
                    S_fin[b, h] = St
            if T == 0:
                S_fin[b, h] = S_init
    return o, S_fin
