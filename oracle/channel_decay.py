"""The delta rule with a per-output-channel decay, in plain NumPy fp64 / complex128.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring): only tests,
the smoke check and the benchmark's CPU baseline use it, and it shares nothing
with the HIP path.

DeltaPhase README, section 2 ("Complex Phase Matrix Delta Memory"), gives the
gated-decay variant that its LaplacePhaseCore implements: the memory is read
through the conjugated key BEFORE any decay, the error against the value is
written along the key, and the old memory is decayed,

    e_t = V_t - read(M_{t-1}, K_t),    M_t = lambda_t M_{t-1} + beta_t (e_t outer K_t).

Section 5 ("Delta-Laplace Phase Memory Core", exact chunkwise-parallel scan)
makes the decay a diagonal diag(r_t) on the memory's output rows, one factor
per value channel.  With the state S [dk, dv] (row = key dimension, S = M^T)
the output rows of M are the columns of S, so for every value channel j:

    e_t[j] = v_t[j] - kread_t^T s_j,      s_j <- r_t[j] s_j + beta_t k_t e_t[j],
    o_t[j] = qread_t^T s_j                (the updated state),

with kread = conj(k), qread = conj(q) for complex data and k, q otherwise.
The decay factors r are real, in (0, 1]; keys may be complex with any modulus
(LaplacePhaseCore's keys are e^{s_t dt}, of modulus e^{sigma dt} <= 1).

Two formulations live here, so that each pins the other:

* ``channel_decay_fwd``: the token loop above.
* ``channel_decay_chunked``: the chunkwise scan of section 5.  Because the decay
  sits on the output side, the coupling between tokens of one chunk is the
  plain Gram Kr K^T, and the decay between tokens u < t factorises in log
  space as exp(c_{t-1} - c_u) with c the running sum of ln r for that channel.
  Each value channel then needs its own unit lower-triangular solve.  Per chunk
  (state s at the chunk start, c_t = sum_{i<=t} ln r_i[j], c_{-1} = 0):

      A_j[t, u] = beta_t (Kr K^T)[t, u] exp(c_{t-1} - c_u)          (u < t)
      (I + A_j) w_j = beta * (v[:, j] - exp(c_{t-1}) (Kr s_j)_t)    (w_t = beta_t e_t)
      o[t, j]  = exp(c_t) (Qr s_j)_t + sum_{u<=t} (Qr K^T)[t, u] exp(c_t - c_u) w_u
      s_j'     = exp(c_{L-1}) s_j + sum_u k_u exp(c_{L-1} - c_u) w_u

  The only library routine is ``scipy.linalg.solve_triangular``.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _as_arrays(q, k, v, r, beta, S0):
    cplx = any(np.iscomplexobj(x) for x in (q, k, v)) or (S0 is not None and np.iscomplexobj(S0))
    dt = np.complex128 if cplx else np.float64
    q, k, v = (np.asarray(x).astype(dt) for x in (q, k, v))
    r = np.asarray(r, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv), dtype=dt) if S0 is None else np.array(S0, dtype=dt)
    return cplx, dt, q, k, v, r, beta, S


def channel_decay_fwd(q, k, v, r, beta, S0=None):
    """q, k [B, T, H, dk]; v, r [B, T, H, dv]; beta [B, T, H]; S0 [B, H, dk, dv] or None.

    Real or complex q, k, v, S0 (r and beta real).  Returns (o [B, T, H, dv],
    S_final [B, H, dk, dv]) in fp64 / complex128.
    """
    cplx, dt, q, k, v, r, beta, S = _as_arrays(q, k, v, r, beta, S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv), dtype=dt)
    for t in range(T):
        kt = k[:, t]
        kread = np.conj(kt) if cplx else kt
        qread = np.conj(q[:, t]) if cplx else q[:, t]
        b = beta[:, t, :, None]
        read = np.einsum("bhij,bhi->bhj", S, kread)       # kread^T S, from the undecayed state
        err = v[:, t] - read                              # error per value channel
        S = S * r[:, t][..., None, :] + kt[..., :, None] * (b * err)[..., None, :]
        o[:, t] = np.einsum("bhij,bhi->bhj", S, qread)
    return o, S


def channel_decay_chunked(q, k, v, r, beta, S0=None, chunk: int = 64):
    """The same forward as a chunkwise scan with one triangular solve per value channel and chunk."""
    cplx, dt, q, k, v, r, beta, S = _as_arrays(q, k, v, r, beta, S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv), dtype=dt)
    for b in range(B):
        for h in range(H):
            s = S[b, h].copy()
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                L = c1 - c0
                K, Q, V = k[b, c0:c1, h], q[b, c0:c1, h], v[b, c0:c1, h]
                Kr = np.conj(K) if cplx else K
                Qr = np.conj(Q) if cplx else Q
                be = beta[b, c0:c1, h]
                c = np.cumsum(np.log(r[b, c0:c1, h]), axis=0)           # [L, dv]
                c_prev = np.vstack([np.zeros((1, dv)), c[:-1]])          # c_{t-1}
                G = Kr @ K.T                                             # plain Gram [L, L]
                P = Qr @ K.T
                KS, QS = Kr @ s, Qr @ s                                  # [L, dv]
                s_next = np.empty_like(s)
                I = np.eye(L)
                strict = np.tril(np.ones((L, L), dtype=bool), -1)
                lower = np.tril(np.ones((L, L), dtype=bool))
                for j in range(dv):
                    dec_read = np.zeros((L, L))
                    dec_read[strict] = np.exp((c_prev[:, j][:, None] - c[:, j][None, :])[strict])
                    A = be[:, None] * G * dec_read
                    rhs = be * (V[:, j] - np.exp(c_prev[:, j]) * KS[:, j])
                    w = solve_triangular(I + A, rhs, lower=True, unit_diagonal=True)
                    dec_out = np.zeros((L, L))
                    dec_out[lower] = np.exp((c[:, j][:, None] - c[:, j][None, :])[lower])
                    o[b, c0:c1, h, j] = np.exp(c[:, j]) * QS[:, j] + (P * dec_out) @ w
                    s_next[:, j] = np.exp(c[-1, j]) * s[:, j] + K.T @ (np.exp(c[-1, j] - c[:, j]) * w)
                s = s_next
            S[b, h] = s
    return o, S
