"""Reverse-mode gradients of the gated delta rule's token loop, in plain NumPy fp64.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring): only tests,
the smoke check and the benchmark's CPU baseline use it, and it shares nothing
with the HIP path.

For real data the forward is, per (batch, head) chain and token t,

    u_t = S_{t-1}^T k_t,
    S_t = alpha_t (S_{t-1} - beta_t k_t u_t^T) + beta_t k_t v_t^T,
    o_t = S_t^T q_t,

the recurrence of DeltaPhase section 2 with the data-dependent forget gate of
the Sykra README ("Architectural Highlights"), gate applied to the whole
Householder-updated state.  Given upstream gradients dO (of o) and dS_T (of
the final state), the chain rule taken token by token in reverse gives, with
G the gradient reaching S_t from later tokens (G = dS_T at t = T):

    D     = G + q_t dO_t^T                      (o_t reads S_t)
    dq_t  = S_t dO_t
    w     = D^T k_t
    dv_t  = beta_t w
    dbeta_t  = w . (v_t - alpha_t u_t)
    dalpha_t = <D, S_{t-1} - beta_t k_t u_t^T>
    dk_t  = D (beta_t v_t - alpha_t beta_t u_t) - alpha_t beta_t S_{t-1} w
    G     <- alpha_t (D - beta_t k_t w^T)       (the gradient reaching S_{t-1})

and dS0 is the final G.

Complex data (DeltaPhase section 2: the readout takes the conjugated key, and
the output the conjugated query): u_t = S_{t-1}^T conj(k_t), o_t = S_t^T
conj(q_t), with real gates.  The loss is real, and the gradient of a complex
input z is dL/dRe(z) + i dL/dIm(z) (so that a change dz moves the loss by
Re(sum conj(grad) dz)); the upstream dO and dS_T are given the same way.  The
same steps then read

    D     = G + q_t dO_t^T
    dq_t  = S_t conj(dO_t)
    w     = D^T conj(k_t)
    dv_t  = beta_t w
    dbeta_t  = Re(conj(w) . (v_t - alpha_t u_t))
    dalpha_t = Re <D, S_{t-1} - beta_t k_t u_t^T>   (<A, B> = sum conj(A) B)
    dk_t  = D conj(y) - alpha_t beta_t S_{t-1} conj(w),  y = beta_t v_t - alpha_t beta_t u_t
    G     <- alpha_t (D - beta_t k_t w^T)

which reduce to the real ones when every value is real (conj is then the
identity).  The pins in tests/test_oracle_backward.py check both against
central finite differences of the C oracle's forward (for complex inputs along
real and imaginary directions separately), not against this derivation.
"""
from __future__ import annotations

import numpy as np


def recurrent_bwd(q, k, v, alpha, beta, S0, dO, dS_final):
    """Gradients of the real loss  Re sum(conj(dO) o) + Re sum(conj(dS_final) S_T)  for the token loop
    (for real data simply sum(o * dO) + sum(S_T * dS_final)).

    q, k [B, T, H, dk]; v, dO [B, T, H, dv]; alpha, beta [B, T, H]; S0 and
    dS_final [B, H, dk, dv] or None (zero).  Real or complex (complex if any of
    q, k, v, S0, dO, dS_final is).  Returns (dq, dk, dv, dalpha, dbeta, dS0) in
    fp64 / complex128 with the shapes of the inputs; dalpha and dbeta are real.
    """
    cplx = any(x is not None and np.iscomplexobj(x) for x in (q, k, v, S0, dO, dS_final))
    dt = np.complex128 if cplx else np.float64
    q, k, v, dO = (np.asarray(x, dtype=dt) for x in (q, k, v, dO))
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    cj = np.conj
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv), dtype=dt) if S0 is None else np.array(S0, dtype=dt)

    # Forward, keeping every state: states[t] = S_t (states[0] = S0).
    states = np.empty((T + 1, B, H, dk, dv), dtype=dt)
    states[0] = S
    for t in range(T):
        kt, vt = k[:, t], v[:, t]
        a, b = alpha[:, t, :, None, None], beta[:, t, :, None, None]
        u = np.einsum("bhij,bhi->bhj", S, cj(kt))
        S = a * (S - b * kt[..., :, None] * u[..., None, :]) + b * kt[..., :, None] * vt[..., None, :]
        states[t + 1] = S

    G = np.zeros((B, H, dk, dv), dtype=dt) if dS_final is None else np.array(dS_final, dtype=dt)
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dalpha, dbeta = np.zeros_like(alpha), np.zeros_like(beta)
    for t in range(T - 1, -1, -1):
        Sp, St = states[t], states[t + 1]
        qt, kt, vt, dot = q[:, t], k[:, t], v[:, t], dO[:, t]
        a, b = alpha[:, t], beta[:, t]
        D = G + qt[..., :, None] * dot[..., None, :]
        dq[:, t] = np.einsum("bhij,bhj->bhi", St, cj(dot))
        u = np.einsum("bhij,bhi->bhj", Sp, cj(kt))
        w = np.einsum("bhij,bhi->bhj", D, cj(kt))
        dv_[:, t] = b[..., None] * w
        dbeta[:, t] = np.real(np.sum(cj(w) * (vt - a[..., None] * u), axis=-1))
        dalpha[:, t] = np.real(np.sum(cj(D) * (Sp - b[..., None, None] * kt[..., :, None] * u[..., None, :]),
                                      axis=(-2, -1)))
        y = b[..., None] * vt - (a * b)[..., None] * u
        dk_[:, t] = (np.einsum("bhij,bhj->bhi", D, cj(y))
                     - (a * b)[..., None] * np.einsum("bhij,bhj->bhi", Sp, cj(w)))
        G = a[..., None, None] * (D - b[..., None, None] * kt[..., :, None] * w[..., None, :])
    return dq, dk_, dv_, dalpha, dbeta, G
