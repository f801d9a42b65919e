"""Naive chunkwise (WY / UT-transform) form of the gated delta rule, NumPy fp64.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see ``oracle/__init__.py``).

This is the second, independent formulation used to pin the token-by-token C
oracle and to provide per-chunk intermediates for unit checks.  It follows the
chunkwise-parallel training scheme the pages describe -- the inner-chunk
recurrence rewritten as matrix products plus one unit-triangular solve per chunk
(Sykra 0.3.3 README, "Architectural Highlights": chunkwise parallel training via
the WY / unit triangular transform; DeltaPhase README, section 1 "Fast
Triangular Solve"), with the data-dependent decay factorised in log space
(DeltaPhase README, section 5, "Exact Chunkwise-Parallel Scan").

Per chunk of length L (the last chunk may be shorter), with S the state at the
chunk start, g_r = sum_{s<=r} ln alpha_s, gamma = exp(g), and
Gamma[r, s] = exp(g_r - g_s) for r >= s (zero above the diagonal; the mask is
applied before the exponential so no factor above 1 is ever formed):

    A   = strict_lower( diag(beta) Kr K^T * Gamma )
    T   = (I + A)^{-1}                       (unit lower triangular solve)
    W   = T diag(beta) (Kr * gamma)
    U   = T diag(beta) V
    Ut  = U - W S
    O   = (Qr * gamma) S + lower( Qr K^T * Gamma ) Ut
    S'  = gamma_L S + (K * exp(g_L - g))^T Ut

Kr, Qr are conj(K), conj(Q) for complex data and K, Q otherwise; K appears
un-conjugated on the write side.  The only library routine used is
``scipy.linalg.solve_triangular``.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_terms(Qc, Kc, Vc, ac, bc, S):
    """Intermediates of one chunk for one chain.  Returns a dict (all fp64/complex128)."""
    L = Kc.shape[0]
    cplx = np.iscomplexobj(Kc) or np.iscomplexobj(Qc) or np.iscomplexobj(Vc) or np.iscomplexobj(S)
    Kr = np.conj(Kc) if cplx else Kc
    Qr = np.conj(Qc) if cplx else Qc
    g = np.cumsum(np.log(ac))
    diff = g[:, None] - g[None, :]
    lower = np.tril(np.ones((L, L), dtype=bool))
    Gam = np.zeros((L, L))
    Gam[lower] = np.exp(diff[lower])
    gamma = np.exp(g)
    A = np.tril(bc[:, None] * (Kr @ Kc.T) * Gam, -1)
    I = np.eye(L)
    T = solve_triangular(I + A, I.astype(A.dtype), lower=True, unit_diagonal=True)
    W = T @ (bc[:, None] * gamma[:, None] * Kr)
    U = T @ (bc[:, None] * Vc)
    Ut = U - W @ S
    P = np.tril(Qr @ Kc.T * Gam)
    O = (Qr * gamma[:, None]) @ S + P @ Ut
    decay_to_end = np.exp(g[-1] - g)
    S_next = gamma[-1] * S + (Kc * decay_to_end[:, None]).T @ Ut
    return dict(g=g, A=A, T=T, W=W, U=U, Ut=Ut, P=P, O=O, S_in=S, S_out=S_next)


def chunked_fwd(q, k, v, alpha, beta, S0=None, chunk: int = 64, keep_terms: bool = False):
    """Chunked forward over [B, T, H, d] inputs.  Returns (o, S_final[, terms]).

    ``terms[(b, h)]`` is the list of per-chunk dicts when ``keep_terms``.
    """
    q, k, v = (np.asarray(x) for x in (q, k, v))
    cplx = any(np.iscomplexobj(x) for x in (q, k, v)) or (S0 is not None and np.iscomplexobj(S0))
    dt = np.complex128 if cplx else np.float64
    q, k, v = (x.astype(dt) for x in (q, k, v))
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv), dtype=dt)
    S_fin = np.zeros((B, H, dk, dv), dtype=dt)
    terms = {}
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv), dtype=dt) if S0 is None else np.asarray(S0[b, h], dtype=dt).copy()
            lst = []
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                tr = chunk_terms(q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h],
                                 alpha[b, c0:c1, h], beta[b, c0:c1, h], S)
                o[b, c0:c1, h] = tr["O"]
                S = tr["S_out"]
                if keep_terms:
                    lst.append(tr)
            S_fin[b, h] = S
            if keep_terms:
                terms[(b, h)] = lst
    if keep_terms:
        return o, S_fin, terms
    return o, S_fin
