"""Facts that pin the CPU oracle to the mathematics, independent of its own code.

Each ``pin_*`` function runs the token-by-token oracle (optionally a given
build of it, so the mutation tests can run the same facts against planted
mistakes) and raises AssertionError when the fact does not hold.  None of them
retypes the oracle's update formula: they compare against closed forms, brute
force, a second formulation, hand-worked values or invariants.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from oracle.bruteforce import bruteforce_fwd
from oracle.chunked import chunked_fwd

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(rng, B, T, H, dk, dv, cplx=False, beta_hi=1.0, alpha_lo=0.3, s0=True):
    """Small random inputs in fp64 (unit-norm keys/queries)."""
    if cplx:
        q = _unit(rng.normal(size=(B, T, H, dk)) + 1j * rng.normal(size=(B, T, H, dk)))
        k = _unit(rng.normal(size=(B, T, H, dk)) + 1j * rng.normal(size=(B, T, H, dk)))
        v = rng.normal(size=(B, T, H, dv)) + 1j * rng.normal(size=(B, T, H, dv))
        S0 = rng.normal(size=(B, H, dk, dv)) + 1j * rng.normal(size=(B, H, dk, dv)) if s0 else None
    else:
        q = _unit(rng.normal(size=(B, T, H, dk)))
        k = _unit(rng.normal(size=(B, T, H, dk)))
        v = rng.normal(size=(B, T, H, dv))
        S0 = rng.normal(size=(B, H, dk, dv)) if s0 else None
    alpha = rng.uniform(alpha_lo, 1.0, size=(B, T, H))
    beta = rng.uniform(0.0, beta_hi, size=(B, T, H))
    return q, k, v, alpha, beta, S0


def fwd(lib, q, k, v, alpha, beta, S0=None):
    o, S, _ = oracle.recurrent_fwd(q, k, v, alpha, beta, S0, threads=1, lib=lib)
    return o, S


# --------------------------------------------------------------------------- F1
def pin_decay_only(lib, cplx=False):
    """beta = 0: pure exponential decay, S_t = gamma_t S0 and o_t = gamma_t S0^T qread_t."""
    rng = np.random.default_rng(11)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 2, 9, 3, 5, 4, cplx=cplx)
    beta[:] = 0.0
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    gam = np.cumprod(alpha, axis=1)  # [B, T, H]
    qr = np.conj(q) if cplx else q
    o_ref = gam[..., None] * np.einsum("bhij,bthi->bthj", S0, qr)
    S_ref = gam[:, -1, :, None, None] * S0
    assert rel(o, o_ref) < 1e-13, rel(o, o_ref)
    assert rel(S, S_ref) < 1e-13, rel(S, S_ref)


# --------------------------------------------------------------------------- F2
def pin_overwrite_retrieval(lib, cplx=False):
    """alpha = beta = 1 with orthonormal keys: querying a key returns its latest written value."""
    rng = np.random.default_rng(12)
    d, T = 8, 30
    Z = rng.normal(size=(d, d)) + (1j * rng.normal(size=(d, d)) if cplx else 0)
    Qm, _ = np.linalg.qr(Z)
    keys = Qm.T  # rows orthonormal (in the Hermitian sense for complex)
    widx = rng.integers(0, d, size=T)
    qidx = rng.integers(0, d, size=T)
    k = keys[widx][None, :, None, :]
    # query with the key whose readout is kread = conj(key) for complex data: o = S^T conj(q)
    q = keys[qidx][None, :, None, :]
    v = rng.normal(size=(1, T, 1, 5)) + (1j * rng.normal(size=(1, T, 1, 5)) if cplx else 0)
    alpha = np.ones((1, T, 1))
    beta = np.ones((1, T, 1))
    o, _ = fwd(lib, q, k, v, alpha, beta, None)
    latest = {}
    for t in range(T):
        latest[widx[t]] = v[0, t, 0]
        want = latest.get(qidx[t], np.zeros(5))
        assert np.allclose(o[0, t, 0], want, atol=1e-12), (t, o[0, t, 0], want)


def pin_self_retrieval(lib, cplx=False):
    """beta = 1, |k| = 1, q = k: o_t = v_t for any alpha and any previous state."""
    rng = np.random.default_rng(13)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 2, 11, 2, 6, 3, cplx=cplx)
    beta[:] = 1.0
    o, _ = fwd(lib, k, k, v, alpha, beta, S0)
    assert rel(o, v) < 1e-13, rel(o, v)


# --------------------------------------------------------------------------- F3
def pin_chunked_agrees(lib, cplx=False, chunks=(1, 4, 16, 64)):
    """The chunkwise WY form (NumPy, scipy triangular solve) equals the token loop."""
    rng = np.random.default_rng(14)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 150, 2, 8, 6, cplx=cplx, beta_hi=2.0 if cplx else 1.0)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    for C in chunks:
        oc, Sc = chunked_fwd(q, k, v, alpha, beta, S0, chunk=C)
        assert rel(oc, o) < 1e-12, (C, rel(oc, o))
        assert rel(Sc, S) < 1e-12, (C, rel(Sc, S))


# --------------------------------------------------------------------------- F4
def pin_bruteforce(lib, cplx=False):
    """Explicit dense transition products agree for T <= 16 (dk != dv catches transposes)."""
    rng = np.random.default_rng(15)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 2, 12, 3, 8, 6, cplx=cplx, beta_hi=2.0)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    ob, Sb = bruteforce_fwd(q, k, v, alpha, beta, S0)
    assert rel(o, ob) < 1e-12, rel(o, ob)
    assert rel(S, Sb) < 1e-12, rel(S, Sb)
    # zero initial state as well (the NULL-S0 path)
    o, S = fwd(lib, q, k, v, alpha, beta, None)
    ob, Sb = bruteforce_fwd(q, k, v, alpha, beta, None)
    assert rel(o, ob) < 1e-12 and rel(S, Sb) < 1e-12


# --------------------------------------------------------------------------- F5
def pin_linearity(lib, cplx=False):
    """Jointly linear in (V, S0); linear in q."""
    rng = np.random.default_rng(16)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 20, 2, 6, 5, cplx=cplx)
    _, _, v2, _, _, S02 = rand_inputs(rng, 1, 20, 2, 6, 5, cplx=cplx)
    c = 0.7 - (0.4j if cplx else 0.0)
    o1, S1 = fwd(lib, q, k, v, alpha, beta, S0)
    o2, S2 = fwd(lib, q, k, v2, alpha, beta, S02)
    o3, S3 = fwd(lib, q, k, v + c * v2, alpha, beta, S0 + c * S02)
    assert rel(o3, o1 + c * o2) < 1e-12 and rel(S3, S1 + c * S2) < 1e-12
    q2 = rand_inputs(rng, 1, 20, 2, 6, 5, cplx=cplx)[0]
    oq, _ = fwd(lib, q + q2, k, v, alpha, beta, S0)
    oq2, _ = fwd(lib, q2, k, v, alpha, beta, S0)
    assert rel(oq, o1 + oq2) < 1e-12


# --------------------------------------------------------------------------- F6
def pin_column_independence(lib, cplx=False):
    """Permuting the value columns of V and S0 permutes the columns of o and S."""
    rng = np.random.default_rng(17)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 25, 2, 6, 5, cplx=cplx)
    perm = rng.permutation(5)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    op, Sp = fwd(lib, q, k, v[..., perm], alpha, beta, S0[..., perm])
    assert rel(op, o[..., perm]) < 1e-13 and rel(Sp, S[..., perm]) < 1e-13


# --------------------------------------------------------------------------- F7
def pin_contraction(lib, cplx=False):
    """|k| = 1, alpha <= 1, beta in [0, 2]: the difference of two states never grows (spectral norm)."""
    rng = np.random.default_rng(18)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 40, 1, 6, 4, cplx=cplx, beta_hi=2.0, alpha_lo=0.9)
    _, _, _, _, _, S0b = rand_inputs(rng, 1, 40, 1, 6, 4, cplx=cplx)
    prev = np.linalg.norm(S0[0, 0] - S0b[0, 0], 2)
    for T in range(1, 41, 3):
        _, Sa = fwd(lib, q[:, :T], k[:, :T], v[:, :T], alpha[:, :T], beta[:, :T], S0)
        _, Sb = fwd(lib, q[:, :T], k[:, :T], v[:, :T], alpha[:, :T], beta[:, :T], S0b)
        cur = np.linalg.norm(Sa[0, 0] - Sb[0, 0], 2)
        assert cur <= prev * (1 + 1e-12), (T, cur, prev)
        prev = cur
    # and with alpha < 1 somewhere the difference strictly shrinks
    assert prev < np.linalg.norm(S0[0, 0] - S0b[0, 0], 2) * 0.999


# --------------------------------------------------------------------------- F8
def pin_reflection_isometry(lib, cplx=False):
    """beta = 2, alpha = 1, v = 0: each step is a Householder reflection, ||S||_F is constant."""
    rng = np.random.default_rng(19)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 30, 2, 7, 5, cplx=cplx)
    beta[:] = 2.0
    alpha[:] = 1.0
    v[:] = 0.0
    _, S = fwd(lib, q, k, v, alpha, beta, S0)
    n0 = np.linalg.norm(S0.reshape(2, -1), axis=1)
    n1 = np.linalg.norm(S.reshape(2, -1), axis=1)
    assert np.allclose(n0, n1, rtol=1e-12), (n0, n1)
    # and the state did change (it is a reflection, not the identity)
    assert rel(S, S0) > 1e-3


# --------------------------------------------------------------------------- F9
def pin_split_invariance(lib, cplx=False):
    """Two calls chained through the final state equal one call."""
    rng = np.random.default_rng(20)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 2, 37, 2, 6, 5, cplx=cplx)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    cut = 13
    oa, Sa = fwd(lib, q[:, :cut], k[:, :cut], v[:, :cut], alpha[:, :cut], beta[:, :cut], S0)
    ob, Sb = fwd(lib, q[:, cut:], k[:, cut:], v[:, cut:], alpha[:, cut:], beta[:, cut:], Sa)
    assert rel(np.concatenate([oa, ob], axis=1), o) < 1e-13 and rel(Sb, S) < 1e-13


# -------------------------------------------------------------------------- F10
def pin_padding_identity(lib, cplx=False):
    """Tokens with alpha = 1, beta = 0, k = 0 leave the state unchanged; their outputs read it."""
    rng = np.random.default_rng(21)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 10, 2, 6, 5, cplx=cplx)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    P = 7
    qp = rand_inputs(rng, 1, P, 2, 6, 5, cplx=cplx)[0]
    cat = lambda a, b: np.concatenate([a, b], axis=1)
    o2, S2 = fwd(lib, cat(q, qp), cat(k, np.zeros_like(qp)), cat(v, rng.normal(size=(1, P, 2, 5))),
                 cat(alpha, np.ones((1, P, 2))), cat(beta, np.zeros((1, P, 2))), S0)
    assert rel(S2, S) < 1e-14 and rel(o2[:, :10], o) < 1e-14
    qr = np.conj(qp) if cplx else qp
    assert rel(o2[:, 10:], np.einsum("bhij,bthi->bthj", S, qr)) < 1e-13


# -------------------------------------------------------------------------- F11
def pin_complex_consistency(lib):
    """Complex data with zero imaginary parts equals real data; conj(inputs) -> conj(outputs)."""
    rng = np.random.default_rng(22)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 20, 2, 6, 5, cplx=False)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    oc, Sc = fwd(lib, q + 0j, k + 0j, v + 0j, alpha, beta, S0 + 0j)
    assert rel(oc, o) < 1e-14 and rel(Sc, S) < 1e-14 and np.abs(oc.imag).max() == 0.0
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 20, 2, 6, 5, cplx=True)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    oc, Sc = fwd(lib, np.conj(q), np.conj(k), np.conj(v), alpha, beta, np.conj(S0))
    assert rel(oc, np.conj(o)) < 1e-13 and rel(Sc, np.conj(S)) < 1e-13


# -------------------------------------------------------------------------- F12
def pin_decode_matches_forward(lib, cplx=False):
    """T single-token decode steps equal one forward over the same tokens."""
    rng = np.random.default_rng(23)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 2, 9, 3, 6, 5, cplx=cplx)
    o, S = fwd(lib, q, k, v, alpha, beta, S0)
    St = S0.reshape(6, 6, 5)
    for t in range(9):
        ot, St = oracle.recurrent_step(q[:, t].reshape(6, 6), k[:, t].reshape(6, 6), v[:, t].reshape(6, 5),
                                       alpha[:, t].reshape(6), beta[:, t].reshape(6), St, threads=1, lib=lib)
        assert rel(ot, o[:, t].reshape(6, 5)) < 1e-13, t
    assert rel(St, S.reshape(6, 6, 5)) < 1e-13


def pin_decode_self_retrieval(lib, cplx=False):
    """Decode step with beta = 1, q = k, |k| = 1 returns v exactly."""
    rng = np.random.default_rng(24)
    q, k, v, alpha, beta, S0 = rand_inputs(rng, 1, 1, 16, 6, 5, cplx=cplx)
    o, _ = oracle.recurrent_step(k[0, 0], k[0, 0], v[0, 0], alpha[0, 0], np.ones(16), S0[0], threads=1, lib=lib)
    assert rel(o, v[0, 0]) < 1e-13


# ------------------------------------------------------------------------ golden
def pin_handworked(lib):
    """Hand-derived tiny cases (tests/golden/handworked.json)."""
    with open(os.path.join(GOLDEN, "handworked.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        cplx = case["dtype"] == "complex"

        def arr(x):
            a = np.asarray(x, dtype=np.float64)
            return a[..., 0] + 1j * a[..., 1] if cplx else a

        q, k, v = arr(case["q"]), arr(case["k"]), arr(case["v"])
        T, dk = q.shape
        dv = v.shape[1]
        alpha = np.asarray(case["alpha"])[None, :, None]
        beta = np.asarray(case["beta"])[None, :, None]
        S0 = arr(case["S0"])[None, None]
        o, S = fwd(lib, q[None, :, None], k[None, :, None], v[None, :, None], alpha, beta, S0)
        assert np.allclose(o[0, :, 0], arr(case["o"]), atol=1e-14), case["name"]
        assert np.allclose(S[0, 0], arr(case["S_final"]), atol=1e-14), case["name"]
        # the decode entry point follows the same hand-worked steps
        St = S0[0]
        for t in range(T):
            ot, St = oracle.recurrent_step(q[t][None], k[t][None], v[t][None], np.array([case["alpha"][t]]),
                                           np.array([case["beta"][t]]), St, threads=1, lib=lib)
            assert np.allclose(ot[0], arr(case["o"])[t], atol=1e-14), (case["name"], t)


def all_pins():
    """(name, callable(lib)) for every pin, real and complex variants."""
    out = [("handworked", pin_handworked), ("complex_consistency", pin_complex_consistency)]
    for cplx in (False, True):
        tag = "c" if cplx else "r"
        for fn in (pin_decay_only, pin_overwrite_retrieval, pin_self_retrieval, pin_chunked_agrees,
                   pin_bruteforce, pin_linearity, pin_column_independence, pin_contraction,
                   pin_reflection_isometry, pin_split_invariance, pin_padding_identity,
                   pin_decode_matches_forward, pin_decode_self_retrieval):
            out.append((f"{fn.__name__[4:]}_{tag}", (lambda f, c: (lambda lib: f(lib, cplx=c)))(fn, cplx)))
    return out
