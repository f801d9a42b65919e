"""Pins for the oracle's reverse-mode gradients (oracle/backward.py), and mutants they must catch.

The gradients are pinned to something other than their own derivation:
* central finite differences, in fp64, of the C oracle's forward (the token
  loop itself) for the scalar  L = sum(o * dO) + sum(S_T * dS_T), along a
  random direction in each input separately; for complex data the same with
  L = Re sum(conj(dO) o) + Re sum(conj(dS_T) S_T), along a real and an
  imaginary direction in each complex input (the gradient's real and
  imaginary parts);
* the closed form at beta = 0, where S_t = gamma_t S0 and o_t = gamma_t S0^T q_t;
* T = 0, where the only gradient is dS0 = dS_T.
Each mutant plants one plausible mistake in a copy of the source (a dropped
term, the wrong state, a missing factor, a flipped sign); some pin must reject
it.  CPU only.
"""
import inspect
import types

import numpy as np
import pytest

import oracle
from oracle import backward as bwd_mod

NAMES = ("q", "k", "v", "alpha", "beta", "S0")


def _inputs(seed, B=1, T=6, H=2, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.normal(size=(B, T, H, dk)), k=rng.normal(size=(B, T, H, dk)) / np.sqrt(dk),
             v=rng.normal(size=(B, T, H, dv)), alpha=rng.uniform(0.4, 0.95, size=(B, T, H)),
             beta=rng.uniform(0.2, 1.8, size=(B, T, H)), S0=rng.normal(size=(B, H, dk, dv)))
    up = dict(dO=rng.normal(size=(B, T, H, dv)), dS=rng.normal(size=(B, H, dk, dv)))
    return x, up


def _loss(x, up):
    o, S, _ = oracle.recurrent_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], threads=1)
    return float(np.sum(o * up["dO"]) + np.sum(S * up["dS"]))


def pin_finite_differences(fn):
    """<grad_X, D> equals (L(X + eps D) - L(X - eps D)) / (2 eps) for every input X."""
    for seed in (1, 2):
        x, up = _inputs(seed)
        grads = dict(zip(NAMES, fn(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], up["dO"], up["dS"])))
        rng = np.random.default_rng(100 + seed)
        for name in NAMES:
            D = rng.normal(size=x[name].shape)
            eps = 1e-6
            xp = dict(x, **{name: x[name] + eps * D})
            xm = dict(x, **{name: x[name] - eps * D})
            fd = (_loss(xp, up) - _loss(xm, up)) / (2 * eps)
            an = float(np.sum(grads[name] * D))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)


def _cinputs(seed, B=1, T=6, H=2, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    c = lambda *sh: rng.normal(size=sh) + 1j * rng.normal(size=sh)  # noqa: E731
    x = dict(q=c(B, T, H, dk), k=c(B, T, H, dk) / np.sqrt(2 * dk), v=c(B, T, H, dv),
             alpha=rng.uniform(0.4, 0.95, size=(B, T, H)), beta=rng.uniform(0.2, 1.8, size=(B, T, H)),
             S0=c(B, H, dk, dv))
    up = dict(dO=c(B, T, H, dv), dS=c(B, H, dk, dv))
    return x, up


def _closs(x, up):
    o, S, _ = oracle.recurrent_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], threads=1)
    return float(np.real(np.sum(np.conj(up["dO"]) * o) + np.sum(np.conj(up["dS"]) * S)))


def pin_finite_differences_complex(fn):
    """For complex inputs the gradient is dL/dRe + i dL/dIm: along a real direction D the loss moves by
    Re sum(conj(grad) D), along an imaginary one i D by Re sum(conj(grad) i D); the real gates as before."""
    for seed in (3, 4):
        x, up = _cinputs(seed)
        grads = dict(zip(NAMES, fn(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], up["dO"], up["dS"])))
        rng = np.random.default_rng(200 + seed)
        for name in NAMES:
            dirs = [1.0, 1j] if np.iscomplexobj(x[name]) else [1.0]
            for ph in dirs:
                D = rng.normal(size=x[name].shape) * ph
                eps = 1e-6
                fd = (_closs(dict(x, **{name: x[name] + eps * D}), up)
                      - _closs(dict(x, **{name: x[name] - eps * D}), up)) / (2 * eps)
                an = float(np.real(np.sum(np.conj(grads[name]) * D)))
                assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, ph, fd, an)


def pin_beta_zero_closed_form(fn):
    """beta = 0: S_t = gamma_t S0, so dq_t = gamma_t S0 dO_t, dS0 = sum_t gamma_t q_t dO_t^T + gamma_T dS_T,
    dalpha_t = sum_{s >= t} (gamma_s / alpha_t) q_s^T S0 dO_s + (gamma_T / alpha_t) <S0, dS_T>,
    dv = dk = 0 and dbeta_t = (D^T k_t) . (v_t - alpha_t S_{t-1}^T k_t)."""
    x, up = _inputs(7, T=5, H=1)
    x["beta"][:] = 0.0
    dq, dk, dv, da, db, dS0 = fn(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], up["dO"], up["dS"])
    a = x["alpha"][0, :, 0]
    gam = np.cumprod(a)
    S0 = x["S0"][0, 0]
    q, dO = x["q"][0, :, 0], up["dO"][0, :, 0]
    T = len(a)
    for t in range(T):
        assert np.allclose(dq[0, t, 0], gam[t] * S0 @ dO[t], atol=1e-13)
    ref = sum(gam[t] * np.outer(q[t], dO[t]) for t in range(T)) + gam[-1] * up["dS"][0, 0]
    assert np.allclose(dS0[0, 0], ref, atol=1e-13)
    assert not dk.any() and not dv.any()
    for t in range(T):
        ref_a = sum(gam[s] / a[t] * q[s] @ S0 @ dO[s] for s in range(t, T)) + gam[-1] / a[t] * np.sum(S0 * up["dS"][0, 0])
        assert abs(da[0, t, 0] - ref_a) <= 1e-12 * max(1.0, abs(ref_a))
    # dbeta_t from its definition: D_t = gamma-weighted future readouts plus dS_T, S_{t-1} = gamma_{t-1} S0
    k, v = x["k"][0, :, 0], x["v"][0, :, 0]
    for t in range(T):
        D = sum(gam[s] / gam[t] * np.outer(q[s], dO[s]) for s in range(t, T)) + gam[-1] / gam[t] * up["dS"][0, 0]
        Sp = (gam[t - 1] if t > 0 else 1.0) * S0
        ref_b = (D.T @ k[t]) @ (v[t] - a[t] * (Sp.T @ k[t]))
        assert abs(db[0, t, 0] - ref_b) <= 1e-12 * max(1.0, abs(ref_b))


def pin_empty_sequence(fn):
    """T = 0: dS0 = dS_T and every per-token gradient is empty."""
    x, up = _inputs(3, T=0)
    out = fn(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], up["dO"], up["dS"])
    assert all(g.size == 0 for g in out[:5])
    assert np.array_equal(out[5], up["dS"])


PINS = [pin_finite_differences, pin_finite_differences_complex, pin_beta_zero_closed_form, pin_empty_sequence]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_pin(pin):
    pin(bwd_mod.recurrent_bwd)


MUTATIONS = {
    "readout_gradient_dropped": ("D = G + qt[..., :, None] * dot[..., None, :]", "D = G + 0 * qt[..., :, None]"),
    "dq_from_previous_state": ('dq[:, t] = np.einsum("bhij,bhj->bhi", St, cj(dot))',
                               'dq[:, t] = np.einsum("bhij,bhj->bhi", Sp, cj(dot))'),
    "dalpha_from_new_state": ("np.sum(cj(D) * (Sp - b", "np.sum(cj(D) * (St - b"),
    "carry_without_alpha": ("G = a[..., None, None] * (D", "G = (D"),
    "carry_without_rank_one": ("G = a[..., None, None] * (D - b[..., None, None] * kt[..., :, None] * w[..., None, :])",
                               "G = a[..., None, None] * D"),
    "dk_second_term_sign": ('- (a * b)[..., None] * np.einsum("bhij,bhj->bhi", Sp, cj(w))',
                            '+ (a * b)[..., None] * np.einsum("bhij,bhj->bhi", Sp, cj(w))'),
    "dbeta_without_alpha": ("(vt - a[..., None] * u)", "(vt - u)"),
    "dv_without_beta": ("dv_[:, t] = b[..., None] * w", "dv_[:, t] = w"),
    "w_from_carry_only": ('w = np.einsum("bhij,bhi->bhj", D, cj(kt))', 'w = np.einsum("bhij,bhi->bhj", G, cj(kt))'),
    "u_from_new_state": ('u = np.einsum("bhij,bhi->bhj", Sp, cj(kt))', 'u = np.einsum("bhij,bhi->bhj", St, cj(kt))'),
    "y_without_beta": ("y = b[..., None] * vt", "y = vt"),
    "dk_transposed_state": ('- (a * b)[..., None] * np.einsum("bhij,bhj->bhi", Sp, cj(w))',
                            '- (a * b)[..., None] * np.einsum("bhji,bhj->bhi", Sp[..., :, :dv], cj(w)[..., :dk])'),
    # complex only: a conjugation dropped or added
    "forward_readout_unconjugated": ('u = np.einsum("bhij,bhi->bhj", S, cj(kt))',
                                     'u = np.einsum("bhij,bhi->bhj", S, kt)'),
    "w_unconjugated_key": ('w = np.einsum("bhij,bhi->bhj", D, cj(kt))', 'w = np.einsum("bhij,bhi->bhj", D, kt)'),
    "dq_unconjugated_upstream": ('St, cj(dot))', 'St, dot)'),
    "dk_unconjugated_y": ('np.einsum("bhij,bhj->bhi", D, cj(y))', 'np.einsum("bhij,bhj->bhi", D, y)'),
    "dk_unconjugated_w": ('np.einsum("bhij,bhj->bhi", Sp, cj(w)))', 'np.einsum("bhij,bhj->bhi", Sp, w))'),
    "dbeta_unconjugated_w": ("np.real(np.sum(cj(w) *", "np.real(np.sum(w *"),
    "dalpha_unconjugated_D": ("np.real(np.sum(cj(D) *", "np.real(np.sum(D *"),
    "carry_conjugated_w": ("kt[..., :, None] * w[..., None, :])", "kt[..., :, None] * cj(w)[..., None, :])"),
}


def _mutant(old, new):
    src = inspect.getsource(bwd_mod)
    assert src.count(old) == 1, old
    ns = types.ModuleType("mutant")
    exec(compile(src.replace(old, new), "mutant", "exec"), ns.__dict__)
    return ns.recurrent_bwd


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_mutant_caught(name):
    fn = _mutant(*MUTATIONS[name])
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(fn)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every backward pin"
