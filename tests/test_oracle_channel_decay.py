"""Pins for the per-output-channel decay oracle (oracle/channel_decay.py), and mutants they must catch.

* r_t = alpha_t on every channel must equal the C oracle's scalar-gated token loop (an independent
  implementation of the same rule).
* Each value column alone equals the C oracle run on that column with alpha = that column's decay
  (columns evolve on their own).
* beta = 0: S_T = S0 diag(prod_t r_t) and o_t = (S0 diag(prod_{s <= t} r_s))^T q_t in closed form.
Shapes use dk != dv, so a transposed operand fails loudly.  CPU only.
"""
import inspect
import types

import numpy as np
import pytest

import oracle
from oracle import channel_decay as cd


def _inputs(seed, B=2, T=9, H=2, dk=5, dv=3):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=q, k=k, v=rng.normal(size=(B, T, H, dv)), r=rng.uniform(0.3, 1.0, size=(B, T, H, dv)),
                beta=rng.uniform(0.1, 1.9, size=(B, T, H)), S0=rng.normal(size=(B, H, dk, dv)))


def pin_scalar_gate_reduction(fn):
    x = _inputs(1)
    alpha = x["r"][..., 0]
    r = np.repeat(alpha[..., None], x["v"].shape[-1], axis=-1)
    o, S = fn(x["q"], x["k"], x["v"], r, x["beta"], x["S0"])
    o_ref, S_ref, _ = oracle.recurrent_fwd(x["q"], x["k"], x["v"], alpha, x["beta"], x["S0"], threads=1)
    assert np.allclose(o, o_ref, atol=1e-12) and np.allclose(S, S_ref, atol=1e-12)


def pin_columns_independent(fn):
    x = _inputs(2)
    o, S = fn(x["q"], x["k"], x["v"], x["r"], x["beta"], x["S0"])
    for j in range(x["v"].shape[-1]):
        o_j, S_j, _ = oracle.recurrent_fwd(x["q"], x["k"], x["v"][..., j:j + 1], x["r"][..., j], x["beta"],
                                           x["S0"][..., j:j + 1], threads=1)
        assert np.allclose(o[..., j:j + 1], o_j, atol=1e-12) and np.allclose(S[..., j:j + 1], S_j, atol=1e-12)


def pin_beta_zero_closed_form(fn):
    x = _inputs(3)
    x["beta"][:] = 0.0
    o, S = fn(x["q"], x["k"], x["v"], x["r"], x["beta"], x["S0"])
    cum = np.cumprod(x["r"], axis=1)  # [B, T, H, dv]
    for t in range(x["q"].shape[1]):
        St = x["S0"] * cum[:, t][:, :, None, :]
        assert np.allclose(o[:, t], np.einsum("bhij,bhi->bhj", St, x["q"][:, t]), atol=1e-12)
    assert np.allclose(S, x["S0"] * cum[:, -1][:, :, None, :], atol=1e-12)


PINS = [pin_scalar_gate_reduction, pin_columns_independent, pin_beta_zero_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_channel_decay_pin(pin):
    pin(cd.channel_decay_fwd)


MUTATIONS = {
    "decay_dropped": ("* r[:, t][..., None, :]", "* 1.0"),
    "decay_on_rows": ("* r[:, t][..., None, :]", "* r[:, t][..., :, None]"),
    "readout_not_decayed": ("S = (S - b * kt[..., :, None] * u[..., None, :]) * r[:, t][..., None, :]",
                            "S = S * r[:, t][..., None, :] - b * kt[..., :, None] * u[..., None, :]"),
    "beta_dropped_on_write": ("+ b * kt[..., :, None] * v[:, t][..., None, :]", "+ kt[..., :, None] * v[:, t][..., None, :]"),
    "output_from_query_key": ('o[:, t] = np.einsum("bhij,bhi->bhj", S, q[:, t])', 'o[:, t] = np.einsum("bhij,bhi->bhj", S, kt)'),
    "readout_with_query": ('u = np.einsum("bhij,bhi->bhj", S, kt)', 'u = np.einsum("bhij,bhi->bhj", S, q[:, t])'),
}


def _mutant(old, new):
    src = inspect.getsource(cd)
    assert src.count(old) == 1, old
    ns = types.ModuleType("mutant")
    exec(compile(src.replace(old, new), "mutant", "exec"), ns.__dict__)
    return ns.channel_decay_fwd


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_channel_decay_mutant_caught(name):
    fn = _mutant(*MUTATIONS[name])
    caught = []
    for pin in PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every channel-decay pin"
