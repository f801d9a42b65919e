"""Pins for the per-output-channel decay oracle (oracle/channel_decay.py), and mutants they must catch.

The rule (DeltaPhase README, section 2, the gated-decay variant of LaplacePhaseCore; section 5 for the
decay on the output rows): per value channel j, e = v[j] - kread^T s_j from the undecayed state, then
s_j <- r[j] s_j + beta k e, o[j] = qread^T s_j.

* Hand-worked cases (tests/golden/channel_decay_handworked.json): a real 2 x 2 state over three tokens and
  a complex 1 x 1 state over two, derived by hand from the page's formulas.
* r = 1 on every channel: the rule is the plain delta rule, so it must equal the C oracle at alpha = 1.
* Each value column alone is an affine recurrence s <- (r I - beta k kread^T) s + beta k v, which is the
  C oracle's gated rule alpha (I - beta' k kread^T) s + beta' k v' with alpha = r, beta' = beta / r and
  v' = r v.  That identity pins every term for general r against the independent C code.
* beta = 0: s_j(t) = (prod_{u<=t} r_u[j]) s_j(0) in closed form.
* The chunkwise scan of section 5 (one triangular solve per value channel) agrees with the token loop for
  chunk lengths 1, 3, 16 and 64, including a ragged tail.
* Complex data with zero imaginary parts equals the real rule; conjugating every complex input conjugates
  every output.
Shapes use dk != dv, so a transposed operand fails loudly.  CPU only.
"""
import inspect
import json
import os
import types

import numpy as np
import pytest

import oracle
from oracle import channel_decay as cd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "channel_decay_handworked.json")


def _inputs(seed, B=2, T=9, H=2, dk=5, dv=3, cplx=False):
    rng = np.random.default_rng(seed)
    if cplx:
        q = rng.normal(size=(B, T, H, dk)) + 1j * rng.normal(size=(B, T, H, dk))
        # Laplace keys: modulus e^{sigma} <= 1 and a phase, per element
        k = np.exp(-rng.uniform(0.0, 0.5, size=(B, T, H, dk)) + 1j * rng.uniform(0, 2 * np.pi, size=(B, T, H, dk)))
        k /= np.sqrt(dk)
        v = rng.normal(size=(B, T, H, dv)) + 1j * rng.normal(size=(B, T, H, dv))
        S0 = rng.normal(size=(B, H, dk, dv)) + 1j * rng.normal(size=(B, H, dk, dv))
    else:
        q = rng.normal(size=(B, T, H, dk))
        k = rng.normal(size=(B, T, H, dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.normal(size=(B, T, H, dv))
        S0 = rng.normal(size=(B, H, dk, dv))
    return dict(q=q, k=k, v=v, r=rng.uniform(0.3, 1.0, size=(B, T, H, dv)),
                beta=rng.uniform(0.1, 1.9, size=(B, T, H)), S0=S0)


def _cx(a):
    a = np.asarray(a, dtype=np.float64)
    return a[..., 0] + 1j * a[..., 1]


def pin_handworked(fn):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        conv = _cx if c["dtype"] == "complex" else (lambda a: np.asarray(a, dtype=np.float64))
        q, k, v = (conv(c[x])[None, :, None] for x in ("q", "k", "v"))
        r = np.asarray(c["r"], dtype=np.float64)[None, :, None]
        beta = np.asarray(c["beta"], dtype=np.float64)[None, :, None]
        S0 = conv(c["S0"])[None, None]
        o, S = fn(q, k, v, r, beta, S0)
        assert np.allclose(o[0, :, 0], conv(c["o"]), atol=1e-12), (c["name"], o[0, :, 0])
        assert np.allclose(S[0, 0], conv(c["S_final"]), atol=1e-12), (c["name"], S[0, 0])


def pin_unit_decay_is_plain_delta_rule(fn):
    for cplx in (False, True):
        x = _inputs(1, cplx=cplx)
        r = np.ones_like(x["r"])
        o, S = fn(x["q"], x["k"], x["v"], r, x["beta"], x["S0"])
        o_ref, S_ref, _ = oracle.recurrent_fwd(x["q"], x["k"], x["v"], np.ones_like(x["beta"]), x["beta"], x["S0"],
                                               threads=1)
        assert np.allclose(o, o_ref, atol=1e-12) and np.allclose(S, S_ref, atol=1e-12), cplx


def pin_column_affine_identity(fn):
    for cplx in (False, True):
        x = _inputs(2, cplx=cplx)
        o, S = fn(x["q"], x["k"], x["v"], x["r"], x["beta"], x["S0"])
        for j in range(x["v"].shape[-1]):
            rj = x["r"][..., j]
            o_j, S_j, _ = oracle.recurrent_fwd(x["q"], x["k"], x["v"][..., j:j + 1] * rj[..., None], rj,
                                               x["beta"] / rj, x["S0"][..., j:j + 1], threads=1)
            assert np.allclose(o[..., j:j + 1], o_j, atol=1e-11), (cplx, j)
            assert np.allclose(S[..., j:j + 1], S_j, atol=1e-11), (cplx, j)


def pin_beta_zero_closed_form(fn):
    x = _inputs(3)
    x["beta"][:] = 0.0
    o, S = fn(x["q"], x["k"], x["v"], x["r"], x["beta"], x["S0"])
    cum = np.cumprod(x["r"], axis=1)  # [B, T, H, dv]
    for t in range(x["q"].shape[1]):
        St = x["S0"] * cum[:, t][:, :, None, :]
        assert np.allclose(o[:, t], np.einsum("bhij,bhi->bhj", St, x["q"][:, t]), atol=1e-12)
    assert np.allclose(S, x["S0"] * cum[:, -1][:, :, None, :], atol=1e-12)


def pin_complex_consistency(fn):
    x = _inputs(4)
    o, S = fn(x["q"], x["k"], x["v"], x["r"], x["beta"], x["S0"])
    c = {n: (x[n] + 0j if n in ("q", "k", "v", "S0") else x[n]) for n in x}
    oc, Sc = fn(c["q"], c["k"], c["v"], c["r"], c["beta"], c["S0"])
    assert np.iscomplexobj(oc) and np.allclose(oc, o, atol=1e-12) and np.allclose(Sc, S, atol=1e-12)
    y = _inputs(5, cplx=True)
    o1, S1 = fn(y["q"], y["k"], y["v"], y["r"], y["beta"], y["S0"])
    o2, S2 = fn(np.conj(y["q"]), np.conj(y["k"]), np.conj(y["v"]), y["r"], y["beta"], np.conj(y["S0"]))
    assert np.allclose(o2, np.conj(o1), atol=1e-12) and np.allclose(S2, np.conj(S1), atol=1e-12)


PINS = [pin_handworked, pin_unit_decay_is_plain_delta_rule, pin_column_affine_identity, pin_beta_zero_closed_form,
        pin_complex_consistency]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_channel_decay_pin(pin):
    pin(cd.channel_decay_fwd)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_channel_decay_chunked_pin(pin):
    pin(lambda *a: cd.channel_decay_chunked(*a, chunk=4))


@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
@pytest.mark.parametrize("cplx", [False, True])
def test_chunked_scan_matches_token_loop(chunk, cplx):
    x = _inputs(6, B=1, T=70, H=2, dk=6, dv=4, cplx=cplx)
    o1, S1 = cd.channel_decay_fwd(x["q"], x["k"], x["v"], x["r"], x["beta"], x["S0"])
    o2, S2 = cd.channel_decay_chunked(x["q"], x["k"], x["v"], x["r"], x["beta"], x["S0"], chunk=chunk)
    assert np.abs(o1 - o2).max() <= 1e-11 * max(1.0, np.abs(o1).max())
    assert np.abs(S1 - S2).max() <= 1e-11 * max(1.0, np.abs(S1).max())


# Textual mutations of the token loop; every one must fail some pin.  "error_from_decayed_state" is the
# Gated-DeltaNet ordering (decay applied before the read), which the page's LaplacePhaseCore does not use.
MUTATIONS = {
    "decay_dropped": ("S = S * r[:, t][..., None, :] +", "S = S * 1.0 +"),
    "decay_on_rows": ("S = S * r[:, t][..., None, :] +", "S = S * r[:, t][..., :, None] +"),
    "error_from_decayed_state": ('read = np.einsum("bhij,bhi->bhj", S, kread)',
                                 'read = np.einsum("bhij,bhi->bhj", S * r[:, t][..., None, :], kread)'),
    "decay_on_write_too": ("S = S * r[:, t][..., None, :] + kt[..., :, None] * (b * err)[..., None, :]",
                           "S = (S + kt[..., :, None] * (b * err)[..., None, :]) * r[:, t][..., None, :]"),
    "beta_dropped_on_write": ("kt[..., :, None] * (b * err)[..., None, :]", "kt[..., :, None] * err[..., None, :]"),
    "output_from_key": ('o[:, t] = np.einsum("bhij,bhi->bhj", S, qread)', 'o[:, t] = np.einsum("bhij,bhi->bhj", S, kread)'),
    "readout_with_query": ('read = np.einsum("bhij,bhi->bhj", S, kread)', 'read = np.einsum("bhij,bhi->bhj", S, qread)'),
    "read_key_not_conjugated": ("kread = np.conj(kt) if cplx else kt", "kread = kt"),
    "write_key_conjugated": ("S = S * r[:, t][..., None, :] + kt[..., :, None]", "S = S * r[:, t][..., None, :] + np.conj(kt)[..., :, None]"),
    "output_before_update": ('        o[:, t] = np.einsum("bhij,bhi->bhj", S, qread)\n', ""),
}


def _mutant(old, new):
    src = inspect.getsource(cd)
    assert src.count(old) == 1, old
    src = src.replace(old, new)
    if old.startswith("        o[:, t]"):  # move the read of o in front of the update
        src = src.replace("        S = S * r[:, t]", '        o[:, t] = np.einsum("bhij,bhi->bhj", S, qread)\n        S = S * r[:, t]')
    ns = types.ModuleType("mutant")
    exec(compile(src, "mutant", "exec"), ns.__dict__)
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
