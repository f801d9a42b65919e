"""Every plausible mistake planted in the C oracle must be caught by at least one pin.

Each mutant is a textual edit of ``oracle/gdn_oracle.c`` compiled into a
temporary library on the CPU; the pins of ``oracle_pins.py`` are then run
against it.  This guards the pins themselves: a pin set that lets a dropped
term, a wrong sign, a wrong index or a transposed operand through would fail
here.  CPU only.
"""
import os
import tempfile

import pytest

import oracle
from oracle_pins import all_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

_REAL_UPDATE = "S[(size_t)i * dv + j] = alpha * (s - beta * k[i] * r[j]) + beta * k[i] * v[j];"
_CPLX_READ = "acc += conj(k[i]) * S[(size_t)i * dv + j];"

# (name, old text, new text, occurrence index to edit or None for all)
MUTANTS = [
    ("alpha_not_on_erase", "alpha * (s - beta * k[i] * r[j])", "alpha * s - beta * k[i] * r[j]", None),
    ("alpha_on_write", "+ beta * k[i] * v[j];", "+ alpha * beta * k[i] * v[j];", None),
    ("erase_sign", "(s - beta * k[i] * r[j])", "(s + beta * k[i] * r[j])", None),
    ("beta_squared_write", "+ beta * k[i] * v[j];", "+ beta * beta * k[i] * v[j];", None),
    ("no_beta_on_erase", "(s - beta * k[i] * r[j])", "(s - k[i] * r[j])", None),
    ("read_with_query", "acc += k[i] * S[(size_t)i * dv + j];", "acc += q[i] * S[(size_t)i * dv + j];", None),
    ("readout_transposed", "acc += S[(size_t)i * dv + j] * q[i];", "acc += S[(size_t)(j % dk) * dv + (i % dv)] * q[i];", None),
    ("outer_product_transposed", _REAL_UPDATE,
     "S[(size_t)i * dv + j] = alpha * (s - beta * k[j % dk] * r[i % dv]) + beta * k[i] * v[j];", None),
    ("initial_state_ignored", "if (S0) memcpy", "if (0) memcpy", None),
    ("alpha_previous_token", "alpha[tok], beta[tok]", "alpha[t > 0 ? tok - H : tok], beta[tok]", None),
    ("beta_previous_token", "alpha[tok], beta[tok]", "alpha[tok], beta[t > 0 ? tok - H : tok]", None),
    ("token_layout_bh_swapped", "size_t tok = ((size_t)b * T + t) * H + h;",
     "size_t tok = ((size_t)(c % B) * T + t) * H + (int)(c / B);", None),
    ("value_from_key_row", "+ beta * k[i] * v[j];", "+ beta * k[i] * v[(j + 1) % dv];", None),
    ("complex_read_not_conj", _CPLX_READ, "acc += k[i] * S[(size_t)i * dv + j];", None),
    ("complex_query_not_conj", "* conj(q[i]);", "* q[i];", None),
    ("complex_write_conj", "cplx s = S[(size_t)i * dv + j];\n            S[(size_t)i * dv + j] = alpha * (s - beta * k[i] * r[j]) + beta * k[i] * v[j];",
     "cplx s = S[(size_t)i * dv + j];\n            S[(size_t)i * dv + j] = alpha * (s - beta * k[i] * r[j]) + beta * conj(k[i]) * v[j];", None),
    ("complex_erase_conj", "cplx s = S[(size_t)i * dv + j];\n            S[(size_t)i * dv + j] = alpha * (s - beta * k[i] * r[j])",
     "cplx s = S[(size_t)i * dv + j];\n            S[(size_t)i * dv + j] = alpha * (s - beta * conj(k[i]) * r[j])", None),
    ("step_gates_swapped", "alpha[n], beta[n], o + (size_t)n * dv", "beta[n], alpha[n], o + (size_t)n * dv", None),
    ("step_state_stride", "step_real(S + (size_t)n * dk * dv", "step_real(S + (size_t)n * dk", None),
]


def _output_before_update(src: str) -> str:
    """Read o from the state before the write (o_t = S_{t-1}^T q) in the real step."""
    start = src.index("static void step_real")
    end = src.index("static void step_cplx")
    body = src[start:end]
    upd_start = body.index("    /* S <- alpha")
    out_start = body.index("    /* o = S^T q")
    out_end = body.rindex("}")
    new_body = body[:upd_start] + body[out_start:out_end] + body[upd_start:out_start] + body[out_end:]
    return src[:start] + new_body + src[end:]


def _apply(src, old, new, which):
    assert old in src, f"mutation anchor not found: {old!r}"
    if which is None:
        return src.replace(old, new)
    parts = src.split(old)
    return old.join(parts[: which + 1]) + new + old.join(parts[which + 1:])


def _mutants():
    src = open(SRC).read()
    out = [(name, _apply(src, old, new, which)) for name, old, new, which in MUTANTS]
    out.append(("output_before_update", _output_before_update(src)))
    return out


@pytest.mark.parametrize("name,msrc", _mutants(), ids=[m[0] for m in _mutants()])
def test_mutant_is_caught(name, msrc, tmp_path):
    csrc = tmp_path / "mutant.c"
    csrc.write_text(msrc)
    so = tmp_path / "libmutant.so"
    oracle.compile_library(str(csrc), str(so))
    lib = oracle.load_library(str(so))
    caught = []
    for pname, pin in all_pins():
        try:
            pin(lib)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pname)
    assert caught, f"mutant {name} passed every pin"
