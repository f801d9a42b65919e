"""Single-token decode step on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from gdn_inputs import WORKLOADS, gen_chunk, gen_decode, gen_decode_workload
from gpu_util import ELEM_TOL, TOL, chain_rel_errors, down, note, run_chunk, torch_dev, up

pytestmark = pytest.mark.gpu


def run_steps(inp, dtype, steps=None):
    """Apply the decode entry point step by step; returns outputs [steps, N, dv] and states after each step."""
    import torch
    import linear_attention_sequence_gated_amd as gdn
    S = up(inp["S"], "f32")
    nsteps = inp["q"].shape[0] if steps is None else steps
    outs, states = [], []
    for t in range(nsteps):
        o = gdn.recurrent_step(up(inp["q"][t], dtype), up(inp["k"][t], dtype), up(inp["v"][t], dtype),
                               up(inp["alpha"][t], "f32"), up(inp["beta"][t], "f32"), S)
        torch.cuda.synchronize()
        outs.append(down(o))
        states.append(down(S))
    return outs, states


def check_steps(name, inp, dtype, outs, states):
    """Every state after every step: relative norm error of o and S per state, and the elementwise
    max|x - ref| / max|ref| per state (bounds as for the chunk forward)."""
    St = inp["S"].astype(np.complex128 if dtype == "c64" else np.float64)
    worst = dict(o=0.0, S=0.0, elem_o=0.0, elem_S=0.0)
    for t in range(len(outs)):
        o_ref, St = oracle.recurrent_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["alpha"][t], inp["beta"][t], St)
        assert np.isfinite(outs[t]).all() and np.isfinite(states[t]).all(), (name, t)
        N = len(St)
        do, dS = outs[t] - o_ref, (states[t] - St).reshape(N, -1)
        Sr = St.reshape(N, -1)
        worst["o"] = max(worst["o"], (np.linalg.norm(do, axis=1) / np.maximum(np.linalg.norm(o_ref, axis=1), 1e-30)).max())
        worst["S"] = max(worst["S"], (np.linalg.norm(dS, axis=1) / np.linalg.norm(Sr, axis=1)).max())
        worst["elem_o"] = max(worst["elem_o"], (np.abs(do).max(axis=1) / np.maximum(np.abs(o_ref).max(axis=1), 1e-30)).max())
        worst["elem_S"] = max(worst["elem_S"], (np.abs(dS).max(axis=1) / np.abs(Sr).max(axis=1)).max())
    print(f"[parity] {name}: max state-step rel err o={worst['o']:.3e} S={worst['S']:.3e} "
          f"elem o={worst['elem_o']:.3e} S={worst['elem_S']:.3e} (tol {TOL[dtype]:g} / {ELEM_TOL[dtype]:g})", flush=True)
    assert worst["o"] <= TOL[dtype] and worst["S"] <= TOL[dtype], (name, worst)
    assert worst["elem_o"] <= ELEM_TOL[dtype] and worst["elem_S"] <= ELEM_TOL[dtype], (name, worst)


@pytest.mark.parametrize("dtype,d,N", [("bf16", 64, 300), ("bf16", 128, 37), ("f32", 64, 129), ("f32", 128, 5),
                                       ("c64", 32, 77)])
def test_decode_small(dtype, d, N):
    torch_dev()
    inp = gen_decode(N, d, d, 6, dtype=dtype, seed=9 + N, beta_scale=2.0 if dtype == "c64" else 1.0)
    note(f"decode dtype={dtype} d={d} N={N}")
    outs, states = run_steps(inp, dtype)
    check_steps(f"decode_{dtype}_{d}", inp, dtype, outs, states)


# Two rounds per workgroup start at 1024 groups of 256 / TPS states (4 states per group for d = 64 and
# complex d = 32, one for d = 128); each N leaves the last workgroup's second round partly or wholly past N.
@pytest.mark.parametrize("dtype,d,N", [("bf16", 64, 4099), ("f32", 64, 4101), ("f32", 128, 1027),
                                       ("c64", 32, 4097)])
def test_decode_two_rounds_ragged(dtype, d, N):
    """Grids large enough for two states per wave, with a last workgroup whose second round is past N
    (it loads state N - 1 and must store nothing): every state compared, including the last one."""
    torch_dev()
    inp = gen_decode(N, d, d, 3, dtype=dtype, seed=31 + N, beta_scale=2.0 if dtype == "c64" else 1.0)
    note(f"decode two rounds dtype={dtype} d={d} N={N}")
    outs, states = run_steps(inp, dtype)
    check_steps(f"decode_rounds_{dtype}_{d}_{N}", inp, dtype, outs, states)


def test_decode_full_workload():
    """4096 states x 64 steps, every state and step compared."""
    torch_dev()
    w = WORKLOADS["decode_4096x64"]
    inp = gen_decode_workload(w)
    note("decode full workload 4096x64")
    outs, states = run_steps(inp, w.dtype)
    check_steps("decode_4096x64", inp, w.dtype, outs, states)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("c64", 32)])
def test_decode_steps_match_chunk_forward(dtype, d):
    """T decode steps on the GPU equal the GPU chunked forward over the same tokens."""
    import torch
    torch_dev()
    B, T, H = 2, 70, 3
    inp = gen_chunk(B, T, H, d, d, dtype=dtype, seed=81, s0_var=0.1, beta_scale=2.0 if dtype == "c64" else 1.0)
    note(f"decode vs chunk dtype={dtype} d={d}")
    o, S = run_chunk(inp, dtype)
    N = B * H
    dec = dict(S=inp["S0"].reshape(N, d, d),
               q=np.stack([inp["q"][:, t].reshape(N, d) for t in range(T)]),
               k=np.stack([inp["k"][:, t].reshape(N, d) for t in range(T)]),
               v=np.stack([inp["v"][:, t].reshape(N, d) for t in range(T)]),
               alpha=np.stack([inp["alpha"][:, t].reshape(N) for t in range(T)]),
               beta=np.stack([inp["beta"][:, t].reshape(N) for t in range(T)]))
    outs, states = run_steps(dec, dtype)
    o_dec = np.stack(outs, axis=1).reshape(B, H, T, d).transpose(0, 2, 1, 3)
    S_dec = states[-1].reshape(B, H, d, d)
    eo, es = chain_rel_errors(o_dec, S_dec, o, S)
    print(f"[parity] decode-vs-chunk {dtype}: o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_deterministic():
    torch_dev()
    inp = gen_decode(512, 64, 64, 2, dtype="bf16", seed=91)
    note("decode determinism")
    o1, s1 = run_steps(inp, "bf16")
    o2, s2 = run_steps(inp, "bf16")
    assert all(np.array_equal(a, b) for a, b in zip(o1, o2)) and all(np.array_equal(a, b) for a, b in zip(s1, s2))
