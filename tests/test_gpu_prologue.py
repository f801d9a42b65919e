"""Prologue entry point on the GPU (through the C ABI) against the fp64 oracle.

The library takes raw q, k and the gate logits: bf16 d64 normalises inside the
single-launch kernel's arithmetic, bf16 d128 (and long d64 sequences) in both
launches of the two-launch path, fp32 d64 and complex64 d32 in a pass over the
rows ahead of the forward.  The oracle applies the same transforms in fp64 to
the same stored values (oracle/prologue.py) and runs the token loop.
"""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, gen_raw_layer, gen_workload
from gpu_util import TOL, assert_close, chain_rel_errors, down, note, torch_dev, up
from oracle.prologue import prologue_fwd

pytestmark = pytest.mark.gpu


def run_prologue(inp, beta_scale, S0=True, S_final_alias=False, dtype="bf16"):
    import torch
    import linear_attention_sequence_gated_amd as gdn
    q, k, v = up(inp["q"], dtype), up(inp["k"], dtype), up(inp["v"], dtype)
    a, b = up(inp["a_logit"], "f32"), up(inp["b_logit"], "f32")
    s0 = up(inp["S0"], "f32") if (S0 and inp.get("S0") is not None) else None
    if S_final_alias and s0 is not None:
        o, S = gdn.chunk_fwd_prologue(q, k, v, a, b, beta_scale, s0, S_final=s0)
    else:
        o, S = gdn.chunk_fwd_prologue(q, k, v, a, b, beta_scale, s0)
    torch.cuda.synchronize()
    return down(o), down(S)


def oracle_prologue(inp, beta_scale):
    return prologue_fwd(inp["q"], inp["k"], inp["v"], inp["a_logit"], inp["b_logit"], beta_scale, inp.get("S0"))


@pytest.mark.parametrize("beta_scale", [1.0, 2.0])
@pytest.mark.parametrize("B,T,H,s0", [(2, 300, 3, None), (1, 129, 2, 0.01), (2, 250, 1, 0.1)])
def test_prologue_small(B, T, H, s0, beta_scale):
    torch_dev()
    inp = gen_raw_layer(B, T, H, 64, seed=17 + T + H, s0_var=s0)
    note(f"prologue B{B} T{T} H{H} s0={s0} beta_scale={beta_scale}")
    o, S = run_prologue(inp, beta_scale)
    o_ref, S_ref = oracle_prologue(inp, beta_scale)
    assert_close(f"prologue_{B}_{T}_{H}_{beta_scale}", "bf16", o, S, o_ref, S_ref)


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 191, 385])
def test_prologue_lengths(T):
    torch_dev()
    inp = gen_raw_layer(2, T, 2, 64, seed=5 + T, s0_var=0.1)
    note(f"prologue lengths T={T}")
    o, S = run_prologue(inp, 2.0)
    if T == 0:  # nothing to process: S_final is S0
        assert np.array_equal(S, inp["S0"])
        return
    o_ref, S_ref = oracle_prologue(inp, 2.0)
    assert_close(f"prologue_len{T}", "bf16", o, S, o_ref, S_ref)


def test_prologue_zero_rows_and_in_place_state():
    """Rows of q or k that are exactly zero stay zero (no division by zero); S_final may alias S0."""
    torch_dev()
    inp = gen_raw_layer(1, 200, 3, 64, seed=23, s0_var=0.1)
    inp["k"][0, 5, 1] = 0.0
    inp["q"][0, 77, 2] = 0.0
    inp["k"][0, 130:140, 0] = 0.0
    note("prologue zero rows, aliased state")
    o, S = run_prologue(inp, 1.0, S_final_alias=True)
    o_ref, S_ref = oracle_prologue(inp, 1.0)
    assert_close("prologue_zero_rows", "bf16", o, S, o_ref, S_ref)


def test_prologue_row_rescaling():
    """Scaling raw q and k rows by powers of two (exact in bf16 and in every fp32 step of the
    normalisation) leaves the outputs unchanged to fp32 rounding."""
    torch_dev()
    inp = gen_raw_layer(2, 190, 2, 64, seed=29, s0_var=0.1)
    rng = np.random.default_rng(1)
    sc = dict(inp)
    for key in ("q", "k"):
        f = (2.0 ** rng.integers(-3, 4, size=inp[key].shape[:3] + (1,))).astype(np.float32)
        sc[key] = inp[key] * f
    note("prologue row rescaling")
    o1, S1 = run_prologue(inp, 2.0)
    o2, S2 = run_prologue(sc, 2.0)
    eo, es = chain_rel_errors(o2, S2, o1, S1)
    print(f"[parity] prologue rescaling: o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 1e-5 and es <= 1e-5


def test_prologue_full_size_all_chains():
    """The 8 x 2048 x 12 d64 layer from raw inputs, as the benchmark runs it; every chain vs the oracle."""
    torch_dev()
    w = WORKLOADS["sykra_layer_bf16_prologue"]
    inp = gen_workload(w)
    note("prologue full size sykra_layer_bf16_prologue")
    o, S = run_prologue(inp, 1.0)
    o_ref, S_ref = oracle_prologue(inp, 1.0)
    assert_close("prologue_full", "bf16", o, S, o_ref, S_ref)


def test_prologue_saturated_logits():
    """Logits far in the tails: alpha ~ e^-40 (state wiped) or ~ 1, beta ~ 0 or ~ beta_scale; random tokens of
    the sequence take each extreme, the rest stay as drawn."""
    torch_dev()
    inp = gen_raw_layer(2, 260, 2, 64, seed=41, s0_var=0.1)
    rng = np.random.default_rng(4)
    pick = rng.random(inp["a_logit"].shape)
    inp["a_logit"] = np.where(pick < 0.1, 40.0, np.where(pick < 0.3, -40.0, inp["a_logit"])).astype(np.float32)
    pick = rng.random(inp["b_logit"].shape)
    inp["b_logit"] = np.where(pick < 0.15, 40.0, np.where(pick < 0.3, -40.0, inp["b_logit"])).astype(np.float32)
    note("prologue saturated logits")
    o, S = run_prologue(inp, 2.0)
    o_ref, S_ref = oracle_prologue(inp, 2.0)
    assert_close("prologue_saturated", "bf16", o, S, o_ref, S_ref)


# Every other supported shape: bf16 d128 (two-launch path, normalised in both launches), fp32 d64 and
# complex64 d32 (row pass, then the plain forward).
DTYPES = [("bf16", 128), ("f32", 64), ("c64", 32)]


@pytest.mark.parametrize("dtype,d", DTYPES)
@pytest.mark.parametrize("beta_scale", [1.0, 2.0])
@pytest.mark.parametrize("B,T,H,s0", [(2, 300, 3, None), (1, 129, 2, 0.01)])
def test_prologue_dtypes_small(dtype, d, B, T, H, s0, beta_scale):
    torch_dev()
    inp = gen_raw_layer(B, T, H, d, seed=31 + T + H + d, s0_var=s0, dtype=dtype)
    note(f"prologue {dtype} d{d} B{B} T{T} H{H} s0={s0} beta_scale={beta_scale}")
    o, S = run_prologue(inp, beta_scale, dtype=dtype)
    o_ref, S_ref = oracle_prologue(inp, beta_scale)
    assert_close(f"prologue_{dtype}{d}_{B}_{T}_{H}_{beta_scale}", dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", DTYPES)
@pytest.mark.parametrize("T", [0, 1, 64, 65, 191])
def test_prologue_dtypes_lengths(dtype, d, T):
    torch_dev()
    inp = gen_raw_layer(2, T, 2, d, seed=7 + T + d, s0_var=0.1, dtype=dtype)
    note(f"prologue {dtype} d{d} lengths T={T}")
    o, S = run_prologue(inp, 2.0, dtype=dtype)
    if T == 0:  # nothing to process: S_final is S0
        assert np.array_equal(S, inp["S0"])
        return
    o_ref, S_ref = oracle_prologue(inp, 2.0)
    assert_close(f"prologue_{dtype}{d}_len{T}", dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", DTYPES)
def test_prologue_dtypes_zero_rows_saturated_and_in_place(dtype, d):
    """Zero rows of q or k stay zero; logits far in the tails; S_final aliasing S0."""
    torch_dev()
    inp = gen_raw_layer(1, 200, 3, d, seed=43 + d, s0_var=0.1, dtype=dtype)
    inp["k"][0, 5, 1] = 0.0
    inp["q"][0, 77, 2] = 0.0
    inp["k"][0, 130:140, 0] = 0.0
    rng = np.random.default_rng(8)
    pick = rng.random(inp["a_logit"].shape)
    inp["a_logit"] = np.where(pick < 0.1, 40.0, np.where(pick < 0.3, -40.0, inp["a_logit"])).astype(np.float32)
    pick = rng.random(inp["b_logit"].shape)
    inp["b_logit"] = np.where(pick < 0.15, 40.0, np.where(pick < 0.3, -40.0, inp["b_logit"])).astype(np.float32)
    note(f"prologue {dtype} d{d} zero rows, saturated logits, aliased state")
    o, S = run_prologue(inp, 2.0, S_final_alias=True, dtype=dtype)
    o_ref, S_ref = oracle_prologue(inp, 2.0)
    assert_close(f"prologue_{dtype}{d}_edges", dtype, o, S, o_ref, S_ref)


def test_prologue_long_d64_sequence_segmented():
    """A long d64 sequence on few chains takes the two-level scan (4 segments): the rows are normalised by the
    factor pass and by the map and output launches alike."""
    import linear_attention_sequence_gated_amd as gdn
    torch_dev()
    B, T, H = 1, 4096, 2
    assert gdn.gdn_chunk_fwd_prologue_workspace_bytes(B, T, H, 64, 64, 64, gdn.GDN_BF16) > B * H * 64 * 6400
    inp = gen_raw_layer(B, T, H, 64, seed=53, s0_var=0.05)
    note("prologue bf16 d64 segmented T=4096")
    o, S = run_prologue(inp, 2.0, S_final_alias=True)
    o_ref, S_ref = oracle_prologue(inp, 2.0)
    assert_close("prologue_bf16_d64_segmented", "bf16", o, S, o_ref, S_ref)


@pytest.mark.parametrize("name", ["long_context_bf16_prologue", "deltaphase_c64_prologue",
                                  "single_head_f32_prologue"])
def test_prologue_dtypes_full_size_all_chains(name):
    """The benchmark's prologue workloads at full size, every chain against the oracle."""
    torch_dev()
    w = WORKLOADS[name]
    inp = gen_workload(w)
    note(f"prologue full size {name}")
    o, S = run_prologue(inp, w.beta_scale, dtype=w.dtype)
    o_ref, S_ref = oracle_prologue(inp, w.beta_scale)
    assert_close(f"prologue_full_{name}", w.dtype, o, S, o_ref, S_ref)
