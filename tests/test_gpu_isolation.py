"""Cross-chain isolation on the GPU: a non-finite input in one (batch, head) chain leaves every other chain's
outputs bit-identical.

Chains never interact in the method, so any difference in another chain means a kernel read or wrote
outside its own rows (a wrong block-index remapping, a shared LDS slot, a stray store).  Each entry point
runs once on clean inputs and once with one chain poisoned, in the launch configuration the benchmark uses
where that matters (the full-size layers).
"""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, bf16_round, gen_chunk, gen_decode, gen_upstream_grads, gen_workload
from gpu_util import down, note, torch_dev, up

pytestmark = pytest.mark.gpu


def _others_identical(clean, dirty, chain_axis_b, chain_axis_h, bad):
    """clean/dirty [..B.., ..H..] arrays: every chain except bad=(b, h) must match bit for bit."""
    c = np.moveaxis(np.asarray(clean), (chain_axis_b, chain_axis_h), (0, 1))
    d = np.moveaxis(np.asarray(dirty), (chain_axis_b, chain_axis_h), (0, 1))
    assert np.isfinite(c).all()
    keep = np.ones(c.shape[:2], dtype=bool)
    keep[bad] = False
    assert np.array_equal(c[keep].view(np.uint8), d[keep].view(np.uint8))
    return d[bad]


def _run_chunk(inp, dtype):
    import torch
    import linear_attention_sequence_gated_amd as gdn
    s0 = up(inp["S0"], "f32") if inp.get("S0") is not None else None
    o, S = gdn.chunk_fwd(up(inp["q"], dtype), up(inp["k"], dtype), up(inp["v"], dtype), up(inp["alpha"], "f32"),
                         up(inp["beta"], "f32"), s0)
    torch.cuda.synchronize()
    return down(o), down(S)


CHUNK_CASES = [
    ("sykra_layer_bf16", "k", (3, 1000, 7, 5), (3, 7)),
    ("long_context_bf16", "v", (1, 9000, 5, 17), (1, 5)),
    ("deltaphase_c64", "alpha", (2, 700, 3), (2, 3)),
    ("small_f32", "q", (1, 150, 4, 0), (1, 4)),
]


@pytest.mark.parametrize("wname,field,where,bad", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_chunk_fwd_chain_isolation(wname, field, where, bad):
    torch_dev()
    if wname == "small_f32":
        inp, dtype = gen_chunk(2, 300, 6, 64, 64, dtype="f32", seed=5, s0_var=0.1), "f32"
    else:
        w = WORKLOADS[wname]
        inp, dtype = gen_workload(w), w.dtype
    note(f"isolation chunk_fwd {wname}: NaN in {field}{where}")
    o1, S1 = _run_chunk(inp, dtype)
    inp[field] = inp[field].copy()
    inp[field][where] = np.nan
    o2, S2 = _run_chunk(inp, dtype)
    bad_o = _others_identical(o1, o2, 0, 2, bad)
    _others_identical(S1, S2, 0, 1, bad)
    assert not np.isfinite(bad_o).all()  # the poison reached its own chain


def test_prologue_chain_isolation():
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    w = WORKLOADS["sykra_layer_bf16_prologue"]
    inp = gen_workload(w)
    note("isolation chunk_fwd_prologue: inf in q of chain (6, 2)")

    def run(x):
        o, S = gdn.chunk_fwd_prologue(up(x["q"], "bf16"), up(x["k"], "bf16"), up(x["v"], "bf16"),
                                      up(x["a_logit"], "f32"), up(x["b_logit"], "f32"), 1.0, None)
        torch.cuda.synchronize()
        return down(o), down(S)

    o1, S1 = run(inp)
    inp["q"] = inp["q"].copy()
    inp["q"][6, 50, 2, 3] = np.inf
    o2, S2 = run(inp)
    assert not np.isfinite(_others_identical(o1, o2, 0, 2, (6, 2))).all()
    _others_identical(S1, S2, 0, 1, (6, 2))


def test_channel_decay_chain_isolation():
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    w = WORKLOADS["sykra_layer_bf16_channel_decay"]
    inp = gen_workload(w)
    note("isolation fwd_channel_decay: NaN in r of chain (4, 9)")

    def run(x):
        o, S = gdn.fwd_channel_decay(up(x["q"], "bf16"), up(x["k"], "bf16"), up(x["v"], "bf16"), up(x["r"], "f32"),
                                     up(x["beta"], "f32"), None)
        torch.cuda.synchronize()
        return down(o), down(S)

    o1, S1 = run(inp)
    inp["r"] = inp["r"].copy()
    inp["r"][4, 10, 9, :] = np.nan
    o2, S2 = run(inp)
    assert not np.isfinite(_others_identical(o1, o2, 0, 2, (4, 9))).all()
    _others_identical(S1, S2, 0, 1, (4, 9))


def test_decode_state_isolation():
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_decode(4096, 64, 64, 1, dtype="bf16", seed=4, s_var=0.1)
    note("isolation recurrent_step: NaN in state 1234")

    def run(S0):
        S = up(S0, "f32")
        o = gdn.recurrent_step(up(inp["q"][0], "bf16"), up(inp["k"][0], "bf16"), up(inp["v"][0], "bf16"),
                               up(inp["alpha"][0], "f32"), up(inp["beta"][0], "f32"), S)
        torch.cuda.synchronize()
        return down(o), down(S)

    o1, S1 = run(inp["S"])
    S0 = inp["S"].copy()
    S0[1234, 7, 9] = np.nan
    o2, S2 = run(S0)
    keep = np.ones(4096, dtype=bool)
    keep[1234] = False
    assert np.array_equal(o1[keep].view(np.uint8), o2[keep].view(np.uint8))
    assert np.array_equal(S1[keep].view(np.uint8), S2[keep].view(np.uint8))
    assert not np.isfinite(o2[1234]).all()


def test_backward_chain_isolation():
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_chunk(2, 200, 6, 64, 64, dtype="bf16", seed=9, s0_var=0.1)
    dO, dS = gen_upstream_grads(2, 200, 6, 64, 64, seed=9, with_dS=True)
    dO = bf16_round(dO)
    note("isolation chunk_bwd: NaN in v of chain (0, 3)")

    def run(x):
        g = gdn.chunk_bwd(up(x["q"], "bf16"), up(x["k"], "bf16"), up(x["v"], "bf16"), up(x["alpha"], "f32"),
                          up(x["beta"], "f32"), up(dO, "bf16"), up(x["S0"], "f32"), up(dS, "f32"))
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in g]

    g1 = run(inp)
    inp["v"] = inp["v"].copy()
    inp["v"][0, 120, 3, 4] = np.nan
    g2 = run(inp)
    for a, b in zip(g1[:5], g2[:5]):
        _others_identical(a, b, 0, 2, (0, 3))
    _others_identical(g1[5], g2[5], 0, 1, (0, 3))
