"""Per-output-channel decay (gdn_fwd_channel_decay) on the GPU through the C ABI, against the fp64 oracle
(oracle/channel_decay.py).  bf16 inputs run the chunk form (16-token sub-chunks, one triangular solve per value
channel); fp32 and complex64 (LaplacePhaseCore-shaped, d = 32) inputs the token loop."""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, gen_channel_decay, gen_workload
from gpu_util import TOL, assert_close, note, torch_dev, up

pytestmark = pytest.mark.gpu


def run(inp, dtype, alias=False):
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    sdt = "c64" if dtype == "c64" else "f32"
    S0 = up(inp["S0"], sdt) if inp.get("S0") is not None else None
    o, S = gdn.fwd_channel_decay(up(inp["q"], dtype), up(inp["k"], dtype), up(inp["v"], dtype), up(inp["r"], "f32"),
                                 up(inp["beta"], "f32"), S0, S_final=S0 if alias else None)
    torch.cuda.synchronize()
    return (o.float() if o.dtype == torch.bfloat16 else o).cpu().numpy(), S.cpu().numpy()


def ref(inp):
    from oracle.channel_decay import channel_decay_fwd
    return channel_decay_fwd(inp["q"], inp["k"], inp["v"], inp["r"], inp["beta"], inp.get("S0"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,H,s0", [(1, 50, 2, None), (2, 300, 3, 0.1)])
def test_channel_decay_small(dtype, B, T, H, s0):
    inp = gen_channel_decay(B, T, H, 64, dtype=dtype, seed=31 + T, s0_var=s0)
    note(f"channel decay {dtype} B{B} T{T} H{H} s0={s0}")
    o, S = run(inp, dtype)
    o_ref, S_ref = ref(inp)
    assert_close(f"chd_{dtype}_{B}_{T}_{H}", dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("T", [0, 1, 2, 65])
def test_channel_decay_lengths_and_alias(T):
    inp = gen_channel_decay(2, T, 2, 64, dtype="f32", seed=7 + T, s0_var=0.5)
    note(f"channel decay T={T}, S_final aliasing S0")
    o, S = run(inp, "f32", alias=True)
    if T == 0:
        assert np.array_equal(S, inp["S0"])
        return
    o_ref, S_ref = ref(inp)
    assert_close(f"chd_len{T}", "f32", o, S, o_ref, S_ref)


def test_channel_decay_unit_decay_equals_delta_rule():
    """r = 1 on every channel: the plain delta rule, i.e. gdn_chunk_fwd at alpha = 1 (two different kernels)."""
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_channel_decay(2, 200, 2, 64, dtype="f32", seed=3, s0_var=0.1)
    inp["r"] = np.ones_like(inp["r"])
    ones = np.ones_like(inp["beta"])
    note("channel decay r = 1 vs the chunk forward at alpha = 1")
    o1, S1 = run(inp, "f32")
    o2, S2 = gdn.chunk_fwd(up(inp["q"], "f32"), up(inp["k"], "f32"), up(inp["v"], "f32"), up(ones, "f32"),
                           up(inp["beta"], "f32"), up(inp["S0"], "f32"))
    torch.cuda.synchronize()
    assert_close("chd_vs_delta_rule", "f32", o1, S1, o2.cpu().numpy(), S2.cpu().numpy())


def test_channel_decay_full_size_all_chains():
    """The 8 x 2048 x 12 d64 bf16 layer with a decay per token and value channel; every chain vs the oracle."""
    w = WORKLOADS["sykra_layer_bf16_channel_decay"]
    inp = gen_workload(w)
    note("channel decay full size")
    o, S = run(inp, "bf16")
    o_ref, S_ref = ref(inp)
    assert_close("chd_full", "bf16", o, S, o_ref, S_ref)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 250])
def test_channel_decay_chunk_form_lengths(T):
    """bf16 (chunk form): lengths around the 16-token sub-chunk, with S0 given and S_final aliasing S0."""
    inp = gen_channel_decay(2, T, 3, 64, dtype="bf16", seed=50 + T, s0_var=0.1)
    note(f"channel decay chunk form T={T}")
    o, S = run(inp, "bf16", alias=True)
    o_ref, S_ref = ref(inp)
    assert_close(f"chd_chunk_len{T}", "bf16", o, S, o_ref, S_ref)


def test_channel_decay_chunk_form_extreme_decays():
    """Decay factors at their extremes on random tokens and channels: r = 1e-6 (the channel is wiped) or 1 (kept),
    beta at 0 or 2; the substitution forms decay products by Horner's rule, so nothing overflows."""
    inp = gen_channel_decay(2, 300, 2, 64, dtype="bf16", seed=61, s0_var=0.1)
    rng = np.random.default_rng(3)
    pr, pb = rng.random(inp["r"].shape), rng.random(inp["beta"].shape)
    inp["r"] = np.where(pr < 0.1, 1e-6, np.where(pr < 0.3, 1.0, inp["r"])).astype(np.float32)
    inp["beta"] = np.where(pb < 0.1, 0.0, np.where(pb < 0.2, 2.0, inp["beta"])).astype(np.float32)
    note("channel decay chunk form, extreme decays")
    o, S = run(inp, "bf16")
    o_ref, S_ref = ref(inp)
    assert_close("chd_chunk_extreme", "bf16", o, S, o_ref, S_ref)


def test_channel_decay_chunk_form_unit_decay_equals_delta_rule():
    """bf16: r = 1 on every channel gives the chunk forward at alpha = 1 (two different kernels, each within the
    bf16 bound of the oracle)."""
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_channel_decay(2, 190, 2, 64, dtype="bf16", seed=8, s0_var=0.1)
    inp["r"] = np.ones_like(inp["r"])
    ones = np.ones_like(inp["beta"])
    note("channel decay chunk form r = 1 vs the chunk forward at alpha = 1")
    o1, S1 = run(inp, "bf16")
    o2, S2 = gdn.chunk_fwd(up(inp["q"], "bf16"), up(inp["k"], "bf16"), up(inp["v"], "bf16"), up(ones, "f32"),
                           up(inp["beta"], "f32"), up(inp["S0"], "f32"))
    torch.cuda.synchronize()
    assert_close("chd_chunk_vs_delta_rule", "bf16", o1, S1, o2.float().cpu().numpy(), S2.cpu().numpy())


@pytest.mark.parametrize("B,T,H,s0", [(1, 50, 2, None), (2, 300, 3, 0.1)])
def test_channel_decay_complex_small(B, T, H, s0):
    inp = gen_channel_decay(B, T, H, 32, dtype="c64", seed=61 + T, s0_var=s0)
    note(f"channel decay c64 B{B} T{T} H{H} s0={s0}")
    o, S = run(inp, "c64")
    o_ref, S_ref = ref(inp)
    assert_close(f"chd_c64_{B}_{T}_{H}", "c64", o, S, o_ref, S_ref)


@pytest.mark.parametrize("T", [0, 1, 3])
def test_channel_decay_complex_lengths_and_alias(T):
    inp = gen_channel_decay(2, T, 2, 32, dtype="c64", seed=70 + T, s0_var=0.5)
    note(f"channel decay c64 T={T}, S_final aliasing S0")
    o, S = run(inp, "c64", alias=True)
    if T == 0:
        assert np.array_equal(S, inp["S0"])
        return
    o_ref, S_ref = ref(inp)
    assert_close(f"chd_c64_len{T}", "c64", o, S, o_ref, S_ref)


def test_channel_decay_complex_unit_decay_equals_delta_rule():
    """Complex data, r = 1: gdn_chunk_fwd's complex kernel at alpha = 1 computes the same rule."""
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_channel_decay(2, 200, 2, 32, dtype="c64", seed=4, s0_var=0.1)
    inp["r"] = np.ones_like(inp["r"])
    ones = np.ones_like(inp["beta"])
    note("channel decay c64 r = 1 vs the complex chunk forward at alpha = 1")
    o1, S1 = run(inp, "c64")
    o2, S2 = gdn.chunk_fwd(up(inp["q"], "c64"), up(inp["k"], "c64"), up(inp["v"], "c64"), up(ones, "f32"),
                           up(inp["beta"], "f32"), up(inp["S0"], "c64"))
    torch.cuda.synchronize()
    assert_close("chd_c64_vs_delta_rule", "c64", o1, S1, o2.cpu().numpy(), S2.cpu().numpy())


def test_channel_decay_complex_full_size_all_chains():
    """The 4 x 4096 x 8 complex d32 layer with LaplacePhaseCore-shaped keys; every chain vs the oracle."""
    w = WORKLOADS["laplace_c64_channel_decay"]
    inp = gen_workload(w)
    note("channel decay c64 full size")
    o, S = run(inp, "c64")
    o_ref, S_ref = ref(inp)
    assert_close("chd_c64_full", "c64", o, S, o_ref, S_ref)
