"""Per-output-channel decay (gdn_fwd_channel_decay) on the GPU through the C ABI, against the fp64 oracle
(oracle/channel_decay.py)."""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, gen_channel_decay, gen_workload
from gpu_util import TOL, assert_close, note, torch_dev, up

pytestmark = pytest.mark.gpu


def run(inp, dtype, alias=False):
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    S0 = up(inp["S0"], "f32") if inp.get("S0") is not None else None
    o, S = gdn.fwd_channel_decay(up(inp["q"], dtype), up(inp["k"], dtype), up(inp["v"], dtype), up(inp["r"], "f32"),
                                 up(inp["beta"], "f32"), S0, S_final=S0 if alias else None)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy()


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


def test_channel_decay_equals_scalar_gate_path():
    """r_t = alpha_t on every channel: the same result as gdn_chunk_fwd (two different kernels)."""
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_channel_decay(2, 200, 2, 64, dtype="f32", seed=3, s0_var=0.1)
    alpha = inp["r"][..., 0].copy()
    inp["r"] = np.repeat(alpha[..., None], 64, axis=-1)
    note("channel decay vs scalar gate")
    o1, S1 = run(inp, "f32")
    o2, S2 = gdn.chunk_fwd(up(inp["q"], "f32"), up(inp["k"], "f32"), up(inp["v"], "f32"), up(alpha, "f32"),
                           up(inp["beta"], "f32"), up(inp["S0"], "f32"))
    torch.cuda.synchronize()
    assert_close("chd_vs_scalar", "f32", o1, S1, o2.cpu().numpy(), S2.cpu().numpy())


def test_channel_decay_full_size_sampled_chains():
    w = WORKLOADS["sykra_layer_bf16_channel_decay"]
    inp = gen_workload(w)
    note("channel decay full size")
    o, S = run(inp, "bf16")
    chains = [(0, 0), (4, 6), (7, 11)]
    sub = {x: np.stack([inp[x][b, :, h] for b, h in chains], axis=1)[None] for x in ("q", "k", "v", "r", "beta")}
    sub["S0"] = None
    o_ref, S_ref = ref(sub)
    o_s = np.stack([o[b, :, h] for b, h in chains], axis=1)[None]
    S_s = np.stack([S[b, h] for b, h in chains])[None]
    assert_close("chd_full", "bf16", o_s, S_s, o_ref, S_ref)
