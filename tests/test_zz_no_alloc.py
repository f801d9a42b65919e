"""gdn_chunk_fwd_noalloc, the entry point for callers that cannot allocate, against gdn_chunk_fwd with a
workspace the caller owns: the same kernels on the same inputs, so outputs and final states must agree bit for
bit (and both match the oracle within the dtype's bounds).  Each case makes two calls in a row, the second with
a smaller input, so the second call runs over the scratch array the first call left behind."""
import numpy as np
import pytest

from gdn_inputs import gen_chunk
from gpu_util import assert_close, down, note, oracle_chunk, torch_dev, up

pytestmark = pytest.mark.gpu

# (name, dtype, d, first (B, T, H), second (B, T, H), extra generator args).  Each takes a path that needs a
# workspace: the bf16 d = 128 two-launch path, the complex path, and the segmented scan.
CASES = [
    ("bf16_d128", "bf16", 128, (2, 700, 3), (1, 300, 2), dict(s0_var=0.01)),
    ("c64", "c64", 32, (2, 600, 2), (1, 130, 1), dict(beta_scale=2.0, s0_var=0.5)),
    ("bf16_d64_segmented", "bf16", 64, (1, 4200, 1), (1, 4100, 1), {}),
]


def _call(noalloc, inp, dtype, d):
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    B, T, H, _ = inp["q"].shape
    tdt = {"bf16": torch.bfloat16, "c64": torch.complex64}[dtype]
    sdt = torch.complex64 if dtype == "c64" else torch.float32
    code = {"bf16": gdn.GDN_BF16, "c64": gdn.GDN_C64}[dtype]
    q, k, v = up(inp["q"], dtype), up(inp["k"], dtype), up(inp["v"], dtype)
    a, b = up(inp["alpha"], "f32"), up(inp["beta"], "f32")
    s0 = up(inp["S0"], "f32") if inp.get("S0") is not None else None
    if not noalloc:
        o, S = gdn.chunk_fwd(q, k, v, a, b, s0)
        torch.cuda.synchronize()
        return down(o), down(S)
    out = torch.empty((B, T, H, d), dtype=tdt, device="cuda")
    S = torch.empty((B, H, d, d), dtype=sdt, device="cuda")
    st = gdn.gdn_chunk_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(),
                                   None if s0 is None else s0.data_ptr(), 64, out.data_ptr(), S.data_ptr(), B, T, H,
                                   d, d, code, torch.cuda.current_stream().cuda_stream)
    assert st == 0, gdn.gdn_status_str(st)
    torch.cuda.synchronize()
    return down(out), down(S)


@pytest.mark.parametrize("name,dtype,d,first,second,extra", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_the_workspace_entry_point(name, dtype, d, first, second, extra):
    torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    for call, (B, T, H) in enumerate((first, second)):
        need = gdn.gdn_chunk_fwd_workspace_bytes(B, T, H, d, d, 64, {"bf16": gdn.GDN_BF16, "c64": gdn.GDN_C64}[dtype])
        assert 0 < need <= gdn.GDN_NOALLOC_MAX_WORKSPACE
        inp = gen_chunk(B, T, H, d, d, dtype=dtype, seed=900 + 10 * call + d, **extra)
        note(f"noalloc {name} call {call}: B{B} T{T} H{H} d{d}")
        o1, S1 = _call(True, inp, dtype, d)
        o2, S2 = _call(False, inp, dtype, d)
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2), (name, call)
        o_ref, S_ref = oracle_chunk(inp)
        assert_close(f"noalloc_{name}_{call}", dtype, o1, S1, o_ref, S_ref)
