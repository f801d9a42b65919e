"""The bf16 two-launch path (factor pass, then state pass) on the GPU through the C ABI.

* The factor records the first launch leaves in the caller's workspace hold, per (chain, chunk),
  Tb = (I + A)^{-1} diag(beta) (rounded to bf16) and the prefix g of log2 alpha; they are compared with
  the oracle's chunk form (oracle/chunked.py), which exposes T for every chunk.
* The segment-parallel two-level scan (taken for long sequences with few chains) against the fp64 token
  loop, with ragged segment and chunk tails, S0 given and S_final aliasing S0.
"""
import numpy as np
import pytest

import oracle
from gdn_inputs import gen_chunk
from gpu_util import assert_close, down, note, oracle_chunk, torch_dev, up
from oracle.chunked import chunked_fwd

pytestmark = pytest.mark.gpu

REC = 6400  # bytes per (chain, chunk) record


def pblk(i, p):
    return i if i < 2 else 2 * i - 2 + p


def decode_records(raw, chains, nch):
    """Workspace bytes -> Tb [chains, nch, 64, 64] (fp32 from bf16) and g [chains, nch, 64]."""
    recs = raw[: chains * nch * REC].reshape(chains, nch, REC)
    bf = recs[..., : 6 * 1024].copy().view(np.uint16).reshape(chains, nch, 6, 64, 8)
    vals = (bf.astype(np.uint32) << 16).view(np.float32)
    Tb = np.zeros((chains, nch, 64, 64), np.float32)
    for i in range(4):
        for p in range(i // 2 + 1):
            blk = vals[:, :, pblk(i, p)]  # [chains, nch, lane, 8]
            for lane in range(64):
                g, c = lane >> 4, lane & 15
                for h in range(2):
                    kt = 2 * p + h
                    if kt > i:
                        assert not blk[:, :, lane, 4 * h:4 * h + 4].any(), "tile above the diagonal must be zero"
                        continue
                    Tb[:, :, 16 * i + c, 16 * kt + 4 * g:16 * kt + 4 * g + 4] = blk[:, :, lane, 4 * h:4 * h + 4]
    g = recs[..., 6 * 1024:].copy().view(np.float32).reshape(chains, nch, 64)
    return Tb, g


# (d, B, T, H): d = 128 always takes the two-launch path; d = 64 does for a long sequence with few chains.
@pytest.mark.parametrize("d,B,T,H", [(128, 2, 150, 3), (128, 2, 77, 3), (64, 1, 4100, 1)])
def test_factor_records_match_the_chunk_form(d, B, T, H):
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_chunk(B, T, H, d, d, dtype="bf16", seed=200 + d, beta_scale=2.0)
    note(f"two-pass factor records d={d} T={T}")
    nch = (T + 63) // 64
    need = gdn.gdn_chunk_fwd_workspace_bytes(B, T, H, d, d, 64, gdn.GDN_BF16)
    assert need >= B * H * nch * REC  # records first, then (segmented scan) the segment maps
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    q, k, v = up(inp["q"], "bf16"), up(inp["k"], "bf16"), up(inp["v"], "bf16")
    a, b = up(inp["alpha"], "f32"), up(inp["beta"], "f32")
    out = torch.empty_like(v)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    st = gdn.gdn_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(), None, 64,
                           out.data_ptr(), S.data_ptr(), B, T, H, d, d, gdn.GDN_BF16, ws.data_ptr(), need,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    Tb, g = decode_records(ws.cpu().numpy(), B * H, nch)
    _, _, terms = chunked_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None, keep_terms=True)
    worst_t = worst_g = 0.0
    for bb in range(B):
        for hh in range(H):
            for n, tr in enumerate(terms[(bb, hh)]):
                L = tr["T"].shape[0]
                beta = inp["beta"][bb, 64 * n:64 * n + L, hh].astype(np.float64)
                ref = np.zeros((64, 64))
                ref[:L, :L] = tr["T"] * beta[None, :]
                got = Tb[bb * H + hh, n]
                worst_t = max(worst_t, np.abs(got - ref).max() / np.abs(ref).max())
                gref = np.full(64, tr["g"][-1] / np.log(2.0))
                gref[:L] = tr["g"] / np.log(2.0)
                worst_g = max(worst_g, np.abs(g[bb * H + hh, n] - gref).max())
    print(f"[parity] factor records d={d}: Tb max err / max |Tb| = {worst_t:.3e}, g max abs err = {worst_g:.3e}",
          flush=True)
    assert worst_t <= 8e-3 and worst_g <= 1e-4


# Shapes that take the segmented scan (one or two chains, long sequences) and their segment counts.
SEGMENTED = [
    ("d128_T4100_one_chain", 1, 4100, 1, 128, 0.01),   # 65 chunks: 4 segments of 17, 17, 17, 14
    ("d128_T8192_two_chains", 2, 8192, 1, 128, None),  # 128 chunks: 8 segments of 16
    ("d64_T16400_one_chain", 1, 16400, 1, 64, 0.1),    # 257 chunks: 16 segments, ragged last chunk
]


@pytest.mark.parametrize("name,B,T,H,d,s0", SEGMENTED, ids=[s[0] for s in SEGMENTED])
def test_segmented_scan(name, B, T, H, d, s0):
    torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    need = gdn.gdn_chunk_fwd_workspace_bytes(B, T, H, d, d, 64, gdn.GDN_BF16)
    nch = (T + 63) // 64
    assert need > B * H * nch * REC, "this shape must take the segmented scan"
    inp = gen_chunk(B, T, H, d, d, dtype="bf16", seed=300 + T, s0_var=s0, alpha_mu=-5.0)
    note(f"segmented scan {name}")
    o, S = gdn.chunk_fwd(up(inp["q"], "bf16"), up(inp["k"], "bf16"), up(inp["v"], "bf16"), up(inp["alpha"], "f32"),
                         up(inp["beta"], "f32"), up(inp["S0"], "f32"))
    import torch
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_chunk(inp)
    assert_close(f"segmented_{name}", "bf16", down(o), down(S), o_ref, S_ref)


def test_segmented_scan_state_in_place():
    """S_final aliasing S0 on the segmented path (the start states are read before the last segment writes)."""
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_chunk(1, 4200, 1, 128, 128, dtype="bf16", seed=77, s0_var=0.01)
    note("segmented scan, S_final aliasing S0")
    s0 = up(inp["S0"], "f32")
    o, S = gdn.chunk_fwd(up(inp["q"], "bf16"), up(inp["k"], "bf16"), up(inp["v"], "bf16"), up(inp["alpha"], "f32"),
                         up(inp["beta"], "f32"), s0, S_final=s0)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_chunk(inp)
    assert_close("segmented_alias", "bf16", down(o), down(S), o_ref, S_ref)


def test_long_sequence_full_size_all_chains():
    """The Sykra layer over one 65536-token sequence (12 chains of 1024 chunks), which takes the segmented scan
    with 10 segments, in the benchmark's launch configuration; every chain against the oracle."""
    torch = torch_dev()
    from gdn_inputs import WORKLOADS, gen_workload
    import linear_attention_sequence_gated_amd as gdn
    w = WORKLOADS["long_sequence_bf16"]
    inp = gen_workload(w)
    need = gdn.gdn_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, 64, gdn.GDN_BF16)
    assert need > w.B * w.H * (w.T // 64) * REC, "the long sequence must take the segmented scan"
    note("segmented scan, long_sequence_bf16 full size")
    o, S = gdn.chunk_fwd(up(inp["q"], "bf16"), up(inp["k"], "bf16"), up(inp["v"], "bf16"), up(inp["alpha"], "f32"),
                         up(inp["beta"], "f32"), None)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_chunk(inp)
    assert_close("full_long_sequence_bf16", "bf16", down(o), down(S), o_ref, S_ref)
