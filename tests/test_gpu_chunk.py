"""Chunked forward on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

from gdn_inputs import WORKLOADS, gen_chunk, gen_workload
from gpu_util import TOL, assert_close, chain_rel_errors, down, note, oracle_chunk, run_chunk, torch_dev, up

pytestmark = pytest.mark.gpu

# (name, dtype, B, T, H, d, extra generator args).  Sizes span several chunks and
# a ragged tail; the oracle finishes each in well under a second.
SMALL = [
    ("f32_single_head_full", "f32", 1, 256, 1, 64, {}),
    ("f32_tail_s0", "f32", 2, 200, 3, 64, dict(s0_var=0.1)),
    ("bf16_d64_tail", "bf16", 2, 300, 3, 64, {}),
    ("bf16_d64_s0", "bf16", 1, 129, 2, 64, dict(s0_var=0.01)),
    # bf16 d64 grids of 16 and 192 workgroups, filled to 256 with cache warm-up
    # workgroups (ragged tails: their loads past T must read nothing)
    ("bf16_d64_warm_16", "bf16", 2, 1000, 4, 64, {}),
    ("bf16_d64_warm_192", "bf16", 8, 333, 12, 64, dict(s0_var=0.01)),
    ("bf16_d128_s0", "bf16", 1, 200, 2, 128, dict(s0_var=0.01, alpha_mu=-5.0)),
    ("bf16_d128_tail", "bf16", 2, 77, 1, 128, {}),
    ("c64_tail", "c64", 2, 200, 2, 32, dict(beta_scale=2.0)),
    ("c64_s0", "c64", 1, 130, 1, 32, dict(beta_scale=2.0, s0_var=0.5)),
]


@pytest.mark.parametrize("name,dtype,B,T,H,d,extra", SMALL, ids=[s[0] for s in SMALL])
def test_chunk_small(name, dtype, B, T, H, d, extra):
    torch_dev()
    inp = gen_chunk(B, T, H, d, d, dtype=dtype, seed=100 + len(name), **extra)
    note(f"chunk {name} B={B} T={T} H={H} d={d}")
    o, S = run_chunk(inp, dtype)
    o_ref, S_ref = oracle_chunk(inp)
    assert_close(name, dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("c64", 32)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 191, 250, 385])
def test_chunk_lengths(dtype, d, T):
    torch_dev()
    inp = gen_chunk(2, T, 2, d, d, dtype=dtype, seed=7 + T, s0_var=0.1,
                    beta_scale=2.0 if dtype == "c64" else 1.0)
    note(f"chunk lengths dtype={dtype} d={d} T={T}")
    o, S = run_chunk(inp, dtype)
    o_ref, S_ref = oracle_chunk(inp)
    assert_close(f"len{T}_{dtype}_{d}", dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("c64", 32)])
def test_chunk_empty_sequence_copies_state(dtype, d):
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_chunk(2, 0, 3, d, d, dtype=dtype, seed=3, s0_var=1.0)
    note(f"chunk T=0 dtype={dtype}")
    sd = torch.complex64 if dtype == "c64" else torch.float32
    q = torch.empty((2, 0, 3, d), dtype={"f32": torch.float32, "bf16": torch.bfloat16, "c64": torch.complex64}[dtype],
                    device="cuda")
    a = torch.empty((2, 0, 3), dtype=torch.float32, device="cuda")
    s0 = up(inp["S0"], "f32")
    _, S = gdn.chunk_fwd(q, q, q, a, a, s0)
    assert np.array_equal(down(S), inp["S0"])
    _, S = gdn.chunk_fwd(q, q, q, a, a, None)
    assert down(S).dtype == (np.complex64 if sd == torch.complex64 else np.float32)
    assert not down(S).any()


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("c64", 32)])
def test_chunk_state_in_place(dtype, d):
    """S_final may alias S0."""
    torch_dev()
    inp = gen_chunk(1, 150, 2, d, d, dtype=dtype, seed=31, s0_var=0.1)
    note(f"chunk in-place state dtype={dtype}")
    o, S = run_chunk(inp, dtype, S_final_alias=True)
    o_ref, S_ref = oracle_chunk(inp)
    assert_close(f"alias_{dtype}", dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("c64", 32)])
def test_chunk_repeated_keys(dtype, d):
    """Associative-recall structure: a small key set written over and over."""
    torch_dev()
    rng = np.random.default_rng(5)
    inp = gen_chunk(2, 320, 2, d, d, dtype=dtype, seed=41, beta_scale=2.0 if dtype == "c64" else 1.0)
    idx = rng.integers(0, 16, size=320)
    inp["k"] = np.ascontiguousarray(inp["k"][:, :16][:, idx])  # token t reuses key idx[t]
    inp["q"] = np.ascontiguousarray(inp["k"][:, rng.permutation(320)])
    note(f"chunk repeated keys dtype={dtype}")
    o, S = run_chunk(inp, dtype)
    o_ref, S_ref = oracle_chunk(inp)
    assert_close(f"repeat_{dtype}", dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("c64", 32)])
def test_chunk_reflection_keeps_norm(dtype, d):
    """beta = 2, alpha = 1, v = 0: Householder reflections keep ||S||_F; matches the oracle too."""
    torch_dev()
    inp = gen_chunk(1, 200, 2, d, d, dtype=dtype, seed=51, s0_var=1.0)
    inp["beta"][:] = 2.0
    inp["alpha"][:] = 1.0
    inp["v"][:] = 0
    note(f"chunk reflection dtype={dtype}")
    o, S = run_chunk(inp, dtype)
    n0 = np.linalg.norm(inp["S0"].reshape(2, -1).astype(np.complex128), axis=1)
    n1 = np.linalg.norm(S.reshape(2, -1).astype(np.complex128), axis=1)
    assert np.allclose(n0, n1, rtol=1e-4), (n0, n1)
    o_ref, S_ref = oracle_chunk(inp)
    assert_close(f"reflect_{dtype}", dtype, o, S, o_ref, S_ref)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("c64", 32)])
def test_chunk_split_invariance(dtype, d):
    """Two calls chained through S_final -> S0 agree with one call."""
    torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    inp = gen_chunk(1, 256, 2, d, d, dtype=dtype, seed=61, s0_var=0.1)
    note(f"chunk split dtype={dtype}")
    o, S = run_chunk(inp, dtype)
    first = {k_: (v_[:, :128] if k_ in ("q", "k", "v", "alpha", "beta") else v_) for k_, v_ in inp.items()}
    o1, S1 = run_chunk(first, dtype)
    second = {k_: (v_[:, 128:] if k_ in ("q", "k", "v", "alpha", "beta") else v_) for k_, v_ in inp.items()}
    second["S0"] = S1
    o2, S2 = run_chunk(second, dtype)
    eo, es = chain_rel_errors(np.concatenate([o1, o2], axis=1), S2, o, S)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


def test_chunk_deterministic():
    torch_dev()
    inp = gen_chunk(2, 300, 3, 64, 64, dtype="bf16", seed=71)
    note("chunk determinism bf16 d64")
    o1, S1 = run_chunk(inp, "bf16")
    o2, S2 = run_chunk(inp, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# ---------------------------------------------------------------- full sizes
FULL = ["sykra_layer_bf16", "long_context_bf16", "deltaphase_c64", "single_head_f32"]


@pytest.mark.parametrize("wname", FULL)
def test_chunk_full_size_all_chains(wname):
    """The workload at its full size, in the launch configuration the benchmark times; every chain is
    recomputed by the oracle and checked element by element."""
    torch_dev()
    w = WORKLOADS[wname]
    inp = gen_workload(w)
    note(f"chunk full size {wname}")
    o, S = run_chunk(inp, w.dtype)
    o_ref, S_ref = oracle_chunk(inp)
    assert_close(f"full_{wname}", w.dtype, o, S, o_ref, S_ref)


def test_chunk_bf16_rows_beyond_32bit_offsets():
    """bf16, d = 64, with T * H * 64 * 2 >= 2^31 bytes in one batch row, so offsets into q, k, v and o
    no longer fit 32 bits and the library runs the fused kernel with 64-bit addressing.  Inputs are drawn
    on the device from a seeded generator, with the distributions of the bf16 layer workload.  The first
    and the last head (whose late rows lie past the 2 GiB offset) are checked against the oracle."""
    import oracle
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    B, T, H, d = 1, 65536, 256, 64
    assert T * H * d * 2 >= 2 ** 31
    note(f"chunk bf16 rows beyond 32-bit offsets: B{B} T{T} H{H} d{d}")
    gen = torch.Generator(device="cuda").manual_seed(2031)

    def unit_rows():
        x = torch.randn((B, T, H, d), generator=gen, device="cuda")
        x /= x.norm(dim=-1, keepdim=True)
        return x.to(torch.bfloat16)

    q, k = unit_rows(), unit_rows()
    v = torch.randn((B, T, H, d), generator=gen, device="cuda").to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((B, T, H), generator=gen, device="cuda"))
    alpha = torch.exp(-torch.nn.functional.softplus(torch.randn((B, T, H), generator=gen, device="cuda") - 4.0))
    o, S = gdn.chunk_fwd(q, k, v, alpha, beta, None)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        chain = lambda t: t[:, :, h:h + 1].float().cpu().numpy()
        o_ref, S_ref, _ = oracle.recurrent_fwd(chain(q), chain(k), chain(v), chain(alpha), chain(beta), None)
        eo, es = chain_rel_errors(chain(o), S[:, h:h + 1].cpu().numpy(), o_ref, S_ref)
        print(f"[parity] bf16 rows beyond 32-bit offsets, head {h}: o={eo:.3e} S={es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (h, eo, es)
