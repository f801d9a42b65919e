"""Backward (gdn_chunk_bwd) on the GPU through the C ABI, against the fp64 oracle's reverse-mode gradients
(oracle/backward.py, pinned by finite differences of the forward)."""
import time

import numpy as np
import pytest

from gdn_inputs import WORKLOADS, bf16_round, gen_chunk, gen_upstream_grads, gen_workload
from gpu_util import note, torch_dev, up

pytestmark = pytest.mark.gpu

# fp32 and complex64 inputs: the token-by-token kernels, fp32 arithmetic on exactly-read inputs.  bf16 inputs:
# the chunk form on the matrix cores, bf16 operands with fp32 accumulation (as in the forward).
TOLS = {"f32": 1e-4, "bf16": 5e-2, "c64": 1e-4}
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def run_bwd(inp, dtype, dO, dS):
    torch = torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    q, k, v = up(inp["q"], dtype), up(inp["k"], dtype), up(inp["v"], dtype)
    a, b = up(inp["alpha"], "f32"), up(inp["beta"], "f32")
    S0 = up(inp["S0"], "f32") if inp.get("S0") is not None else None
    g = gdn.chunk_bwd(q, k, v, a, b, up(dO, dtype), S0, up(dS, "f32") if dS is not None else None)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in g]


def oracle_bwd(inp, dO, dS):
    from oracle.backward import recurrent_bwd
    return recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp.get("S0"), dO, dS)


def per_chain_errors(x, ref, name):
    """Max over (b, h) chains of ||x - ref|| / ||ref|| and of max|x - ref| / max|ref|, over that chain's entries."""
    cplx = np.iscomplexobj(x) or np.iscomplexobj(ref)
    x, ref = (np.asarray(y, np.complex128 if cplx else np.float64) for y in (x, ref))
    if name == "dS0":
        xs, rs = x.reshape(-1, x.shape[-2] * x.shape[-1]), ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    else:  # [B, T, H, ...] -> chains
        xs = np.moveaxis(x, 2, 1).reshape(x.shape[0] * x.shape[2], -1)
        rs = np.moveaxis(ref, 2, 1).reshape(ref.shape[0] * ref.shape[2], -1)
    if not len(xs) or not xs.shape[1]:
        return 0.0, 0.0
    den = np.maximum(np.linalg.norm(rs, axis=1), 1e-30)
    norm = float(np.max(np.linalg.norm(xs - rs, axis=1) / den))
    elem = float(np.max(np.abs(xs - rs).max(axis=1) / np.maximum(np.abs(rs).max(axis=1), 1e-30)))
    return norm, elem


def assert_grads(tag, got, ref, dtype):
    tol = TOLS[dtype]
    errs = {n: per_chain_errors(g, r, n) for n, g, r in zip(NAMES, got, ref)}
    print(f"[parity] {tag}: " + " ".join(f"{n}={e[0]:.2e}/{e[1]:.2e}" for n, e in errs.items())
          + f" (norm / elem, tol {tol:g})", flush=True)
    for n, g in zip(NAMES, got):
        assert np.isfinite(g).all(), (tag, n)
    assert all(e[0] <= tol and e[1] <= tol for e in errs.values()), (tag, errs)


def _case(B, T, H, dtype, seed, s0, dS, d=64):
    inp = gen_chunk(B, T, H, d, d, dtype=dtype, seed=seed, s0_var=0.1 if s0 else None,
                    beta_scale=2.0 if dtype == "c64" else 1.0)
    dO, dSf = gen_upstream_grads(B, T, H, d, d, seed=seed, with_dS=dS, dtype="c64" if dtype == "c64" else "f32")
    if dtype == "bf16":
        dO = bf16_round(dO)
    return inp, dO, dSf


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,H,s0,dS", [(1, 20, 2, False, False), (2, 77, 3, True, True), (1, 200, 2, True, False)])
def test_backward_small(dtype, B, T, H, s0, dS):
    inp, dO, dSf = _case(B, T, H, dtype, 11 + T, s0, dS)
    note(f"backward {dtype} B{B} T{T} H{H} S0={s0} dS={dS}")
    assert_grads(f"bwd_{dtype}_{B}_{T}_{H}", run_bwd(inp, dtype, dO, dSf), oracle_bwd(inp, dO, dSf), dtype)


@pytest.mark.parametrize("T", [0, 1, 7, 8, 9, 64, 65])
def test_backward_lengths(T):
    inp, dO, dSf = _case(2, T, 2, "bf16", 3 + T, True, True)
    note(f"backward lengths T={T}")
    got = run_bwd(inp, "bf16", dO, dSf)
    if T == 0:  # only dS0 = dS_T
        assert np.array_equal(got[5], dSf)
        return
    assert_grads(f"bwd_len{T}", got, oracle_bwd(inp, dO, dSf), "bf16")


def test_backward_deterministic():
    inp, dO, dSf = _case(2, 100, 2, "bf16", 5, True, True)
    note("backward determinism")
    g1, g2 = run_bwd(inp, "bf16", dO, dSf), run_bwd(inp, "bf16", dO, dSf)
    assert all(np.array_equal(a, b) for a, b in zip(g1, g2))


@pytest.mark.timeout(600)
def test_backward_full_size_all_chains():
    """The 8 x 2048 x 12 d64 bf16 layer on the GPU; every chain recomputed by the oracle (two batch rows at a
    time, to bound the oracle's memory for the states it keeps)."""
    w = WORKLOADS["sykra_layer_bf16"]
    inp = gen_workload(w)
    dO, dSf = gen_upstream_grads(w.B, w.T, w.H, w.dk, w.dv, seed=w.seed, with_dS=True)
    dO = bf16_round(dO)
    note("backward full size sykra_layer_bf16")
    t0 = time.perf_counter()
    got = run_bwd(inp, "bf16", dO, dSf)
    print(f"[backward] full size call + copies {time.perf_counter() - t0:.3f} s", flush=True)
    for b0 in range(0, w.B, 2):
        sl = slice(b0, b0 + 2)
        sub = {x: (None if inp[x] is None else inp[x][sl]) for x in inp}
        ref = oracle_bwd(sub, dO[sl], dSf[sl])
        assert_grads(f"bwd_full_rows{b0}-{b0 + 1}", [g[sl] for g in got], ref, "bf16")


def test_backward_extreme_gates():
    """Gates at their extremes on random tokens: alpha = 1e-6 (state wiped) or 1, beta = 0 or 2 (a full
    Householder reflection); the rest as drawn."""
    inp, dO, dSf = _case(2, 150, 2, "f32", 77, True, True)
    rng = np.random.default_rng(8)
    pa, pb = rng.random(inp["alpha"].shape), rng.random(inp["beta"].shape)
    inp["alpha"] = np.where(pa < 0.1, 1e-6, np.where(pa < 0.3, 1.0, inp["alpha"])).astype(np.float32)
    inp["beta"] = np.where(pb < 0.15, 0.0, np.where(pb < 0.3, 2.0, inp["beta"])).astype(np.float32)
    note("backward extreme gates")
    assert_grads("bwd_extreme", run_bwd(inp, "f32", dO, dSf), oracle_bwd(inp, dO, dSf), "f32")


@pytest.mark.parametrize("B,T,H,s0,dS", [(1, 20, 2, False, False), (2, 77, 3, True, True), (1, 200, 2, True, False)])
def test_backward_d128(B, T, H, s0, dS):
    """bf16 d = 128: the chunk form with its gradient pass in two launches (value columns, then rows and keys)."""
    inp, dO, dSf = _case(B, T, H, "bf16", 21 + T, s0, dS, d=128)
    note(f"backward d128 B{B} T{T} H{H} S0={s0} dS={dS}")
    assert_grads(f"bwd_d128_{B}_{T}_{H}", run_bwd(inp, "bf16", dO, dSf), oracle_bwd(inp, dO, dSf), "bf16")


@pytest.mark.parametrize("T", [0, 1, 64, 65, 130])
def test_backward_d128_lengths(T):
    inp, dO, dSf = _case(2, T, 2, "bf16", 40 + T, True, True, d=128)
    note(f"backward d128 lengths T={T}")
    got = run_bwd(inp, "bf16", dO, dSf)
    if T == 0:  # only dS0 = dS_T
        assert np.array_equal(got[5], dSf)
        return
    assert_grads(f"bwd_d128_len{T}", got, oracle_bwd(inp, dO, dSf), "bf16")


@pytest.mark.timeout(600)
def test_backward_d128_long():
    """A longer d = 128 case, 16 chunks per chain, with the long-context gate recipe (alpha logits ~ N(-5, 1))
    and S0 given; every chain against the oracle."""
    inp = gen_chunk(1, 1000, 4, 128, 128, dtype="bf16", seed=2, alpha_mu=-5.0, s0_var=0.01)
    dO, dSf = gen_upstream_grads(1, 1000, 4, 128, 128, seed=2, with_dS=True)
    dO = bf16_round(dO)
    note("backward d128 long")
    assert_grads("bwd_d128_long", run_bwd(inp, "bf16", dO, dSf), oracle_bwd(inp, dO, dSf), "bf16")


# Long single-chain sequences: the backward's forward state pass takes the two-level scan (segment maps,
# their combine, then every segment's chunk states from its true start state), with ragged segment and
# chunk tails.  (name, T, d): 65 chunks split into 4 segments (17, 17, 17, 14), 257 into 16 (15 of 17, one of 2).
BWD_SEGMENTED = [("d64_T4100", 4100, 64), ("d128_T4100", 4100, 128), ("d64_T16400", 16400, 64)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,T,d", BWD_SEGMENTED, ids=[s[0] for s in BWD_SEGMENTED])
def test_backward_segmented_scan(name, T, d):
    torch_dev()
    import linear_attention_sequence_gated_amd as gdn
    nch = (T + 63) // 64
    rec = 6400  # bytes of one chunk's factor record; more workspace than the records means segment maps
    assert gdn.gdn_chunk_fwd_workspace_bytes(1, T, 1, d, d, 64, gdn.GDN_BF16) > nch * rec, \
        "this shape must take the segmented scan"
    inp = gen_chunk(1, T, 1, d, d, dtype="bf16", seed=40 + d, alpha_mu=-5.0, s0_var=0.1)
    dO, dSf = gen_upstream_grads(1, T, 1, d, d, seed=40 + d, with_dS=True)
    dO = bf16_round(dO)
    note(f"backward segmented {name}")
    assert_grads(f"bwd_segmented_{name}", run_bwd(inp, "bf16", dO, dSf), oracle_bwd(inp, dO, dSf), "bf16")


# Complex data, d = 32 (the phasor memory): the token-by-token kernel in fp32, gradients dL/dRe + i dL/dIm.
@pytest.mark.parametrize("B,T,H,s0,dS", [(1, 20, 2, False, False), (2, 77, 3, True, True), (1, 200, 2, True, False)])
def test_backward_complex(B, T, H, s0, dS):
    inp, dO, dSf = _case(B, T, H, "c64", 31 + T, s0, dS, d=32)
    note(f"backward complex B{B} T{T} H{H} S0={s0} dS={dS}")
    assert_grads(f"bwd_c64_{B}_{T}_{H}", run_bwd(inp, "c64", dO, dSf), oracle_bwd(inp, dO, dSf), "c64")


@pytest.mark.parametrize("T", [0, 1, 7, 8, 9, 65])
def test_backward_complex_lengths(T):
    inp, dO, dSf = _case(2, T, 2, "c64", 50 + T, True, True, d=32)
    note(f"backward complex lengths T={T}")
    got = run_bwd(inp, "c64", dO, dSf)
    if T == 0:  # only dS0 = dS_T
        assert np.array_equal(got[5], dSf)
        return
    assert_grads(f"bwd_c64_len{T}", got, oracle_bwd(inp, dO, dSf), "c64")


def test_backward_complex_extreme_gates():
    """Complex data with gates at their extremes on random tokens: alpha = 1e-6 or 1, beta = 0 or 2."""
    inp, dO, dSf = _case(2, 150, 2, "c64", 78, True, True, d=32)
    rng = np.random.default_rng(9)
    pa, pb = rng.random(inp["alpha"].shape), rng.random(inp["beta"].shape)
    inp["alpha"] = np.where(pa < 0.1, 1e-6, np.where(pa < 0.3, 1.0, inp["alpha"])).astype(np.float32)
    inp["beta"] = np.where(pb < 0.15, 0.0, np.where(pb < 0.3, 2.0, inp["beta"])).astype(np.float32)
    note("backward complex extreme gates")
    assert_grads("bwd_c64_extreme", run_bwd(inp, "c64", dO, dSf), oracle_bwd(inp, dO, dSf), "c64")


@pytest.mark.timeout(600)
def test_backward_complex_full_size_all_chains():
    """The 4 x 4096 x 8 complex phasor layer; every chain recomputed by the oracle (one batch row at a time)."""
    w = WORKLOADS["deltaphase_c64_bwd"]
    inp = gen_workload(w)
    dO, dSf = gen_upstream_grads(w.B, w.T, w.H, w.dk, w.dv, seed=w.seed, with_dS=True, dtype="c64")
    note("backward full size deltaphase_c64_bwd")
    got = run_bwd(inp, "c64", dO, dSf)
    for b0 in range(w.B):
        sl = slice(b0, b0 + 1)
        sub = {x: (None if inp[x] is None else inp[x][sl]) for x in inp}
        assert_grads(f"bwd_c64_full_row{b0}", [g[sl] for g in got], oracle_bwd(sub, dO[sl], dSf[sl]), "c64")
