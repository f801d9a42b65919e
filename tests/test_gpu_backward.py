"""Backward (gdn_chunk_bwd) on the GPU through the C ABI, against the fp64 oracle's reverse-mode gradients
(oracle/backward.py, pinned by finite differences of the forward)."""
import time

import numpy as np
import pytest

from gdn_inputs import WORKLOADS, bf16_round, gen_chunk, gen_upstream_grads, gen_workload
from gpu_util import note, take_chains, torch_dev, up

pytestmark = pytest.mark.gpu

TOL = 1e-4  # fp32 arithmetic on exactly-read inputs, both dtypes
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


def per_chain_rel(x, ref, name):
    """Max over (b, h) chains of ||x - ref|| / ||ref||, over that chain's entries."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if name == "dS0":
        xs, rs = x.reshape(-1, x.shape[-2] * x.shape[-1]), ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    else:  # [B, T, H, ...] -> chains
        xs = np.moveaxis(x, 2, 1).reshape(x.shape[0] * x.shape[2], -1)
        rs = np.moveaxis(ref, 2, 1).reshape(ref.shape[0] * ref.shape[2], -1)
    den = np.maximum(np.linalg.norm(rs, axis=1), 1e-30)
    return float(np.max(np.linalg.norm(xs - rs, axis=1) / den)) if len(xs) else 0.0


def assert_grads(tag, got, ref):
    errs = {n: per_chain_rel(g, r, n) for n, g, r in zip(NAMES, got, ref)}
    print(f"[parity] {tag}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, g in zip(NAMES, got):
        assert np.isfinite(g).all(), (tag, n)
    assert all(e <= TOL for e in errs.values()), (tag, errs)


def _case(B, T, H, dtype, seed, s0, dS):
    inp = gen_chunk(B, T, H, 64, 64, dtype=dtype, seed=seed, s0_var=0.1 if s0 else None)
    dO, dSf = gen_upstream_grads(B, T, H, 64, 64, seed=seed, with_dS=dS)
    if dtype == "bf16":
        dO = bf16_round(dO)
    return inp, dO, dSf


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,H,s0,dS", [(1, 20, 2, False, False), (2, 77, 3, True, True), (1, 200, 2, True, False)])
def test_backward_small(dtype, B, T, H, s0, dS):
    inp, dO, dSf = _case(B, T, H, dtype, 11 + T, s0, dS)
    note(f"backward {dtype} B{B} T{T} H{H} S0={s0} dS={dS}")
    assert_grads(f"bwd_{dtype}_{B}_{T}_{H}", run_bwd(inp, dtype, dO, dSf), oracle_bwd(inp, dO, dSf))


@pytest.mark.parametrize("T", [0, 1, 7, 8, 9, 64, 65])
def test_backward_lengths(T):
    inp, dO, dSf = _case(2, T, 2, "bf16", 3 + T, True, True)
    note(f"backward lengths T={T}")
    got = run_bwd(inp, "bf16", dO, dSf)
    if T == 0:  # only dS0 = dS_T
        assert np.array_equal(got[5], dSf)
        return
    assert_grads(f"bwd_len{T}", got, oracle_bwd(inp, dO, dSf))


def test_backward_deterministic():
    inp, dO, dSf = _case(2, 100, 2, "bf16", 5, True, True)
    note("backward determinism")
    g1, g2 = run_bwd(inp, "bf16", dO, dSf), run_bwd(inp, "bf16", dO, dSf)
    assert all(np.array_equal(a, b) for a, b in zip(g1, g2))


def test_backward_full_size_sampled_chains():
    """The 8 x 2048 x 12 d64 bf16 layer, all chains on the GPU; sampled chains recomputed by the oracle."""
    w = WORKLOADS["sykra_layer_bf16"]
    inp = gen_workload(w)
    dO, dSf = gen_upstream_grads(w.B, w.T, w.H, w.dk, w.dv, seed=w.seed, with_dS=True)
    dO = bf16_round(dO)
    note("backward full size sykra_layer_bf16")
    t0 = time.perf_counter()
    got = run_bwd(inp, "bf16", dO, dSf)
    print(f"[backward] full size call + copies {time.perf_counter() - t0:.3f} s", flush=True)
    chains = [(0, 0), (5, 9)]
    sub = take_chains(inp, chains)
    dO_s = np.stack([dO[b, :, h] for b, h in chains], axis=1)[None]
    dS_s = np.stack([dSf[b, h] for b, h in chains])[None]
    ref = oracle_bwd(sub, dO_s, dS_s)
    pick = [np.stack([g[b, :, h] for b, h in chains], axis=1)[None] for g in got[:5]]
    pick.append(np.stack([got[5][b, h] for b, h in chains])[None])
    assert_grads("bwd_full", pick, ref)


def test_backward_extreme_gates():
    """Gates at their extremes on random tokens: alpha = 1e-6 (state wiped) or 1, beta = 0 or 2 (a full
    Householder reflection); the rest as drawn."""
    inp, dO, dSf = _case(2, 150, 2, "f32", 77, True, True)
    rng = np.random.default_rng(8)
    pa, pb = rng.random(inp["alpha"].shape), rng.random(inp["beta"].shape)
    inp["alpha"] = np.where(pa < 0.1, 1e-6, np.where(pa < 0.3, 1.0, inp["alpha"])).astype(np.float32)
    inp["beta"] = np.where(pb < 0.15, 0.0, np.where(pb < 0.3, 2.0, inp["beta"])).astype(np.float32)
    note("backward extreme gates")
    assert_grads("bwd_extreme", run_bwd(inp, "f32", dO, dSf), oracle_bwd(inp, dO, dSf))
