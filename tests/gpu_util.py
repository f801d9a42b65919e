"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI, run the oracle on the same stored values, compare chain by chain."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle

# Tolerances: relative Frobenius error of each chain's output [T, dv] and final
# state [dk, dv].  fp32 / complex64 inputs: 1e-4.  bf16 inputs with fp32
# accumulation: 2e-2 (normwise).
TOL = {"f32": 1e-4, "c64": 1e-4, "bf16": 2e-2}


def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import linear_attention_sequence_gated_amd as gdn
    gdn.load()  # where a GPU is present the library must load; a missing build is an error, not a skip
    return torch


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def up(x, dtype: str):
    """numpy (already in stored precision) -> device tensor of the stored dtype."""
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16" and t.dtype == torch.float32:
        t = t.to(torch.bfloat16)
    return t.to("cuda")


def down(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def run_chunk(inp, dtype, S0=True, S_final_alias=False):
    import torch
    import linear_attention_sequence_gated_amd as gdn
    q, k, v = up(inp["q"], dtype), up(inp["k"], dtype), up(inp["v"], dtype)
    a, b = up(inp["alpha"], "f32"), up(inp["beta"], "f32")
    s0 = up(inp["S0"], "f32") if (S0 and inp.get("S0") is not None) else None
    if S_final_alias and s0 is not None:
        o, S = gdn.chunk_fwd(q, k, v, a, b, s0, S_final=s0)
    else:
        o, S = gdn.chunk_fwd(q, k, v, a, b, s0)
    torch.cuda.synchronize()
    return down(o), down(S)


def chain_rel_errors(o, S, o_ref, S_ref):
    """Max over chains of the relative Frobenius error of o[b,:,h] and S[b,h]."""
    B, T, H, _ = o_ref.shape
    eo, es = 0.0, 0.0
    for bb in range(B):
        for hh in range(H):
            r = o_ref[bb, :, hh]
            n = np.linalg.norm(r)
            if n > 0:
                eo = max(eo, np.linalg.norm(o[bb, :, hh] - r) / n)
            rs = S_ref[bb, hh]
            ns = np.linalg.norm(rs)
            if ns > 0:
                es = max(es, np.linalg.norm(S[bb, hh] - rs) / ns)
    return eo, es


def oracle_chunk(inp, threads=0):
    o, S, _ = oracle.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp.get("S0"),
                                   threads=threads)
    return o, S


def assert_close(name, dtype, o, S, o_ref, S_ref):
    eo, es = chain_rel_errors(o, S, o_ref, S_ref)
    tol = TOL[dtype]
    print(f"[parity] {name}: max chain rel err o={eo:.3e} S={es:.3e} (tol {tol:g})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all(), name
    assert eo <= tol and es <= tol, (name, eo, es, tol)


def take_chains(inp, chains):
    """Inputs restricted to a list of (b, h) chains, as a [1, T, len, d] batch."""
    out = {}
    for key in ("q", "k", "v"):
        out[key] = np.stack([inp[key][b, :, h] for b, h in chains], axis=1)[None]
    for key in ("alpha", "beta"):
        out[key] = np.stack([inp[key][b, :, h] for b, h in chains], axis=1)[None]
    out["S0"] = None if inp.get("S0") is None else np.stack([inp["S0"][b, h] for b, h in chains])[None]
    return out
