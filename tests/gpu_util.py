"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI, run the oracle on the same stored values, compare chain by chain."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle

# Tolerances, per (b, h) chain.
#   norm  relative Frobenius error of the chain's output [T, dv] and of its final state [dk, dv]
#         (the normwise bound: 1e-4 for fp32 / complex64 inputs, 2e-2 for bf16 inputs with fp32
#         accumulation);
#   token max over tokens of ||o_t - ref_t|| / (||ref_t|| + 0.1 rms_t ||ref_t||): a single wrong token row
#         cannot hide in the chain's norm.  2.5x the normwise bound: a row carries the same few roundings of
#         bf16 operands (2^-9 relative each) as the whole chain, without averaging over rows;
#   elem  max |o - ref| / max |ref| over the chain's output, and the same over its state: a single wrong
#         element at 2% of the chain's largest entry fails a bf16 check.  Equal to the normwise bound.
TOL = {"f32": 1e-4, "c64": 1e-4, "bf16": 2e-2}
TOKEN_TOL = {d: 2.5 * t for d, t in TOL.items()}
ELEM_TOL = dict(TOL)


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


def _chains(x):
    """[B, T, H, ...] -> [B*H, T, prod(...)] (one row per chain)."""
    x = np.asarray(x)
    B, T, H = x.shape[:3]
    return np.moveaxis(x, 2, 1).reshape(B * H, T, -1)


def chain_rel_errors(o, S, o_ref, S_ref):
    """Max over chains of the relative Frobenius error of o[b,:,h] and S[b,h]."""
    m = chain_metrics(o, S, o_ref, S_ref)
    return m["norm_o"].max(initial=0.0), m["norm_S"].max(initial=0.0)


def chain_metrics(o, S, o_ref, S_ref):
    """Per-chain error metrics (arrays over the B*H chains): norm_o, norm_S, token, elem_o, elem_S."""
    oc, rc = _chains(o), _chains(o_ref)
    C, T = rc.shape[:2]
    Sc = np.asarray(S).reshape(C, -1)
    Src = np.asarray(S_ref).reshape(C, -1)
    out = {k: np.zeros(C) for k in ("norm_o", "norm_S", "token", "elem_o", "elem_S")}
    for c in range(C):  # chain by chain keeps the fp64 temporaries small at full size
        r = rc[c].astype(np.complex128 if np.iscomplexobj(rc) else np.float64)
        d = oc[c] - r
        rown = np.linalg.norm(r, axis=1)
        n = np.linalg.norm(rown)
        if n > 0:
            out["norm_o"][c] = np.linalg.norm(d) / n
            floor = 0.1 * n / np.sqrt(T)
            out["token"][c] = np.max(np.linalg.norm(d, axis=1) / (rown + floor))
            out["elem_o"][c] = np.abs(d).max() / np.abs(r).max()
        rs = Src[c]
        ns = np.linalg.norm(rs)
        if ns > 0:
            ds = Sc[c] - rs
            out["norm_S"][c] = np.linalg.norm(ds) / ns
            out["elem_S"][c] = np.abs(ds).max() / np.abs(rs).max()
    return out


def oracle_chunk(inp, threads=0):
    o, S, _ = oracle.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp.get("S0"),
                                   threads=threads)
    return o, S


def assert_close(name, dtype, o, S, o_ref, S_ref):
    """Every chain within the normwise, per-token and elementwise bounds for its dtype; logs the worst of each."""
    assert np.isfinite(o).all() and np.isfinite(S).all(), name
    m = chain_metrics(o, S, o_ref, S_ref)
    worst = {k: float(v.max(initial=0.0)) for k, v in m.items()}
    print(f"[parity] {name}: {len(m['norm_o'])} chains, max rel err o={worst['norm_o']:.3e} "
          f"S={worst['norm_S']:.3e} token={worst['token']:.3e} elem o={worst['elem_o']:.3e} "
          f"S={worst['elem_S']:.3e} (tol {TOL[dtype]:g} / {TOKEN_TOL[dtype]:g} / {ELEM_TOL[dtype]:g})", flush=True)
    assert worst["norm_o"] <= TOL[dtype] and worst["norm_S"] <= TOL[dtype], (name, worst)
    assert worst["token"] <= TOKEN_TOL[dtype], (name, worst)
    assert worst["elem_o"] <= ELEM_TOL[dtype] and worst["elem_S"] <= ELEM_TOL[dtype], (name, worst)


def take_chains(inp, chains):
    """Inputs restricted to a list of (b, h) chains, as a [1, T, len, d] batch."""
    out = {}
    for key in ("q", "k", "v"):
        out[key] = np.stack([inp[key][b, :, h] for b, h in chains], axis=1)[None]
    for key in ("alpha", "beta"):
        out[key] = np.stack([inp[key][b, :, h] for b, h in chains], axis=1)[None]
    out["S0"] = None if inp.get("S0") is None else np.stack([inp["S0"][b, h] for b, h in chains])[None]
    return out
