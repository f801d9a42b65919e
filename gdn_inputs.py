"""Seeded synthetic inputs for the gated delta rule, shared by the tests and the benchmark.

This module only draws random numbers and stores them in the precision the
kernels read.  It holds none of the method's arithmetic; both the HIP path and
the CPU oracle consume exactly the arrays returned here.

Recipe (all draws from ``numpy.random.default_rng(seed)``, in this order):

real workloads
    q, k ~ N(0, 1)  [B, T, H, dk], each token's vector scaled to unit L2 norm (fp64)
    v    ~ N(0, 1)  [B, T, H, dv]
    beta  = beta_scale * sigmoid(N(0, 1))          [B, T, H]
    alpha = exp(-softplus(N(alpha_mu, 1)))         [B, T, H]
    S0   ~ N(0, s0_var) [B, H, dk, dv] when s0_var is given (variance, not std)
complex workloads
    theta_q, theta_k ~ U(0, 2 pi) [B, T, H, dk];  q = exp(i theta_q) / sqrt(dk), same for k
    v = (N(0, 1/2) + i N(0, 1/2))  [B, T, H, dv]    (circular complex normal, unit variance)
    beta, alpha as above; S0 complex normal with variance s0_var when given
decode
    S ~ N(0, s_var) [N, dk, dv] fp32, then for each step (step index outermost) the
    token draws q, k, v, beta-logit, alpha-logit as in the real recipe with B*T*H -> N.
raw layer inputs (for the fused-prologue entry point)
    q, k ~ N(0, 1) [B, T, H, dk], each token's vector scaled by its own U(0.25, 4)
         factor (not normalised)
    v    ~ N(0, 1) [B, T, H, dv]
    b    ~ N(0, 1), a ~ N(alpha_mu, 1)  [B, T, H]   (the logits, stored as drawn)
    S0   as above when s0_var is given

Storage: q, k, v are cast fp64 -> fp32 -> bf16 (round to nearest even) for bf16
workloads, fp32 / complex64 otherwise; alpha, beta and states are fp32
(complex64 states for complex data).  Arrays are returned as float32/complex64
NumPy arrays whose values are exactly representable in the stored dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returns float32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    return (r.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload shape.  ``kind`` is 'chunk', 'prologue' (raw layer inputs), 'backward', 'channel' or 'decode'."""
    name: str
    kind: str
    dtype: str  # 'f32', 'bf16' or 'c64'
    B: int = 1
    T: int = 1
    H: int = 1
    dk: int = 64
    dv: int = 64
    chunk: int = 64
    alpha_mu: float = -4.0
    beta_scale: float = 1.0
    s0_var: float | None = None
    N: int = 0
    steps: int = 0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads, shaped like the models the pages describe.
WORKLOADS = {
    "single_head_f32": Workload(
        "single_head_f32", "chunk", "f32", B=1, T=256, H=1, dk=64, dv=64, seed=0,
        note="one head, T=256, d=64, fp32, zero initial state"),
    "sykra_layer_bf16": Workload(
        "sykra_layer_bf16", "chunk", "bf16", B=8, T=2048, H=12, dk=64, dv=64, seed=1,
        note="Sykra-shaped layer: hidden 768 = 12 heads x 64, chunk 64, bf16 q/k/v"),
    "long_context_bf16": Workload(
        "long_context_bf16", "chunk", "bf16", B=2, T=16384, H=16, dk=128, dv=128, seed=2,
        alpha_mu=-5.0, s0_var=0.01, note="long context, d=128, slow decay, nonzero S0"),
    "long_sequence_bf16": Workload(
        "long_sequence_bf16", "chunk", "bf16", B=1, T=65536, H=12, dk=64, dv=64, seed=5,
        note="the Sykra-shaped layer over one 65536-token sequence (the longest length DeltaPhase times)"),
    "deltaphase_c64": Workload(
        "deltaphase_c64", "chunk", "c64", B=4, T=4096, H=8, dk=32, dv=32, seed=3,
        beta_scale=2.0, note="complex phasor keys/queries, beta in (0, 2)"),
    "sykra_layer_bf16_prologue": Workload(
        "sykra_layer_bf16_prologue", "prologue", "bf16", B=8, T=2048, H=12, dk=64, dv=64, seed=1,
        note="the Sykra-shaped layer from raw inputs: q, k not normalised, gate logits a, b"),
    "long_context_bf16_prologue": Workload(
        "long_context_bf16_prologue", "prologue", "bf16", B=2, T=16384, H=16, dk=128, dv=128, seed=2,
        alpha_mu=-5.0, s0_var=0.01, note="the long-context d=128 layer from raw inputs"),
    "deltaphase_c64_prologue": Workload(
        "deltaphase_c64_prologue", "prologue", "c64", B=4, T=4096, H=8, dk=32, dv=32, seed=3, beta_scale=2.0,
        note="the complex phasor layer from raw inputs: phasor rows of any modulus, beta = 2 sigmoid(b)"),
    "single_head_f32_prologue": Workload(
        "single_head_f32_prologue", "prologue", "f32", B=1, T=256, H=1, dk=64, dv=64, seed=0,
        note="one fp32 head from raw inputs"),
    "sykra_layer_bf16_bwd": Workload(
        "sykra_layer_bf16_bwd", "backward", "bf16", B=8, T=2048, H=12, dk=64, dv=64, seed=1,
        note="gradients of the Sykra-shaped layer (inputs as sykra_layer_bf16, upstream dO, dS_T ~ N(0,1))"),
    "long_context_bf16_bwd": Workload(
        "long_context_bf16_bwd", "backward", "bf16", B=2, T=16384, H=16, dk=128, dv=128, seed=2,
        alpha_mu=-5.0, s0_var=0.01,
        note="gradients of the long-context d=128 layer (inputs as long_context_bf16, upstream dO, dS_T ~ N(0,1))"),
    "deltaphase_c64_bwd": Workload(
        "deltaphase_c64_bwd", "backward", "c64", B=4, T=4096, H=8, dk=32, dv=32, seed=3, beta_scale=2.0,
        note="gradients of the complex phasor layer (inputs as deltaphase_c64, complex upstream dO, dS_T)"),
    "sykra_layer_bf16_channel_decay": Workload(
        "sykra_layer_bf16_channel_decay", "channel", "bf16", B=8, T=2048, H=12, dk=64, dv=64, seed=1,
        note="the Sykra-shaped layer with a decay per token and value channel (DeltaPhase section 5)"),
    "laplace_c64_channel_decay": Workload(
        "laplace_c64_channel_decay", "channel", "c64", B=4, T=4096, H=8, dk=32, dv=32, seed=6,
        note="LaplacePhaseCore-shaped: complex keys e^{(sigma + i omega) dt} / sqrt(32), decay per token and "
             "value channel (DeltaPhase section 5)"),
    "decode_4096x64": Workload(
        "decode_4096x64", "decode", "bf16", N=4096, dk=64, dv=64, steps=64, seed=4,
        s0_var=0.1, note="4096 independent 64x64 states, 64 single-token steps"),
}


def _store(x, dtype: str):
    if dtype == "bf16":
        return bf16_round(x.astype(np.float32))
    if dtype == "c64":
        return x.astype(np.complex64)
    return x.astype(np.float32)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def gen_chunk(B, T, H, dk, dv, dtype="f32", seed=0, alpha_mu=-4.0, beta_scale=1.0, s0_var=None):
    """Inputs for the chunked forward.  Returns dict q, k, v, alpha, beta, S0 (None if absent)."""
    rng = np.random.default_rng(seed)
    if dtype == "c64":
        th_q = rng.uniform(0.0, 2.0 * np.pi, (B, T, H, dk))
        th_k = rng.uniform(0.0, 2.0 * np.pi, (B, T, H, dk))
        q = np.exp(1j * th_q) / np.sqrt(dk)
        k = np.exp(1j * th_k) / np.sqrt(dk)
        v = rng.normal(0.0, np.sqrt(0.5), (B, T, H, dv)) + 1j * rng.normal(0.0, np.sqrt(0.5), (B, T, H, dv))
    else:
        q = _unit_rows(rng.normal(0.0, 1.0, (B, T, H, dk)))
        k = _unit_rows(rng.normal(0.0, 1.0, (B, T, H, dk)))
        v = rng.normal(0.0, 1.0, (B, T, H, dv))
    beta = beta_scale * _sigmoid(rng.normal(0.0, 1.0, (B, T, H)))
    alpha = np.exp(-_softplus(rng.normal(alpha_mu, 1.0, (B, T, H))))
    S0 = None
    if s0_var is not None:
        sd = np.sqrt(s0_var)
        if dtype == "c64":
            S0 = (rng.normal(0.0, sd * np.sqrt(0.5), (B, H, dk, dv))
                  + 1j * rng.normal(0.0, sd * np.sqrt(0.5), (B, H, dk, dv))).astype(np.complex64)
        else:
            S0 = rng.normal(0.0, sd, (B, H, dk, dv)).astype(np.float32)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
                alpha=alpha.astype(np.float32), beta=beta.astype(np.float32), S0=S0)


def gen_raw_layer(B, T, H, d, seed=0, alpha_mu=-4.0, s0_var=None, dtype="bf16"):
    """Raw q, k, v and fp32 logits for the fused-prologue entry point.

    Real dtypes: q, k ~ N(0, 1) rows, each row scaled by its own U(0.25, 4) factor (not normalised), v ~ N(0, 1).
    Complex: q, k rows of unit phasors e^{i theta}, theta ~ U(0, 2 pi), each row scaled by its own U(0.25, 4)
    factor (the transforms normalise them to e^{i theta} / sqrt(d)), v complex normal.  Logits b ~ N(0, 1),
    a ~ N(alpha_mu, 1).  Returns dict q, k, v (values in stored precision), a_logit, b_logit, S0 (None if
    absent)."""
    rng = np.random.default_rng(seed)
    if dtype == "c64":
        q = np.exp(1j * rng.uniform(0.0, 2.0 * np.pi, (B, T, H, d))) * rng.uniform(0.25, 4.0, (B, T, H, 1))
        k = np.exp(1j * rng.uniform(0.0, 2.0 * np.pi, (B, T, H, d))) * rng.uniform(0.25, 4.0, (B, T, H, 1))
        v = rng.normal(0.0, np.sqrt(0.5), (B, T, H, d)) + 1j * rng.normal(0.0, np.sqrt(0.5), (B, T, H, d))
    else:
        q = rng.normal(0.0, 1.0, (B, T, H, d)) * rng.uniform(0.25, 4.0, (B, T, H, 1))
        k = rng.normal(0.0, 1.0, (B, T, H, d)) * rng.uniform(0.25, 4.0, (B, T, H, 1))
        v = rng.normal(0.0, 1.0, (B, T, H, d))
    b = rng.normal(0.0, 1.0, (B, T, H))
    a = rng.normal(alpha_mu, 1.0, (B, T, H))
    S0 = None
    if s0_var is not None:
        sd = np.sqrt(s0_var)
        if dtype == "c64":
            S0 = (rng.normal(0.0, sd * np.sqrt(0.5), (B, H, d, d))
                  + 1j * rng.normal(0.0, sd * np.sqrt(0.5), (B, H, d, d))).astype(np.complex64)
        else:
            S0 = rng.normal(0.0, sd, (B, H, d, d)).astype(np.float32)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype), a_logit=a.astype(np.float32),
                b_logit=b.astype(np.float32), S0=S0)


def gen_upstream_grads(B, T, H, dk, dv, seed=0, with_dS=True, dtype="f32"):
    """Upstream gradients for the backward: dO ~ N(0, 1) [B, T, H, dv] stored in fp32 (cast to the
    forward's dtype by the caller) and, if asked, dS_T ~ N(0, 1) [B, H, dk, dv] fp32.  dtype 'c64': complex
    normal, real and imaginary parts N(0, 1/2) each, stored as complex64."""
    rng = np.random.default_rng(seed + 1000)
    if dtype == "c64":
        s = np.sqrt(0.5)
        dO = (rng.normal(0.0, s, (B, T, H, dv)) + 1j * rng.normal(0.0, s, (B, T, H, dv))).astype(np.complex64)
        dS = ((rng.normal(0.0, s, (B, H, dk, dv)) + 1j * rng.normal(0.0, s, (B, H, dk, dv))).astype(np.complex64)
              if with_dS else None)
        return dO, dS
    dO = rng.normal(0.0, 1.0, (B, T, H, dv)).astype(np.float32)
    dS = rng.normal(0.0, 1.0, (B, H, dk, dv)).astype(np.float32) if with_dS else None
    return dO, dS


def gen_channel_decay(B, T, H, d, dtype="bf16", seed=0, alpha_mu=-4.0, s0_var=None):
    """Inputs for the per-output-channel decay: q, k unit-norm rows and v ~ N(0, 1) as in gen_chunk,
    beta = sigmoid(N(0, 1)) [B, T, H], and r = exp(-softplus(N(alpha_mu, 1))) drawn per token and value
    channel [B, T, H, d] (fp32).  Returns dict q, k, v, r, beta, S0."""
    base = gen_chunk(B, T, H, d, d, dtype=dtype, seed=seed, alpha_mu=alpha_mu, s0_var=s0_var)
    rng = np.random.default_rng(seed + 2000)
    logit = rng.normal(alpha_mu, 1.0, (B, T, H, d))
    r = np.exp(-(np.maximum(logit, 0.0) + np.log1p(np.exp(-np.abs(logit)))))
    k = base["k"]
    if dtype == "c64":
        # LaplacePhaseCore-shaped keys e^{(sigma + i omega) dt} / sqrt(d): the unit phasors of gen_chunk times
        # a per-element modulus e^{sigma dt} with sigma dt ~ U(-0.5, 0].
        k = (k * np.exp(-rng.uniform(0.0, 0.5, k.shape))).astype(np.complex64)
    return dict(q=base["q"], k=k, v=base["v"], r=r.astype(np.float32), beta=base["beta"], S0=base["S0"])


def gen_workload(w: Workload, **overrides):
    """Inputs for a named chunk workload (fields may be overridden, e.g. T=...)."""
    p = dict(B=w.B, T=w.T, H=w.H, dk=w.dk, dv=w.dv, dtype=w.dtype, seed=w.seed,
             alpha_mu=w.alpha_mu, beta_scale=w.beta_scale, s0_var=w.s0_var)
    p.update(overrides)
    if w.kind == "channel":
        return gen_channel_decay(p["B"], p["T"], p["H"], p["dk"], dtype=p["dtype"], seed=p["seed"],
                                 alpha_mu=p["alpha_mu"], s0_var=p["s0_var"])
    if w.kind == "prologue":
        return gen_raw_layer(p["B"], p["T"], p["H"], p["dk"], seed=p["seed"], alpha_mu=p["alpha_mu"],
                             s0_var=p["s0_var"], dtype=p["dtype"])
    return gen_chunk(**p)


def gen_decode(N, dk, dv, steps, dtype="bf16", seed=4, s_var=0.1, alpha_mu=-4.0, beta_scale=1.0):
    """Inputs for repeated decode steps.

    Returns dict S [N, dk, dv] and per-step q, k [steps, N, dk], v [steps, N, dv],
    alpha, beta [steps, N].
    """
    rng = np.random.default_rng(seed)
    sd = np.sqrt(s_var)
    if dtype == "c64":
        S = (rng.normal(0.0, sd * np.sqrt(0.5), (N, dk, dv))
             + 1j * rng.normal(0.0, sd * np.sqrt(0.5), (N, dk, dv))).astype(np.complex64)
    else:
        S = rng.normal(0.0, sd, (N, dk, dv)).astype(np.float32)
    qs, ks, vs, bs, as_ = [], [], [], [], []
    for _ in range(steps):
        if dtype == "c64":
            q = np.exp(1j * rng.uniform(0.0, 2.0 * np.pi, (N, dk))) / np.sqrt(dk)
            k = np.exp(1j * rng.uniform(0.0, 2.0 * np.pi, (N, dk))) / np.sqrt(dk)
            v = rng.normal(0.0, np.sqrt(0.5), (N, dv)) + 1j * rng.normal(0.0, np.sqrt(0.5), (N, dv))
        else:
            q = _unit_rows(rng.normal(0.0, 1.0, (N, dk)))
            k = _unit_rows(rng.normal(0.0, 1.0, (N, dk)))
            v = rng.normal(0.0, 1.0, (N, dv))
        bs.append(beta_scale * _sigmoid(rng.normal(0.0, 1.0, (N,))))
        as_.append(np.exp(-_softplus(rng.normal(alpha_mu, 1.0, (N,)))))
        qs.append(_store(q, dtype)); ks.append(_store(k, dtype)); vs.append(_store(v, dtype))
    return dict(S=S, q=np.stack(qs), k=np.stack(ks), v=np.stack(vs),
                alpha=np.stack(as_).astype(np.float32), beta=np.stack(bs).astype(np.float32))


def gen_decode_workload(w: Workload, **overrides):
    p = dict(N=w.N, dk=w.dk, dv=w.dv, steps=w.steps, dtype=w.dtype, seed=w.seed,
             s_var=w.s0_var, alpha_mu=w.alpha_mu, beta_scale=w.beta_scale)
    p.update(overrides)
    return gen_decode(**p)
