"""The C-ABI library loads, exports every symbol include/gdn.h declares, and rejects
bad arguments before launching anything.  CPU only: no call here reaches a kernel
(every call either fails validation or has nothing to do)."""
import os
import re

import pytest

import linear_attention_sequence_gated_amd as gdn
from linear_attention_sequence_gated_amd import gdn as raw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000  # a 16-byte aligned fake address; validation rejects before any use


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = gdn.load()
    names = declared_functions()
    assert set(names) == set(raw.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(8):
        assert gdn.gdn_status_str(s).startswith("GDN_")
    assert "unknown" in gdn.gdn_status_str(99)


def chunk(**kw):
    args = dict(q=A, k=A, v=A, alpha=A, beta=A, S0=None, chunk=64, out=A, S_final=A, B=2, T=128, H=3, dk=64,
                dv=64, dtype=gdn.GDN_BF16, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return gdn.gdn_chunk_fwd(**args)


def step(**kw):
    args = dict(q=A, k=A, v=A, alpha=A, beta=A, S=A, out=A, N=16, dk=64, dv=64, dtype=gdn.GDN_BF16, stream=None)
    args.update(kw)
    return gdn.gdn_recurrent_step(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), raw.GDN_ERR_DTYPE),
    (dict(dtype=-1), raw.GDN_ERR_DTYPE),
    (dict(B=-1), raw.GDN_ERR_SHAPE),
    (dict(T=-5), raw.GDN_ERR_SHAPE),
    (dict(dk=0), raw.GDN_ERR_SHAPE),
    (dict(B=1 << 20, T=1 << 20, H=1 << 10), raw.GDN_ERR_SHAPE),
    (dict(chunk=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(dk=96, dv=96), raw.GDN_ERR_UNSUPPORTED),
    (dict(dk=64, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_F32, dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64, dk=64, dv=64), raw.GDN_ERR_UNSUPPORTED),
    (dict(q=None), raw.GDN_ERR_NULL),
    (dict(alpha=None), raw.GDN_ERR_NULL),
    (dict(out=None), raw.GDN_ERR_NULL),
    (dict(k=A + 8), raw.GDN_ERR_ALIGN),
    (dict(S0=A + 4), raw.GDN_ERR_ALIGN),
    (dict(S_final=A + 2), raw.GDN_ERR_ALIGN),
])
def test_chunk_argument_errors(kw, status):
    assert chunk(**kw) == status


def test_chunk_empty_is_noop():
    # no chains: nothing to launch, even with NULL inputs
    assert chunk(B=0, q=None, k=None, v=None, alpha=None, beta=None, out=None, S_final=None) == raw.GDN_OK
    assert chunk(H=0) == raw.GDN_OK


def prologue(**kw):
    args = dict(q=A, k=A, v=A, a_logit=A, b_logit=A, beta_scale=2.0, S0=None, chunk=64, out=A, S_final=A, B=2,
                T=128, H=3, dk=64, dv=64, dtype=gdn.GDN_BF16, stream=None)
    args.update(kw)
    return gdn.gdn_chunk_fwd_prologue(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), raw.GDN_ERR_DTYPE),
    (dict(T=-1), raw.GDN_ERR_SHAPE),
    (dict(beta_scale=-0.5), raw.GDN_ERR_SHAPE),
    (dict(beta_scale=2.5), raw.GDN_ERR_SHAPE),
    (dict(beta_scale=float("nan")), raw.GDN_ERR_SHAPE),
    (dict(chunk=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_F32), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64, dk=32, dv=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(B=1, T=1 << 22, H=64), raw.GDN_ERR_UNSUPPORTED),
    (dict(a_logit=None), raw.GDN_ERR_NULL),
    (dict(b_logit=None), raw.GDN_ERR_NULL),
    (dict(q=A + 8), raw.GDN_ERR_ALIGN),
    (dict(b_logit=A + 4), raw.GDN_ERR_ALIGN),
])
def test_prologue_argument_errors(kw, status):
    assert prologue(**kw) == status


def test_prologue_empty_is_noop():
    assert prologue(B=0, q=None, k=None, v=None, a_logit=None, b_logit=None, out=None, S_final=None) == raw.GDN_OK


def backward(**kw):
    args = dict(q=A, k=A, v=A, alpha=A, beta=A, S0=None, grad_out=A, grad_S_final=None, grad_q=A, grad_k=A, grad_v=A,
                grad_alpha=A, grad_beta=A, grad_S0=A, B=2, T=128, H=3, dk=64, dv=64, dtype=gdn.GDN_F32, workspace=A,
                workspace_bytes=1 << 30, stream=None)
    args.update(kw)
    return gdn.gdn_chunk_bwd(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), raw.GDN_ERR_DTYPE),
    (dict(H=-1), raw.GDN_ERR_SHAPE),
    (dict(dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dk=64, dv=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64, dk=32, dv=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(B=1, T=1 << 22, H=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(grad_out=None), raw.GDN_ERR_NULL),
    (dict(grad_beta=None), raw.GDN_ERR_NULL),
    (dict(alpha=None), raw.GDN_ERR_NULL),
    (dict(grad_k=A + 4), raw.GDN_ERR_ALIGN),
    (dict(workspace=None), raw.GDN_ERR_WORKSPACE),
    (dict(workspace_bytes=2 * 3 * 16 * 64 * 64 * 4 - 1), raw.GDN_ERR_WORKSPACE),
])
def test_backward_argument_errors(kw, status):
    assert backward(**kw) == status


def test_backward_empty_and_workspace_query():
    assert backward(B=0, q=None, k=None, v=None, alpha=None, beta=None, grad_out=None, grad_q=None, grad_k=None,
                    grad_v=None, grad_alpha=None, grad_beta=None, grad_S0=None, workspace=None,
                    workspace_bytes=0) == raw.GDN_OK
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 128, 3, 64, 64, gdn.GDN_BF16) == 2 * 3 * 16 * 64 * 64 * 4
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 129, 3, 64, 64, gdn.GDN_F32) == 2 * 3 * 17 * 64 * 64 * 4
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 0, 3, 64, 64, gdn.GDN_F32) == 0
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 128, 3, 64, 64, gdn.GDN_C64) == 0


def channel(**kw):
    args = dict(q=A, k=A, v=A, r=A, beta=A, S0=None, out=A, S_final=A, B=2, T=100, H=3, dk=64, dv=64,
                dtype=gdn.GDN_BF16, stream=None)
    args.update(kw)
    return gdn.gdn_fwd_channel_decay(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), raw.GDN_ERR_DTYPE),
    (dict(B=-2), raw.GDN_ERR_SHAPE),
    (dict(dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64, dk=32, dv=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(r=None), raw.GDN_ERR_NULL),
    (dict(out=None), raw.GDN_ERR_NULL),
    (dict(r=A + 4), raw.GDN_ERR_ALIGN),
])
def test_channel_decay_argument_errors(kw, status):
    assert channel(**kw) == status


def test_channel_decay_empty_is_noop():
    assert channel(H=0, q=None, k=None, v=None, r=None, beta=None, out=None, S_final=None) == raw.GDN_OK


def test_workspace_query():
    assert gdn.gdn_chunk_fwd_workspace_bytes(8, 2048, 12, 64, 64, 64, gdn.GDN_BF16) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), raw.GDN_ERR_DTYPE),
    (dict(N=-1), raw.GDN_ERR_SHAPE),
    (dict(dk=48, dv=48), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64), raw.GDN_ERR_UNSUPPORTED),
    (dict(S=None), raw.GDN_ERR_NULL),
    (dict(v=None), raw.GDN_ERR_NULL),
    (dict(out=A + 8), raw.GDN_ERR_ALIGN),
])
def test_step_argument_errors(kw, status):
    assert step(**kw) == status


def test_step_empty_is_noop():
    assert step(N=0, q=None, S=None) == raw.GDN_OK


def test_torch_helper_rejects_bad_shapes_on_cpu():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # host tensors are refused before any HIP call
        gdn.chunk_fwd(q, q, q, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1))
    with pytest.raises(TypeError):
        gdn.chunk_fwd(q.to(torch.float16), q, q, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1))
    with pytest.raises(ValueError):
        gdn.recurrent_step(q[0, 0], q[0, 0], q[0, 0], torch.zeros(1), torch.zeros(1), torch.zeros(1, 64, 64))
