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


def declared_functions(header="gdn.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_every_header_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["gdn.h", "gdn_peak.h"]


def test_peak_library_exports_its_header():
    """libgdn_peak.so (the benchmark's measured-peak loops) exports what include/gdn_peak.h declares and
    rejects bad arguments without launching."""
    import ctypes
    from linear_attention_sequence_gated_amd import build as gbuild
    lib = ctypes.CDLL(gbuild.PEAK_LIB)
    names = declared_functions("gdn_peak.h")
    assert names == ["gdn_peak_mfma_loop", "gdn_peak_read"]
    fn = lib.gdn_peak_mfma_loop
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert fn(3, 10, 1, A, None) == -1
    assert fn(0, 0, 1, A, None) == -1
    assert fn(0, 10, 0, A, None) == -1
    assert fn(1, 10, 1, None, None) == -1
    rd = lib.gdn_peak_read
    rd.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert rd(None, 1024, 1, A, None) == -1
    assert rd(A + 4, 1024, 1, A, None) == -1
    assert rd(A, 1024, 0, A, None) == -1
    assert rd(A, 1024, 1, None, None) == -1


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
    (dict(B=1 << 10, T=1, H=1 << 10), raw.GDN_ERR_SHAPE),  # 2^20 chains x 4096 threads: past the launch limit
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


def test_chunk_bf16_d128_needs_its_workspace():
    need = gdn.gdn_chunk_fwd_workspace_bytes(2, 128, 3, 128, 128, 64, gdn.GDN_BF16)
    assert need == 2 * 3 * 2 * 6400
    assert chunk(dk=128, dv=128, workspace=None, workspace_bytes=0) == raw.GDN_ERR_WORKSPACE
    assert chunk(dk=128, dv=128, workspace=A, workspace_bytes=need - 1) == raw.GDN_ERR_WORKSPACE


def test_long_sequence_few_chains_takes_the_segmented_scan():
    # one 65536-token sequence of a 12-head d = 64 layer: 12 chains leave most CUs idle, so the call runs
    # the two-level scan with 10 segments (factor records, segment maps [dk, dk + dv], start states): 103
    # chunks per segment, the map launch in two rounds of the 256 CUs and the output launch in one
    need = gdn.gdn_chunk_fwd_workspace_bytes(1, 65536, 12, 64, 64, 64, gdn.GDN_BF16)
    assert need == 12 * 1024 * 6400 + 12 * 10 * (64 * 128 + 64 * 64) * 4


def prologue(**kw):
    args = dict(q=A, k=A, v=A, a_logit=A, b_logit=A, beta_scale=2.0, S0=None, chunk=64, out=A, S_final=A, B=2,
                T=128, H=3, dk=64, dv=64, dtype=gdn.GDN_BF16, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return gdn.gdn_chunk_fwd_prologue(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), raw.GDN_ERR_DTYPE),
    (dict(T=-1), raw.GDN_ERR_SHAPE),
    (dict(beta_scale=-0.5), raw.GDN_ERR_SHAPE),
    (dict(beta_scale=2.5), raw.GDN_ERR_SHAPE),
    (dict(beta_scale=float("nan")), raw.GDN_ERR_SHAPE),
    (dict(chunk=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(dk=128, dv=128), raw.GDN_ERR_WORKSPACE),                # d128 runs the two-launch path
    (dict(dtype=gdn.GDN_F32), raw.GDN_ERR_WORKSPACE),             # fp32: the row pass writes to the workspace
    (dict(dtype=gdn.GDN_C64, dk=32, dv=32), raw.GDN_ERR_WORKSPACE),
    (dict(dtype=gdn.GDN_F32, dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),  # fp32: d = 64 only
    (dict(dtype=gdn.GDN_C64), raw.GDN_ERR_UNSUPPORTED),         # complex: d = 32 only
    (dict(dk=32, dv=32), raw.GDN_ERR_UNSUPPORTED),                # real: d = 64 only
    (dict(dtype=gdn.GDN_C64, dk=32, dv=64), raw.GDN_ERR_UNSUPPORTED),
    (dict(B=1, T=1 << 22, H=64), raw.GDN_ERR_UNSUPPORTED),
    # d128 factor grid: 2^26 chunks x 64 threads reach the launch limit; one chunk fewer per chain still fits
    (dict(B=1 << 10, T=1 << 18, H=16, dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(B=1 << 10, T=(1 << 18) - 64, H=16, dk=128, dv=128), raw.GDN_ERR_WORKSPACE),
    (dict(a_logit=None), raw.GDN_ERR_NULL),
    (dict(b_logit=None), raw.GDN_ERR_NULL),
    (dict(q=A + 8), raw.GDN_ERR_ALIGN),
    (dict(b_logit=A + 4), raw.GDN_ERR_ALIGN),
])
def test_prologue_argument_errors(kw, status):
    assert prologue(**kw) == status


def test_prologue_workspace_sizes():
    """bf16 needs what the plain forward needs, plus 1/|k| per token (256 bytes per chunk) on the
    two-launch path;
    fp32 and complex64 hold the transformed q, k (256-byte rows) and the two gates, each rounded up to 256 bytes,
    and complex64 adds the forward's own workspace."""
    rows = 2 * 128 * 3
    rowpass = 2 * (rows * 256) + 2 * ((rows * 4 + 255) // 256 * 256)
    assert gdn.gdn_chunk_fwd_prologue_workspace_bytes(2, 128, 3, 64, 64, 64, gdn.GDN_BF16) == 0
    assert gdn.gdn_chunk_fwd_prologue_workspace_bytes(2, 128, 3, 128, 128, 64, gdn.GDN_BF16) == 2 * 3 * 2 * (6400 + 256)
    assert gdn.gdn_chunk_fwd_prologue_workspace_bytes(2, 128, 3, 64, 64, 64, gdn.GDN_F32) == rowpass
    assert gdn.gdn_chunk_fwd_prologue_workspace_bytes(2, 128, 3, 32, 32, 64, gdn.GDN_C64) == rowpass + 2 * 3 * 2 * 57600
    assert gdn.gdn_chunk_fwd_prologue_workspace_bytes(2, 128, 3, 64, 64, 64, gdn.GDN_C64) == 0   # unsupported
    need = gdn.gdn_chunk_fwd_prologue_workspace_bytes(2, 128, 3, 64, 64, 64, gdn.GDN_F32)
    assert prologue(dtype=gdn.GDN_F32, workspace=A, workspace_bytes=need - 1) == raw.GDN_ERR_WORKSPACE
    assert prologue(dtype=gdn.GDN_F32, workspace=A + 8, workspace_bytes=need) == raw.GDN_ERR_ALIGN


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
    (dict(B=1 << 11, T=1, H=1 << 12), raw.GDN_ERR_SHAPE),  # 2^23 chains x 512 threads
    (dict(dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),              # fp32: d = 64 only
    # bf16 d128 gradient grid: 2^23 chunks x 512 threads reach the launch limit; one chunk fewer per chain fits
    (dict(dtype=gdn.GDN_BF16, B=1 << 10, T=1 << 15, H=16, dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_BF16, B=1 << 10, T=(1 << 15) - 64, H=16, dk=128, dv=128), raw.GDN_ERR_WORKSPACE),
    (dict(dtype=gdn.GDN_BF16, dk=128, dv=64), raw.GDN_ERR_UNSUPPORTED),
    (dict(dk=64, dv=32), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64), raw.GDN_ERR_UNSUPPORTED),         # complex: d = 32 only
    (dict(dk=32, dv=32), raw.GDN_ERR_UNSUPPORTED),                # real: d = 64 only
    (dict(dtype=gdn.GDN_C64, dk=32, dv=64), raw.GDN_ERR_UNSUPPORTED),
    (dict(B=1, T=1 << 22, H=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64, dk=32, dv=32, B=1, T=1 << 22, H=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64, dk=32, dv=32, workspace=None), raw.GDN_ERR_WORKSPACE),
    (dict(dtype=gdn.GDN_C64, dk=32, dv=32, workspace_bytes=2 * 3 * 16 * 32 * 32 * 8 - 1), raw.GDN_ERR_WORKSPACE),
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
    # bf16: the matrix-core path -- two 6400-byte records, a bf16 start state and a bf16 end gradient per chunk
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 128, 3, 64, 64, gdn.GDN_BF16) == 2 * 3 * 2 * (2 * 6400 + 2 * 8192)
    # bf16 d = 128: also U and dX (bf16 64 x 128) and 64 fp32 dg terms per chunk
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 128, 3, 128, 128, gdn.GDN_BF16) == \
        2 * 3 * 2 * (2 * 6400 + 2 * 128 * 128 * 2 + 2 * 64 * 128 * 2 + 64 * 4)
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 0, 3, 128, 128, gdn.GDN_BF16) == 0
    # fp32: the token-by-token pass in 8 column groups -- the state every 8 tokens, and each group's share
    # of dq, dk (64 floats each) and of dalpha, dbeta per token-head
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 129, 3, 64, 64, gdn.GDN_F32) == \
        2 * 3 * 17 * 64 * 64 * 4 + 8 * (2 * 129 * 3) * (2 * 64 + 2) * 4
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 0, 3, 64, 64, gdn.GDN_F32) == 0
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 128, 3, 64, 64, gdn.GDN_C64) == 0
    # complex64 d = 32: the same in 8 column groups of 4 columns, complex values
    assert gdn.gdn_chunk_bwd_workspace_bytes(2, 129, 3, 32, 32, gdn.GDN_C64) == \
        2 * 3 * 17 * 32 * 32 * 8 + 8 * (2 * 129 * 3) * (2 * 32 * 2 + 2) * 4


def channel(**kw):
    args = dict(q=A, k=A, v=A, r=A, beta=A, S0=None, out=A, S_final=A, B=2, T=100, H=3, dk=64, dv=64,
                dtype=gdn.GDN_BF16, stream=None)
    args.update(kw)
    return gdn.gdn_fwd_channel_decay(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), raw.GDN_ERR_DTYPE),
    (dict(B=-2), raw.GDN_ERR_SHAPE),
    (dict(B=1 << 10, T=1, H=1 << 12), raw.GDN_ERR_SHAPE),  # 2^22 chains x 1024 threads
    (dict(dk=128, dv=128), raw.GDN_ERR_UNSUPPORTED),
    (dict(dtype=gdn.GDN_C64), raw.GDN_ERR_UNSUPPORTED),         # complex: d = 32 only
    (dict(dk=32, dv=32), raw.GDN_ERR_UNSUPPORTED),                # real: d = 64 only
    (dict(dtype=gdn.GDN_C64, dk=32, dv=64), raw.GDN_ERR_UNSUPPORTED),
    (dict(r=None), raw.GDN_ERR_NULL),
    (dict(out=None), raw.GDN_ERR_NULL),
    (dict(r=A + 4), raw.GDN_ERR_ALIGN),
])
def test_channel_decay_argument_errors(kw, status):
    assert channel(**kw) == status


def test_channel_decay_empty_is_noop():
    assert channel(H=0, q=None, k=None, v=None, r=None, beta=None, out=None, S_final=None) == raw.GDN_OK


def test_workspace_query():
    # d = 64 bf16 with enough chains and fp32: the fused kernels keep everything on chip
    assert gdn.gdn_chunk_fwd_workspace_bytes(8, 2048, 12, 64, 64, 64, gdn.GDN_BF16) == 0
    # d = 128 bf16: one 6400-byte factor record per (chain, chunk)
    assert gdn.gdn_chunk_fwd_workspace_bytes(2, 16384, 16, 128, 128, 64, gdn.GDN_BF16) == 2 * 16 * 256 * 6400
    assert gdn.gdn_chunk_fwd_workspace_bytes(1, 65, 1, 64, 64, 64, gdn.GDN_F32) == 0
    assert gdn.gdn_chunk_fwd_workspace_bytes(2, 0, 3, 64, 64, 64, gdn.GDN_BF16) == 0
    # a long sequence with few chains adds the segment maps and start states of the two-level scan
    G = 16  # 1 chain x 8 slices: 15 x 16 map workgroups and 16 x 8 output workgroups fit 256 CUs
    assert gdn.gdn_chunk_fwd_workspace_bytes(1, 65536, 1, 128, 128, 64, gdn.GDN_BF16) == \
        1024 * 6400 + G * (128 * 256 + 128 * 128) * 4


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), raw.GDN_ERR_DTYPE),
    (dict(N=-1), raw.GDN_ERR_SHAPE),
    (dict(N=1 << 24), raw.GDN_ERR_SHAPE),  # 2^24 states x 256 threads
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


def test_torch_helpers_reject_non_contiguous_q():
    """A transposed (non-contiguous) q is refused by every helper, not read as if it were dense."""
    torch = pytest.importorskip("torch")
    qt = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16).transpose(1, 2)  # [1, 4, 2, 64], strided
    x = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    g = torch.zeros(1, 4, 2)
    for call in (lambda: gdn.chunk_fwd(qt, x, x, g, g),
                 lambda: gdn.chunk_fwd_prologue(qt, x, x, g, g),
                 lambda: gdn.chunk_bwd(qt, x, x, g, g, x),
                 lambda: gdn.fwd_channel_decay(qt, x, x, torch.zeros(1, 4, 2, 64), g)):
        with pytest.raises(ValueError, match="q: must be contiguous"):
            call()
    q2 = torch.zeros(64, 3, dtype=torch.bfloat16).t()  # [3, 64], strided
    with pytest.raises(ValueError, match="q: must be contiguous"):
        gdn.recurrent_step(q2, q2.contiguous(), q2.contiguous(), torch.zeros(3), torch.zeros(3), torch.zeros(3, 64, 64))


def test_noalloc_rejects_sizes_past_its_scratch():
    """gdn_chunk_fwd_noalloc refuses a call whose workspace exceeds its fixed scratch array, before any HIP call,
    and reports argument errors as gdn_chunk_fwd does."""
    args = dict(q=A, k=A, v=A, alpha=A, beta=A, S0=None, chunk=64, out=A, S_final=A, B=4, T=65536, H=16, dk=128,
                dv=128, dtype=gdn.GDN_BF16, stream=None)
    assert gdn.gdn_chunk_fwd_workspace_bytes(4, 65536, 16, 128, 128, 64, gdn.GDN_BF16) > gdn.GDN_NOALLOC_MAX_WORKSPACE
    assert gdn.gdn_chunk_fwd_noalloc(**args) == raw.GDN_ERR_WORKSPACE
    assert gdn.gdn_chunk_fwd_noalloc(**dict(args, dtype=9)) == raw.GDN_ERR_DTYPE
    assert gdn.gdn_chunk_fwd_noalloc(**dict(args, B=-1)) == raw.GDN_ERR_SHAPE
    assert gdn.gdn_chunk_fwd_noalloc(**dict(args, B=0, q=None, k=None, v=None, alpha=None, beta=None, out=None,
                                            S_final=None)) == raw.GDN_OK
