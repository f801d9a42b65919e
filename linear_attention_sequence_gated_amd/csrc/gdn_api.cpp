// gdn_api.cpp -- the C ABI of libgdn (declared in include/gdn.h).
//
// Validates every argument before anything is enqueued (no HIP call happens on
// an argument error), then dispatches to the kernels.  The library holds no
// allocations and no per-call state.
#include <stdint.h>

#include "../../include/gdn.h"
#include "gdn_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool chunk_supported(int dtype, int dk, int dv) {
  if (dk != dv) return false;
  switch (dtype) {
    case GDN_BF16: return dk == 64 || dk == 128;
    case GDN_F32: return dk == 64;
    case GDN_C64: return dk == 32;
    default: return false;
  }
}

bool step_supported(int dtype, int dk, int dv) {
  if (dk != dv) return false;
  switch (dtype) {
    case GDN_BF16:
    case GDN_F32: return dk == 64 || dk == 128;
    case GDN_C64: return dk == 32;
    default: return false;
  }
}

// Kernels for bf16 whose rows are addressable with 32-bit buffer offsets (one
// batch row of q, k, v and out under 2^31 bytes):
//   d = 128: the two-launch path (factor pass, then state pass);
//   d = 64: the three-stage pipelined kernel, unless the chains are too few to
//   fill the CUs and the sequence is long: then the two-launch path with the
//   segment-parallel two-level scan.
// Rows past 32-bit offsets take the fused kernel.
bool rows_fit(int T, int H, int dk) { return (long long)T * H * dk * 2 < (1LL << 31); }

gdn::ChunkArgs shape_args(int B, int T, int H, int dk, int dv, int dtype) {
  gdn::ChunkArgs a{};
  a.B = B;
  a.T = T;
  a.H = H;
  a.dk = dk;
  a.dv = dv;
  a.dtype = dtype;
  return a;
}

bool two_path(int B, int T, int H, int dk, int dv, int dtype) {
  if (dtype != GDN_BF16 || dk != dv || (dk != 64 && dk != 128) || !rows_fit(T, H, dk)) return false;
  // the factor pass runs 64 threads per chunk
  if ((long long)B * H * ((T + 63) / 64) * 64 >= (1LL << 32)) return false;
  return dk == 128 || gdn::chunk_two_segments(shape_args(B, T, H, dk, dv, dtype)) > 1;
}

// The backward's matrix-core path: bf16, d = 64 (T > 0) or 128 (any T), rows
// addressable with 32-bit offsets (fp32 gradient rows included) and the chunk
// grid (512 threads per chunk at d = 128) in range.  fp32 inputs take the token-by-token kernel (fp32
// throughout, d = 64).
bool grad_path(int B, int T, int H, int dk, int dv, int dtype) {
  if (dtype != GDN_BF16 || dk != dv || (dk != 64 && dk != 128) || (dk == 64 && T <= 0)) return false;
  if ((long long)T * H * dk * 4 >= (1LL << 31)) return false;
  return (long long)B * H * ((T + 63) / 64) * 512 < (1LL << 32);
}

// Largest element count any single tensor may have (keeps every index in range).
constexpr long long kMaxElems = 1LL << 40;

// Launch limits.  A launch may hold fewer than 2^32 work-items along x.  The
// chunk kernels run at most 4096 threads per (batch, head) chain (eight
// 512-thread workgroups), the backward kernels at most 512 (the fp32 token
// backward: eight 64-lane column groups), the channel-decay kernels at most
// 1024 (the bf16 chunk form: two 448-thread workgroups), and the decode
// kernel at most 256 per state.
// The grids that scale with the chunk count are bounded where their path is
// chosen.  Sizes past these bounds are argument errors,
// reported before anything is launched.
constexpr long long kMaxWorkItems = 1LL << 32;
bool chains_fit(long long chains, long long threads_per_chain) {
  return chains * threads_per_chain < kMaxWorkItems;
}

}  // namespace

extern "C" {

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK: success";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: a size is negative or too large";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: dtype must be GDN_F32, GDN_BF16 or GDN_C64";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: chunk or head dimensions not supported";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime reported an error";
    default: return "GDN: unknown status code";
  }
}

size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (B < 0 || T < 0 || H < 0 || chunk != 64 || !chunk_supported(dtype, dk, dv)) return 0;
  // The complex path and the bf16 two-launch path hand per-chunk factors from
  // one launch to the next; the fused kernels keep every intermediate on chip.
  if (dtype == GDN_C64) return gdn::chunk_cx_workspace_bytes(B, T, H);
  if (two_path(B, T, H, dk, dv, dtype)) return gdn::chunk_two_workspace_bytes(shape_args(B, T, H, dk, dv, dtype));
  return 0;
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                  const void* S0, int chunk, void* out, void* S_final, int B, int T, int H, int dk, int dv,
                  int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)B * T * H * (dk > dv ? dk : dv) > kMaxElems || (long long)B * H * dk * dv > kMaxElems)
    return GDN_ERR_SHAPE;
  if (chunk != 64 || !chunk_supported(dtype, dk, dv)) return GDN_ERR_UNSUPPORTED;
  if (!chains_fit((long long)B * H, 4096)) return GDN_ERR_SHAPE;
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !alpha || !beta || !out)) return GDN_ERR_NULL;
  const void* ptrs[] = {q, k, v, alpha, beta, S0, out, S_final, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::ChunkArgs a{q, k, v, alpha, beta, S0, out, S_final, B, T, H, dk, dv, dtype, stream};
  if (two_path(B, T, H, dk, dv, dtype)) return gdn::launch_chunk_two(a, workspace) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  if (dtype == GDN_BF16 && dk == 64 && rows_fit(T, H, dk))
    return gdn::launch_chunk_pipe(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  if (dtype == GDN_C64) return gdn::launch_chunk_cx(a, workspace) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  return gdn::launch_chunk_fwd(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_chunk_fwd_prologue_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (B < 0 || T < 0 || H < 0 || chunk != 64 || !chunk_supported(dtype, dk, dv)) return 0;
  // bf16: the transforms are fused into the forward's own kernels; the
  // two-launch path also hands 1 / |k| per token from its factor pass to its
  // state pass.  fp32 and complex64: a pass over the rows writes the
  // transformed q, k and the gates for the forward to read.
  if (dtype == GDN_BF16)
    return two_path(B, T, H, dk, dv, dtype) ? gdn::chunk_two_prologue_workspace_bytes(shape_args(B, T, H, dk, dv, dtype))
                                            : 0;
  size_t b = gdn::prologue_rows_workspace_bytes((long)B * T * H);
  if (dtype == GDN_C64) b += gdn::chunk_cx_workspace_bytes(B, T, H);
  return b;
}

int gdn_chunk_fwd_prologue(const void* q, const void* k, const void* v, const float* a_logit,
                           const float* b_logit, float beta_scale, const void* S0, int chunk, void* out,
                           void* S_final, int B, int T, int H, int dk, int dv, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)B * T * H * (dk > dv ? dk : dv) > kMaxElems || (long long)B * H * dk * dv > kMaxElems)
    return GDN_ERR_SHAPE;
  if (chunk != 64 || !chunk_supported(dtype, dk, dv)) return GDN_ERR_UNSUPPORTED;
  if (!(beta_scale >= 0.f && beta_scale <= 2.f)) return GDN_ERR_SHAPE;
  if (!chains_fit((long long)B * H, 4096)) return GDN_ERR_SHAPE;
  // bf16 runs on the buffer-resource kernels only (rows under 2^31 bytes; at
  // d = 128 the two-launch path).
  const bool two = two_path(B, T, H, dk, dv, dtype);
  if (dtype == GDN_BF16 && (!rows_fit(T, H, dk) || (dk == 128 && !two))) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !a_logit || !b_logit || !out)) return GDN_ERR_NULL;
  const void* ptrs[] = {q, k, v, a_logit, b_logit, S0, out, S_final, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  const size_t need = gdn_chunk_fwd_prologue_workspace_bytes(B, T, H, dk, dv, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::ChunkArgs a{q, k, v, a_logit, b_logit, S0, out, S_final, B, T, H, dk, dv, dtype, stream};
  a.prologue = 1;
  a.beta_scale = beta_scale;
  if (dtype == GDN_BF16) {
    if (two) return gdn::launch_chunk_two(a, workspace) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    return gdn::launch_chunk_pipe(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  }
  gdn::ChunkArgs f{};
  if (gdn::launch_prologue_rows(a, workspace, &f) != hipSuccess) return GDN_ERR_HIP;
  if (dtype == GDN_C64) {
    void* cx = static_cast<char*>(workspace) + gdn::prologue_rows_workspace_bytes((long)B * T * H);
    return gdn::launch_chunk_cx(f, cx) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  }
  return gdn::launch_chunk_fwd(f) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype) {
  if (B < 0 || T < 0 || H < 0) return 0;
  if (dtype == GDN_C64) return dk == 32 && dv == 32 ? gdn::tok_bwd_workspace_bytes(B, T, H, true) : 0;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return 0;
  if (grad_path(B, T, H, dk, dv, dtype)) return gdn::chunk_grad_workspace_bytes(B, T, H, dk);
  if (dtype == GDN_F32) return dk == 64 && dv == 64 ? gdn::tok_bwd_workspace_bytes(B, T, H, false) : 0;
  if (dk != 64 || dv != 64) return 0;
  return gdn::chunk_bwd_workspace_bytes(B, T, H);
}

int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                  const float* S0, const void* grad_out, const float* grad_S_final, float* grad_q, float* grad_k,
                  float* grad_v, float* grad_alpha, float* grad_beta, float* grad_S0, int B, int T, int H, int dk,
                  int dv, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)B * T * H * (dk > dv ? dk : dv) > kMaxElems || (long long)B * H * dk * dv > kMaxElems ||
      !chains_fit((long long)B * H, 512))
    return GDN_ERR_SHAPE;
  const bool mfma = grad_path(B, T, H, dk, dv, dtype);
  const bool cx = dtype == GDN_C64;
  if ((long long)T * H * 4 >= (1LL << 31) && !mfma) return GDN_ERR_UNSUPPORTED;
  if (cx ? (dk != 32 || dv != 32) : (!mfma && (dk != 64 || dv != 64))) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !alpha || !beta || !grad_out || !grad_q || !grad_k || !grad_v || !grad_alpha ||
                 !grad_beta))
    return GDN_ERR_NULL;
  const void* ptrs[] = {q,      k,      v,      alpha,      beta,      S0,      grad_out, grad_S_final,
                        grad_q, grad_k, grad_v, grad_alpha, grad_beta, grad_S0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  // complex64 and fp32: the token-by-token pass split by column groups; bf16:
  // the chunk form (the token kernel only for T == 0 and rows past 32-bit
  // offsets)
  const bool tok = cx || dtype == GDN_F32;
  const size_t need = tok    ? gdn::tok_bwd_workspace_bytes(B, T, H, cx)
                      : mfma ? gdn::chunk_grad_workspace_bytes(B, T, H, dk)
                             : gdn::chunk_bwd_workspace_bytes(B, T, H);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::BwdArgs a{q,      k,      v,      alpha,      beta,      S0,      grad_out, grad_S_final, grad_q, grad_k,
                 grad_v, grad_alpha, grad_beta, grad_S0, workspace, B, T, H, dtype, stream};
  a.D = dk;
  if (tok) return gdn::launch_tok_bwd(a, cx) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  if (mfma) return gdn::launch_chunk_grad(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  return gdn::launch_chunk_bwd(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_fwd_channel_decay(const void* q, const void* k, const void* v, const float* r, const float* beta,
                          const float* S0, void* out, float* S_final, int B, int T, int H, int dk, int dv, int dtype,
                          void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)B * T * H * (dk > dv ? dk : dv) > kMaxElems || (long long)B * H * dk * dv > kMaxElems ||
      !chains_fit((long long)B * H, 1024))
    return GDN_ERR_SHAPE;
  if (dk != dv || (dtype == GDN_C64 ? dk != 32 : dk != 64)) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !r || !beta || !out)) return GDN_ERR_NULL;
  const void* ptrs[] = {q, k, v, r, beta, S0, out, S_final};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::ChannelArgs a{q, k, v, r, beta, S0, out, S_final, B, T, H, dtype, stream};
  // bf16: the chunk form (per-channel triangular solves, the state on the
  // matrix cores) while rows are addressable with 32-bit buffer offsets;
  // otherwise, and for fp32 inputs, the token loop.
  if (dtype == GDN_BF16 && (long long)T * H * dk * 4 < (1LL << 31))
    return gdn::launch_channel_chunk(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  return gdn::launch_channel_decay(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_recurrent_step(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                       void* S, void* out, int N, int dk, int dv, int dtype, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (N < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)N * dk * dv > kMaxElems || !chains_fit(N, 256)) return GDN_ERR_SHAPE;
  if (!step_supported(dtype, dk, dv)) return GDN_ERR_UNSUPPORTED;
  if (N == 0) return GDN_OK;
  if (!q || !k || !v || !alpha || !beta || !S || !out) return GDN_ERR_NULL;
  const void* ptrs[] = {q, k, v, alpha, beta, S, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDN_ERR_ALIGN;
  gdn::StepArgs a{q, k, v, alpha, beta, S, out, N, dk, dv, dtype, stream};
  return gdn::launch_recurrent_step(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
