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

// Largest element count any single tensor may have (keeps every index in range).
constexpr long long kMaxElems = 1LL << 40;

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
  // The real kernels keep every intermediate on chip; the complex path hands
  // per-chunk factors from one launch to the next.
  if (dtype == GDN_C64) return gdn::chunk_cx_workspace_bytes(B, T, H);
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
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !alpha || !beta || !out)) return GDN_ERR_NULL;
  const void* ptrs[] = {q, k, v, alpha, beta, S0, out, S_final, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::ChunkArgs a{q, k, v, alpha, beta, S0, out, S_final, B, T, H, dk, dv, dtype, stream};
  // The pipelined bf16 kernel addresses one batch row of q/k/v/out with 32-bit
  // buffer offsets; larger rows use the fused kernel.
  const bool pipe_fits = (long long)T * H * (dk > dv ? dk : dv) * 2 < (1LL << 31);
  if (dtype == GDN_BF16 && pipe_fits) return gdn::launch_chunk_pipe(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  if (dtype == GDN_C64) return gdn::launch_chunk_cx(a, workspace) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  return gdn::launch_chunk_fwd(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_chunk_fwd_prologue(const void* q, const void* k, const void* v, const float* a_logit,
                           const float* b_logit, float beta_scale, const void* S0, int chunk, void* out,
                           void* S_final, int B, int T, int H, int dk, int dv, int dtype, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)B * T * H * (dk > dv ? dk : dv) > kMaxElems || (long long)B * H * dk * dv > kMaxElems)
    return GDN_ERR_SHAPE;
  if (chunk != 64 || dtype != GDN_BF16 || dk != 64 || dv != 64) return GDN_ERR_UNSUPPORTED;
  if (!(beta_scale >= 0.f && beta_scale <= 2.f)) return GDN_ERR_SHAPE;
  if ((long long)T * H * dk * 2 >= (1LL << 31)) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !a_logit || !b_logit || !out)) return GDN_ERR_NULL;
  const void* ptrs[] = {q, k, v, a_logit, b_logit, S0, out, S_final};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::ChunkArgs a{q, k, v, a_logit, b_logit, S0, out, S_final, B, T, H, dk, dv, dtype, stream};
  a.prologue = 1;
  a.beta_scale = beta_scale;
  return gdn::launch_chunk_pipe(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype) {
  if (B < 0 || T < 0 || H < 0 || (dtype != GDN_F32 && dtype != GDN_BF16) || dk != 64 || dv != 64) return 0;
  return gdn::chunk_bwd_workspace_bytes(B, T, H);
}

int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                  const float* S0, const void* grad_out, const float* grad_S_final, float* grad_q, float* grad_k,
                  float* grad_v, float* grad_alpha, float* grad_beta, float* grad_S0, int B, int T, int H, int dk,
                  int dv, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)B * T * H * (dk > dv ? dk : dv) > kMaxElems || (long long)B * H * dk * dv > kMaxElems ||
      (long long)B * H >= (1LL << 31))
    return GDN_ERR_SHAPE;
  if (dtype == GDN_C64 || dk != 64 || dv != 64 || (long long)T * H * 4 >= (1LL << 31)) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !alpha || !beta || !grad_out || !grad_q || !grad_k || !grad_v || !grad_alpha ||
                 !grad_beta))
    return GDN_ERR_NULL;
  const void* ptrs[] = {q,      k,      v,      alpha,      beta,      S0,      grad_out, grad_S_final,
                        grad_q, grad_k, grad_v, grad_alpha, grad_beta, grad_S0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  const size_t need = gdn::chunk_bwd_workspace_bytes(B, T, H);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::BwdArgs a{q,      k,      v,      alpha,      beta,      S0,      grad_out, grad_S_final, grad_q, grad_k,
                 grad_v, grad_alpha, grad_beta, grad_S0, workspace, B, T, H, dtype, stream};
  return gdn::launch_chunk_bwd(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_fwd_channel_decay(const void* q, const void* k, const void* v, const float* r, const float* beta,
                          const float* S0, void* out, float* S_final, int B, int T, int H, int dk, int dv, int dtype,
                          void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)B * T * H * (dk > dv ? dk : dv) > kMaxElems || (long long)B * H * dk * dv > kMaxElems ||
      (long long)B * H * 4 >= (1LL << 31))
    return GDN_ERR_SHAPE;
  if (dtype == GDN_C64 || dk != 64 || dv != 64) return GDN_ERR_UNSUPPORTED;
  const bool tokens = (long long)B * T * H > 0;
  if (tokens && (!q || !k || !v || !r || !beta || !out)) return GDN_ERR_NULL;
  const void* ptrs[] = {q, k, v, r, beta, S0, out, S_final};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_ALIGN;
  if ((long long)B * H == 0) return GDN_OK;
  gdn::ChannelArgs a{q, k, v, r, beta, S0, out, S_final, B, T, H, dtype, stream};
  return gdn::launch_channel_decay(a) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_recurrent_step(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                       void* S, void* out, int N, int dk, int dv, int dtype, void* stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_C64) return GDN_ERR_DTYPE;
  if (N < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if ((long long)N * dk * dv > kMaxElems) return GDN_ERR_SHAPE;
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
