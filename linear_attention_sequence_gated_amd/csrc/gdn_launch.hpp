// gdn_launch.hpp -- internal interface between the C ABI layer and the kernels.
// Arguments arrive here already validated (shapes, alignment, supported set).
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>

namespace gdn {

// Launches `kernel` and returns the status of this launch itself.  (The
// runtime's last-error slot may hold an earlier, unrelated error from the
// caller's own HIP calls, so it is neither read nor cleared here.)
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                                Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  // fewer than 2^32 work-items along x: the argument checks keep every launch
  // inside this; a grid past it is refused rather than truncated
  if ((unsigned long long)grid.x * block.x >= (1ULL << 32)) return hipErrorInvalidConfiguration;
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const void* S0;
  void* out;
  void* S_final;
  int B, T, H, dk, dv, dtype;
  void* stream;
  // Fused prologue (bf16 pipelined and two-launch kernels): q and k raw,
  // alpha and beta hold the logits a and b; beta = beta_scale * sigmoid(b).
  int prologue = 0;
  float beta_scale = 1.f;
};

struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  void* S;
  void* out;
  int N, dk, dv, dtype;
  void* stream;
};

// Reverse-mode gradients of the chunk forward; gradient outputs are fp32
// (complex64 for complex data, as float pairs).  dS_final, S0 and dS0 may be
// NULL.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* S0;
  const void* dout;
  const float* dS_final;
  float* dq;
  float* dk;
  float* dv;
  float* dalpha;
  float* dbeta;
  float* dS0;
  void* workspace;
  int B, T, H, dtype;
  void* stream;
  int D = 64;  // dk = dv
};

// Forward with a per-output-channel decay r [B, T, H, dv] (real dtypes, d = 64).
struct ChannelArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* r;
  const float* beta;
  const float* S0;
  void* out;
  float* S_final;
  int B, T, H, dtype;
  void* stream;
};

hipError_t launch_chunk_fwd(const ChunkArgs& a);   // fused kernel, real dtypes
hipError_t launch_chunk_pipe(const ChunkArgs& a);  // pipelined kernel, bf16 only (fused prologue)
// bf16, d = 64 or 128: the chunk-parallel factor pass, then the state pass
// (segmented for long sequences with few chains).  Per-chunk factors and the
// segment maps go through `workspace`.
size_t chunk_two_workspace_bytes(const ChunkArgs& a);
size_t chunk_two_prologue_workspace_bytes(const ChunkArgs& a);  // + 1 / |k|, 1 / |q| per token
int chunk_two_segments(const ChunkArgs& a);  // segments of the two-level scan (1: none)
hipError_t launch_chunk_two(const ChunkArgs& a, void* workspace);
// The same forward for the gradient pass: also writes the Tb^T records to
// `recT` and every chunk's start state (bf16 [chains][nch][dk][dv]) to `Sck`;
// a.out may be NULL (no output written).
hipError_t launch_chunk_two_states(const ChunkArgs& a, void* workspace, void* recT, void* Sck);
hipError_t launch_recurrent_step(const StepArgs& a);
// Complex64, head size 32: three launches (prep, state scan, output) that
// exchange per-chunk intermediates through `workspace`.
// Input transforms of the layer for the fp32 and complex64 forwards (rows of
// 64 floats): normalised q, k and the gates written to the workspace; *fwd
// receives `a` with q, k, alpha, beta pointing there.
size_t prologue_rows_workspace_bytes(long rows);
hipError_t launch_prologue_rows(const ChunkArgs& a, void* workspace, ChunkArgs* fwd);
size_t chunk_cx_workspace_bytes(int B, int T, int H);
hipError_t launch_chunk_cx(const ChunkArgs& a, void* workspace);
// Backward: forward checkpoints every 8 tokens in `workspace`.
size_t chunk_bwd_workspace_bytes(int B, int T, int H);
hipError_t launch_chunk_bwd(const BwdArgs& a);
// Token-by-token reverse pass split by column groups: fp32 data (d = 64) or
// complex64 data (d = 32; pointers hold complex64 as float pairs, alpha, beta
// and their gradients real).
size_t tok_bwd_workspace_bytes(int B, int T, int H, bool complex_data);
hipError_t launch_tok_bwd(const BwdArgs& a, bool complex_data);
// bf16, d = 64 or 128: the chunk form on the matrix cores (the forward's
// factor and state passes, the adjoint scan, the chunk-parallel gradients).
// T = 0 copies dS_final (or zeros) to dS0.
size_t chunk_grad_workspace_bytes(int B, int T, int H, int D);
hipError_t launch_chunk_grad(const BwdArgs& a);
hipError_t launch_channel_decay(const ChannelArgs& a);  // token loop (fp32 inputs)
hipError_t launch_channel_chunk(const ChannelArgs& a);  // chunk form on the matrix cores (bf16 inputs)

}  // namespace gdn
