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
  // Fused prologue (d64 bf16 pipelined kernel only): q and k raw, alpha and
  // beta hold the logits a and b; beta = beta_scale * sigmoid(b).
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

// Reverse-mode gradients of the chunk forward (real dtypes, d = 64); all
// gradient outputs are fp32.  dS_final, S0 and dS0 may be NULL.
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
hipError_t launch_chunk_pipe(const ChunkArgs& a);  // pipelined kernel, bf16 only
hipError_t launch_recurrent_step(const StepArgs& a);
// Complex64, head size 32: three launches (prep, state scan, output) that
// exchange per-chunk intermediates through `workspace`.
size_t chunk_cx_workspace_bytes(int B, int T, int H);
hipError_t launch_chunk_cx(const ChunkArgs& a, void* workspace);
// Backward: forward checkpoints every 8 tokens in `workspace`.
size_t chunk_bwd_workspace_bytes(int B, int T, int H);
hipError_t launch_chunk_bwd(const BwdArgs& a);
hipError_t launch_channel_decay(const ChannelArgs& a);

}  // namespace gdn
