// gdn_launch.hpp -- internal interface between the C ABI layer and the kernels.
// Arguments arrive here already validated (shapes, alignment, supported set).
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

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

hipError_t launch_chunk_fwd(const ChunkArgs& a);   // fused kernel, every dtype
hipError_t launch_chunk_pipe(const ChunkArgs& a);  // pipelined kernel, bf16 only
hipError_t launch_recurrent_step(const StepArgs& a);

}  // namespace gdn
