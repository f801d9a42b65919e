// noalloc.hip -- gdn_chunk_fwd for callers that cannot allocate device memory
// (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc).  The workspace the chunk forward needs (per-chunk factors, the
// segment maps of the two-level scan, the complex path's hand-off buffers)
// comes from one file-scope device array of fixed size instead of the caller.
//
// The array lives in this translation unit only, so a process that never
// calls the entry point never loads it.  Each device keeps its own copy, from
// the first call on that device until the process ends.  Its address on each
// device is looked up once, with that device current, and kept; the array's
// name is never passed to a kernel (in host code it only stands in for the
// symbol).  Every call on one device shares the array: calls that overlap on
// one device (different streams, different host threads without ordering)
// race on it.  Nothing in it needs to start at zero: every launch that reads
// a part of it reads only what an earlier launch of the same call wrote.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"

namespace {

constexpr size_t kScratchBytes = GDN_NOALLOC_MAX_WORKSPACE;  // 128 MiB per device
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of the array, or NULL on error.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                          const void* S0, int chunk, void* out, void* S_final, int B, int T, int H, int dk, int dv,
                          int dtype, void* stream) {
  // Sizes are validated by gdn_chunk_fwd; the query returns 0 for anything it rejects.
  const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype);
  if (need > kScratchBytes) return GDN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return GDN_ERR_HIP;
  }
  return gdn_chunk_fwd(q, k, v, alpha, beta, S0, chunk, out, S_final, B, T, H, dk, dv, dtype, ws, need, stream);
}

}  // extern "C"
