// channel_decay.hip -- the delta rule with a per-output-channel decay, real
// data, d_k = d_v = 64 (fp32 or bf16 q, k, v; fp32 decay, beta and state).
//
// DeltaPhase README, section 5 (LaplacePhaseCore): the decay diag(r_t) acts on
// the value channels of the memory.  With the state S [dk, dv] it scales the
// columns, applied to the Householder-updated state:
//   S_t = (I - beta_t k_t k_t^T) S_{t-1} diag(r_t) + beta_t k_t v_t^T,
//   o_t = S_t^T q_t.
// Column j of S evolves on its own:
//   s_j <- r_j s_j + k (beta (v_j - r_j k^T s_j)),   o_j = q^T s_j,
// so the kernel needs no communication between columns.  A lane quad holds
// one column: lane l of wave w owns column 16 w + l / 4 and rows
// 16 (l % 4) .. + 15.  k^T s_j and q^T s_j are 16-term in-lane sums and two
// DPP adds.  Keys and queries are read from global memory by every lane
// (16 consecutive elements each), eight tokens ahead of their use; there is no
// LDS and no barrier.  Waves are independent: one workgroup of one wave per
// (chain, 16-column slice).
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_lane.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace chd {

using lane::quad_sum;
using lane::Row;

constexpr int D = 64;  // head dimension
constexpr int R = 16;  // rows per lane

__device__ __forceinline__ float f32(float x) { return x; }
__device__ __forceinline__ float f32(__hip_bfloat16 x) { return __bfloat162float(x); }
__device__ __forceinline__ void st(float* p, float x) { *p = x; }
__device__ __forceinline__ void st(__hip_bfloat16* p, float x) { *p = __float2bfloat16(x); }

template <class IT>
__global__ __launch_bounds__(64) void channel_decay_kernel(const IT* __restrict__ q, const IT* __restrict__ k,
                                                           const IT* __restrict__ v, const float* __restrict__ r,
                                                           const float* __restrict__ beta,
                                                           const float* __restrict__ S0, IT* __restrict__ out,
                                                           float* __restrict__ Sf, int T, int H) {
  const int l = threadIdx.x, slice = blockIdx.x & 3, chain = blockIdx.x >> 2;
  const int b = chain / H, h = chain % H;
  const int c = 16 * slice + (l >> 2), rq = l & 3, i0 = R * rq;
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };

  float s[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) s[ii] = S0 ? S0[((size_t)chain * D + i0 + ii) * D + c] : 0.f;

  // This lane's inputs of one token (t clamped into [0, T), valid when T > 0),
  // kept as stored until used so that loading the next token never waits.
  struct Tok {
    Row<IT> k, q;
    IT v;
    float r, be;
  };
  auto load = [&](int t) {
    Tok x;
    const size_t rt = tok(max(0, min(t, T - 1)));
    x.k.load(k + rt * D + i0);
    x.q.load(q + rt * D + i0);
    x.v = v[rt * D + c];
    x.r = r[rt * D + c];
    x.be = beta[rt];
    return x;
  };

  // One token on s; o is stored by the quad's first lane.
  auto step = [&](const Tok& x, int t) {
    float u = 0.f;
#pragma unroll
    for (int ii = 0; ii < R; ++ii) u += x.k[ii] * s[ii];
    u = quad_sum(u);
    const float y = x.be * (f32(x.v) - x.r * u);
    float o = 0.f;
#pragma unroll
    for (int ii = 0; ii < R; ++ii) {
      s[ii] = x.r * s[ii] + x.k[ii] * y;
      o += x.q[ii] * s[ii];
    }
    o = quad_sum(o);
    if (rq == 0) st(out + tok(t) * D + c, o);
  };

  // Inputs are loaded PF tokens ahead (a token takes well under a memory
  // latency), in a ring of registers indexed at compile time; the loads are
  // unconditional (clamped), so the compiler's in-order load counts are static.
  constexpr int PF = 8;
  if (T > 0) {  // T = 0: the input buffers may be empty
    Tok ring[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[p] = load(p);
    for (int t = 0; t < T; t += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        if (t + p < T) step(ring[p], t + p);
        ring[p] = load(t + p + PF);
      }
    }
  }
  if (Sf) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) Sf[((size_t)chain * D + i0 + ii) * D + c] = s[ii];
  }
}

}  // namespace chd

hipError_t launch_channel_decay(const ChannelArgs& a) {
  const dim3 grid((unsigned)((long)a.B * a.H * 4)), block(64);
  if (a.dtype == kDtBF16)
    return launch_kernel(chd::channel_decay_kernel<__hip_bfloat16>, grid, block, (hipStream_t)a.stream,
                         (const __hip_bfloat16*)a.q, (const __hip_bfloat16*)a.k, (const __hip_bfloat16*)a.v, a.r,
                         a.beta, a.S0, (__hip_bfloat16*)a.out, a.S_final, a.T, a.H);
  return launch_kernel(chd::channel_decay_kernel<float>, grid, block, (hipStream_t)a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, a.r, a.beta, a.S0, (float*)a.out, a.S_final, a.T, a.H);
}

}  // namespace gdn
