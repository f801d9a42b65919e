// prologue.hip -- the layer's input transforms for the fp32 and complex64
// chunk forwards, as one pass over the token rows ahead of the forward.
//
// Per token and head (DeltaPhase README, section 1 "Extended Householder Beta
// Range" for beta; Sykra 0.3.3 README, "Architectural Highlights", for the
// data-dependent forget gate, read as a logistic map of a logit):
//
//   q <- q / max(|q|, 1e-12),  k <- k / max(|k|, 1e-12)   (L2 over the key
//        dimension; for complex rows the Hermitian norm sum |q_i|^2, the
//        length of the row read as real and imaginary parts)
//   alpha = exp(-softplus(a)) = 1 / (1 + e^a),  beta = bscale * sigmoid(b)
//
// Both supported shapes store a row as 64 floats (fp32 d = 64, or complex64
// d = 32 as interleaved re, im), and the squared norm of either is the sum of
// the squares of those 64 floats.  Sixteen lanes take one row, a 16-byte piece
// each, and the row's norm is summed across them with DPP (row_piece_sum).  The transformed
// q, k and the gates go to the caller's workspace, where the forward reads
// them.  alpha is kept at or above the smallest normal float, so that its
// logarithm in the forward stays finite for logits up to the float range
// (a gate that small already wipes the state).
#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "gdn_pipe.hpp"

namespace gdn {
namespace pro {

// One 256-thread workgroup takes 16 rows per round, grid-stride over the rows.
__global__ __launch_bounds__(256) void rows_kernel(const float4* __restrict__ q, const float4* __restrict__ k,
                                                   const float* __restrict__ a, const float* __restrict__ b,
                                                   float bscale, float4* __restrict__ qh, float4* __restrict__ kh,
                                                   float* __restrict__ alpha, float* __restrict__ beta, long rows) {
  const int piece = threadIdx.x & 15;
  const long stride = (long)gridDim.x * 16;
  for (long r = (long)blockIdx.x * 16 + (threadIdx.x >> 4); r < rows; r += stride) {
    const float4 x = q[r * 16 + piece], y = k[r * 16 + piece];
    const float sx = pipe::row_piece_sum<16>(x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w);
    const float sy = pipe::row_piece_sum<16>(y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w);
    const float ix = __builtin_amdgcn_rsqf(fmaxf(sx, 1e-24f)), iy = __builtin_amdgcn_rsqf(fmaxf(sy, 1e-24f));
    qh[r * 16 + piece] = make_float4(x.x * ix, x.y * ix, x.z * ix, x.w * ix);
    kh[r * 16 + piece] = make_float4(y.x * iy, y.y * iy, y.z * iy, y.w * iy);
    if (piece == 0) {
      constexpr float kLog2e = 1.4426950408889634f;
      const float al = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a[r] * kLog2e));
      alpha[r] = fmaxf(al, 1.17549435e-38f);
      beta[r] = bscale * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-b[r] * kLog2e));
    }
  }
}

}  // namespace pro

namespace {
constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}

size_t prologue_rows_workspace_bytes(long rows) { return 2 * align256((size_t)rows * 256) + 2 * align256((size_t)rows * 4); }

hipError_t launch_prologue_rows(const ChunkArgs& a, void* workspace, ChunkArgs* fwd) {
  const long rows = (long)a.B * a.T * a.H;
  char* ws = static_cast<char*>(workspace);
  float* qh = reinterpret_cast<float*>(ws);
  float* kh = reinterpret_cast<float*>(ws + align256((size_t)rows * 256));
  float* al = reinterpret_cast<float*>(ws + 2 * align256((size_t)rows * 256));
  float* be = reinterpret_cast<float*>(ws + 2 * align256((size_t)rows * 256) + align256((size_t)rows * 4));
  *fwd = a;
  fwd->q = qh;
  fwd->k = kh;
  fwd->alpha = al;
  fwd->beta = be;
  fwd->prologue = 0;
  if (rows == 0) return hipSuccess;
  const long blocks = (rows + 15) / 16;
  const unsigned grid = (unsigned)(blocks < (1L << 20) ? blocks : (1L << 20));
  return launch_kernel(pro::rows_kernel, dim3(grid), dim3(256), (hipStream_t)a.stream,
                       static_cast<const float4*>(a.q), static_cast<const float4*>(a.k), a.alpha, a.beta, a.beta_scale,
                       reinterpret_cast<float4*>(qh), reinterpret_cast<float4*>(kh), al, be, rows);
}

}  // namespace gdn
