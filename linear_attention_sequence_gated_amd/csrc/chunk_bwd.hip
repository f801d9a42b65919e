// chunk_bwd.hip -- reverse-mode gradients of the gated delta rule, real data,
// d_k = d_v = 64 (fp32 or bf16 inputs, fp32 arithmetic and gradients).
//
// Per (batch, head) chain the forward is u_t = S_{t-1}^T k_t,
// S_t = alpha_t (S_{t-1} - beta_t k_t u_t^T) + beta_t k_t v_t^T and
// o_t = S_t^T q_t (DeltaPhase section 2; forget gate of the Sykra README,
// "Architectural Highlights").  Token by token in reverse, with G the
// gradient reaching S_t from later tokens:
//   D = G + q_t dO_t^T,  w = D^T k_t,  y = beta_t v_t - alpha_t beta_t u_t,
//   dq_t = S_t dO_t = alpha_t S_{t-1} dO_t + k_t (y . dO_t),
//   dk_t = D y - alpha_t beta_t S_{t-1} w,  dv_t = beta_t w,
//   dbeta_t = w . (v_t - alpha_t u_t),
//   dalpha_t = <D, S_{t-1}> - beta_t (w . u_t),
//   G <- alpha_t (D - beta_t k_t w^T);  dS0 is the last G.
//
// One wave per chain; lane j owns column j of S and of G (64 registers
// each).  Column sums (u, w) are in-lane; the two row sums per token (for dq
// and dk) go through a padded LDS buffer.  S_{t-1} is needed in reverse
// order, so a first pass runs the forward and checkpoints S every 8 tokens to
// the workspace; the reverse pass recomputes each 8-token block from its
// checkpoint into LDS (128 KB) and walks it backwards.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace bwd {

constexpr int D = 64;      // head dimension (d_k = d_v)
constexpr int SUB = 8;     // tokens per checkpoint block
constexpr int LDR = D + 1; // row stride of the row-sum buffer (conflict-free both ways)

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __hip_bfloat16* p) { return __bfloat162float(*p); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <class IT>
__global__ __launch_bounds__(64) void bwd_kernel(const IT* __restrict__ q, const IT* __restrict__ k,
                                                 const IT* __restrict__ v, const float* __restrict__ alpha,
                                                 const float* __restrict__ beta, const float* __restrict__ S0,
                                                 const IT* __restrict__ dO, const float* __restrict__ dSf,
                                                 float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                                                 float* __restrict__ dalpha, float* __restrict__ dbeta,
                                                 float* __restrict__ dS0, float* __restrict__ ckpt, int T, int H) {
  __shared__ float st[SUB][D][D];  // S_{t-1} of each token of the block, [i][j]
  __shared__ float red[D * LDR];   // row sums: lane j writes column j, lane i reads row i
  __shared__ float kv[D], qv[D];   // k_t and q_t, read by every lane
  const int j = threadIdx.x, chain = blockIdx.x, b = chain / H, h = chain % H;
  const int nsub = (T + SUB - 1) / SUB;
  float* const ck = ckpt + (size_t)chain * nsub * D * D;
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };

  float s[D];
#pragma unroll
  for (int i = 0; i < D; ++i) s[i] = S0 ? S0[((size_t)chain * D + i) * D + j] : 0.f;

  // One forward token on s (column j of the state); k_t is left in kv.
  auto forward = [&](int t) {
    const size_t r = tok(t);
    __syncthreads();  // earlier readers of kv are done
    kv[j] = ld(k + r * D + j);
    __syncthreads();
    const float a = alpha[r], be = beta[r], vj = ld(v + r * D + j);
    float u = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) u += s[i] * kv[i];
    const float y = be * vj - a * be * u;
#pragma unroll
    for (int i = 0; i < D; ++i) s[i] = a * s[i] + kv[i] * y;
  };

  // Pass 1: checkpoints S at the start of every block.
  for (int c = 0; c < nsub; ++c) {
#pragma unroll
    for (int i = 0; i < D; ++i) ck[((size_t)c * D + i) * D + j] = s[i];
    const int mend = min(SUB, T - c * SUB);
    for (int m = 0; m < mend; ++m) forward(c * SUB + m);
  }

  // Pass 2: blocks in reverse; g is column j of G.
  float g[D];
#pragma unroll
  for (int i = 0; i < D; ++i) g[i] = dSf ? dSf[((size_t)chain * D + i) * D + j] : 0.f;
  for (int c = nsub - 1; c >= 0; --c) {
    const int mend = min(SUB, T - c * SUB);
#pragma unroll
    for (int i = 0; i < D; ++i) s[i] = ck[((size_t)c * D + i) * D + j];
    for (int m = 0; m < mend; ++m) {
#pragma unroll
      for (int i = 0; i < D; ++i) st[m][i][j] = s[i];
      if (m + 1 < mend) forward(c * SUB + m);  // the block's last state is not needed
    }
    for (int m = mend - 1; m >= 0; --m) {
      const size_t r = tok(c * SUB + m);
      __syncthreads();  // st written, earlier readers of kv / qv / red done
      kv[j] = ld(k + r * D + j);
      qv[j] = ld(q + r * D + j);
      __syncthreads();
      const float a = alpha[r], be = beta[r], vj = ld(v + r * D + j), doj = ld(dO + r * D + j);
      float u = 0.f, w = 0.f, dsp = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        g[i] += qv[i] * doj;  // D = G + q dO^T
        u += st[m][i][j] * kv[i];
        w += g[i] * kv[i];
        dsp += g[i] * st[m][i][j];
      }
      const float y = be * vj - a * be * u;
      dv[r * D + j] = be * w;
      const float db = wave_sum(w * (vj - a * u));
      const float da = wave_sum(dsp - be * w * u);
      const float ydo = wave_sum(y * doj);
      if (j == 0) {
        dbeta[r] = db;
        dalpha[r] = da;
      }
      // Row sums over the columns: sum_j S_{t-1}[i][j] dO_j, then
      // sum_j (D[i][j] y_j - alpha beta S_{t-1}[i][j] w_j).
#pragma unroll
      for (int i = 0; i < D; ++i) red[i * LDR + j] = st[m][i][j] * doj;
      __syncthreads();
      float r1 = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) r1 += red[j * LDR + x];
      __syncthreads();
      const float ab = a * be;
#pragma unroll
      for (int i = 0; i < D; ++i) red[i * LDR + j] = g[i] * y - ab * st[m][i][j] * w;
      __syncthreads();
      float r2 = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) r2 += red[j * LDR + x];
      dq[r * D + j] = a * r1 + kv[j] * ydo;  // lane j now stands for row j
      dk[r * D + j] = r2;
#pragma unroll
      for (int i = 0; i < D; ++i) g[i] = a * (g[i] - be * kv[i] * w);
    }
  }
  if (dS0) {
#pragma unroll
    for (int i = 0; i < D; ++i) dS0[((size_t)chain * D + i) * D + j] = g[i];
  }
}

}  // namespace bwd

size_t chunk_bwd_workspace_bytes(int B, int T, int H) {
  return (size_t)B * H * ((T + bwd::SUB - 1) / bwd::SUB) * bwd::D * bwd::D * sizeof(float);
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
  const dim3 grid((unsigned)((long)a.B * a.H)), block(64);
  if (a.dtype == kDtBF16)
    return launch_kernel(bwd::bwd_kernel<__hip_bfloat16>, grid, block, (hipStream_t)a.stream,
                         (const __hip_bfloat16*)a.q, (const __hip_bfloat16*)a.k, (const __hip_bfloat16*)a.v, a.alpha,
                         a.beta, a.S0, (const __hip_bfloat16*)a.dout, a.dS_final, a.dq, a.dk, a.dv, a.dalpha, a.dbeta,
                         a.dS0, (float*)a.workspace, a.T, a.H);
  return launch_kernel(bwd::bwd_kernel<float>, grid, block, (hipStream_t)a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, a.alpha, a.beta, a.S0, (const float*)a.dout, a.dS_final,
                       a.dq, a.dk, a.dv, a.dalpha, a.dbeta, a.dS0, (float*)a.workspace, a.T, a.H);
}

}  // namespace gdn
