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
// and dk) go through a padded LDS buffer, each lane writing its column as a
// row of it.  The workgroup is one wave, so LDS exchanges between its lanes
// are ordered with wavefront-scope fences: a workgroup barrier's fence would
// also wait for every global load and store in flight.  S_{t-1} is needed in reverse
// order, so a first pass runs the forward and checkpoints S every 8 tokens to
// the workspace; the reverse pass recomputes each 8-token block from its
// checkpoint into LDS (136 KB) and walks it backwards.  Each chain is one
// wave alone on its CU, so nothing hides a load's latency: every token's
// inputs are loaded while the token before it (in the direction of the walk)
// is computed.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace bwd {

constexpr int D = 64;      // head dimension (d_k = d_v)
constexpr int SUB = 8;     // tokens per checkpoint block
constexpr int LDC = D + 4; // row stride of the LDS column buffers (16-byte rows, conflict-free)

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __hip_bfloat16* p) { return __bfloat162float(*p); }

// Orders this wave's earlier LDS writes before its later LDS reads in every
// lane (wavefront-scope release / acquire around a wave barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
  __shared__ __attribute__((aligned(16))) float st[SUB][D][LDC];  // S_{t-1} of each token of the block, [j][i]
  __shared__ __attribute__((aligned(16))) float red[D * LDC];      // row sums: lane j writes [j][*], lane i reads [*][i]
  __shared__ float kv[D], qv[D];   // k_t and q_t, read by every lane
  const int j = threadIdx.x, chain = blockIdx.x, b = chain / H, h = chain % H;
  const int nsub = (T + SUB - 1) / SUB;
  float* const ck = ckpt + (size_t)chain * nsub * D * D;
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };

  float s[D];
#pragma unroll
  for (int i = 0; i < D; ++i) s[i] = S0 ? S0[((size_t)chain * D + i) * D + j] : 0.f;

  // Lane j's inputs of one token (t clamped into [0, T), so always a valid
  // address when T > 0; never called when T = 0).
  struct Tok {
    float k, q, v, dO, a, be;
  };
  auto load = [&](int t, bool back) {
    Tok x;
    const size_t r = tok(max(0, min(t, T - 1)));
    x.k = ld(k + r * D + j);
    x.v = ld(v + r * D + j);
    x.a = alpha[r];
    x.be = beta[r];
    x.q = back ? ld(q + r * D + j) : 0.f;
    x.dO = back ? ld(dO + r * D + j) : 0.f;
    return x;
  };

  // One forward token on s (column j of the state).
  auto forward = [&](const Tok& x) {
    wave_sync();  // earlier readers of kv are done
    kv[j] = x.k;
    wave_sync();
    float u = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) u += s[i] * kv[i];
    const float y = x.be * x.v - x.a * x.be * u;
#pragma unroll
    for (int i = 0; i < D; ++i) s[i] = x.a * s[i] + kv[i] * y;
  };

  // Pass 1: checkpoints S at the start of every block.
  {
    Tok cur{};
    if (T > 0) cur = load(0, false);  // T = 0: the input buffers may be empty
    for (int t = 0; t < T; ++t) {
      if (t % SUB == 0) {
#pragma unroll
        for (int i = 0; i < D; ++i) ck[((size_t)(t / SUB) * D + i) * D + j] = s[i];
      }
      const Tok nxt = load(t + 1, false);
      forward(cur);
      cur = nxt;
    }
  }

  // Pass 2: blocks in reverse; g is column j of G.
  float g[D];
#pragma unroll
  for (int i = 0; i < D; ++i) g[i] = dSf ? dSf[((size_t)chain * D + i) * D + j] : 0.f;
  for (int c = nsub - 1; c >= 0; --c) {
    const int mend = min(SUB, T - c * SUB);
#pragma unroll
    for (int i = 0; i < D; ++i) s[i] = ck[((size_t)c * D + i) * D + j];
    Tok cur = load(c * SUB, false);
    for (int m = 0; m < mend; ++m) {
#pragma unroll
      for (int i = 0; i < D; ++i) st[m][j][i] = s[i];
      if (m + 1 < mend) {  // the block's last state is not needed
        const Tok nxt = load(c * SUB + m + 1, false);
        forward(cur);
        cur = nxt;
      }
    }
    cur = load(c * SUB + mend - 1, true);
    for (int m = mend - 1; m >= 0; --m) {
      const size_t r = tok(c * SUB + m);
      const Tok nxt = load(c * SUB + m - 1, true);
      wave_sync();  // st written, earlier readers of kv / qv / red done
      kv[j] = cur.k;
      qv[j] = cur.q;
      wave_sync();
      const float a = cur.a, be = cur.be, vj = cur.v, doj = cur.dO;
      float u = 0.f, w = 0.f, dsp = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        g[i] += qv[i] * doj;  // D = G + q dO^T
        u += st[m][j][i] * kv[i];
        w += g[i] * kv[i];
        dsp += g[i] * st[m][j][i];
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
      for (int i = 0; i < D; ++i) red[j * LDC + i] = st[m][j][i] * doj;
      wave_sync();
      float r1 = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) r1 += red[x * LDC + j];
      wave_sync();
      const float ab = a * be;
#pragma unroll
      for (int i = 0; i < D; ++i) red[j * LDC + i] = g[i] * y - ab * st[m][j][i] * w;
      wave_sync();
      float r2 = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) r2 += red[x * LDC + j];
      dq[r * D + j] = a * r1 + kv[j] * ydo;  // lane j now stands for row j
      dk[r * D + j] = r2;
#pragma unroll
      for (int i = 0; i < D; ++i) g[i] = a * (g[i] - be * kv[i] * w);
      cur = nxt;
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
