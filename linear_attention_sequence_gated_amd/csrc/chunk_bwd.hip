// chunk_bwd.hip -- reverse-mode gradients of the gated delta rule, real data,
// d_k = d_v = 64, bf16 inputs, fp32 arithmetic and gradients: the token-loop
// pass for the bf16 calls the chunk form does not take (T == 0, and layers
// whose gradient rows pass 32-bit offsets).
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
// Four waves per chain (256 threads).  Thread (w, l) owns column
// c = 16 w + l / 4 and rows 16 (l % 4) .. + 15 of the state S and of the
// carried gradient G, 16 registers each.  Column sums (u, w) are a 16-term
// in-lane sum and two DPP adds within the lane quad that holds the column;
// wave sums are DPP adds within rows of 16 lanes and four lane reads.  The two row sums per token (for dq
// and dk) go through LDS: every thread writes its 16 products of each, then
// thread (w, l) sums row l over the 16 columns of wave w, and wave 0 adds the
// four partial sums.  S_{t-1} is needed in reverse order: a first pass runs
// the forward and checkpoints S every 8 tokens to the workspace (column-major
// per chain); the reverse pass recomputes each 8-token block from its
// checkpoint into registers (8 x 16 per thread) and walks it backwards.
// Barriers wait for LDS only (a workgroup barrier's fence would also wait for
// every global load and store in flight), and each token's inputs are loaded
// while the token before it in the walk is computed.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_lane.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace bwd {

using lane::quad_sum;
using lane::wave_sum;

constexpr int D = 64;       // head dimension (d_k = d_v)
constexpr int SUB = 8;      // tokens per checkpoint block
constexpr int NWV = 4;      // waves per chain
constexpr int R = 16;       // rows per thread
constexpr int LDC = D + 4;  // row stride of the product buffers (16-byte rows)

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __hip_bfloat16* p) { return __bfloat162float(*p); }
__device__ __forceinline__ float f32(float x) { return x; }

// Raw buffer resource over `bytes` bytes from `base`.  The gates are read
// through it so that their (uniform) loads are vector-memory loads: a scalar
// load would be counted with LDS traffic, and every barrier's LDS wait would
// then also wait for the next token's gates.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_rsrc(const float* base, size_t end, size_t begin) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, end > begin ? (int)(end - begin) : 0,
                                           0x00020000);
}
__device__ __forceinline__ float f32(__hip_bfloat16 x) { return __bfloat162float(x); }

// All waves of the workgroup meet; LDS writes before it are visible after it.
// Global loads and stores in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <class IT>
__global__ __launch_bounds__(256) void bwd_kernel(const IT* __restrict__ q, const IT* __restrict__ k,
                                                  const IT* __restrict__ v, const float* __restrict__ alpha,
                                                  const float* __restrict__ beta, const float* __restrict__ S0,
                                                  const IT* __restrict__ dO, const float* __restrict__ dSf,
                                                  float* __restrict__ dq, float* __restrict__ dk,
                                                  float* __restrict__ dv, float* __restrict__ dalpha,
                                                  float* __restrict__ dbeta, float* __restrict__ dS0,
                                                  float* __restrict__ ckpt, int T, int H) {
  __shared__ __attribute__((aligned(16))) float kv[2][D], qv[2][D];  // k_t, q_t (double-buffered by token)
  __shared__ __attribute__((aligned(16))) float red[2][D * LDC];     // [column][row] products for the row sums
  __shared__ float rowp[2][NWV][D];                                  // per-wave partial row sums
  // Per-wave partial dbeta, dalpha and y . dO, double-buffered by token: the
  // other waves write the next token's partials before the first barrier of
  // the next step, while wave 0 may still be reading this token's.
  __shared__ float scal[2][3][NWV];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = 16 * w + (l >> 2), rq = l & 3, i0 = R * rq;
  const int chain = blockIdx.x, b = chain / H, h = chain % H;
  const int nsub = (T + SUB - 1) / SUB;
  float* const ck = ckpt + (size_t)chain * nsub * D * D;
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };
  const size_t gbase = (size_t)b * T * H + h;
  const __amdgpu_buffer_rsrc_t ra = gate_rsrc(alpha + gbase, (size_t)T * H * 4, (size_t)h * 4);
  const __amdgpu_buffer_rsrc_t rb = gate_rsrc(beta + gbase, (size_t)T * H * 4, (size_t)h * 4);

  // This thread's inputs of one token: k and q element l (wave 0 puts them
  // in LDS for every thread), v and dO of column c, the gates.  t is clamped
  // into [0, T), so the address is valid whenever T > 0.  Values are kept as
  // stored and converted where used, and every wave issues the same loads:
  // the compiler's in-order load counts are then static, and no wave waits
  // for the next token's loads where it only needs this token's.
  struct Tok {
    IT k, q, v, dO;
    float a, be;
  };
  auto load = [&](int t, bool back) {
    Tok x{};
    const int tc = max(0, min(t, T - 1));
    const size_t r = tok(tc);
    x.k = k[r * D + l];
    if (back) x.q = q[r * D + l];
    x.v = v[r * D + c];
    if (back) x.dO = dO[r * D + c];
    x.a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, tc * H * 4, 0, 0));
    x.be = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, tc * H * 4, 0, 0));
    return x;
  };

  float s[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) s[ii] = S0 ? S0[((size_t)chain * D + i0 + ii) * D + c] : 0.f;

  int par = 0;  // LDS buffer parity, flipped per token
  // One forward token on s.
  auto forward = [&](const Tok& x) {
    if (w == 0) kv[par][l] = f32(x.k);
    lds_barrier();
    float kk[R];
#pragma unroll
    for (int ii = 0; ii < R; ++ii) kk[ii] = kv[par][i0 + ii];
    float u = 0.f;
#pragma unroll
    for (int ii = 0; ii < R; ++ii) u += s[ii] * kk[ii];
    u = quad_sum(u);
    const float y = x.be * f32(x.v) - x.a * x.be * u;
#pragma unroll
    for (int ii = 0; ii < R; ++ii) s[ii] = x.a * s[ii] + kk[ii] * y;
    par ^= 1;
  };

  // Pass 1: checkpoints S at the start of every block.
  {
    Tok cur{};
    if (T > 0) cur = load(0, false);  // T = 0: the input buffers may be empty
    for (int t = 0; t < T; ++t) {
      if (t % SUB == 0) {
#pragma unroll
        for (int ii = 0; ii < R; ++ii) ck[((size_t)(t / SUB) * D + c) * D + i0 + ii] = s[ii];
      }
      const Tok nxt = load(t + 1, false);
      forward(cur);
      cur = nxt;
    }
  }

  // Pass 2: blocks in reverse.
  float g[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) g[ii] = dSf ? dSf[((size_t)chain * D + i0 + ii) * D + c] : 0.f;
  float nck[R];  // the next block's checkpoint, loaded during this block's walk
  if (nsub > 0) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) nck[ii] = ck[((size_t)(nsub - 1) * D + c) * D + i0 + ii];
  }
  for (int cb = nsub - 1; cb >= 0; --cb) {
    const int t0 = cb * SUB, mend = min(SUB, T - t0);
#pragma unroll
    for (int ii = 0; ii < R; ++ii) s[ii] = nck[ii];
    float sp[SUB][R];  // S_{t-1} of each token of the block
    const Tok wfirst = load(t0 + mend - 1, true);  // the walk's first token, in flight during the recompute
    Tok cur = load(t0, false);
#pragma unroll
    for (int m = 0; m < SUB; ++m) {
      if (m < mend) {
#pragma unroll
        for (int ii = 0; ii < R; ++ii) sp[m][ii] = s[ii];
        if (m + 1 < mend) {  // the block's last state is not needed
          const Tok nxt = load(t0 + m + 1, false);
          forward(cur);
          cur = nxt;
        }
      }
    }
    cur = wfirst;
    const int cbn = max(cb - 1, 0);
#pragma unroll
    for (int ii = 0; ii < R; ++ii) nck[ii] = ck[((size_t)cbn * D + c) * D + i0 + ii];
    if (w == 0) {  // the walk's first token; later ones are staged before the step's last barrier
      kv[par][l] = f32(cur.k);
      qv[par][l] = f32(cur.q);
    }
    lds_barrier();
#pragma unroll
    for (int m = SUB - 1; m >= 0; --m) {
      if (m < mend) {
        const size_t r = tok(t0 + m);
        const Tok nxt = load(t0 + m - 1, true);
        const float a = cur.a, be = cur.be, vc = f32(cur.v), doc = f32(cur.dO), ab = a * be;
        float kk[R];
        float u = 0.f, wc = 0.f, dsp = 0.f;
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          kk[ii] = kv[par][i0 + ii];
          g[ii] += qv[par][i0 + ii] * doc;  // D = G + q dO^T
          u += sp[m][ii] * kk[ii];
          wc += g[ii] * kk[ii];
          dsp += g[ii] * sp[m][ii];
        }
        u = quad_sum(u);
        wc = quad_sum(wc);
        const float y = be * vc - ab * u;
        if (rq == 0) dv[r * D + c] = be * wc;
        const float lead = rq == 0 ? 1.f : 0.f;  // one copy of each per-column term
        const float db = wave_sum(lead * wc * (vc - a * u));
        const float da = wave_sum(dsp - lead * be * wc * u);
        const float yd = wave_sum(lead * y * doc);
        if (l == 0) {
          scal[par][0][w] = db;
          scal[par][1][w] = da;
          scal[par][2][w] = yd;
        }
        // Row sums over the columns: sum_c S_{t-1}[i][c] dO_c and
        // sum_c (D[i][c] y_c - alpha beta S_{t-1}[i][c] w_c).
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          red[0][c * LDC + i0 + ii] = sp[m][ii] * doc;
          red[1][c * LDC + i0 + ii] = g[ii] * y - ab * sp[m][ii] * wc;
        }
        lds_barrier();
        float p1 = 0.f, p2 = 0.f;  // row l over the columns of wave w
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          p1 += red[0][(16 * w + x) * LDC + l];
          p2 += red[1][(16 * w + x) * LDC + l];
        }
        rowp[0][w][l] = p1;
        rowp[1][w][l] = p2;
        if (w == 0 && m > 0) {  // the next token's k and q (that buffer's readers are two steps back)
          kv[par ^ 1][l] = f32(nxt.k);
          qv[par ^ 1][l] = f32(nxt.q);
        }
        lds_barrier();
        if (w == 0) {
          const float r1 = rowp[0][0][l] + rowp[0][1][l] + rowp[0][2][l] + rowp[0][3][l];
          const float r2 = rowp[1][0][l] + rowp[1][1][l] + rowp[1][2][l] + rowp[1][3][l];
          const float ydo = scal[par][2][0] + scal[par][2][1] + scal[par][2][2] + scal[par][2][3];
          dq[r * D + l] = a * r1 + f32(cur.k) * ydo;  // cur.k is k_l here
          dk[r * D + l] = r2;
          if (l == 0) {
            dbeta[r] = scal[par][0][0] + scal[par][0][1] + scal[par][0][2] + scal[par][0][3];
            dalpha[r] = scal[par][1][0] + scal[par][1][1] + scal[par][1][2] + scal[par][1][3];
          }
        }
#pragma unroll
        for (int ii = 0; ii < R; ++ii) g[ii] = a * (g[ii] - be * kk[ii] * wc);
        par ^= 1;
        cur = nxt;
      }
    }
  }
  if (dS0) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) dS0[((size_t)chain * D + i0 + ii) * D + c] = g[ii];
  }
}

}  // namespace bwd

size_t chunk_bwd_workspace_bytes(int B, int T, int H) {
  return (size_t)B * H * ((T + bwd::SUB - 1) / bwd::SUB) * bwd::D * bwd::D * sizeof(float);
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
  if (a.dtype != kDtBF16) return hipErrorInvalidValue;  // fp32 runs the column-group pass
  const dim3 grid((unsigned)((long)a.B * a.H)), block(bwd::NWV * 64);
  return launch_kernel(bwd::bwd_kernel<__hip_bfloat16>, grid, block, (hipStream_t)a.stream,
                       (const __hip_bfloat16*)a.q, (const __hip_bfloat16*)a.k, (const __hip_bfloat16*)a.v, a.alpha,
                       a.beta, a.S0, (const __hip_bfloat16*)a.dout, a.dS_final, a.dq, a.dk, a.dv, a.dalpha, a.dbeta,
                       a.dS0, (float*)a.workspace, a.T, a.H);
}

}  // namespace gdn
