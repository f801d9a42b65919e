// bwd_cx.hip -- reverse-mode gradients of the gated delta rule for complex
// data, d_k = d_v = 32 (complex64 inputs, fp32 arithmetic, complex64 and fp32
// gradients).
//
// Per (batch, head) chain the forward is u_t = S_{t-1}^T conj(k_t),
// S_t = alpha_t (S_{t-1} - beta_t k_t u_t^T) + beta_t k_t v_t^T and
// o_t = S_t^T conj(q_t): the phase memory of DeltaPhase section 2 (readout with
// the conjugated key, output with the conjugated query), with real gates (the
// forget gate of the Sykra README, "Architectural Highlights").  For the real
// loss L, the gradient of a complex value z is dL/dRe z + i dL/dIm z; with G
// the gradient reaching S_t from later tokens, token by token in reverse:
//   D = G + q_t dO_t^T,  w = D^T conj(k_t),  y = beta_t v_t - alpha_t beta_t u_t,
//   dq_t = S_t conj(dO_t) = alpha_t S_{t-1} conj(dO_t) + k_t (y . conj(dO_t)),
//   dk_t = D conj(y) - alpha_t beta_t S_{t-1} conj(w),  dv_t = beta_t w,
//   dbeta_t = Re(conj(w) . (v_t - alpha_t u_t)),
//   dalpha_t = Re <D, S_{t-1}> - beta_t Re(conj(w) . u_t)   (<A, B> = sum conj(A) B),
//   G <- alpha_t (D - beta_t k_t w^T);  dS0 is the last G.
//
// Two waves per chain (128 threads).  Thread (w, l) owns column
// c = 16 w + l / 4 and rows 8 (l % 4) .. + 7 of S and of G, 8 complex
// registers each; column sums are an in-lane sum and two DPP adds within the
// lane quad that holds the column; the row sums for dq and dk go through LDS.
// S_{t-1} is needed in reverse order: a first pass runs the forward and
// checkpoints S every 8 tokens to the workspace; the reverse pass recomputes
// each 8-token block from its checkpoint into registers and walks it
// backwards.  Barriers wait for LDS only, and each token's inputs are loaded
// while the token before it in the walk is computed.
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_lane.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace bwdcx {

using lane::quad_sum;
using lane::wave_sum;

constexpr int D = 32;       // complex head dimension (d_k = d_v)
constexpr int SUB = 8;      // tokens per checkpoint block
constexpr int NWV = 2;      // waves per chain
constexpr int R = 8;        // rows per thread
constexpr int LDC = D + 1;  // row stride (complex) of the product buffers

struct cf {
  float x, y;
};
__device__ __forceinline__ cf cadd(cf a, cf b) { return {a.x + b.x, a.y + b.y}; }
__device__ __forceinline__ cf csub(cf a, cf b) { return {a.x - b.x, a.y - b.y}; }
__device__ __forceinline__ cf cscale(float s, cf a) { return {s * a.x, s * a.y}; }
__device__ __forceinline__ cf cmul(cf a, cf b) { return {a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x}; }
// a conj(b)
__device__ __forceinline__ cf cmulc(cf a, cf b) { return {a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y}; }
// Re(conj(a) b)
__device__ __forceinline__ float cdotr(cf a, cf b) { return a.x * b.x + a.y * b.y; }
__device__ __forceinline__ cf cquad(cf a) { return {quad_sum(a.x), quad_sum(a.y)}; }
__device__ __forceinline__ cf cwave(cf a) { return {wave_sum(a.x), wave_sum(a.y)}; }
__device__ __forceinline__ cf ld(const float2* p) {
  const float2 v = *p;
  return {v.x, v.y};
}
__device__ __forceinline__ void st(float2* p, cf a) { *p = make_float2(a.x, a.y); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_rsrc(const float* base, size_t end, size_t begin) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, end > begin ? (int)(end - begin) : 0,
                                           0x00020000);
}

// All waves meet; LDS writes before it are visible after it.  Global loads
// and stores in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(128) void bwd_cx_kernel(const float2* __restrict__ q, const float2* __restrict__ k,
                                                     const float2* __restrict__ v, const float* __restrict__ alpha,
                                                     const float* __restrict__ beta, const float2* __restrict__ S0,
                                                     const float2* __restrict__ dO, const float2* __restrict__ dSf,
                                                     float2* __restrict__ dq, float2* __restrict__ dk,
                                                     float2* __restrict__ dv, float* __restrict__ dalpha,
                                                     float* __restrict__ dbeta, float2* __restrict__ dS0,
                                                     float2* __restrict__ ckpt, int T, int H) {
  __shared__ float2 kv[2][D], qv[2][D];     // k_t, q_t (double-buffered by token)
  __shared__ float2 red[2][D * LDC];        // [column][row] products for the row sums
  __shared__ float2 rowp[2][NWV][D];        // per-wave partial row sums
  __shared__ float scal[2][4][NWV];         // per-wave dbeta, dalpha, y . conj(dO) (re, im), by token parity
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = 16 * w + (l >> 2), rq = l & 3, i0 = R * rq;
  const int chain = blockIdx.x, b = chain / H, h = chain % H;
  const int nsub = (T + SUB - 1) / SUB;
  float2* const ck = ckpt + (size_t)chain * nsub * D * D;
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };
  const size_t gbase = (size_t)b * T * H + h;
  const __amdgpu_buffer_rsrc_t ra = gate_rsrc(alpha + gbase, (size_t)T * H * 4, (size_t)h * 4);
  const __amdgpu_buffer_rsrc_t rb = gate_rsrc(beta + gbase, (size_t)T * H * 4, (size_t)h * 4);

  // One token's inputs for this thread: k and q element l % 32 (wave 0 puts
  // them in LDS), v and dO of column c, the gates; t clamped into [0, T).
  struct Tok {
    cf k, q, v, dO;
    float a, be;
  };
  const int e = l & (D - 1);
  auto load = [&](int t, bool back) {
    Tok x{};
    const int tc = max(0, min(t, T - 1));
    const size_t r = tok(tc);
    x.k = ld(k + r * D + e);
    if (back) x.q = ld(q + r * D + e);
    x.v = ld(v + r * D + c);
    if (back) x.dO = ld(dO + r * D + c);
    x.a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, tc * H * 4, 0, 0));
    x.be = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, tc * H * 4, 0, 0));
    return x;
  };

  cf s[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) s[ii] = S0 ? ld(S0 + ((size_t)chain * D + i0 + ii) * D + c) : cf{0.f, 0.f};

  int par = 0;
  // One forward token on s: u = S^T conj(k), S <- alpha S + k (beta v - alpha beta u)^T.
  auto forward = [&](const Tok& x) {
    if (w == 0 && l < D) kv[par][l] = make_float2(x.k.x, x.k.y);
    lds_barrier();
    cf kk[R];
#pragma unroll
    for (int ii = 0; ii < R; ++ii) {
      const float2 t2 = kv[par][i0 + ii];
      kk[ii] = {t2.x, t2.y};
    }
    cf u{0.f, 0.f};
#pragma unroll
    for (int ii = 0; ii < R; ++ii) u = cadd(u, cmulc(s[ii], kk[ii]));
    u = cquad(u);
    const cf y = csub(cscale(x.be, x.v), cscale(x.a * x.be, u));
#pragma unroll
    for (int ii = 0; ii < R; ++ii) s[ii] = cadd(cscale(x.a, s[ii]), cmul(kk[ii], y));
    par ^= 1;
  };

  // Pass 1: checkpoints S at the start of every block.
  {
    Tok cur{};
    if (T > 0) cur = load(0, false);
    for (int t = 0; t < T; ++t) {
      if (t % SUB == 0) {
#pragma unroll
        for (int ii = 0; ii < R; ++ii) st(ck + ((size_t)(t / SUB) * D + c) * D + i0 + ii, s[ii]);
      }
      const Tok nxt = load(t + 1, false);
      forward(cur);
      cur = nxt;
    }
  }

  // Pass 2: blocks in reverse.
  cf g[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) g[ii] = dSf ? ld(dSf + ((size_t)chain * D + i0 + ii) * D + c) : cf{0.f, 0.f};
  cf nck[R];
  if (nsub > 0) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) nck[ii] = ld(ck + ((size_t)(nsub - 1) * D + c) * D + i0 + ii);
  }
  for (int cb = nsub - 1; cb >= 0; --cb) {
    const int t0 = cb * SUB, mend = min(SUB, T - t0);
#pragma unroll
    for (int ii = 0; ii < R; ++ii) s[ii] = nck[ii];
    cf sp[SUB][R];
    const Tok wfirst = load(t0 + mend - 1, true);
    Tok cur = load(t0, false);
#pragma unroll
    for (int m = 0; m < SUB; ++m) {
      if (m < mend) {
#pragma unroll
        for (int ii = 0; ii < R; ++ii) sp[m][ii] = s[ii];
        if (m + 1 < mend) {
          const Tok nxt = load(t0 + m + 1, false);
          forward(cur);
          cur = nxt;
        }
      }
    }
    cur = wfirst;
    const int cbn = max(cb - 1, 0);
#pragma unroll
    for (int ii = 0; ii < R; ++ii) nck[ii] = ld(ck + ((size_t)cbn * D + c) * D + i0 + ii);
    if (w == 0 && l < D) {
      kv[par][l] = make_float2(cur.k.x, cur.k.y);
      qv[par][l] = make_float2(cur.q.x, cur.q.y);
    }
    lds_barrier();
#pragma unroll
    for (int m = SUB - 1; m >= 0; --m) {
      if (m < mend) {
        const size_t r = tok(t0 + m);
        const Tok nxt = load(t0 + m - 1, true);
        const float a = cur.a, be = cur.be, ab = a * be;
        const cf vc = cur.v, doc = cur.dO;
        cf kk[R];
        cf u{0.f, 0.f}, wc{0.f, 0.f};
        float dsp = 0.f;
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          const float2 k2 = kv[par][i0 + ii], q2 = qv[par][i0 + ii];
          kk[ii] = {k2.x, k2.y};
          g[ii] = cadd(g[ii], cmul({q2.x, q2.y}, doc));  // D = G + q dO^T
          u = cadd(u, cmulc(sp[m][ii], kk[ii]));
          wc = cadd(wc, cmulc(g[ii], kk[ii]));
          dsp += cdotr(g[ii], sp[m][ii]);
        }
        u = cquad(u);
        wc = cquad(wc);
        const cf y = csub(cscale(be, vc), cscale(ab, u));
        if (rq == 0) st(dv + r * D + c, cscale(be, wc));
        const float lead = rq == 0 ? 1.f : 0.f;  // one copy of each per-column term
        const float db = wave_sum(lead * cdotr(wc, csub(vc, cscale(a, u))));
        const float da = wave_sum(dsp - lead * be * cdotr(wc, u));
        const cf yd = cwave(cscale(lead, cmulc(y, doc)));
        if (l == 0) {
          scal[par][0][w] = db;
          scal[par][1][w] = da;
          scal[par][2][w] = yd.x;
          scal[par][3][w] = yd.y;
        }
        // Row sums over the columns: sum_c S_{t-1}[i][c] conj(dO_c) and
        // sum_c (D[i][c] conj(y_c) - alpha beta S_{t-1}[i][c] conj(w_c)).
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          const cf p1 = cmulc(sp[m][ii], doc);
          const cf p2 = csub(cmulc(g[ii], y), cscale(ab, cmulc(sp[m][ii], wc)));
          red[0][c * LDC + i0 + ii] = make_float2(p1.x, p1.y);
          red[1][c * LDC + i0 + ii] = make_float2(p2.x, p2.y);
        }
        lds_barrier();
        if (l < D) {  // row l over the columns of wave w
          cf p1{0.f, 0.f}, p2{0.f, 0.f};
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const float2 a1 = red[0][(16 * w + x) * LDC + l], a2 = red[1][(16 * w + x) * LDC + l];
            p1 = cadd(p1, {a1.x, a1.y});
            p2 = cadd(p2, {a2.x, a2.y});
          }
          rowp[0][w][l] = make_float2(p1.x, p1.y);
          rowp[1][w][l] = make_float2(p2.x, p2.y);
        }
        if (w == 0 && l < D && m > 0) {  // the next token's k and q (that buffer's readers are two steps back)
          kv[par ^ 1][l] = make_float2(nxt.k.x, nxt.k.y);
          qv[par ^ 1][l] = make_float2(nxt.q.x, nxt.q.y);
        }
        lds_barrier();
        if (w == 0 && l < D) {
          const float2 a0 = rowp[0][0][l], a1 = rowp[0][1][l], b0 = rowp[1][0][l], b1 = rowp[1][1][l];
          const cf r1{a0.x + a1.x, a0.y + a1.y}, r2{b0.x + b1.x, b0.y + b1.y};
          const cf ydo{scal[par][2][0] + scal[par][2][1], scal[par][3][0] + scal[par][3][1]};
          st(dq + r * D + l, cadd(cscale(a, r1), cmul(cur.k, ydo)));  // cur.k is k_l here
          st(dk + r * D + l, r2);
          if (l == 0) {
            dbeta[r] = scal[par][0][0] + scal[par][0][1];
            dalpha[r] = scal[par][1][0] + scal[par][1][1];
          }
        }
#pragma unroll
        for (int ii = 0; ii < R; ++ii) g[ii] = cscale(a, csub(g[ii], cmul(cscale(be, kk[ii]), wc)));
        par ^= 1;
        cur = nxt;
      }
    }
  }
  if (dS0) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) st(dS0 + ((size_t)chain * D + i0 + ii) * D + c, g[ii]);
  }
}

}  // namespace bwdcx

size_t chunk_bwd_cx_workspace_bytes(int B, int T, int H) {
  return (size_t)B * H * ((T + bwdcx::SUB - 1) / bwdcx::SUB) * bwdcx::D * bwdcx::D * sizeof(float2);
}

hipError_t launch_chunk_bwd_cx(const BwdArgs& a) {
  const dim3 grid((unsigned)((long)a.B * a.H)), block(bwdcx::NWV * 64);
  return launch_kernel(bwdcx::bwd_cx_kernel, grid, block, (hipStream_t)a.stream, (const float2*)a.q,
                       (const float2*)a.k, (const float2*)a.v, a.alpha, a.beta, (const float2*)a.S0,
                       (const float2*)a.dout, (const float2*)a.dS_final, (float2*)a.dq, (float2*)a.dk, (float2*)a.dv,
                       a.dalpha, a.dbeta, (float2*)a.dS0, (float2*)a.workspace, a.T, a.H);
}

}  // namespace gdn
