// tok_bwd.hip -- reverse-mode gradients of the gated delta rule token by
// token, for fp32 data (d = 64) and complex64 data (d = 32); fp32 arithmetic.
//
// Per (batch, head) chain the forward is u_t = S_{t-1}^T kr_t,
// S_t = alpha_t (S_{t-1} - beta_t k_t u_t^T) + beta_t k_t v_t^T and
// o_t = S_t^T qr_t, with kr = k, qr = q for real data and kr = conj(k),
// qr = conj(q) for complex data (DeltaPhase section 2: the phase memory reads
// with the conjugated key; forget gate of the Sykra README, "Architectural
// Highlights").  For the real loss L, the gradient of a complex value z is
// dL/dRe z + i dL/dIm z.  With G the gradient reaching S_t from later tokens,
// token by token in reverse (conj is the identity for real data):
//   D = G + q_t dO_t^T,  w = D^T conj(k_t),  y = beta_t v_t - alpha_t beta_t u_t,
//   dq_t = S_t conj(dO_t) = alpha_t S_{t-1} conj(dO_t) + k_t (y . conj(dO_t)),
//   dk_t = D conj(y) - alpha_t beta_t S_{t-1} conj(w),  dv_t = beta_t w,
//   dbeta_t = Re(conj(w) . (v_t - alpha_t u_t)),
//   dalpha_t = Re <D, S_{t-1}> - beta_t Re(conj(w) . u_t),
//   G <- alpha_t (D - beta_t k_t w^T);  dS0 is the last G.
//
// The columns of S (value channels) evolve independently, in the forward and
// in this reverse pass: only dq, dk, dalpha and dbeta sum over them, and they
// are linear in those sums.  So each chain is split into groups of NCW
// columns (8 for fp32, 4 for complex64), one wave each (no workgroup barrier
// on the token chain).  Lane l owns column NCW g + l / L of its group g and
// rows R (l % L) .. + R - 1 (L = 64 / NCW lanes per column, R = D / L);
// column sums are L-lane DPP sums, the row sums over the wave's columns go
// through an LDS transpose within the wave.  A wave issues one vector
// instruction per 4 cycles, so a token step costs about one lane's
// instructions: the complex chain runs as eight waves of 4 columns (2 rows
// per lane), not four of 8.  Each wave writes its
// group's share of dq, dk, dalpha and dbeta to the workspace, and a second
// launch adds the groups' shares.  S_{t-1} is needed in reverse order: a first
// pass runs the forward and checkpoints the group's columns every 8 tokens; the
// reverse pass recomputes each 8-token block from its checkpoint into
// registers and walks it backwards.  Inputs are staged in LDS a block at a
// time, loaded from memory one block (8 tokens) ahead of their use.
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_lane.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace tbwd {

constexpr int SUB = 8;  // tokens per checkpoint block
typedef float f4 __attribute__((ext_vector_type(4)));

// Real and complex scalars with the same operations (conj is the identity for real).
struct rf {
  float x;
};
struct cf {
  float x, y;
};
__device__ __forceinline__ rf operator+(rf a, rf b) { return {a.x + b.x}; }
__device__ __forceinline__ rf operator-(rf a, rf b) { return {a.x - b.x}; }
__device__ __forceinline__ rf operator*(float s, rf a) { return {s * a.x}; }
__device__ __forceinline__ rf mul(rf a, rf b) { return {a.x * b.x}; }
__device__ __forceinline__ rf mulc(rf a, rf b) { return {a.x * b.x}; }  // a conj(b)
__device__ __forceinline__ float dotr(rf a, rf b) { return a.x * b.x; }  // Re(conj(a) b)
__device__ __forceinline__ cf operator+(cf a, cf b) { return {a.x + b.x, a.y + b.y}; }
__device__ __forceinline__ cf operator-(cf a, cf b) { return {a.x - b.x, a.y - b.y}; }
__device__ __forceinline__ cf operator*(float s, cf a) { return {s * a.x, s * a.y}; }
__device__ __forceinline__ cf mul(cf a, cf b) { return {a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x}; }
__device__ __forceinline__ cf mulc(cf a, cf b) { return {a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y}; }
__device__ __forceinline__ float dotr(cf a, cf b) { return a.x * b.x + a.y * b.y; }

// Sum over the L consecutive lanes of a column, L = 8 or 16: xor 1, xor 2 by
// quad_perm, then the half-row mirror (and for 16 lanes the row mirror), each
// reading a partner whose partial sum covers the other half once the smaller
// groups agree; every lane of the column ends with the same value.
template <int ctrl> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xf, 0xf, true));
}
template <int L> __device__ __forceinline__ float colsum(float v) {
  static_assert(L == 8 || L == 16, "column width");
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  if constexpr (L == 16) v += dpp<0x140>(v);
  return v;
}
template <int L> __device__ __forceinline__ rf colsum(rf a) { return {colsum<L>(a.x)}; }
template <int L> __device__ __forceinline__ cf colsum(cf a) { return {colsum<L>(a.x), colsum<L>(a.y)}; }
__device__ __forceinline__ rf wsum(rf a) { return {lane::wave_sum(a.x)}; }
__device__ __forceinline__ cf wsum(cf a) { return {lane::wave_sum(a.x), lane::wave_sum(a.y)}; }

// Orders this wave's LDS accesses across its lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool CX> struct Cfg {
  using S = typename std::conditional<CX, cf, rf>::type;
  static constexpr int D = CX ? 32 : 64;  // head dimension (d_k = d_v)
  static constexpr int NCW = CX ? 4 : 8;  // columns per wave
  static constexpr int L = 64 / NCW;      // lanes per column
  static constexpr int R = D / L;         // rows per lane
  static constexpr int NG = D / NCW;      // column groups (waves) per chain
  static constexpr int W = CX ? 2 : 1;    // floats per element
  static constexpr int P = 2 * D;         // partial elements per token: dq, dk
};

template <bool CX> __device__ __forceinline__ typename Cfg<CX>::S ld(const float* p) {
  if constexpr (CX) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    return cf{v.x, v.y};
  } else {
    return rf{*p};
  }
}
__device__ __forceinline__ void stv(float* p, rf a) { *p = a.x; }
__device__ __forceinline__ void stv(float* p, cf a) { *reinterpret_cast<float2*>(p) = make_float2(a.x, a.y); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_rsrc(const float* base, size_t end, size_t begin) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, end > begin ? (int)(end - begin) : 0,
                                           0x00020000);
}

// One 8-token block of inputs staged in LDS: k and q rows, this group's
// columns of v and dO, the gates.
template <bool CX> struct Blk {
  static constexpr int D = Cfg<CX>::D, W = Cfg<CX>::W, NCW = Cfg<CX>::NCW;
  float k[SUB][D * W], q[SUB][D * W], v[SUB][NCW * W], dO[SUB][NCW * W], a[SUB], be[SUB];
};

// Element pointers are float pointers; element e of a complex array is at 2 e.
template <bool CX>
__global__ __launch_bounds__(64) void tok_bwd_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                     const float* __restrict__ v, const float* __restrict__ alpha,
                                                     const float* __restrict__ beta, const float* __restrict__ S0,
                                                     const float* __restrict__ dO, const float* __restrict__ dSf,
                                                     float* __restrict__ dv, float* __restrict__ dS0,
                                                     float* __restrict__ part, float* __restrict__ partg,
                                                     float* __restrict__ ckpt, int T, int H) {
  using C = Cfg<CX>;
  using S = typename C::S;
  constexpr int D = C::D, R = C::R, NG = C::NG, W = C::W, NCW = C::NCW, L = C::L;
  constexpr int KPL = SUB * D * W / 4 / 64;  // float4 of a k (or q) block per lane: 2
  constexpr int VPL = SUB * NCW * W / 64;    // floats of a v (or dO) block per lane: 1 or 2
  static_assert(KPL * 256 == SUB * D * W && VPL * 64 == SUB * NCW * W, "block shapes");
  __shared__ __attribute__((aligned(16))) Blk<CX> buf[2];
  __shared__ __attribute__((aligned(16))) float red[2][NCW][D * W + 4];  // [product][column][row] for the row sums
  const int l = threadIdx.x;
  // A chain's groups on one XCD (the hardware deals consecutive blocks to the
  // eight XCDs in turn), so its k and q rows are fetched once into that L2.
  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int grp = bid % NG, chain = bid / NG, b = chain / H, h = chain % H;
  const int cl = l / L, c = grp * NCW + cl, rq = l % L, i0 = R * rq;
  const int nsub = (T + SUB - 1) / SUB;
  const size_t ntok = (size_t)(gridDim.x / NG) * T;
  // checkpoints of this group's columns: [nsub][NCW][D]
  float* const ck = ckpt + (size_t)bid * nsub * NCW * D * W;
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };
  const size_t gbase = (size_t)b * T * H + h;
  const __amdgpu_buffer_rsrc_t ra = gate_rsrc(alpha + gbase, (size_t)T * H * 4, (size_t)h * 4);
  const __amdgpu_buffer_rsrc_t rb = gate_rsrc(beta + gbase, (size_t)T * H * 4, (size_t)h * 4);

  // A block's inputs in registers, loaded one block ahead of its use; tokens
  // past T read token T - 1 (never used).
  struct Regs {
    f4 k[KPL], q[KPL];
    float v[VPL], dO[VPL], g;
  };
  auto load_block = [&](int blk, bool back) {
    Regs x{};
    const int t0 = blk * SUB;
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
      const int f = (l + 64 * u) * 4, m = f / (D * W), e = f % (D * W);  // token of the block, float of its row
      const size_t r = tok(min(t0 + m, T - 1));
      x.k[u] = *reinterpret_cast<const f4*>(k + r * D * W + e);
      if (back) x.q[u] = *reinterpret_cast<const f4*>(q + r * D * W + e);
    }
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int f = l + 64 * u, m = f / (NCW * W), e = f % (NCW * W);
      const size_t r = tok(min(t0 + m, T - 1));
      x.v[u] = v[r * D * W + grp * NCW * W + e];
      if (back) x.dO[u] = dO[r * D * W + grp * NCW * W + e];
    }
    const int m = l & 7, tc = min(t0 + m, T - 1);
    x.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(l < 8 ? ra : rb, tc * H * 4, 0, 0));
    return x;
  };
  auto store_block = [&](const Regs& x, Blk<CX>& B, bool back) {
#pragma unroll
    for (int u = 0; u < KPL; ++u) {
      const int f = (l + 64 * u) * 4, m = f / (D * W), e = f % (D * W);
      *reinterpret_cast<f4*>(&B.k[m][e]) = x.k[u];
      if (back) *reinterpret_cast<f4*>(&B.q[m][e]) = x.q[u];
    }
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int f = l + 64 * u, m = f / (NCW * W), e = f % (NCW * W);
      B.v[m][e] = x.v[u];
      if (back) B.dO[m][e] = x.dO[u];
    }
    if (l < 8) B.a[l] = x.g;
    else if (l < 16) B.be[l - 8] = x.g;
  };
  auto krow = [&](const Blk<CX>& B, int m, S (&dst)[R], bool isq) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) dst[ii] = ld<CX>(&(isq ? B.q : B.k)[m][(i0 + ii) * W]);
  };

  S s[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) s[ii] = S0 ? ld<CX>(S0 + (((size_t)chain * D + i0 + ii) * D + c) * W) : S{};

  // One forward token m of block B on s: u = S^T conj(k), S <- alpha S + k (beta v - alpha beta u)^T.
  auto forward = [&](const Blk<CX>& B, int m) {
    S kk[R];
    krow(B, m, kk, false);
    const float a = B.a[m], be = B.be[m];
    S u{};
#pragma unroll
    for (int ii = 0; ii < R; ++ii) u = u + mulc(s[ii], kk[ii]);
    u = colsum<L>(u);
    const S y = be * ld<CX>(&B.v[m][cl * W]) - (a * be) * u;
#pragma unroll
    for (int ii = 0; ii < R; ++ii) s[ii] = a * s[ii] + mul(kk[ii], y);
  };
  auto ckp = [&](int blk, int ii) { return ck + (((size_t)blk * NCW + cl) * D + i0 + ii) * W; };

  // Pass 1: the forward, checkpointing S at the start of every block.
  if (nsub > 0) {
    Regs x = load_block(0, false);
    for (int blk = 0; blk < nsub; ++blk) {
      Blk<CX>& B = buf[blk & 1];
      store_block(x, B, false);
      wave_sync();
      if (blk + 1 < nsub) x = load_block(blk + 1, false);
#pragma unroll
      for (int ii = 0; ii < R; ++ii) stv(ckp(blk, ii), s[ii]);
      const int mend = min(SUB, T - blk * SUB);
#pragma unroll
      for (int m = 0; m < SUB; ++m)
        if (m < mend) forward(B, m);
    }
  }

  // Pass 2: blocks in reverse.
  S g[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) g[ii] = dSf ? ld<CX>(dSf + (((size_t)chain * D + i0 + ii) * D + c) * W) : S{};
  constexpr int NRD = 2 * D / 64;  // row sums per lane: 2 (real, D = 64) or 1 (complex, D = 32)
  if (nsub > 0) {
    Regs x = load_block(nsub - 1, true);
    S nck[R];
#pragma unroll
    for (int ii = 0; ii < R; ++ii) nck[ii] = ld<CX>(ckp(nsub - 1, ii));
    for (int cb = nsub - 1; cb >= 0; --cb) {
      Blk<CX>& B = buf[cb & 1];
      wave_sync();  // the walk two blocks back has finished reading this buffer
      store_block(x, B, true);
      wave_sync();
      if (cb > 0) x = load_block(cb - 1, true);
      const int t0 = cb * SUB, mend = min(SUB, T - t0);
#pragma unroll
      for (int ii = 0; ii < R; ++ii) s[ii] = nck[ii];
      S sp[SUB][R];
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        if (m < mend) {
#pragma unroll
          for (int ii = 0; ii < R; ++ii) sp[m][ii] = s[ii];
          if (m + 1 < mend) forward(B, m);
        }
      }
      const int cbn = max(cb - 1, 0);
#pragma unroll
      for (int ii = 0; ii < R; ++ii) nck[ii] = ld<CX>(ckp(cbn, ii));
#pragma unroll
      for (int m = SUB - 1; m >= 0; --m) {
        if (m < mend) {
          const size_t r = tok(t0 + m);
          const float a = B.a[m], be = B.be[m], ab = a * be;
          const S vc = ld<CX>(&B.v[m][cl * W]), doc = ld<CX>(&B.dO[m][cl * W]);
          S kk[R], qq[R];
          krow(B, m, kk, false);
          krow(B, m, qq, true);
          S u{}, wc{};
          float dsp = 0.f;
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            g[ii] = g[ii] + mul(qq[ii], doc);  // D = G + q dO^T
            u = u + mulc(sp[m][ii], kk[ii]);
            wc = wc + mulc(g[ii], kk[ii]);
            dsp += dotr(g[ii], sp[m][ii]);
          }
          u = colsum<L>(u);
          wc = colsum<L>(wc);
          const S y = be * vc - ab * u;
          if (rq == 0) stv(dv + (r * D + c) * W, be * wc);
          const float lead = rq == 0 ? 1.f : 0.f;  // one copy of each per-column term
          const float db = lane::wave_sum(lead * dotr(wc, vc - a * u));
          const float da = lane::wave_sum(dsp - lead * be * dotr(wc, u));
          const S yd = wsum(lead * mulc(y, doc));
          // Row sums over the wave's columns through LDS: sum_c S_{t-1}[i][c] conj(dO_c) and
          // sum_c (D[i][c] conj(y_c) - alpha beta S_{t-1}[i][c] conj(w_c)).
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            stv(&red[0][cl][(i0 + ii) * W], mulc(sp[m][ii], doc));
            stv(&red[1][cl][(i0 + ii) * W], mulc(g[ii], y) - ab * mulc(sp[m][ii], wc));
          }
          wave_sync();
          float* const pr = part + ((size_t)grp * ntok + r) * C::P * W;
#pragma unroll
          for (int n = 0; n < NRD; ++n) {
            const int e = l + 64 * n;           // 0 .. 2 D - 1
            const int pi = e / D, row = e % D;  // product, row
            S acc{};
#pragma unroll
            for (int xc = 0; xc < NCW; ++xc) acc = acc + ld<CX>(&red[pi][xc][row * W]);
            // dq share: alpha sum_c S conj(dO) + k_row (y . conj(dO)); dk share: the second sum
            if (pi == 0) acc = a * acc + mul(ld<CX>(&B.k[m][row * W]), yd);
            stv(pr + (size_t)e * W, acc);
          }
          if (l == 0) {
            float* const pg = partg + ((size_t)grp * ntok + r) * 2;
            pg[0] = da;
            pg[1] = db;
          }
          wave_sync();
#pragma unroll
          for (int ii = 0; ii < R; ++ii) g[ii] = a * (g[ii] - be * mul(kk[ii], wc));
        }
      }
    }
  }
  if (dS0) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) stv(dS0 + (((size_t)chain * D + i0 + ii) * D + c) * W, g[ii]);
  }
}

// dq, dk, dalpha, dbeta: the column groups' shares added, per token-head.
template <bool CX>
__global__ __launch_bounds__(256) void tok_bwd_sum_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ partg, float* __restrict__ dq,
                                                          float* __restrict__ dk, float* __restrict__ dalpha,
                                                          float* __restrict__ dbeta, long ntok) {
  using C = Cfg<CX>;
  constexpr int D = C::D, W = C::W, PW = C::P * W, NG = C::NG;
  const long per = (long)PW + 2;  // floats per token-head: shares of dq, dk, then dalpha, dbeta
  const long total = ntok * per;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long t = i / per, e = i % per;
    float acc = 0.f;
    if (e < PW) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) acc += part[((size_t)gi * ntok + t) * PW + e];
      if (e < D * W)
        dq[t * D * W + e] = acc;
      else
        dk[t * D * W + e - D * W] = acc;
    } else {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) acc += partg[((size_t)gi * ntok + t) * 2 + (e - PW)];
      (e == PW ? dalpha : dbeta)[t] = acc;
    }
  }
}

}  // namespace tbwd

template <bool CX> static size_t tok_bwd_bytes(int B, int T, int H, size_t* ck_bytes) {
  using C = tbwd::Cfg<CX>;
  const size_t chains = (size_t)B * H, nsub = (T + tbwd::SUB - 1) / tbwd::SUB;
  const size_t ck = chains * C::NG * nsub * C::NCW * C::D * C::W * 4;
  const size_t ntok = (size_t)B * T * H;
  if (ck_bytes) *ck_bytes = ck;
  return ck + C::NG * ntok * (C::P * C::W + 2) * 4;
}

size_t tok_bwd_workspace_bytes(int B, int T, int H, bool complex_data) {
  return complex_data ? tok_bwd_bytes<true>(B, T, H, nullptr) : tok_bwd_bytes<false>(B, T, H, nullptr);
}

template <bool CX> static hipError_t launch_tok(const BwdArgs& a) {
  using C = tbwd::Cfg<CX>;
  size_t ck_bytes = 0;
  tok_bwd_bytes<CX>(a.B, a.T, a.H, &ck_bytes);
  char* ws = static_cast<char*>(a.workspace);
  float* ck = reinterpret_cast<float*>(ws);
  const size_t ntok = (size_t)a.B * a.T * a.H;
  float* part = reinterpret_cast<float*>(ws + ck_bytes);
  float* partg = part + C::NG * ntok * C::P * C::W;
  hipStream_t st = (hipStream_t)a.stream;
  hipError_t e = launch_kernel(tbwd::tok_bwd_kernel<CX>, dim3((unsigned)((long)a.B * a.H * C::NG)), dim3(64), st,
                               (const float*)a.q, (const float*)a.k, (const float*)a.v, a.alpha, a.beta, a.S0,
                               (const float*)a.dout, a.dS_final, a.dv, a.dS0, part, partg, ck, a.T, a.H);
  if (e != hipSuccess || ntok == 0) return e;
  const long total = (long)ntok * (C::P * C::W + 2);
  const long blocks = (total + 255) / 256;
  return launch_kernel(tbwd::tok_bwd_sum_kernel<CX>, dim3((unsigned)(blocks < (1L << 20) ? blocks : (1L << 20))),
                       dim3(256), st, (const float*)part, (const float*)partg, a.dq, a.dk, a.dalpha, a.dbeta,
                       (long)ntok);
}

hipError_t launch_tok_bwd(const BwdArgs& a, bool complex_data) {
  return complex_data ? launch_tok<true>(a) : launch_tok<false>(a);
}

}  // namespace gdn
