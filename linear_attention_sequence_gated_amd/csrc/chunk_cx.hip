// chunk_cx.hip -- complex64 chunked forward for head size 32, in three launches.
//
// The method is the chunkwise WY / unit-triangular form of the gated delta
// rule with the read side conjugated (DeltaPhase README, section 1 "Fast
// Triangular Solve" and section 2 on the complex memory; section 5 "Exact
// Chunkwise-Parallel Scan" for the log-space decay).  Per chunk of C = 64
// tokens, with S the state at the chunk start, Kr = conj(K), Qr = conj(Q):
//   A  = strict_lower(diag(beta) Kr K^T * Gamma),   T = (I + A)^{-1},
//   W  = T diag(beta gamma) Kr,   U = T diag(beta) V,   Ut = U - W S,
//   O  = diag(gamma) Qr S + lower(Qr K^T * Gamma) Ut,
//   S <- gamma_C S + (diag(lambda) K)^T Ut,   lambda_t = gamma_C / gamma_t.
//
// One workgroup per (batch, head) walking all chunks leaves most of the chip
// idle at few heads, and every chunk's Gram, inverse and W/U products sit on
// the sequential path.  Here only the state recurrence is sequential, in the
// form of an affine map per chunk (substitute Ut into the state update):
//   S <- M_n S + B_n,   M_n = gamma_C I - (diag(lambda) K)^T W,
//                       B_n = (diag(lambda) K)^T U.
//   1. prep (one workgroup per chunk): gates, Gram tiles, diagonal inverses,
//      block substitution for W and U, then M_n and B_n; writes -W, U, M_n,
//      B_n and the decay prefix to a workspace;
//   2. scan (one workgroup per (chain, 8 value columns)): S <- M_n S + B_n
//      chunk after chunk, writing each chunk-start state S_n;
//   3. out (one workgroup per chunk): Ut = U - W S_n, P = Qr K^T * Gamma and
//      O = diag(gamma) Qr S_n + P Ut.
//
// Complex products in the prep and out kernels use separate real/imaginary
// planes and four real fp32 MFMA products (cmma).  The scan kernel instead
// packs 8 complex columns into the 16 MFMA columns as interleaved (re, im)
// pairs: for X complex with real form Xr = [re, im] pairs, a complex product
// M X equals the real product [Mre | Mim] [X ; swz(X)], where swz maps each
// pair (x, y) to (-y, x).  swz is one DPP lane swap plus a sign flip, so the
// state stays in accumulator registers and feeds the next product directly.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace cx {

constexpr int D = 32;         // key = value head size (complex elements)
constexpr int LDK = D + 4;    // LDS row stride (floats) of a [64][32] plane
constexpr int LD16 = 16 + 4;  // LDS row stride of a 16x16 tile
constexpr int szK = 64 * LDK, szTri = 10 * 16 * LD16;

// Workspace of one chunk, in floats.
constexpr int wG = 64;           // log2 cumulative decay within the chunk
constexpr int wNW = 2 * 64 * D;  // -W, planes [re|im][t][d]
constexpr int wU = 64 * D * 2;   // U: [t][e] interleaved (re, im)
constexpr int wM = 2 * D * D;    // M_n, planes [re|im][d][d']
constexpr int wB = D * D * 2;    // B_n: [d][e] interleaved
constexpr int wS = D * D * 2;    // chunk-start state [d][e] interleaved
constexpr int oG = 0, oNW = oG + wG, oU = oNW + wNW, oM = oU + wU, oB = oM + wM, oS = oB + wB;
constexpr int kChunkFloats = oS + wS;
static_assert(8 * 2 * 256 <= 2 * szK, "Ut tiles fit in the K planes of the output kernel");
static_assert(oNW % 4 == 0 && oU % 4 == 0 && oM % 4 == 0 && oB % 4 == 0 && oS % 4 == 0 && kChunkFloats % 4 == 0,
              "16-byte aligned workspace sections");

__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }

using M = LdsMat<true, float>;
using CS = CSub<true, float>;
using CA = Acc<true>;

// c += sum_{s < n} op(a[s]) op(b[s]) for complex planar sub-blocks, op
// conjugating when CA / CB is set, with three real matrix products per
// sub-block instead of four (Gauss): with sa, sb = -1 for a conjugated
// operand, P1 = ar br, P2 = ai bi, P3 = (ar + sa ai)(br + sb bi) give
// re = P1 - sa sb P2 and im = P3 - P1 - sa sb P2.  The three products are
// accumulated over all sub-blocks before they are combined.
template <bool CA, bool CB, int NMAX>
__device__ __forceinline__ void cmma3(Acc<true>& c, const CSub<true, float> (&a)[NMAX],
                                      const CSub<true, float> (&b)[NMAX], int n) {
  f32x4 p1{0.f, 0.f, 0.f, 0.f}, p2 = p1, p3 = p1;
#pragma unroll
  for (int s = 0; s < NMAX; ++s) {
    if (s < n) {
      const f32x4 as = CA ? a[s].v[0] - a[s].v[1] : a[s].v[0] + a[s].v[1];
      const f32x4 bs = CB ? b[s].v[0] - b[s].v[1] : b[s].v[0] + b[s].v[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s].v[0][j], b[s].v[0][j], p1, 0, 0, 0);
        p2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s].v[1][j], b[s].v[1][j], p2, 0, 0, 0);
        p3 = __builtin_amdgcn_mfma_f32_16x16x4f32(as[j], bs[j], p3, 0, 0, 0);
      }
    }
  }
  constexpr float sg = (CA != CB) ? -1.f : 1.f;  // sa * sb
  c.v[0] += p1 - sg * p2;
  c.v[1] += p3 - p1 - sg * p2;
}

// Row-major token index of (b, t, h) in a [B, T, H, ...] tensor.
__device__ __forceinline__ size_t tok(int b, int t, int h, int T, int H) { return ((size_t)b * T + t) * H + h; }

// Loads one 64-token tile of a [B, T, H, 32] complex tensor into planar LDS
// rows (row t, columns d), zero beyond T.  256 threads, 4 float4 each.
__device__ __forceinline__ void load_tile(const float* __restrict__ src, float* re, float* im, int b, int h, int c0,
                                          int T, int H, int tid) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int unit = tid + 256 * u, row = unit >> 4, cu = unit & 15, t = c0 + row;
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < T) f = *reinterpret_cast<const float4*>(src + tok(b, t, h, T, H) * (2 * D) + 4 * cu);
    *reinterpret_cast<float2*>(re + row * LDK + 2 * cu) = make_float2(f.x, f.z);
    *reinterpret_cast<float2*>(im + row * LDK + 2 * cu) = make_float2(f.y, f.w);
  }
}

// ============================================================== 1. prep
// Value of lane M of each 16-lane row, in every lane of that row.
template <int M> __device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + M, 0xF, 0xF, true));
}

// Forward-substitution steps M .. 14 for a complex 16 x 16 unit lower-triangular
// inverse held by rows: t_c += (-A[c][M]) t_M for every row c.
template <int M>
__device__ __forceinline__ void inv_rows(f32x4& tr, f32x4& ti, const float (&nar)[16], const float (&nai)[16]) {
  if constexpr (M < 15) {
    f32x4 br, bi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      br[j] = row_bcast<M>(tr[j]);
      bi[j] = row_bcast<M>(ti[j]);
    }
    const float ar = nar[M], ai = nai[M];
    tr += ar * br - ai * bi;
    ti += ar * bi + ai * br;
    inv_rows<M + 1>(tr, ti, nar, nai);
  }
}
constexpr int LDT = 64 + 4;  // LDS row stride of a [32][64] plane
constexpr int szKT = D * LDT;
// LDS of the prep kernel: the K planes, the -A tiles and the gates.  Each
// diagonal inverse overwrites its own diagonal tile of -A, and (diag(lambda)
// K)^T is formed over the -A tiles once every wave has finished its
// substitution, so three workgroups fit in a CU.
constexpr int kPrepFloats = 2 * szK + 2 * szTri + 4 * 64;
static_assert(2 * szKT <= 2 * szTri, "(diag(lambda) K)^T fits over the -A tiles");

// Prefetched operands of one prep chunk for one thread.
struct PrepIn {
  float4 k[4];  // this thread's four 16-byte units of the K tile
  float a, b;   // alpha, beta of token l
};

// Persistent, like the output kernel: chunks blockIdx.x, + gridDim.x, ...,
// with the next chunk's K and gates loaded during the current one.  V is
// loaded at the start of its chunk and first used after the Gram tiles and
// the inverses.  Three workgroups per CU.
__global__ __launch_bounds__(256, 3) void cx_prep_kernel(const float* __restrict__ kg, const float* __restrict__ vg,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta, float* __restrict__ ws,
                                                      int T, int H, int nch, int total) {
  __shared__ __attribute__((aligned(16))) float smem[kPrepFloats];
  float* const sK = smem;                 // planes re, im
  float* const sA = sK + 2 * szK;         // -A, packed lower 16x16 tiles, 2 planes;
                                          // diagonal tiles become (I + A_ii)^{-1}
  float* const sKT = sA;                  // (diag(lambda) K)^T, 2 planes, after the substitution
  float* const s_g2 = sA + 2 * szTri;     // log2 cumulative decay
  float* const s_beta = s_g2 + 64;
  float* const s_gam = s_g2 + 128;
  float* const s_lam = s_g2 + 192;
  const M mK{sK, LDK, szK};
  auto tileA = [&](int i, int j) { return M{sA + tri(i, j) * 16 * LD16, LD16, szTri}; };
  auto tileT = [&](int i) { return tileA(i, i); };  // (I + A_ii)^{-1} once inverted

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, c = l & 15;
  // Loads are unconditional: rows past T are clamped and their values replaced
  // when used (padding token: k = v = 0, alpha = 1, beta = 0, which leaves the
  // state unchanged).
  auto load_in = [&](PrepIn& r, int n) {
    const int chain = n / nch, c0 = 64 * (n % nch), b = chain / H, h = chain % H;
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int unit = tid + 256 * uu, t = min(c0 + (unit >> 4), T - 1), cu = unit & 15;
      r.k[uu] = *reinterpret_cast<const float4*>(kg + tok(b, t, h, T, H) * (2 * D) + 4 * cu);
    }
    const int t = min(c0 + l, T - 1);
    r.a = alpha[tok(b, t, h, T, H)];
    r.b = beta[tok(b, t, h, T, H)];
  };

  PrepIn r;
  load_in(r, blockIdx.x);
  for (int n = blockIdx.x; n < total; n += gridDim.x) {
  // Lane indices re-derived from an opaque copy of the thread index, so that
  // the many per-lane LDS addresses below are formed per chunk instead of being
  // held in registers across the loop.
  int tid_it = tid;
  asm volatile("" : "+v"(tid_it));
  const int l = tid_it & 63, g = l >> 4, c = l & 15;
  const int chain = n / nch, c0 = 64 * (n % nch), b = chain / H, h = chain % H;
  float* const wsn = ws + (size_t)n * kChunkFloats;
  // Value rows for the U column tile 16 (w & 1) + c (waves 2, 3 use them), in
  // accumulator layout.
  float2 vv[4][4];
  {
    const int vcol = 16 * (w & 1) + c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = min(c0 + 16 * i + 4 * g + j, T - 1);
        vv[i][j] = *reinterpret_cast<const float2*>(vg + tok(b, t, h, T, H) * (2 * D) + 2 * vcol);
      }
  }

  // ---------------------------------------------------- this chunk's operands
  // K tile to LDS; value rows for this wave's U column tile, in accumulator layout.
#pragma unroll
  for (int uu = 0; uu < 4; ++uu) {
    const int unit = tid + 256 * uu, row = unit >> 4, cu = unit & 15;
    const float4 f = c0 + row < T ? r.k[uu] : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float2*>(sK + row * LDK + 2 * cu) = make_float2(f.x, f.z);
    *reinterpret_cast<float2*>(sK + szK + row * LDK + 2 * cu) = make_float2(f.y, f.w);
  }
  const bool tin = c0 + l < T;
  const float pa = tin ? r.a : 1.f, pb = tin ? r.b : 0.f;
  // ---------------------------------------------------- next chunk's operands, in flight from here on
  load_in(r, min(n + (int)gridDim.x, total - 1));
  if (w == 0) {
    float x = log2f(pa);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (l >= off) x += y;
    }
    const float glast = __shfl(x, 63, 64);
    s_g2[l] = x;
    s_beta[l] = pb;
    s_gam[l] = exp2f(x);
    s_lam[l] = exp2f(glast - x);
    wsn[oG + l] = x;
  }
  lds_barrier();

  // ---------------------------------------------------- Gram tiles -> -A
  for (int m = 0; m < 3; ++m) {
    const int tt = w + 4 * m;
    if (tt >= 10) break;
    const int ti = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;
    const int tj = tt - tri(ti, 0);
    CS a[2], bk[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      a[d] = csub_rows(mK, 16 * tj + c, 16 * d);
      bk[d] = csub_rows(mK, 16 * ti + c, 16 * d);
    }
    CA acc = acc_zero<true>();
    cmma3<false, true, 2>(acc, a, bk, 2);  // [s][r] = k_s . conj(k_r)
    const int r = 16 * ti + c;
    const float gr = s_g2[r], br = s_beta[r];
    CA va;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 16 * tj + 4 * g + j;
      const float fa = r > s ? br * exp2f(gr - s_g2[s]) : 0.f;
#pragma unroll
      for (int p = 0; p < 2; ++p) va.v[p][j] = -fa * acc.v[p][j];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *reinterpret_cast<f32x4*>(sA + p * szTri + tt * 16 * LD16 + c * LD16 + 4 * g) = va.v[p];
  }
  lds_barrier();

  // ---------------------------------------------------- diagonal inverses
  // Wave w inverts (I + A_ww) by forward substitution over rows: lane (g, c)
  // owns row c, complex columns 4g .. 4g + 3.  Once row m is final it is
  // broadcast along each 16-lane row (DPP row_newbcast) and added, scaled by
  // -A[c][m], to every row (rows c <= m have A[c][m] = 0).  The inverse
  // replaces the tile: only this wave reads it, and all its reads come first.
  {
    const float* At = sA + tri(w, w) * 16 * LD16 + c * LD16;
    float nar[16], nai[16];  // -A[c][m], row c of the tile
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 vr = *reinterpret_cast<const f32x4*>(At + 4 * q);
      const f32x4 vi = *reinterpret_cast<const f32x4*>(At + szTri + 4 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        nar[4 * q + j] = vr[j];
        nai[4 * q + j] = vi[j];
      }
    }
    f32x4 tr, ti{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) tr[j] = c == 4 * g + j ? 1.f : 0.f;
    inv_rows<0>(tr, ti, nar, nai);
    *reinterpret_cast<f32x4*>(sA + tri(w, w) * 16 * LD16 + c * LD16 + 4 * g) = tr;
    *reinterpret_cast<f32x4*>(sA + szTri + tri(w, w) * 16 * LD16 + c * LD16 + 4 * g) = ti;
  }
  lds_barrier();

  // ---------------------------------------------------- block substitution
  // X = (I + A)^{-1} R by 16-row blocks: X_i = T_ii (R_i - sum_{i'<i} A_ii' X_i').
  CA X[4];
  auto substitute = [&](auto getR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      CA y = getR(i);
      if (i > 0) {
        CS a[3], xb[3];
#pragma unroll
        for (int ip = 0; ip < 3; ++ip) {
          if (ip < i) {
            a[ip] = csub_rows(tileA(i, ip), c, 0);
            xb[ip] = csub_from_acc<true, float>(X[ip]);
          } else {
            a[ip] = csub_zero<true, float>();
            xb[ip] = csub_zero<true, float>();
          }
        }
        cmma3<false, false, 3>(y, a, xb, i);
      }
      CS at[1] = {csub_rows(tileT(i), c, 0)};
      CS yb[1] = {csub_from_acc<true, float>(y)};
      X[i] = acc_zero<true>();
      cmma3<false, false, 1>(X[i], at, yb, 1);
    }
  };
  // Rows 16 dd .. 16 dd + 15 of (diag(lambda) K)^T X for this wave's column tile.
  const M mKT{sKT, LDT, szKT};
  auto kl_times_x = [&](int dd) {
    CS a[4], xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = csub_rows(mKT, 16 * dd + c, 16 * i);
      xb[i] = csub_from_acc<true, float>(X[i]);
    }
    CA acc = acc_zero<true>();
    cmma3<false, false, 4>(acc, a, xb, 4);
    return acc;
  };
  if (w < 2) {
    // W column tile w: R = diag(beta gamma) conj(K); the workspace keeps -W.
    const int col = 16 * w + c;
    substitute([&](int i) {
      CA y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * i + 4 * g + j;
        const float sc = s_beta[t] * s_gam[t];
        y.v[0][j] = sc * sK[t * LDK + col];
        y.v[1][j] = -sc * sK[szK + t * LDK + col];
      }
      return y;
    });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int p = 0; p < 2; ++p) wsn[oNW + p * (64 * D) + (16 * i + 4 * g + j) * D + col] = -X[i].v[p][j];
  } else {
    // U column tile w - 2: R = diag(beta) V.
    const int col = 16 * (w - 2) + c;
    substitute([&](int i) {
      CA y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float be = s_beta[16 * i + 4 * g + j];
        // padding rows have beta = 0, which also clears their (clamped) values
        y.v[0][j] = be * vv[i][j].x;
        y.v[1][j] = be * vv[i][j].y;
      }
      return y;
    });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float2*>(wsn + oU + ((16 * i + 4 * g + j) * D + col) * 2) =
            make_float2(X[i].v[0][j], X[i].v[1][j]);
  }
  lds_barrier();  // every wave is done with the -A tiles and the inverses

  // (diag(lambda) K)^T over the -A tiles, for M_n and B_n.  Consecutive lanes
  // take consecutive key columns so the transposing reads are conflict free.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int unit = tid + 256 * u, d = unit & 31, t4 = 4 * ((unit >> 5) & 15), p = unit >> 9;
    const float* src = sK + p * szK + d;
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = s_lam[t4 + j] * src[(t4 + j) * LDK];
    *reinterpret_cast<f32x4*>(sKT + p * szKT + d * LDT + t4) = o;
  }
  lds_barrier();

  if (w < 2) {
    // M_n column tile w: gamma_C I - (diag(lambda) K)^T W.
    const int col = 16 * w + c;
    const float gC = s_gam[63];
#pragma unroll
    for (int dd = 0; dd < 2; ++dd) {
      const CA m = kl_times_x(dd);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 16 * dd + 4 * g + j;
        wsn[oM + d * D + col] = (d == col ? gC : 0.f) - m.v[0][j];
        wsn[oM + D * D + d * D + col] = -m.v[1][j];
      }
    }
  } else {
    // B_n column tile w - 2: (diag(lambda) K)^T U.
    const int col = 16 * (w - 2) + c;
#pragma unroll
    for (int dd = 0; dd < 2; ++dd) {
      const CA bn = kl_times_x(dd);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float2*>(wsn + oB + ((16 * dd + 4 * g + j) * D + col) * 2) =
            make_float2(bn.v[0][j], bn.v[1][j]);
    }
  }
  lds_barrier();  // every wave is done with this chunk's LDS tables
  }
}

// ============================================================== 2. scan
// Real form of 8 complex value columns: lane column c holds part (c & 1) of
// complex column e0 + c / 2.  swz(x) at column c is -x[c + 1] for even c and
// x[c - 1] for odd c: the DPP quad permutation [1, 0, 3, 2] swaps lane pairs.
__device__ __forceinline__ float swz(float x, uint32_t smask) {
  const int y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true);
  return __int_as_float(y ^ smask);
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operands of one scan step for one wave: wave w = dd + 2 kh forms rows
// 16 dd .. 16 dd + 15 of M_n S from the key rows 16 kh .. 16 kh + 15 of S.
struct ScanIn {
  f32x4 m[2];  // [plane]: M_n row 16 dd + c, columns 16 kh + 4g .. + 3
  float b[4];  // B_n rows 16 dd + 4g + j, real column c of the slice
};

__device__ __forceinline__ void scan_load(ScanIn& r, const float* __restrict__ wn, int dd, int kh, int g, int c,
                                          int e0) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
    r.m[p] = *reinterpret_cast<const f32x4*>(wn + oM + p * (D * D) + (16 * dd + c) * D + 16 * kh + 4 * g);
#pragma unroll
  for (int j = 0; j < 4; ++j) r.b[j] = wn[oB + (16 * dd + 4 * g + j) * (2 * D) + 2 * e0 + c];
}

__global__ __launch_bounds__(256) void cx_scan_kernel(const float* S0, float* Sf, float* __restrict__ ws, int nch) {
  __shared__ __attribute__((aligned(16))) f32x4 sPart[2][4][64];  // [parity][wave][lane]
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, c = l & 15;
  const int dd = w & 1, kh = w >> 1;
  const int chain = blockIdx.x >> 2, e0 = 8 * (blockIdx.x & 3);
  const uint32_t smask = (c & 1) ? 0u : 0x80000000u;
  float* const wsc = ws + (size_t)chain * nch * kChunkFloats;
  const size_t sbase = (size_t)chain * (2 * D * D) + 2 * e0 + c;

  // Key rows 16 kh .. 16 kh + 15 of the state slice, real form:
  // Sk[j] = S_real[16 kh + 4g + j][c].
  f32x4 Sk;
#pragma unroll
  for (int j = 0; j < 4; ++j) Sk[j] = S0 ? S0[sbase + (16 * kh + 4 * g + j) * (2 * D)] : 0.f;

  auto step = [&](const ScanIn& r, int n) {
    float* const wn = wsc + (size_t)n * kChunkFloats;
    // Chunk-start state: both waves holding key rows 16 kh .. store them (the
    // same values), so the loop has no conditional memory path.
#pragma unroll
    for (int j = 0; j < 4; ++j) wn[oS + (16 * kh + 4 * g + j) * (2 * D) + 2 * e0 + c] = Sk[j];
    f32x4 part = kh == 0 ? f32x4{r.b[0], r.b[1], r.b[2], r.b[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      part = mfma4(r.m[0][j], Sk[j], part);
      part = mfma4(r.m[1][j], swz(Sk[j], smask), part);
    }
    const int par = n & 1;
    sPart[par][w][l] = part;
    lds_barrier();
    // rows 16 kh .. of the new state: the two waves with dd == kh
    Sk = sPart[par][kh][l] + sPart[par][kh + 2][l];
  };

  // Loads run three chunks ahead of the state (four register sets).  The main
  // loop body is unconditional, with loads clamped to the last chunk, so the
  // compiler keeps the later loads in flight at every wait; the last 0..3
  // chunks run from the sets already loaded.
  if (nch > 0) {
    auto ld = [&](ScanIn& r, int m) { scan_load(r, wsc + (size_t)min(m, nch - 1) * kChunkFloats, dd, kh, g, c, e0); };
    ScanIn r0, r1, r2, r3;
    ld(r0, 0);
    ld(r1, 1);
    ld(r2, 2);
    int n = 0;
    for (; n + 4 <= nch; n += 4) {
      ld(r3, n + 3);
      step(r0, n);
      ld(r0, n + 4);
      step(r1, n + 1);
      ld(r1, n + 5);
      step(r2, n + 2);
      ld(r2, n + 6);
      step(r3, n + 3);
    }
    if (n < nch) step(r0, n);
    if (n + 1 < nch) step(r1, n + 1);
    if (n + 2 < nch) step(r2, n + 2);
  }
  if (dd == 0 && Sf != nullptr) {
#pragma unroll
    for (int j = 0; j < 4; ++j) Sf[sbase + (16 * kh + 4 * g + j) * (2 * D)] = Sk[j];
  }
}

// ============================================================== 3. out
constexpr int kOutFloats = 4 * szK + 2 * szTri + 2 * 64;

// Prefetched operands of one output chunk for one thread.
struct OutIn {
  float4 q[4], k[4];   // this thread's four 16-byte units of the Q and K tiles
  float g;             // log2 decay prefix of token l (wave 0)
};

// Persistent: each workgroup takes chunks blockIdx.x, + gridDim.x, ...  The
// next chunk's Q and K tiles are loaded while the current one is computed,
// into the registers the current one has just been moved out of; the
// workspace operands are loaded at the start of a chunk and first used after
// the P tiles.  Loads are unconditional (rows past T are clamped, then
// zeroed), so the loop has no conditional load path.
__global__ __launch_bounds__(256, 2) void cx_out_kernel(const float* __restrict__ qg, const float* __restrict__ kg,
                                                        const float* __restrict__ ws, float* __restrict__ og, int T,
                                                        int H, int nch, int total) {
  __shared__ __attribute__((aligned(16))) float smem[kOutFloats];
  float* const sQ = smem;             // planes re, im
  float* const sK = sQ + 2 * szK;
  float* const sP = sK + 2 * szK;     // P, packed lower 16x16 tiles, 2 planes
  float* const s_g2 = sP + 2 * szTri;
  float* const s_gam = s_g2 + 64;
  const M mQ{sQ, LDK, szK}, mK{sK, LDK, szK};
  auto tileP = [&](int i, int j) { return M{sP + tri(i, j) * 16 * LD16, LD16, szTri}; };
  // Ut tiles (row block i, column tile u) go to the K planes once P no longer
  // needs them, stored transposed so that a B operand is one 16-byte read per plane.
  float* const sU = sK;
  auto tileU = [&](int i, int uu, int p) { return sU + ((i * 2 + uu) * 2 + p) * 256; };

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, c = l & 15;
  // This wave's output column tile u and row blocks {0, 3} (waves 0, 1) or
  // {1, 2} (waves 2, 3): equal work.
  const int u = w & 1, col = 16 * u + c;
  auto rowblk = [&](int k) { return w < 2 ? 3 * k : 1 + k; };

  auto load_in = [&](OutIn& r, int n) {
    const int chain = n / nch, c0 = 64 * (n % nch), b = chain / H, h = chain % H;
    const float* const wsn = ws + (size_t)n * kChunkFloats;
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int unit = tid + 256 * uu, t = min(c0 + (unit >> 4), T - 1), cu = unit & 15;
      r.q[uu] = *reinterpret_cast<const float4*>(qg + tok(b, t, h, T, H) * (2 * D) + 4 * cu);
      r.k[uu] = *reinterpret_cast<const float4*>(kg + tok(b, t, h, T, H) * (2 * D) + 4 * cu);
    }
    r.g = wsn[oG + l];
  };

  OutIn r;
  load_in(r, blockIdx.x);
  for (int n = blockIdx.x; n < total; n += gridDim.x) {
    const int chain = n / nch, c0 = 64 * (n % nch), b = chain / H, h = chain % H;
    const float* const wsn = ws + (size_t)n * kChunkFloats;
    // ---------------------------------------------------- workspace operands (used after the P tiles):
    // B operand S_n (rows d, columns of tile u); for this wave's two row
    // blocks, U and the A operands of -W.
    CS sb[2], nw[2][2];
    CA ut[2];
#pragma unroll
    for (int dd = 0; dd < 2; ++dd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 x = *reinterpret_cast<const float2*>(wsn + oS + ((16 * dd + 4 * g + j) * D + col) * 2);
        sb[dd].v[0][j] = x.x;
        sb[dd].v[1][j] = x.y;
      }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = rowblk(k);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 x = *reinterpret_cast<const float2*>(wsn + oU + ((16 * i + 4 * g + j) * D + col) * 2);
        ut[k].v[0][j] = x.x;
        ut[k].v[1][j] = x.y;
      }
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          nw[k][dd].v[p] =
              *reinterpret_cast<const f32x4*>(wsn + oNW + p * (64 * D) + (16 * i + c) * D + 16 * dd + 4 * g);
    }
    // ---------------------------------------------------- this chunk's Q, K tiles and decay
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int unit = tid + 256 * uu, row = unit >> 4, cu = unit & 15;
      const bool in = c0 + row < T;
      const float4 fq = in ? r.q[uu] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 fk = in ? r.k[uu] : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float2*>(sQ + row * LDK + 2 * cu) = make_float2(fq.x, fq.z);
      *reinterpret_cast<float2*>(sQ + szK + row * LDK + 2 * cu) = make_float2(fq.y, fq.w);
      *reinterpret_cast<float2*>(sK + row * LDK + 2 * cu) = make_float2(fk.x, fk.z);
      *reinterpret_cast<float2*>(sK + szK + row * LDK + 2 * cu) = make_float2(fk.y, fk.w);
    }
    if (w == 0) {
      s_g2[l] = r.g;
      s_gam[l] = exp2f(r.g);
    }
    // ---------------------------------------------------- next chunk's Q, K tiles, in flight from here on
    load_in(r, min(n + (int)gridDim.x, total - 1));
    lds_barrier();

    // ---------------------------------------------------- P tiles
    for (int m = 0; m < 3; ++m) {
      const int tt = w + 4 * m;
      if (tt >= 10) break;
      const int ti = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;
      const int tj = tt - tri(ti, 0);
      CS a[2], bq[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        a[d] = csub_rows(mK, 16 * tj + c, 16 * d);
        bq[d] = csub_rows(mQ, 16 * ti + c, 16 * d);
      }
      CA acc = acc_zero<true>();
      cmma3<false, true, 2>(acc, a, bq, 2);  // [s][r] = k_s . conj(q_r)
      const int rr = 16 * ti + c;
      const float gr = s_g2[rr];
      CA vp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ss = 16 * tj + 4 * g + j;
        const float gam = rr >= ss ? exp2f(gr - s_g2[ss]) : 0.f;
#pragma unroll
        for (int p = 0; p < 2; ++p) vp.v[p][j] = gam * acc.v[p][j];
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
        *reinterpret_cast<f32x4*>(sP + p * szTri + tt * 16 * LD16 + c * LD16 + 4 * g) = vp.v[p];
    }
    // ---------------------------------------------------- Ut = U + (-W) S_n, this wave's two tiles
#pragma unroll
    for (int k = 0; k < 2; ++k) cmma3<false, false, 2>(ut[k], nw[k], sb, 2);
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int p = 0; p < 2; ++p) *reinterpret_cast<f32x4*>(tileU(rowblk(k), u, p) + c * 16 + 4 * g) = ut[k].v[p];
    lds_barrier();
    CS ub[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < 2; ++p) ub[i].v[p] = *reinterpret_cast<const f32x4*>(tileU(i, u, p) + c * 16 + 4 * g);

    // ---------------------------------------------------- output tiles
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = rowblk(k);
      CA o = acc_zero<true>();
      CS a[2];
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) a[dd] = csub_rows(mQ, 16 * i + c, 16 * dd);
      cmma3<true, false, 2>(o, a, sb, 2);  // conj(Q) S
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gm = s_gam[16 * i + 4 * g + j];
        o.v[0][j] *= gm;
        o.v[1][j] *= gm;
      }
      CS pa[4], ubb[4];
#pragma unroll
      for (int ip = 0; ip < 4; ++ip) {
        if (ip <= i) {
          pa[ip] = csub_rows(tileP(i, ip), c, 0);
          ubb[ip] = ub[ip];
        } else {
          pa[ip] = csub_zero<true, float>();
          ubb[ip] = csub_zero<true, float>();
        }
      }
      cmma3<false, false, 4>(o, pa, ubb, i + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = c0 + 16 * i + 4 * g + j;
        if (t < T)
          *reinterpret_cast<float2*>(og + (tok(b, t, h, T, H) * D + col) * 2) = make_float2(o.v[0][j], o.v[1][j]);
      }
    }
    lds_barrier();  // every wave is done with this chunk's Q, K, P and Ut tiles
  }
}

}  // namespace cx

size_t chunk_cx_workspace_bytes(int B, int T, int H) {
  const size_t nch = ((size_t)T + 63) / 64;
  return (size_t)B * H * nch * cx::kChunkFloats * sizeof(float);
}

// `per_cu` resident workgroups per CU for the persistent chunk kernels.
static unsigned persistent_grid(unsigned nblk, unsigned per_cu) {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 256;
  const unsigned want = per_cu * (unsigned)ncu;
  return nblk < want ? nblk : want;
}

hipError_t launch_chunk_cx(const ChunkArgs& a, void* workspace) {
  const int nch = (a.T + 63) / 64;
  const int nchains = a.B * a.H;
  const hipStream_t st = (hipStream_t)a.stream;
  float* ws = static_cast<float*>(workspace);
  const unsigned nblk = (unsigned)((long)nchains * nch);
  hipError_t e = hipSuccess;
  if (nblk > 0) {
    e = launch_kernel(cx::cx_prep_kernel, dim3(persistent_grid(nblk, 3)), dim3(256), st, static_cast<const float*>(a.k),
                      static_cast<const float*>(a.v), a.alpha, a.beta, ws, a.T, a.H, nch, (int)nblk);
    if (e != hipSuccess) return e;
  }
  e = launch_kernel(cx::cx_scan_kernel, dim3((unsigned)nchains * 4), dim3(256), st,
                    static_cast<const float*>(a.S0), static_cast<float*>(a.S_final), ws, nch);
  if (e != hipSuccess || nblk == 0) return e;
  return launch_kernel(cx::cx_out_kernel, dim3(persistent_grid(nblk, 2)), dim3(256), st, static_cast<const float*>(a.q),
                       static_cast<const float*>(a.k), static_cast<const float*>(ws), static_cast<float*>(a.out),
                       a.T, a.H, nch, (int)nblk);
}

}  // namespace gdn
