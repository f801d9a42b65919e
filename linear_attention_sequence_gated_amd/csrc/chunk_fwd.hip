// chunk_fwd.hip -- fused chunkwise gated delta-rule forward for gfx950.
//
// Method (per head, chunk of C = 64 tokens, S = state at the chunk start):
//   g_r = sum_{s<=r} log alpha_s (log-space cumulative decay), gamma = exp(g),
//   Gamma_rs = exp(g_r - g_s) for r >= s, masked to 0 above the diagonal
//   before the exponential, so no factor above one is ever formed;
//   A = strict_lower(diag(beta) Kr K^T * Gamma),  T = (I + A)^{-1},
//   W = T diag(beta)(Kr * gamma),  U = T diag(beta) V,  Ut = U - W S,
//   O = (Qr * gamma) S + lower(Qr K^T * Gamma) Ut,
//   S <- gamma_C S + (K * exp(g_C - g))^T Ut,
// with Kr = conj(K), Qr = conj(Q) for complex data.  This is the chunkwise
// WY / unit-triangular transform of the gated delta rule (Sykra 0.3.3
// README, "Architectural Highlights": chunkwise parallel training; DeltaPhase
// README, section 1 "Fast Triangular Solve", and section 5 "Exact
// Chunkwise-Parallel Scan" for the log-space decay factorisation).
//
// Design (one workgroup of 4 waves per (batch, head, value slice)):
//   * q/k/v tiles of the next chunk are prefetched into registers with 16-byte
//     global loads while the current chunk is computed, then staged into LDS.
//   * Gram tiles K Kr^T and K Qr^T (lower 16x16 tiles only) run on MFMA; the
//     transposed accumulator rows let each lane store 4 consecutive columns of
//     A and P with one vector write.
//   * (I + A)^{-1} is never formed beyond its four 16x16 diagonal blocks,
//     which are inverted by forward substitution in fp32 registers.  W and U
//     come from block forward substitution whose intermediate blocks stay in
//     MFMA accumulators and feed the next product directly.
//   * The state slice S (dk x 16 per wave) lives in accumulator registers for
//     the whole sequence; U - W S, the output and the state update all consume
//     it without going through LDS.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int DT> struct InT;
template <> struct InT<kDtF32> { typedef float el; static constexpr int comps = 1; };
template <> struct InT<kDtBF16> { typedef __bf16 el; static constexpr int comps = 1; };
template <> struct InT<kDtC64> { typedef float el; static constexpr int comps = 2; };

constexpr int align16(int x) { return (x + 15) & ~15; }

// Lower-triangular 16x16 tile (i >= j) -> packed index.
__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }

template <int DT, int DK, int NV> struct ChunkCfg {
  static constexpr bool CX = DT == kDtC64;
  using Op = std::conditional_t<DT == kDtBF16, __bf16, float>;
  using El = typename InT<DT>::el;
  static constexpr int NPL = CX ? 2 : 1;
  static constexpr int NDT = DK / 16;  // key-dim tiles
  static constexpr int NWS = NV / 16;  // waves that own state columns
  static constexpr int PAD = sizeof(Op) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PAD, LDV = NV + PAD, LDT = 64 + PAD, LD16 = 16 + PAD;
  static constexpr int szK = 64 * LDK, szV = 64 * LDV, szKt = DK * LDT;
  static constexpr int szTri = 10 * 16 * LD16, szTd = 4 * 16 * LD16;
  static constexpr int oK = 0, oQ = oK + NPL * szK, oKt = oQ + NPL * szK, oV = oKt + NPL * szKt;
  static constexpr int oW = oV + NPL * szV, oA = oW + NPL * szK, oP = oA + NPL * szTri, oTd = oP + NPL * szTri;
  static constexpr int nOp = oTd + NPL * szTd;
  static constexpr bool kDiagCopy = !std::is_same_v<Op, float>;  // fp32 copy of diag A blocks
  static constexpr int szAd = 4 * 16 * 17;
  static constexpr int fOff = align16(nOp * (int)sizeof(Op));
  static constexpr int bytes = fOff + (4 * 64 + (kDiagCopy ? NPL * szAd : 0)) * 4;
  static constexpr int ELB = (int)sizeof(El) * InT<DT>::comps;  // bytes per element
  static constexpr int RBK = DK * ELB, RBV = NV * ELB;           // bytes per tile row
  static constexpr int UPRK = RBK / 16, UPRV = RBV / 16;         // 16-byte units per row
  static constexpr int NUK = 64 * UPRK / 256, NUV = 64 * UPRV / 256;
  static constexpr int EPU = 16 / ELB;                           // elements per unit
  static_assert(NUK * 256 == 64 * UPRK && NUV * 256 == 64 * UPRV, "tile rows must split evenly");
  static_assert(NWS <= 4 && NDT >= 1, "bad shape");
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Write one 16-byte global unit (EPU elements) into row `row`, columns
// [col, col + EPU) of an LDS matrix.
template <int DT, class Op, bool CX>
__device__ __forceinline__ void unit_to_rows(const uint4& u, const LdsMat<CX, Op>& m, int row, int col) {
  if constexpr (DT == kDtBF16) {
    *reinterpret_cast<uint4*>(m.at(0, row, col)) = u;
  } else if constexpr (DT == kDtF32) {
    *reinterpret_cast<uint4*>(m.at(0, row, col)) = u;
  } else {
    const float* f = reinterpret_cast<const float*>(&u);
    *reinterpret_cast<float2*>(m.at(0, row, col)) = make_float2(f[0], f[2]);
    *reinterpret_cast<float2*>(m.at(1, row, col)) = make_float2(f[1], f[3]);
  }
}

// Same unit, written transposed: element e goes to row col + e, column `row`.
template <int DT, class Op, bool CX>
__device__ __forceinline__ void unit_to_cols(const uint4& u, const LdsMat<CX, Op>& m, int row, int col) {
  if constexpr (DT == kDtBF16) {
    const __bf16* e = reinterpret_cast<const __bf16*>(&u);
#pragma unroll
    for (int i = 0; i < 8; ++i) *m.at(0, col + i, row) = e[i];
  } else if constexpr (DT == kDtF32) {
    const float* e = reinterpret_cast<const float*>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i) *m.at(0, col + i, row) = e[i];
  } else {
    const float* f = reinterpret_cast<const float*>(&u);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *m.at(0, col + i, row) = f[2 * i];
      *m.at(1, col + i, row) = f[2 * i + 1];
    }
  }
}

template <int DT, int DK, int NV>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(
    const void* __restrict__ qg, const void* __restrict__ kg, const void* __restrict__ vg,
    const float* __restrict__ alpha, const float* __restrict__ beta, const void* S0g, void* __restrict__ outg,
    void* Sfg, int T, int H, int DV, int nslices) {
  using Cf = ChunkCfg<DT, DK, NV>;
  using Op = typename Cf::Op;
  using El = typename Cf::El;
  constexpr bool CX = Cf::CX;
  constexpr int NPL = Cf::NPL, NDT = Cf::NDT, NWS = Cf::NWS, LD16 = Cf::LD16;

  __shared__ __attribute__((aligned(16))) char smem[Cf::bytes];
  Op* sop = reinterpret_cast<Op*>(smem);
  float* sf = reinterpret_cast<float*>(smem + Cf::fOff);
  float* s_g2 = sf;          // log2 cumulative decay within the chunk
  float* s_beta = sf + 64;   // beta_t
  float* s_gam = sf + 128;   // gamma_t = 2^{g2_t}
  float* s_lam = sf + 192;   // 2^{g2_last - g2_t}
  float* s_ad = sf + 256;    // bf16 engine: A diagonal blocks in fp32

  const LdsMat<CX, Op> mK{sop + Cf::oK, Cf::LDK, Cf::szK};
  const LdsMat<CX, Op> mQ{sop + Cf::oQ, Cf::LDK, Cf::szK};
  const LdsMat<CX, Op> mKt{sop + Cf::oKt, Cf::LDT, Cf::szKt};
  const LdsMat<CX, Op> mV{sop + Cf::oV, Cf::LDV, Cf::szV};
  const LdsMat<CX, Op> mW{sop + Cf::oW, Cf::LDK, Cf::szK};  // holds -W
  Op* const sA = sop + Cf::oA;    // -A, packed lower 16x16 tiles
  Op* const sP = sop + Cf::oP;    // P, packed lower 16x16 tiles
  Op* const sTd = sop + Cf::oTd;  // (I + A_ii)^{-1}, 4 tiles

  auto tileA = [&](int i, int j) { return LdsMat<CX, Op>{sA + tri(i, j) * 16 * LD16, LD16, Cf::szTri}; };
  auto tileP = [&](int i, int j) { return LdsMat<CX, Op>{sP + tri(i, j) * 16 * LD16, LD16, Cf::szTri}; };
  auto tileT = [&](int i) { return LdsMat<CX, Op>{sTd + i * 16 * LD16, LD16, Cf::szTd}; };

  // Block -> (chain, slice).  Workgroups are dispatched round-robin over the 8
  // XCDs; remap so that consecutive logical ids (the slices of one chain, the
  // heads of one batch row) share an XCD and its L2.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int slice = bid % nslices;
  const int chain = bid / nslices;
  const int b = chain / H, h = chain % H;
  const int dv0 = slice * NV;

  // w is made explicitly uniform so that branches on it are scalar branches:
  // matrix-core instructions do not honour the exec mask.
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, c = l & 15;

  // ------------------------------------------------------------ prefetch
  uint4 pk[Cf::NUK], pq[Cf::NUK], pv[Cf::NUV];
  float pa = 1.f, pb = 0.f;
  auto prefetch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < Cf::NUK; ++u) {
      const int unit = tid + 256 * u, row = unit / Cf::UPRK, cu = unit % Cf::UPRK, t = c0 + row;
      if (t < T) {
        const size_t tok = ((size_t)b * T + t) * H + h;
        pk[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(kg) + tok * Cf::RBK + cu * 16);
        pq[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(qg) + tok * Cf::RBK + cu * 16);
      } else {
        pk[u] = make_uint4(0, 0, 0, 0);
        pq[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < Cf::NUV; ++u) {
      const int unit = tid + 256 * u, row = unit / Cf::UPRV, cu = unit % Cf::UPRV, t = c0 + row;
      if (t < T) {
        const size_t tok = ((size_t)b * T + t) * H + h;
        pv[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(vg) + (tok * DV + dv0) * Cf::ELB + cu * 16);
      } else {
        pv[u] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 64) {
      const int t = c0 + tid;
      if (t < T) {
        const size_t tok = ((size_t)b * T + t) * H + h;
        pa = alpha[tok];
        pb = beta[tok];
      } else {  // padding token: alpha = 1, beta = 0 leaves the state unchanged
        pa = 1.f;
        pb = 0.f;
      }
    }
  };

  // ------------------------------------------------------------ state
  Acc<CX> S[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) S[d] = acc_zero<CX>();
  if (w < NWS && S0g != nullptr) {
    const float* s0 = static_cast<const float*>(S0g);
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t idx = ((size_t)chain * DK + 16 * d + 4 * g + j) * DV + dv0 + 16 * w + c;
        if constexpr (CX) {
          S[d].v[0][j] = s0[2 * idx];
          S[d].v[1][j] = s0[2 * idx + 1];
        } else {
          S[d].v[0][j] = s0[idx];
        }
      }
  }

  const int nchunks = (T + 63) / 64;
  if (nchunks > 0) prefetch(0);

  for (int n = 0; n < nchunks; ++n) {
    const int c0 = n * 64;
    // ---------------------------------------------------- stage + gate scan
#pragma unroll
    for (int u = 0; u < Cf::NUK; ++u) {
      const int unit = tid + 256 * u, row = unit / Cf::UPRK, col = (unit % Cf::UPRK) * Cf::EPU;
      unit_to_rows<DT>(pk[u], mK, row, col);
      unit_to_rows<DT>(pq[u], mQ, row, col);
      unit_to_cols<DT>(pk[u], mKt, row, col);
    }
#pragma unroll
    for (int u = 0; u < Cf::NUV; ++u) {
      const int unit = tid + 256 * u, row = unit / Cf::UPRV, col = (unit % Cf::UPRV) * Cf::EPU;
      unit_to_rows<DT>(pv[u], mV, row, col);
    }
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
    }
    if (n + 1 < nchunks) prefetch(c0 + 64);
    lds_barrier();

    // ---------------------------------------------------- Gram tiles -> A, P
    for (int m = 0; m < 3; ++m) {
      const int tt = w + 4 * m;
      if (tt >= 10) break;
      const int ti = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;
      const int tj = tt - tri(ti, 0);
      CSub<CX, Op> a[NDT], bk[NDT], bq[NDT];
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        a[d] = csub_rows(mK, 16 * tj + c, 16 * d);
        bk[d] = csub_rows(mK, 16 * ti + c, 16 * d);
        bq[d] = csub_rows(mQ, 16 * ti + c, 16 * d);
      }
      Acc<CX> accG = acc_zero<CX>(), accP = acc_zero<CX>();
      cmma<CX, Op, false, true, NDT>(accG, a, bk, NDT);  // [s][r] = k_s . conj(k_r)
      cmma<CX, Op, false, true, NDT>(accP, a, bq, NDT);  // [s][r] = k_s . conj(q_r)
      const int r = 16 * ti + c;
      const float gr = s_g2[r], br = s_beta[r];
      Acc<CX> va, vp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 16 * tj + 4 * g + j;
        const float gam = exp2f(r >= s ? gr - s_g2[s] : -INFINITY);
        const float fa = r > s ? br * gam : 0.f;
#pragma unroll
        for (int p = 0; p < NPL; ++p) {
          va.v[p][j] = -fa * accG.v[p][j];
          vp.v[p][j] = gam * accP.v[p][j];
        }
      }
#pragma unroll
      for (int p = 0; p < NPL; ++p) {
        *reinterpret_cast<Sub<Op>*>(sA + p * Cf::szTri + tt * 16 * LD16 + c * LD16 + 4 * g) = sub_from_acc<Op>(va.v[p]);
        *reinterpret_cast<Sub<Op>*>(sP + p * Cf::szTri + tt * 16 * LD16 + c * LD16 + 4 * g) = sub_from_acc<Op>(vp.v[p]);
        if constexpr (Cf::kDiagCopy) {
          if (ti == tj) {
#pragma unroll
            for (int j = 0; j < 4; ++j) s_ad[p * Cf::szAd + ti * 16 * 17 + c * 17 + 4 * g + j] = -va.v[p][j];
          }
        }
      }
    }
    lds_barrier();

    // ---------------------------------------------------- diagonal inverses
    // Wave w inverts (I + A_ww): lane c < 16 owns column c and runs forward
    // substitution, subtracting A[r][s] * t[s] from every later row r once t[s]
    // is final.
    if (l < 16) {
      auto Aget = [&](int p, int r, int s) -> float {
        if constexpr (Cf::kDiagCopy) return s_ad[p * Cf::szAd + w * 16 * 17 + r * 17 + s];
        else return -static_cast<float>(sA[p * Cf::szTri + tri(w, w) * 16 * LD16 + r * LD16 + s]);
      };
      if constexpr (!CX) {
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = r == c ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < 15; ++s)
#pragma unroll
          for (int r = s + 1; r < 16; ++r) t[r] -= Aget(0, r, s) * t[s];
#pragma unroll
        for (int r = 0; r < 16; ++r) sTd[w * 16 * LD16 + r * LD16 + c] = static_cast<Op>(t[r]);
      } else {
        float tr[16], tim[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          tr[r] = r == c ? 1.f : 0.f;
          tim[r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < 15; ++s)
#pragma unroll
          for (int r = s + 1; r < 16; ++r) {
            const float ar = Aget(0, r, s), ai = Aget(1, r, s);
            tr[r] -= ar * tr[s] - ai * tim[s];
            tim[r] -= ar * tim[s] + ai * tr[s];
          }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sTd[w * 16 * LD16 + r * LD16 + c] = tr[r];
          sTd[Cf::szTd + w * 16 * LD16 + r * LD16 + c] = tim[r];
        }
      }
    }
    lds_barrier();

    // ---------------------------------------------------- block substitution
    // X = (I + A)^{-1} R one 16-row block at a time:
    //   X_i = T_ii (R_i - sum_{i' < i} A_{i i'} X_{i'}).
    auto substitute = [&](auto getR, Acc<CX>(&X)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Acc<CX> y = getR(i);
        if (i > 0) {
          CSub<CX, Op> a[3], xb[3];
#pragma unroll
          for (int ip = 0; ip < 3; ++ip) {
            if (ip < i) {
              a[ip] = csub_rows(tileA(i, ip), c, 0);
              xb[ip] = csub_from_acc<CX, Op>(X[ip]);
            } else {
              a[ip] = csub_zero<CX, Op>();
              xb[ip] = csub_zero<CX, Op>();
            }
          }
          cmma<CX, Op, false, false, 3>(y, a, xb, i);
        }
        CSub<CX, Op> at[1] = {csub_rows(tileT(i), c, 0)};
        CSub<CX, Op> yb[1] = {csub_from_acc<CX, Op>(y)};
        X[i] = acc_zero<CX>();
        cmma<CX, Op, false, false, 1>(X[i], at, yb, 1);
      }
    };

    Acc<CX> U[4];
    for (int cw = w; cw < NDT; cw += 4) {
      Acc<CX> X[4];
      substitute(
          [&](int i) {  // R = diag(beta * gamma) conj(K), column tile cw
            Acc<CX> y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int t = 16 * i + 4 * g + j;
              const float sc = s_beta[t] * s_gam[t];
              y.v[0][j] = sc * static_cast<float>(*mK.at(0, t, 16 * cw + c));
              if constexpr (CX) y.v[1][j] = -sc * static_cast<float>(*mK.at(1, t, 16 * cw + c));
            }
            return y;
          },
          X);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int p = 0; p < NPL; ++p) *mW.at(p, 16 * i + 4 * g + j, 16 * cw + c) = static_cast<Op>(-X[i].v[p][j]);
    }
    if (w < NWS) {
      substitute(
          [&](int i) {  // R = diag(beta) V, this wave's 16 value columns
            Acc<CX> y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int t = 16 * i + 4 * g + j;
#pragma unroll
              for (int p = 0; p < NPL; ++p) y.v[p][j] = s_beta[t] * static_cast<float>(*mV.at(p, t, 16 * w + c));
            }
            return y;
          },
          U);
    }
    lds_barrier();

    // ---------------------------------------------------- state pass
    if (w < NWS) {
      CSub<CX, Op> sb[NDT];
#pragma unroll
      for (int d = 0; d < NDT; ++d) sb[d] = csub_from_acc<CX, Op>(S[d]);
      // Ut = U - W S
      Acc<CX> Ut[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Ut[i] = U[i];
        CSub<CX, Op> a[NDT];
#pragma unroll
        for (int d = 0; d < NDT; ++d) a[d] = csub_rows(mW, 16 * i + c, 16 * d);
        cmma<CX, Op, false, false, NDT>(Ut[i], a, sb, NDT);
      }
      // O = diag(gamma) Qr S + P Ut
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Acc<CX> o = acc_zero<CX>();
        CSub<CX, Op> a[NDT];
#pragma unroll
        for (int d = 0; d < NDT; ++d) a[d] = csub_rows(mQ, 16 * i + c, 16 * d);
        cmma<CX, Op, true, false, NDT>(o, a, sb, NDT);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gm = s_gam[16 * i + 4 * g + j];
#pragma unroll
          for (int p = 0; p < NPL; ++p) o.v[p][j] *= gm;
        }
        CSub<CX, Op> pa_[4], ub[4];
#pragma unroll
        for (int ip = 0; ip < 4; ++ip) {
          if (ip <= i) {
            pa_[ip] = csub_rows(tileP(i, ip), c, 0);
            ub[ip] = csub_from_acc<CX, Op>(Ut[ip]);
          } else {
            pa_[ip] = csub_zero<CX, Op>();
            ub[ip] = csub_zero<CX, Op>();
          }
        }
        cmma<CX, Op, false, false, 4>(o, pa_, ub, i + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = c0 + 16 * i + 4 * g + j;
          if (t < T) {
            const size_t idx = (((size_t)b * T + t) * H + h) * DV + dv0 + 16 * w + c;
            if constexpr (CX) {
              float* out = static_cast<float*>(outg);
              *reinterpret_cast<float2*>(out + 2 * idx) = make_float2(o.v[0][j], o.v[1][j]);
            } else {
              static_cast<El*>(outg)[idx] = static_cast<El>(o.v[0][j]);
            }
          }
        }
      }
      // S <- gamma_C S + K^T diag(lambda) Ut
      const float gC = s_gam[63];
      CSub<CX, Op> ul[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Acc<CX> tmp = Ut[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lm = s_lam[16 * i + 4 * g + j];
#pragma unroll
          for (int p = 0; p < NPL; ++p) tmp.v[p][j] *= lm;
        }
        ul[i] = csub_from_acc<CX, Op>(tmp);
      }
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
#pragma unroll
        for (int p = 0; p < NPL; ++p) S[d].v[p] *= gC;
        CSub<CX, Op> a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = csub_rows(mKt, 16 * d + c, 16 * i);
        cmma<CX, Op, false, false, 4>(S[d], a, ul, 4);
      }
    }
    lds_barrier();
  }

  if (w < NWS && Sfg != nullptr) {
    float* sfo = static_cast<float*>(Sfg);
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t idx = ((size_t)chain * DK + 16 * d + 4 * g + j) * DV + dv0 + 16 * w + c;
        if constexpr (CX) {
          *reinterpret_cast<float2*>(sfo + 2 * idx) = make_float2(S[d].v[0][j], S[d].v[1][j]);
        } else {
          sfo[idx] = S[d].v[0][j];
        }
      }
  }
}

template <int DT, int DK, int NV>
static hipError_t launch_fused(const ChunkArgs& a) {
  const int nslices = a.dv / NV;
  const long nblk = (long)a.B * a.H * nslices;
  return launch_kernel(chunk_fwd_kernel<DT, DK, NV>, dim3((unsigned)nblk), dim3(256), (hipStream_t)a.stream, a.q, a.k,
                       a.v, a.alpha, a.beta, a.S0, a.out, a.S_final, a.T, a.H, a.dv, nslices);
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  if (a.dtype == kDtBF16 && a.dk == 64) return launch_fused<kDtBF16, 64, 64>(a);
  if (a.dtype == kDtBF16 && a.dk == 128) return launch_fused<kDtBF16, 128, 64>(a);
  if (a.dtype == kDtF32 && a.dk == 64) return launch_fused<kDtF32, 64, 64>(a);
  return hipErrorInvalidValue;
}

}  // namespace gdn
