// chunk_grad.hip -- gradients of the bf16 chunk forward (d_k = d_v = 64) on
// the matrix cores, in the chunk form.
//
// The forward, per chunk of C = 64 tokens with state S at its start (Sykra
// README, "Architectural Highlights": chunkwise parallel training, data-
// dependent forget gating; DeltaPhase README, section 1 "Fast Triangular
// Solve" and section 5, the log-space factorisation of the decay): with the
// gate prefix gamma_t = prod_{i<=t} alpha_i, lambda_t = gamma_C / gamma_t,
//   X = V - diag(gamma) K S,          U = Tb X,  Tb = (I + diag(beta) Gt)^{-1} diag(beta),
//   O = diag(gamma) Q S + P U,        P = (Q K^T) o M (M_tu = gamma_t / gamma_u, u <= t),
//   S' = gamma_C S + K^T diag(lambda) U,
// where Gt = (K K^T) o M below the diagonal.  Reverse mode, with dO and dS'
// (the gradient reaching the chunk's end state) given:
//   dU = P^T dO + diag(lambda) K dS',  dX = Tb^T dU  (= dV),
//   dS = gamma_C dS' + Q^T diag(gamma) dO - K^T diag(gamma) dX   (to the chunk's start),
//   dY = dU - Gt^T dX,  R = X - Gt U,  dbeta_t = dY_t . R_t,
//   dP = (dO U^T) o [u <= t],  dGt = -(dX U^T) o [u < t],
//   D1 = dP o M,  D2 = dGt o M,
//   dQ = D1 K + diag(gamma) dO S^T,
//   dK = D1^T Q + (D2 + D2^T) K + diag(lambda) U dS'^T - diag(gamma) dX S^T,
// and the gradient of the log-gate prefix g_t = ln gamma_t,
//   dg_t = gamma_t (QS)_t . dO_t - gamma_t (KS)_t . dX_t - Z_t . U_t
//          + rowsum_t(dP o P + dGt o Gt) - colsum_t(dP o P + dGt o Gt)
//          + [t = C - 1] (gamma_C <dS', S> + sum_u Z_u . U_u),   Z = diag(lambda) K dS',
// so that d ln alpha_i = sum_{t >= i} dg_t within the chunk.  (dY and R are
// formed without dividing by beta: dY = (I + A)^{-T} dU from (I + A)^T dY = dU,
// and R_t = U_t / beta_t read from (I + A) U = diag(beta) X.)
//
// Three passes after the forward's factor pass (which also writes Tb^T):
//   1. the forward state pass, storing every chunk's start state S_n (bf16);
//   2. this file's adjoint scan: dS carried from the last chunk to the first,
//      storing every chunk's end gradient dS'_n (bf16) and returning dS0 --
//      the same recurrence as the forward state pass, transposed;
//   3. this file's gradient pass: one workgroup per (chain, chunk), all
//      chunks at once, everything above from S_n and dS'_n.
// Products take bf16 operands with fp32 accumulation, as the forward does.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "gdn_lane.hpp"
#include "gdn_pipe.hpp"

namespace gdn {
namespace grad {
using namespace pipe;

__device__ __forceinline__ float bf_at(const u32x2& v, int j) { return j & 1 ? hi_f(v[j >> 1]) : lo_f(v[j >> 1]); }

// Sum over the lane's row of 16 (every lane of the row receives it).
__device__ __forceinline__ float row16_sum(float x) {
  return lane::dpp_add<lane::kRowRor8>(lane::dpp_add<lane::kRowRor4>(lane::quad_sum(x)));
}

// Sum over the four rows of 16 at the lane's column position.
__device__ __forceinline__ float col4_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

__device__ __forceinline__ int clampc(int m, int n) { return __builtin_amdgcn_readfirstlane(max(0, min(m, n - 1))); }

// Steps k = -2 .. n (at least) with a barrier after each, in whole triples;
// step(phase, k) has phase = (k + 2) % 3 at compile time.
template <class Step>
__device__ __forceinline__ void run_steps(int n, Step&& step) {
  __builtin_assume(n >= 0);
  for (int k = -2; k <= n; k += 3) {
    step(ic<0>{}, k);
    stage_barrier();
    step(ic<1>{}, k + 1);
    stage_barrier();
    step(ic<2>{}, k + 2);
    stage_barrier();
  }
}

// ------------------------------------------------------------ adjoint scan
// One workgroup per (chain, NV value columns).  Waves: NC consumers (16 columns
// each, dS in matrix-core accumulators in the key order of the forward state
// pass), the E wave (P^T dO of the next chunk, handed over through LDS) and the
// loaders.  Chunks run last to first; in step k the loaders publish chunk
// k + 2, the E wave works on chunk k + 1 and the consumers on chunk k (local
// indices; chunk n = nch - 1 - k).
template <int DK, int NC>
struct AdjCfg {
  static constexpr int NV = 16 * NC, NDT = DK / 16, NKP = DK / 32, LDV = NV + 8;
  static constexpr int wE = NC, wL = NC + 1;
  static constexpr int NLOAD = DK == 64 ? 2 : 3;  // (K and Q rows | dO, Tb^T, g) or (K | Q | dO, Tb^T, g)
  static constexpr int kThreads = (NC + 1 + NLOAD) * 64;
  // stage slot (bytes): K rows, Q rows, dO tile, Tb^T blocks, gate table
  static constexpr int oK = 0, oQ = 64 * DK * 2, oV = 2 * 64 * DK * 2, oTb = oV + 64 * LDV * 2, oGt = oTb + 6 * 1024;
  static constexpr int gGam = 0, gLam = 64, gG = 128, gGC = 192, szG = 196;  // floats
  static constexpr int szSlot = oGt + szG * 4;
  static constexpr int oE = 3 * szSlot, szE = NC * 4 * 64 * 16;  // E hand-off, two slots
  static constexpr int bytes = oE + 2 * szE;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(szSlot % 16 == 0 && oTb % 16 == 0 && oGt % 16 == 0, "16-byte alignment");
};

struct AdjArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* dO;
  const char* recT;   // Tb^T records [chains][nch]
  const float* dSf;   // [chains][DK][DV] or NULL
  __bf16* dSck;       // [chains][nch][DK][DV]: the gradient at each chunk's end
  float* dS0;         // [chains][DK][DV] or NULL
  int T, H, DV, nch;
};

template <int DK, int NC, int ROLE>
__device__ __forceinline__ void adj_load_role(const AdjArgs& a, int chain, int dv0, char* smem, int l) {
  using Cf = AdjCfg<DK, NC>;
  const int T = a.T, H = a.H, DV = a.DV, nch = a.nch;
  const int b = chain / H, h = chain % H;
  const size_t tokbase = (size_t)b * T * H + h;
  auto first_tok = [&](int m) { return (nch - 1 - clampc(m, nch)) * 64; };
  constexpr bool kRows = ROLE < Cf::NLOAD - 1;
  constexpr int NROW = DK == 64 ? 2 : 1;
  constexpr int NU = DK / 8, NPL = NU;
  constexpr int NVU = Cf::NV / 8, NVL = NVU;
  if constexpr (kRows) {
    const uint32_t span = span_bytes((size_t)T * H * DK * 2, (size_t)h * DK * 2);
    const __bf16* src[NROW];
    int ldst[NROW];
    if constexpr (DK == 64) {
      src[0] = a.k;
      src[1] = a.q;
      ldst[0] = Cf::oK / 2;
      ldst[1] = Cf::oQ / 2;
    } else {
      src[0] = ROLE == 0 ? a.k : a.q;
      ldst[0] = ROLE == 0 ? Cf::oK / 2 : Cf::oQ / 2;
    }
    __amdgpu_buffer_rsrc_t rs[NROW];
#pragma unroll
    for (int m = 0; m < NROW; ++m) rs[m] = make_rsrc(src[m] + tokbase * DK, span);
    const int rowK = H * DK * 2;
    int vof[NPL], lof[NPL];
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int unit = l + 64 * u, row = unit / NU, pc = unit % NU;
      vof[u] = row * rowK + 16 * pc;
      lof[u] = row_off<DK>(row, 8 * pc);
    }
    u32x4 st[3][NROW][NPL];
    auto load = [&](auto sc, int m) {
      constexpr int s = decltype(sc)::value;
#pragma unroll
      for (int r = 0; r < NROW; ++r)
#pragma unroll
        for (int u = 0; u < NPL; ++u)
          st[s][r][u] =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[r], vof[u], first_tok(m) * rowK, 0));
    };
    load(ic<0>{}, 0);
    issue_fence();
    load(ic<1>{}, 1);
    issue_fence();
    load(ic<2>{}, 2);
    issue_fence();
    run_steps(nch, [&](auto pc, int k) {
      constexpr int ph = decltype(pc)::value;
      if (k + 2 < nch) {
        __bf16* const R = reinterpret_cast<__bf16*>(smem + ph * Cf::szSlot);
#pragma unroll
        for (int r = 0; r < NROW; ++r)
#pragma unroll
          for (int u = 0; u < NPL; ++u) *reinterpret_cast<u32x4*>(R + ldst[r] + lof[u]) = st[ph][r][u];
      }
      issue_fence();
      load(ic<ph>{}, k + 5);
    });
  } else {
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(a.dO + tokbase * DV + dv0, span_bytes((size_t)T * H * DV * 2, ((size_t)h * DV + dv0) * 2));
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.recT + (size_t)chain * nch * kRecBytes, (uint32_t)nch * kRecBytes);
    const int rowV = H * DV * 2;
    int vof[NVL], lof[NVL];
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int unit = l + 64 * u, row = unit / NVU, cu = unit % NVU;
      vof[u] = row * rowV + 16 * cu;
      lof[u] = row * Cf::LDV + 8 * cu;
    }
    struct Set {
      u32x4 v[NVL], tb[6];
      float gv;
    };
    Set st[3];
    auto load = [&](auto sc, int m) {
      constexpr int s = decltype(sc)::value;
      const int n = nch - 1 - clampc(m, nch);
#pragma unroll
      for (int u = 0; u < NVL; ++u)
        st[s].v[u] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vof[u], n * 64 * rowV, 0));
#pragma unroll
      for (int e = 0; e < 6; ++e)
        st[s].tb[e] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, kRecTb + e * 1024 + l * 16, n * kRecBytes, 0));
      st[s].gv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, kRecG + 4 * l, n * kRecBytes, 0));
    };
    load(ic<0>{}, 0);
    issue_fence();
    load(ic<1>{}, 1);
    issue_fence();
    load(ic<2>{}, 2);
    issue_fence();
    run_steps(nch, [&](auto pc, int k) {
      constexpr int ph = decltype(pc)::value;
      if (k + 2 < nch) {
        char* const R = smem + ph * Cf::szSlot;
        __bf16* const Rb = reinterpret_cast<__bf16*>(R);
        float* const Gt = reinterpret_cast<float*>(R + Cf::oGt);
#pragma unroll
        for (int u = 0; u < NVL; ++u) *reinterpret_cast<u32x4*>(Rb + Cf::oV / 2 + lof[u]) = st[ph].v[u];
#pragma unroll
        for (int e = 0; e < 6; ++e) *reinterpret_cast<u32x4*>(R + Cf::oTb + e * 1024 + l * 16) = st[ph].tb[e];
        const float gl = st[ph].gv;
        const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), 63));
        Gt[Cf::gGam + l] = __builtin_amdgcn_exp2f(gl);
        Gt[Cf::gLam + l] = __builtin_amdgcn_exp2f(gC - gl);
        Gt[Cf::gG + l] = gl;
        if (l == 63) Gt[Cf::gGC] = __builtin_amdgcn_exp2f(gC);
      }
      issue_fence();
      load(ic<ph>{}, k + 5);
    });
  }
}

// P^T as A operands of block row i: pairs (2p, 2p + 1) of k blocks, from the
// accumulators of P blocks (j, i) = Q_j K_i^T, which hold P[16j + 4g + r][16i + c]
// -- the A order of P^T.  Decay M_tu = 2^(g_t - g_u) for u <= t, zero above.
template <int NKP>
__device__ __forceinline__ void p_transposed(const u32x4 (&qq)[4][NKP], const u32x4 (&kk)[4][NKP], const float* gtab,
                                             int g, int c, u32x4 (&PT)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float gu = gtab[16 * i + c];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x2 hv[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int j = 2 * p + hh;
        if (j < i) {
          hv[hh] = z4();
          continue;
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp) acc = mma32(qq[j][kp], kk[i][kp], acc);
        const f32x4 gt = *reinterpret_cast<const f32x4*>(gtab + 16 * j + 4 * g);
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = 4 * g + r + 16 * j >= 16 * i + c ? acc[r] * __builtin_amdgcn_exp2f(gt[r] - gu) : 0.f;
        hv[hh] = cvt4(v);
      }
      PT[i][p] = pair(hv[0], hv[1]);
    }
  }
}

template <int DK, int NC>
__device__ __forceinline__ void adj_e_role(const AdjArgs& a, char* smem, int l) {
  using Cf = AdjCfg<DK, NC>;
  constexpr int NKP = Cf::NKP;
  const int g = l >> 4, c = l & 15;
  run_steps(a.nch, [&](auto pc, int k) {
    constexpr int slot = (decltype(pc)::value + 2) % 3;  // chunk k + 1
    const int m = k + 1;
    if (m < 0 || m >= a.nch) return;
    const char* const R = smem + slot * Cf::szSlot;
    const __bf16* const Rb = reinterpret_cast<const __bf16*>(R);
    const float* const Gt = reinterpret_cast<const float*>(R + Cf::oGt);
    u32x4 kk[4][NKP], qq[4][NKP];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        kk[i][p] = *reinterpret_cast<const u32x4*>(Rb + Cf::oK / 2 + row_off<DK>(16 * i + c, 32 * p + 8 * g));
        qq[i][p] = *reinterpret_cast<const u32x4*>(Rb + Cf::oQ / 2 + row_off<DK>(16 * i + c, 32 * p + 8 * g));
      }
    u32x2 dd[NC][4];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dd[cb][j] = ld4_tr(Rb + Cf::oV / 2 + (16 * j + 4 * g + (c >> 2)) * Cf::LDV + 16 * cb + 4 * (c & 3));
    u32x4 PT[4][2];
    p_transposed<NKP>(qq, kk, Gt + Cf::gG, g, c, PT);
    float* const E = reinterpret_cast<float*>(smem + Cf::oE + (m & 1) * Cf::szE);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const u32x4 d01 = pair(dd[cb][0], dd[cb][1]), d23 = pair(dd[cb][2], dd[cb][3]);
      f32x4 e[4];
      e[0] = mma32(PT[0][1], d23, mma32(PT[0][0], d01, zero4()));
      e[1] = mma32(PT[1][1], d23, mma32(PT[1][0], d01, zero4()));
      e[2] = mma32(PT[2][1], d23, zero4());
      e[3] = mma32(PT[3][1], d23, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(E + ((cb * 4 + i) * 64 + l) * 4) = e[i];
    }
  });
}

template <int DK, int NC>
__device__ __forceinline__ void adj_consumer(const AdjArgs& a, int chain, int dv0, char* smem, int w, int l) {
  using Cf = AdjCfg<DK, NC>;
  constexpr int NDT = Cf::NDT, NKP = Cf::NKP;
  const int g = l >> 4, c = l & 15, col = dv0 + 16 * w + c;
  f32x4 S[NDT];
  u32x2 sfr[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) S[d][j] = a.dSf ? a.dSf[((size_t)chain * DK + key_row(d, g, j)) * a.DV + col] : 0.f;
    sfr[d] = cvt4(S[d]);
  }
  run_steps(a.nch, [&](auto pc, int k) {
    constexpr int slot = (decltype(pc)::value + 1) % 3;  // chunk k
    if (k < 0 || k >= a.nch) return;
    const int n = a.nch - 1 - k;
    // The gradient at the end of chunk n, for the gradient pass (32-bit
    // offsets through a buffer resource, formed here).
    {
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(a.dSck + ((size_t)chain * a.nch + n) * DK * a.DV + dv0 + 16 * w, (uint32_t)(DK * a.DV * 2));
#pragma unroll
      for (int d = 0; d < NDT; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned u = sfr[d][j >> 1];
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)((j & 1) ? u >> 16 : u), rs,
                                                (key_row(d, g, j) * a.DV + c) * 2, 0, 0);
        }
    }
    const char* const R = smem + slot * Cf::szSlot;
    const __bf16* const Rb = reinterpret_cast<const __bf16*>(R);
    const float* const Gt = reinterpret_cast<const float*>(R + Cf::oGt);
    const float* const E = reinterpret_cast<const float*>(smem + Cf::oE + (k & 1) * Cf::szE);
    // At d = 128 the K rows are read per 16-row block and half of the update's
    // K^T operands after the Tb^T product (register budget, as in the forward).
    constexpr int KRB = DK == 128 ? 1 : 4, KTB = DK == 128 ? 4 : NDT;
    auto krow = [&](int i, u32x4 (&dst)[NKP]) {
#pragma unroll
      for (int p = 0; p < NKP; ++p)
        dst[p] = *reinterpret_cast<const u32x4*>(Rb + Cf::oK / 2 + row_off<DK>(16 * i + c, 32 * p + 8 * g));
    };
    u32x4 kr[KRB][NKP];
    u32x2 dd[4];
    f32x4 gm[4], lm[4], ee[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < KRB) krow(i, kr[i < KRB ? i : 0]);
      dd[i] = ld4_tr(Rb + Cf::oV / 2 + (16 * i + 4 * g + (c >> 2)) * Cf::LDV + 16 * w + 4 * (c & 3));
      gm[i] = *reinterpret_cast<const f32x4*>(Gt + Cf::gGam + 16 * i + 4 * g);
      lm[i] = *reinterpret_cast<const f32x4*>(Gt + Cf::gLam + 16 * i + 4 * g);
      ee[i] = *reinterpret_cast<const f32x4*>(E + ((w * 4 + i) * 64 + l) * 4);
    }
    u32x4 tt[6];
#pragma unroll
    for (int e = 0; e < 6; ++e) tt[e] = *reinterpret_cast<const u32x4*>(R + Cf::oTb + e * 1024 + l * 16);
    issue_fence();
    // dU = E + lambda * (K dS')
    u32x2 du[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 ki[NKP];
      if (i < KRB) {
#pragma unroll
        for (int p = 0; p < NKP; ++p) ki[p] = kr[i < KRB ? i : 0][p];
      } else {
        krow(i, ki);
      }
      f32x4 z = zero4();
#pragma unroll
      for (int p = 0; p < NKP; ++p) z = mma32(ki[p], pair(sfr[2 * p], sfr[2 * p + 1]), z);
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = ee[i][j] + lm[i][j] * z[j];
      du[i] = cvt4(x);
    }
    // The update's Q side needs only dO: dS <- gamma_C dS + Q^T (gamma dO) runs
    // while the Tb^T product is formed (Q^T read in the key order of the
    // accumulators, one key block at a time).
    const float gC = Gt[Cf::gGC];
    {
      u32x2 W1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 x1;
#pragma unroll
        for (int j = 0; j < 4; ++j) x1[j] = gm[i][j] * bf_at(dd[i], j);
        W1[i] = cvt4(x1);
      }
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        u32x2 qt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          qt[i] = ld4_tr(Rb + Cf::oQ / 2 +
                         row_off<DK>(16 * i + 4 * g + (c >> 2), 32 * (d / 2) + 4 * (d % 2) + 8 * (c & 3)));
        f32x4 sd = S[d];
#pragma unroll
        for (int j = 0; j < 4; ++j) sd[j] *= gC;
        sd = mma2(qt[0], qt[1], W1[0], W1[1], sd);
        S[d] = mma2(qt[2], qt[3], W1[2], W1[3], sd);
      }
    }
    // K^T operands of the update, in flight during the Tb^T product.
    auto ktr = [&](int d, u32x2 (&dst)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = ld4_tr(Rb + Cf::oK / 2 +
                        row_off<DK>(16 * i + 4 * g + (c >> 2), 32 * (d / 2) + 4 * (d % 2) + 8 * (c & 3)));
    };
    u32x2 kt[KTB][4];
#pragma unroll
    for (int d = 0; d < KTB; ++d) ktr(d, kt[d]);
    issue_fence();
    // dX = Tb^T dU (block row i sums k blocks i .. 3)
    const u32x4 d01 = pair(du[0], du[1]), d23 = pair(du[2], du[3]);
    f32x4 X[4];
    X[0] = mma32(tt[qblk(0, 1)], d23, mma32(tt[qblk(0, 0)], d01, zero4()));
    X[1] = mma32(tt[qblk(1, 1)], d23, mma32(tt[qblk(1, 0)], d01, zero4()));
    X[2] = mma32(tt[qblk(2, 1)], d23, zero4());
    X[3] = mma32(tt[qblk(3, 1)], d23, zero4());
    u32x2 W2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 x2;
#pragma unroll
      for (int j = 0; j < 4; ++j) x2[j] = -gm[i][j] * X[i][j];
      W2[i] = cvt4(x2);
    }
    // ... - K^T (gamma dX)
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      u32x2 kd[4];
      if (d < KTB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kd[i] = kt[d < KTB ? d : 0][i];
      } else {
        ktr(d, kd);
      }
      f32x4 sd = mma2(kd[0], kd[1], W2[0], W2[1], S[d]);
      sd = mma2(kd[2], kd[3], W2[2], W2[3], sd);
      S[d] = sd;
      sfr[d] = cvt4(sd);
    }
  });
  if (a.dS0) {
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) a.dS0[((size_t)chain * DK + key_row(d, g, j)) * a.DV + col] = S[d][j];
  }
}

template <int DK, int NC>
__global__ __launch_bounds__((AdjCfg<DK, NC>::kThreads), 1) void adj_kernel(AdjArgs a) {
  using Cf = AdjCfg<DK, NC>;
  __shared__ __attribute__((aligned(16))) char smem[Cf::bytes];
  // Slices of one chain are neighbours on one XCD (consecutive blocks go to
  // the eight XCDs in turn), so their shared rows are fetched once into its L2.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int nsl = a.DV / Cf::NV, chain = bid / nsl, dv0 = (bid % nsl) * Cf::NV;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  if (w < NC)
    adj_consumer<DK, NC>(a, chain, dv0, smem, w, l);
  else if (w == Cf::wE)
    adj_e_role<DK, NC>(a, smem, l);
  else if (w == Cf::wL)
    adj_load_role<DK, NC, 0>(a, chain, dv0, smem, l);
  else if (w == Cf::wL + 1)
    adj_load_role<DK, NC, 1>(a, chain, dv0, smem, l);
  else if constexpr (Cf::NLOAD > 2)
    adj_load_role<DK, NC, 2>(a, chain, dv0, smem, l);
}

// ----------------------------------------------------------- gradient pass
// One workgroup of four waves per (chain, chunk).  The chunk's K, Q, V, dO
// rows and its S_n, dS'_n sit in LDS as bf16 64 x 64 matrices with swizzled
// rows; Tb and Tb^T come straight from the records as A operands.
//   phase 0, wave w = token rows 16w .. 16w + 15 of the C x C factors: P^T,
//     Gt^T and Gt as A operands (decayed and masked), shared through LDS;
//   phase 1, wave w = value columns 16w .. 16w + 15: KS, QS, X, U, Z, dU, dX,
//     dY, R; dV; row partials of dbeta and dg; then U and dX to LDS;
//   phase 2, wave w = token rows 16w .. 16w + 15: dP, dGt against P and Gt,
//     D1 and D2 + D2^T to LDS, row and column partials of dg;
//   phase 3, wave w = key columns 16w .. 16w + 15: dQ and dK;
//   phase 4, wave 0: dg, its suffix sums over the chunk, dalpha and dbeta.
// Decays 2^(g_t - g_u) between different 16-token blocks are products of two
// table entries (each at most 1): ge[b][t] = 2^(g_t - g_e) and fs[u] =
// 2^(g_e - g_u), with e the last token of u's block b; within a block they are
// formed directly.
struct GradCfg {
  static constexpr int MAT = 64 * 64 * 2;  // one bf16 matrix
  static constexpr int mK = 0, mQ = 1, mV = 2, mD1 = 2, mO = 3, mS = 4, mDS = 5, mU = 6, mX = 7, mM2 = 8, NMAT = 9;
  // operand blocks of phase 0/1 (lane order, 1 KB each), in matrices that are free until phase 1 ends
  static constexpr int bPT = mM2, bGT = mU, bGL = mX;
  // fp32 arrays after the matrices: g (log2 prefix), beta, gamma, lambda, fs,
  // ge[3], per-wave dg, column, dbeta partials, phase 2 row sums, per-wave
  // Z.U totals and <dS', S> partials
  static constexpr int fG = 0, fB = 64, fGam = 128, fLam = 192, fFs = 256, fGe = 320, fDG = 512, fCP = fDG + 256,
                       fDB = fCP + 256, fRP = fDB + 256, fZS = fRP + 64, fSS = fZS + 4, szF = fSS + 4;
  static constexpr int oF = NMAT * MAT;
  static constexpr int bytes = oF + szF * 4;
  static_assert(bytes <= 80 * 1024, "two workgroups per CU");
};

struct GradArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dO;
  const float* alpha;
  const float* beta;
  const char* rec;     // Tb records [chains][nch]
  const char* recT;    // Tb^T records
  const __bf16* Sck;   // [chains][nch][64][64] chunk start states
  const __bf16* dSck;  // [chains][nch][64][64] chunk end gradients
  float* dq;
  float* dk;
  float* dv;
  float* dalpha;
  float* dbeta;
  int T, H, nch;
  // d = 128 only: the hand-off between its two launches, per (chain, chunk):
  // U and dX (bf16 [64][128]) and the value-side dg terms (fp32 [64])
  __bf16* Uw;
  __bf16* Xw;
  float* dgA;
};

__device__ __forceinline__ __bf16* mat(char* smem, int m) { return reinterpret_cast<__bf16*>(smem + m * GradCfg::MAT); }

// LDS matrices of W bf16 columns with swizzled rows (row_off<W>).
// A or B operand piece: 8 consecutive elements of row r from column e0.
template <int W = 64>
__device__ __forceinline__ u32x4 rowp(const __bf16* M, int r, int e0) {
  return *reinterpret_cast<const u32x4*>(M + row_off<W>(r, e0));
}
// Column piece: M[r0 + e][c0 + c] for e = 0..7 in lane (g, c) (r0 may depend
// on g), through two transposed reads.
template <int W = 64>
__device__ __forceinline__ u32x4 colp(const __bf16* M, int r0, int c0, int c) {
  const u32x2 lo = ld4_tr(M + row_off<W>(r0 + (c >> 2), c0 + 4 * (c & 3)));
  const u32x2 hi = ld4_tr(M + row_off<W>(r0 + 4 + (c >> 2), c0 + 4 * (c & 3)));
  return pair(lo, hi);
}
// Accumulator-layout piece: M[r0 + 4g + j][c0 + c], j = 0..3.
template <int W = 64>
__device__ __forceinline__ u32x2 accp(const __bf16* M, int r0, int c0, int g, int c) {
  return ld4_tr(M + row_off<W>(r0 + 4 * g + (c >> 2), c0 + 4 * (c & 3)));
}
// Stores an accumulator tile (rows r0 + 4g + j, column c0 + c) as bf16.
template <int W = 64>
__device__ __forceinline__ void st_acc(__bf16* M, int r0, int c0, int g, int c, const f32x4& v) {
  const u32x2 b = cvt4(v);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    M[row_off<W>(r0 + 4 * g + j, c0 + c)] =
        __builtin_bit_cast(__bf16, (unsigned short)((j & 1) ? b[j >> 1] >> 16 : b[j >> 1]));
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Decay 2^(g_t - g_u) for token t of block J and token u of block I, J > I,
// from the tables ge (3 x 64) and fs (64).
__device__ __forceinline__ float cross_decay(const float* ge, const float* fs, int I, int t, int u) {
  return ge[64 * I + t] * fs[u];
}
__device__ __forceinline__ float cross_decay(const float* F, int I, int t, int u) {
  return cross_decay(F + GradCfg::fGe, F + GradCfg::fFs, I, t, u);
}

// Gate tables of a chunk, by one wave from its g (log2 prefix, lane t):
// g, gamma, lambda, fs and ge (3 x 64) at the given offsets of F.  Returns g_C.
__device__ __forceinline__ float gate_tables(float* F, float gl, int l, int oG, int oGam, int oLam, int oFs, int oGe) {
  auto at = [&](int src_lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), src_lane));
  };
  const float e0 = at(15), e1 = at(31), e2 = at(47), gC = at(63);
  const int blk = l >> 4;
  const float gend = blk == 0 ? e0 : blk == 1 ? e1 : blk == 2 ? e2 : gC;
  F[oG + l] = gl;
  F[oGam + l] = __builtin_amdgcn_exp2f(gl);
  F[oLam + l] = __builtin_amdgcn_exp2f(gC - gl);
  F[oFs + l] = __builtin_amdgcn_exp2f(gend - gl);
  F[oGe + l] = __builtin_amdgcn_exp2f(blk > 0 ? gl - e0 : -INFINITY);
  F[oGe + 64 + l] = __builtin_amdgcn_exp2f(blk > 1 ? gl - e1 : -INFINITY);
  F[oGe + 128 + l] = __builtin_amdgcn_exp2f(blk > 2 ? gl - e2 : -INFINITY);
  return gC;
}

__global__ __launch_bounds__(256, 2) void grad_kernel(GradArgs a) {
  using Cf = GradCfg;
  __shared__ __attribute__((aligned(16))) char smem[Cf::bytes];
  float* const F = reinterpret_cast<float*>(smem + Cf::oF);
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, nch = a.nch;
  const int id = blockIdx.x;
  const int h = id % H, bn = id / H, n = bn % nch, b = bn / nch;
  const int chain = b * H + h, t0 = n * 64;
  const size_t tokbase = (size_t)b * T * H + h;
  const int rowB = H * 64 * 2;
  const uint32_t spanR = span_bytes((size_t)T * H * 128, (size_t)h * 128);
  const char* const rec = a.rec + ((size_t)chain * nch + n) * kRecBytes;
  const char* const recT = a.recT + ((size_t)chain * nch + n) * kRecBytes;

  // ---- loads: the chunk's rows (zero past T), the states, g and beta; wave 0
  // forms the gate tables
  {
    const __bf16* src[4] = {a.k, a.q, a.v, a.dO};
    const int dstm[4] = {Cf::mK, Cf::mQ, Cf::mV, Cf::mO};
    u32x4 x[4][2], s[2][2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(src[m] + tokbase * 64, spanR);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int unit = tid + 256 * u, row = unit >> 3, pc = unit & 7;
        x[m][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, row * rowB + 16 * pc, t0 * rowB, 0));
      }
    }
    const __bf16* st[2] = {a.Sck + ((size_t)chain * nch + n) * 4096, a.dSck + ((size_t)chain * nch + n) * 4096};
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < 2; ++u) s[m][u] = reinterpret_cast<const u32x4*>(st[m])[tid + 256 * u];
    if (w == 0) {
      const float gl = reinterpret_cast<const float*>(rec + kRecG)[l];
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + tokbase, span_bytes((size_t)T * H * 4, (size_t)h * 4));
      F[Cf::fB + l] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, l * H * 4, t0 * H * 4, 0));
      auto at = [&](int src_lane) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), src_lane));
      };
      const float e0 = at(15), e1 = at(31), e2 = at(47), gC = at(63);
      const int blk = l >> 4;
      const float gend = blk == 0 ? e0 : blk == 1 ? e1 : blk == 2 ? e2 : gC;
      F[Cf::fG + l] = gl;
      F[Cf::fGam + l] = __builtin_amdgcn_exp2f(gl);
      F[Cf::fLam + l] = __builtin_amdgcn_exp2f(gC - gl);
      F[Cf::fFs + l] = __builtin_amdgcn_exp2f(gend - gl);
      F[Cf::fGe + l] = __builtin_amdgcn_exp2f(blk > 0 ? gl - e0 : -INFINITY);
      F[Cf::fGe + 64 + l] = __builtin_amdgcn_exp2f(blk > 1 ? gl - e1 : -INFINITY);
      F[Cf::fGe + 128 + l] = __builtin_amdgcn_exp2f(blk > 2 ? gl - e2 : -INFINITY);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int unit = tid + 256 * u, row = unit >> 3, pc = unit & 7;
        *reinterpret_cast<u32x4*>(mat(smem, dstm[m]) + row_off<64>(row, 8 * pc)) = x[m][u];
      }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int unit = tid + 256 * u, row = unit >> 3, pc = unit & 7;
        *reinterpret_cast<u32x4*>(mat(smem, m == 0 ? Cf::mS : Cf::mDS) + row_off<64>(row, 8 * pc)) = s[m][u];
      }
  }
  __syncthreads();

  const __bf16* const mK = mat(smem, Cf::mK);
  const __bf16* const mQ = mat(smem, Cf::mQ);
  const __bf16* const mO = mat(smem, Cf::mO);
  const __bf16* const mS = mat(smem, Cf::mS);
  const __bf16* const mDS = mat(smem, Cf::mDS);
  const float* const gt = F + Cf::fG;
  const float gC = gt[63];
  auto blob = [&](int area, int i, int p) { return reinterpret_cast<u32x4*>(smem + area * Cf::MAT + (i * 2 + p) * 1024) + l; };

  // ---- phase 0: block row I = w of P^T, Gt^T (k blocks J >= I) and Gt (J <= I)
  {
    const int I = w;
    u32x4 kI[2], kr[4][2], qr[4][2];
#pragma unroll
    for (int p = 0; p < 2; ++p) kI[p] = rowp(mK, 16 * I + c, 32 * p + 8 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        kr[j][p] = rowp(mK, 16 * j + c, 32 * p + 8 * g);
        qr[j][p] = rowp(mQ, 16 * j + c, 32 * p + 8 * g);
      }
    const float gu = gt[16 * I + c];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x2 hP[2], hT[2], hL[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int J = 2 * p + hh;
        hP[hh] = hT[hh] = hL[hh] = z4();
        // raw Gram block: lane (g, c) holds G[16J + 4g + r][16I + c]
        f32x4 G = zero4();
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) G = mma32(kr[J][kp], kI[kp], G);
        if (J >= I) {
          // P^T and Gt^T of block (I, J): t = 16J + 4g + r (row of P, Gt), u = 16I + c
          f32x4 P = zero4();
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) P = mma32(qr[J][kp], kI[kp], P);
          const f32x4 gj = ld4f(gt + 16 * J + 4 * g);
          f32x4 vP, vT;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * J + 4 * g + r, u = 16 * I + c;
            const float m = J > I ? cross_decay(F, I, t, u) : __builtin_amdgcn_exp2f(t >= u ? gj[r] - gu : -INFINITY);
            vP[r] = P[r] * m;
            vT[r] = t > u ? G[r] * m : 0.f;
          }
          hP[hh] = cvt4(vP);
          hT[hh] = cvt4(vT);
        }
        if (J <= I) {
          // Gt of block (I, J): row t = 16I + c, column u = 16J + 4g + r, G symmetric
          const f32x4 gj = ld4f(gt + 16 * J + 4 * g);
          f32x4 vL;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + c, u = 16 * J + 4 * g + r;
            const float m = I > J ? cross_decay(F, J, t, u) : __builtin_amdgcn_exp2f(t > u ? gu - gj[r] : -INFINITY);
            vL[r] = G[r] * m;
          }
          hL[hh] = cvt4(vL);
        }
      }
      *blob(Cf::bPT, I, p) = pair(hP[0], hP[1]);
      *blob(Cf::bGT, I, p) = pair(hT[0], hT[1]);
      *blob(Cf::bGL, I, p) = pair(hL[0], hL[1]);
    }
  }
  __syncthreads();

  // ---- phase 1: value columns cw .. cw + 15
  {
    const int cw = 16 * w;
    auto krow = [&](u32x4 (&kr)[4][2], const __bf16* M) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p) kr[i][p] = rowp(M, 16 * i + c, 32 * p + 8 * g);
    };
    u32x4 sB[2], dsB[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      sB[p] = colp(mS, 32 * p + 8 * g, cw, c);
      dsB[p] = colp(mDS, 32 * p + 8 * g, cw, c);
    }
    // <dS', S> over this wave's columns
    {
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += lo_f(sB[p][e]) * lo_f(dsB[p][e]) + hi_f(sB[p][e]) * hi_f(dsB[p][e]);
      ss = lane::wave_sum(ss);
      if (l == 0) F[Cf::fSS + w] = ss;
    }
    u32x2 oB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) oB[i] = accp(mO, 16 * i, cw, g, c);
    float dgr[4][4];  // dg terms of the lane's rows 16i + 4g + j, this column
    // (a) gamma QS . dO; (b) KS, X = V - gamma KS, U = Tb X
    f32x4 KS[4], X[4], U[4];
    u32x2 ub[4];
    {
      u32x4 qr[4][2], kr[4][2];
      krow(qr, mQ);
      krow(kr, mK);
      u32x2 xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 vB = accp(mat(smem, Cf::mV), 16 * i, cw, g, c);
        f32x4 qs = zero4(), ks = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          qs = mma32(qr[i][p], sB[p], qs);
          ks = mma32(kr[i][p], sB[p], ks);
        }
        const f32x4 gm = ld4f(F + Cf::fGam + 16 * i + 4 * g);
        KS[i] = ks;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dgr[i][j] = gm[j] * qs[j] * bf_at(oB[i], j);
          X[i][j] = bf_at(vB, j) - gm[j] * ks[j];
        }
        xb[i] = cvt4(X[i]);
      }
      u32x4 tb[6];
#pragma unroll
      for (int e = 0; e < 6; ++e) tb[e] = reinterpret_cast<const u32x4*>(rec + kRecTb + e * 1024)[l];
      const u32x4 x01 = pair(xb[0], xb[1]), x23 = pair(xb[2], xb[3]);
      U[0] = mma32(tb[pblk(0, 0)], x01, zero4());
      U[1] = mma32(tb[pblk(1, 0)], x01, zero4());
      U[2] = mma32(tb[pblk(2, 1)], x23, mma32(tb[pblk(2, 0)], x01, zero4()));
      U[3] = mma32(tb[pblk(3, 1)], x23, mma32(tb[pblk(3, 0)], x01, zero4()));
#pragma unroll
      for (int i = 0; i < 4; ++i) ub[i] = cvt4(U[i]);
    }
    // (c) Z = lambda K dS', dU = P^T dO + Z
    f32x4 dU[4], Z[4];
    {
      u32x4 kr[4][2];
      krow(kr, mK);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 z = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p) z = mma32(kr[i][p], dsB[p], z);
        const f32x4 lm = ld4f(F + Cf::fLam + 16 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) Z[i][j] = lm[j] * z[j];
      }
      const u32x4 o01 = pair(oB[0], oB[1]), o23 = pair(oB[2], oB[3]);
      dU[0] = mma32(*blob(Cf::bPT, 0, 1), o23, mma32(*blob(Cf::bPT, 0, 0), o01, Z[0]));
      dU[1] = mma32(*blob(Cf::bPT, 1, 1), o23, mma32(*blob(Cf::bPT, 1, 0), o01, Z[1]));
      dU[2] = mma32(*blob(Cf::bPT, 2, 1), o23, Z[2]);
      dU[3] = mma32(*blob(Cf::bPT, 3, 1), o23, Z[3]);
    }
    // (d) dX = Tb^T dU (= dV); the -gamma KS . dX - Z . U row terms
    f32x4 DX[4];
    u32x2 dxb[4];
    float zsum = 0.f;
    {
      u32x2 dub[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dub[i] = cvt4(dU[i]);
      u32x4 tt[6];
#pragma unroll
      for (int e = 0; e < 6; ++e) tt[e] = reinterpret_cast<const u32x4*>(recT + kRecTb + e * 1024)[l];
      const u32x4 d01 = pair(dub[0], dub[1]), d23 = pair(dub[2], dub[3]);
      DX[0] = mma32(tt[qblk(0, 1)], d23, mma32(tt[qblk(0, 0)], d01, zero4()));
      DX[1] = mma32(tt[qblk(1, 1)], d23, mma32(tt[qblk(1, 0)], d01, zero4()));
      DX[2] = mma32(tt[qblk(2, 1)], d23, zero4());
      DX[3] = mma32(tt[qblk(3, 1)], d23, zero4());
      const __amdgpu_buffer_rsrc_t rdv =
          make_rsrc(a.dv + tokbase * 64 + cw, span_bytes((size_t)T * H * 256, ((size_t)h * 64 + cw) * 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dxb[i] = cvt4(DX[i]);
        const f32x4 gm = ld4f(F + Cf::fGam + 16 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * i + 4 * g + j;
          // (through a scalar: a bit cast of a vector element was compiled as a cast of element 0)
          const float dvv = DX[i][j];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dvv), rdv, r * H * 256 + 4 * c,
                                                t0 * H * 256, 0);
          const float zu = Z[i][j] * U[i][j];
          zsum += zu;
          dgr[i][j] -= gm[j] * KS[i][j] * dvv + zu;
        }
      }
    }
    // (e) dY = dU - Gt^T dX, R = X - Gt U, dbeta = dY . R; the row sums
    {
      const u32x4 x01 = pair(dxb[0], dxb[1]), x23 = pair(dxb[2], dxb[3]);
      const u32x4 u01 = pair(ub[0], ub[1]), u23 = pair(ub[2], ub[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 t = mma32(*blob(Cf::bGT, i, 1), x23, mma32(*blob(Cf::bGT, i, 0), x01, zero4()));
        const f32x4 rr = mma32(*blob(Cf::bGL, i, 1), u23, mma32(*blob(Cf::bGL, i, 0), u01, zero4()));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * i + 4 * g + j;
          const float db = row16_sum((dU[i][j] - t[j]) * (X[i][j] - rr[j]));
          const float dg = row16_sum(dgr[i][j]);
          if (c == 0) {
            F[Cf::fDB + 64 * w + r] = db;
            F[Cf::fDG + 64 * w + r] = dg;
          }
        }
      }
      zsum = lane::wave_sum(zsum);
      if (l == 0) F[Cf::fZS + w] = zsum;
    }
    __syncthreads();  // every wave is done with the phase 0 blocks before U and dX overwrite them
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st_acc(mat(smem, Cf::mU), 16 * i, cw, g, c, U[i]);
      st_acc(mat(smem, Cf::mX), 16 * i, cw, g, c, DX[i]);
    }
  }
  __syncthreads();

  // ---- phase 2: token rows 16I .. 16I + 15, I = w
  {
    const int I = w;
    __bf16* const mD1 = mat(smem, Cf::mD1);
    __bf16* const mM2 = mat(smem, Cf::mM2);
    const __bf16* const mU = mat(smem, Cf::mU);
    const __bf16* const mX = mat(smem, Cf::mX);
    u32x4 oR[2], xR[2], qI[2], kI[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      oR[p] = rowp(mO, 16 * I + c, 32 * p + 8 * g);
      xR[p] = rowp(mX, 16 * I + c, 32 * p + 8 * g);
      qI[p] = rowp(mQ, 16 * I + c, 32 * p + 8 * g);
      kI[p] = rowp(mK, 16 * I + c, 32 * p + 8 * g);
    }
    const f32x4 gI = ld4f(gt + 16 * I + 4 * g);
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > I) {  // above the diagonal: D1 is zero, and this wave reports no column terms there
        st_acc(mD1, 16 * I, 16 * J, g, c, zero4());
        if (g == 0) F[Cf::fCP + 64 * w + 16 * J + c] = 0.f;
        continue;
      }
      f32x4 dP = zero4(), dG = zero4(), P = zero4(), G = zero4();
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32x4 uJ = rowp(mU, 16 * J + c, 32 * p + 8 * g);
        const u32x4 kJ = rowp(mK, 16 * J + c, 32 * p + 8 * g);
        dP = mma32(oR[p], uJ, dP);
        dG = mma32(xR[p], uJ, dG);
        P = mma32(qI[p], kJ, P);
        G = mma32(kI[p], kJ, G);
      }
      const float gu = gt[16 * J + c];
      f32x4 d1, d2;
      float cs = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ti = 16 * I + 4 * g + r, uj = 16 * J + c;
        const float m = I > J ? cross_decay(F, J, ti, uj) : __builtin_amdgcn_exp2f(ti >= uj ? gI[r] - gu : -INFINITY);
        const float ms = ti > uj ? m : 0.f;
        d1[r] = dP[r] * m;
        d2[r] = -dG[r] * ms;
        const float e = d1[r] * P[r] + d2[r] * G[r];  // dP o P + dGt o Gt (the decay sits on one factor)
        rs[r] += e;
        cs += e;
      }
      cs = col4_sum(cs);
      if (g == 0) F[Cf::fCP + 64 * w + 16 * J + c] = cs;
      st_acc(mD1, 16 * I, 16 * J, g, c, d1);
      // D2 + D2^T: the strictly lower entries, and their mirror images
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ti = 16 * I + 4 * g + r, uj = 16 * J + c;
        const __bf16 val = __builtin_bit_cast(__bf16, (unsigned short)(cvt2(d2[r], 0.f) & 0xffffu));
        if (J < I || ti > uj) {
          mM2[row_off<64>(ti, uj)] = val;
          mM2[row_off<64>(uj, ti)] = val;
        } else if (ti == uj) {
          mM2[row_off<64>(ti, uj)] = __builtin_bit_cast(__bf16, (unsigned short)0);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = row16_sum(rs[r]);
      if (c == 0) F[Cf::fRP + 16 * I + 4 * g + r] = v;
    }
  }
  __syncthreads();

  // ---- phase 3: key columns kw .. kw + 15
  {
    const int kw = 16 * w;
    const __bf16* const mD1 = mat(smem, Cf::mD1);
    const __bf16* const mM2 = mat(smem, Cf::mM2);
    const __bf16* const mU = mat(smem, Cf::mU);
    const __bf16* const mX = mat(smem, Cf::mX);
    u32x4 kB[2], qB[2], sR[2], dsR[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      kB[p] = colp(mK, 32 * p + 8 * g, kw, c);
      qB[p] = colp(mQ, 32 * p + 8 * g, kw, c);
      sR[p] = rowp(mS, kw + c, 32 * p + 8 * g);
      dsR[p] = rowp(mDS, kw + c, 32 * p + 8 * g);
    }
    const __amdgpu_buffer_rsrc_t rdq =
        make_rsrc(a.dq + tokbase * 64 + kw, span_bytes((size_t)T * H * 256, ((size_t)h * 64 + kw) * 4));
    const __amdgpu_buffer_rsrc_t rdk =
        make_rsrc(a.dk + tokbase * 64 + kw, span_bytes((size_t)T * H * 256, ((size_t)h * 64 + kw) * 4));
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 q1 = zero4(), q2 = zero4(), k1 = zero4(), k3 = zero4(), k4 = zero4();
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        q1 = mma32(rowp(mD1, 16 * I + c, 32 * p + 8 * g), kB[p], q1);
        q2 = mma32(rowp(mO, 16 * I + c, 32 * p + 8 * g), sR[p], q2);
        k1 = mma32(colp(mD1, 32 * p + 8 * g, 16 * I, c), qB[p], k1);
        k1 = mma32(rowp(mM2, 16 * I + c, 32 * p + 8 * g), kB[p], k1);
        k3 = mma32(rowp(mU, 16 * I + c, 32 * p + 8 * g), dsR[p], k3);
        k4 = mma32(rowp(mX, 16 * I + c, 32 * p + 8 * g), sR[p], k4);
      }
      const f32x4 gm = ld4f(F + Cf::fGam + 16 * I + 4 * g), lm = ld4f(F + Cf::fLam + 16 * I + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * I + 4 * g + j;
        const float dqv = q1[j] + gm[j] * q2[j];
        const float dkv = k1[j] + lm[j] * k3[j] - gm[j] * k4[j];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dqv), rdq, r * H * 256 + 4 * c, t0 * H * 256, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dkv), rdk, r * H * 256 + 4 * c, t0 * H * 256, 0);
      }
    }
  }

  // ---- phase 4: dg, d ln alpha as suffix sums, dalpha and dbeta
  __syncthreads();
  if (w == 0) {
    const int t = l;
    float dg = 0.f, db = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      dg += F[Cf::fDG + 64 * v + t] - F[Cf::fCP + 64 * v + t];
      db += F[Cf::fDB + 64 * v + t];
    }
    dg += F[Cf::fRP + t];
    if (t == 63) {
      const float ss = (F[Cf::fSS] + F[Cf::fSS + 1]) + (F[Cf::fSS + 2] + F[Cf::fSS + 3]);
      const float zt = (F[Cf::fZS] + F[Cf::fZS + 1]) + (F[Cf::fZS + 2] + F[Cf::fZS + 3]);
      dg += __builtin_amdgcn_exp2f(gC) * ss + zt;
    }
    const float pre = wave_prefix_sum(dg);
    const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pre), 63));
    const float dla = tot - pre + dg;
    const uint32_t spanG = span_bytes((size_t)T * H * 4, (size_t)h * 4);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.alpha + tokbase, spanG);
    const float al = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, t * H * 4, t0 * H * 4, 0));
    const __amdgpu_buffer_rsrc_t rda = make_rsrc(a.dalpha + tokbase, spanG);
    const __amdgpu_buffer_rsrc_t rdb = make_rsrc(a.dbeta + tokbase, spanG);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dla / al), rda, t * H * 4, t0 * H * 4, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, db), rdb, t * H * 4, t0 * H * 4, 0);
  }
}

// ------------------------------------------------ gradient pass at d = 128
// The d = 64 workgroup holds K, Q, V, dO, S, dS', U, dX and the C x C
// factors at once (79 KB).  At d = 128 the two states alone take 64 KB, so the
// pass runs as two launches per (chain, chunk), handing U, dX (bf16) and the
// value-side dg terms over through the workspace:
//   cols: phases 0 and 1, eight waves (one per 16 value columns): dV, dbeta;
//   rows: phases 2 to 4, four waves: dQ, dK, dalpha.  There the S and dS'
//         rows are B operands read straight from global memory (16 contiguous
//         bytes each), and only 64-column matrices sit in LDS.
struct Grad128Cfg {
  static constexpr int D = 128;
  static constexpr int MAT = 64 * D * 2;  // a 64 x 128 bf16 matrix
  // cols launch (bytes): K, Q, V, dO; S, dS' (128 x 128); phase 0 operand blocks (PT, GT, GL)
  static constexpr int cK = 0, cQ = MAT, cV = 2 * MAT, cO = 3 * MAT, cS = 4 * MAT, cDS = 6 * MAT, cBL = 8 * MAT;
  static constexpr int cF = cBL + 3 * 8192;
  // fp32 arrays: g, beta, gamma, lambda, fs, ge[3]; per-wave dg and dbeta partials; Z.U and <dS', S> per wave
  static constexpr int fG = 0, fB = 64, fGam = 128, fLam = 192, fFs = 256, fGe = 320, fDG = 512, fDB = fDG + 512,
                       fZS = fDB + 512, fSS = fZS + 8, szF = fSS + 8;
  static constexpr int cBytes = cF + szF * 4;
  // rows launch (bytes): K, Q, dO, U, dX (64 x 128), D1 and D2 + D2^T (64 x 64)
  static constexpr int rK = 0, rQ = MAT, rO = 2 * MAT, rU = 3 * MAT, rX = 4 * MAT, rD1 = 5 * MAT, rM2 = rD1 + 8192,
                       rF = rM2 + 8192;
  // fp32 arrays: g, gamma, lambda, fs, ge[3], the cols launch's dg terms, column partials [4][64], row sums
  static constexpr int hG = 0, hGam = 64, hLam = 128, hFs = 192, hGe = 256, hDA = 448, hCP = 512, hRP = 768,
                       szH = 832;
  static constexpr int rBytes = rF + szH * 4;
  static_assert(cBytes <= 160 * 1024 && rBytes <= 160 * 1024, "LDS budget");
};

__global__ __launch_bounds__(512, 1) void grad_cols_kernel(GradArgs a) {
  using Cf = Grad128Cfg;
  constexpr int D = Cf::D;
  __shared__ __attribute__((aligned(16))) char smem[Cf::cBytes];
  float* const F = reinterpret_cast<float*>(smem + Cf::cF);
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, nch = a.nch;
  const int id = blockIdx.x;
  const int h = id % H, bn = id / H, n = bn % nch, b = bn / nch;
  const int chain = b * H + h, t0 = n * 64;
  const size_t tokbase = (size_t)b * T * H + h, ck = (size_t)chain * nch + n;
  const int rowB = H * D * 2;
  const uint32_t spanR = span_bytes((size_t)T * H * D * 2, (size_t)h * D * 2);
  const char* const rec = a.rec + ck * kRecBytes;
  const char* const recT = a.recT + ck * kRecBytes;
  auto M = [&](int off) { return reinterpret_cast<__bf16*>(smem + off); };

  // ---- loads
  {
    const __bf16* src[4] = {a.k, a.q, a.v, a.dO};
    const int dst[4] = {Cf::cK, Cf::cQ, Cf::cV, Cf::cO};
    u32x4 x[4][2], st[2][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(src[m] + tokbase * D, spanR);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int unit = tid + 512 * u, row = unit >> 4, pc = unit & 15;
        x[m][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, row * rowB + 16 * pc, t0 * rowB, 0));
      }
    }
    const u32x4* ss[2] = {reinterpret_cast<const u32x4*>(a.Sck + ck * D * D),
                          reinterpret_cast<const u32x4*>(a.dSck + ck * D * D)};
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) st[m][u] = ss[m][tid + 512 * u];
    if (w == 0) {
      const float gl = reinterpret_cast<const float*>(rec + kRecG)[l];
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + tokbase, span_bytes((size_t)T * H * 4, (size_t)h * 4));
      F[Cf::fB + l] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, l * H * 4, t0 * H * 4, 0));
      gate_tables(F, gl, l, Cf::fG, Cf::fGam, Cf::fLam, Cf::fFs, Cf::fGe);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int unit = tid + 512 * u, row = unit >> 4, pc = unit & 15;
        *reinterpret_cast<u32x4*>(M(dst[m]) + row_off<D>(row, 8 * pc)) = x[m][u];
      }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int unit = tid + 512 * u, row = unit >> 4, pc = unit & 15;
        *reinterpret_cast<u32x4*>(M(m == 0 ? Cf::cS : Cf::cDS) + row_off<D>(row, 8 * pc)) = st[m][u];
      }
  }
  __syncthreads();

  const __bf16* const mK = M(Cf::cK);
  const __bf16* const mQ = M(Cf::cQ);
  const __bf16* const mO = M(Cf::cO);
  const float* const gt = F + Cf::fG;
  const float gC = gt[63];
  auto blob = [&](int which, int i, int p) {
    return reinterpret_cast<u32x4*>(smem + Cf::cBL + which * 8192 + (i * 2 + p) * 1024) + l;
  };

  // ---- phase 0: waves 0-3 P^T of block row w, waves 4-7 Gt^T and Gt of block row w - 4
  {
    const int I = w & 3;
    const bool pwave = w < 4;
    u32x4 kI[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) kI[p] = rowp<D>(mK, 16 * I + c, 32 * p + 8 * g);
    const float gu = gt[16 * I + c];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x2 h0[2], h1[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int J = 2 * p + hh;
        h0[hh] = h1[hh] = z4();
        const __bf16* const src = pwave ? mQ : mK;
        f32x4 acc = zero4();
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) acc = mma32(rowp<D>(src, 16 * J + c, 32 * kp + 8 * g), kI[kp], acc);
        const f32x4 gj = ld4f(gt + 16 * J + 4 * g);
        if (J >= I) {  // P^T / Gt^T block (I, J): t = 16J + 4g + r, u = 16I + c
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * J + 4 * g + r, u = 16 * I + c;
            const float m = J > I ? cross_decay(F + Cf::fGe, F + Cf::fFs, I, t, u)
                                  : __builtin_amdgcn_exp2f(t >= u ? gj[r] - gu : -INFINITY);
            v[r] = (pwave || t > u) ? acc[r] * m : 0.f;
          }
          h0[hh] = cvt4(v);
        }
        if (!pwave && J <= I) {  // Gt block (I, J): t = 16I + c, u = 16J + 4g + r (G symmetric)
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + c, u = 16 * J + 4 * g + r;
            const float m = I > J ? cross_decay(F + Cf::fGe, F + Cf::fFs, J, t, u)
                                  : __builtin_amdgcn_exp2f(t > u ? gu - gj[r] : -INFINITY);
            v[r] = acc[r] * m;
          }
          h1[hh] = cvt4(v);
        }
      }
      if (pwave) {
        *blob(0, I, p) = pair(h0[0], h0[1]);
      } else {
        *blob(1, I, p) = pair(h0[0], h0[1]);
        *blob(2, I, p) = pair(h1[0], h1[1]);
      }
    }
  }
  __syncthreads();

  // ---- phase 1: value columns cw .. cw + 15
  const int cw = 16 * w;
  f32x4 U[4], DX[4];
  {
    const __bf16* const mS = M(Cf::cS);
    const __bf16* const mDS = M(Cf::cDS);
    u32x4 sB[4], dsB[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      sB[p] = colp<D>(mS, 32 * p + 8 * g, cw, c);
      dsB[p] = colp<D>(mDS, 32 * p + 8 * g, cw, c);
    }
    {
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += lo_f(sB[p][e]) * lo_f(dsB[p][e]) + hi_f(sB[p][e]) * hi_f(dsB[p][e]);
      ss = lane::wave_sum(ss);
      if (l == 0) F[Cf::fSS + w] = ss;
    }
    u32x2 oB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) oB[i] = accp<D>(mO, 16 * i, cw, g, c);
    float dgr[4][4];
    f32x4 KS[4], X[4];
    u32x2 ub[4];
    {
      u32x2 xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 vB = accp<D>(M(Cf::cV), 16 * i, cw, g, c);
        f32x4 qs = zero4(), ks = zero4();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          qs = mma32(rowp<D>(mQ, 16 * i + c, 32 * p + 8 * g), sB[p], qs);
          ks = mma32(rowp<D>(mK, 16 * i + c, 32 * p + 8 * g), sB[p], ks);
        }
        const f32x4 gm = ld4f(F + Cf::fGam + 16 * i + 4 * g);
        KS[i] = ks;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dgr[i][j] = gm[j] * qs[j] * bf_at(oB[i], j);
          X[i][j] = bf_at(vB, j) - gm[j] * ks[j];
        }
        xb[i] = cvt4(X[i]);
      }
      u32x4 tb[6];
#pragma unroll
      for (int e = 0; e < 6; ++e) tb[e] = reinterpret_cast<const u32x4*>(rec + kRecTb + e * 1024)[l];
      const u32x4 x01 = pair(xb[0], xb[1]), x23 = pair(xb[2], xb[3]);
      U[0] = mma32(tb[pblk(0, 0)], x01, zero4());
      U[1] = mma32(tb[pblk(1, 0)], x01, zero4());
      U[2] = mma32(tb[pblk(2, 1)], x23, mma32(tb[pblk(2, 0)], x01, zero4()));
      U[3] = mma32(tb[pblk(3, 1)], x23, mma32(tb[pblk(3, 0)], x01, zero4()));
#pragma unroll
      for (int i = 0; i < 4; ++i) ub[i] = cvt4(U[i]);
    }
    f32x4 dU[4], Z[4];
    {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 z = zero4();
#pragma unroll
        for (int p = 0; p < 4; ++p) z = mma32(rowp<D>(mK, 16 * i + c, 32 * p + 8 * g), dsB[p], z);
        const f32x4 lm = ld4f(F + Cf::fLam + 16 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) Z[i][j] = lm[j] * z[j];
      }
      const u32x4 o01 = pair(oB[0], oB[1]), o23 = pair(oB[2], oB[3]);
      dU[0] = mma32(*blob(0, 0, 1), o23, mma32(*blob(0, 0, 0), o01, Z[0]));
      dU[1] = mma32(*blob(0, 1, 1), o23, mma32(*blob(0, 1, 0), o01, Z[1]));
      dU[2] = mma32(*blob(0, 2, 1), o23, Z[2]);
      dU[3] = mma32(*blob(0, 3, 1), o23, Z[3]);
    }
    u32x2 dxb[4];
    float zsum = 0.f;
    {
      u32x2 dub[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dub[i] = cvt4(dU[i]);
      u32x4 tt[6];
#pragma unroll
      for (int e = 0; e < 6; ++e) tt[e] = reinterpret_cast<const u32x4*>(recT + kRecTb + e * 1024)[l];
      const u32x4 d01 = pair(dub[0], dub[1]), d23 = pair(dub[2], dub[3]);
      DX[0] = mma32(tt[qblk(0, 1)], d23, mma32(tt[qblk(0, 0)], d01, zero4()));
      DX[1] = mma32(tt[qblk(1, 1)], d23, mma32(tt[qblk(1, 0)], d01, zero4()));
      DX[2] = mma32(tt[qblk(2, 1)], d23, zero4());
      DX[3] = mma32(tt[qblk(3, 1)], d23, zero4());
      const __amdgpu_buffer_rsrc_t rdv =
          make_rsrc(a.dv + tokbase * D + cw, span_bytes((size_t)T * H * D * 4, ((size_t)h * D + cw) * 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dxb[i] = cvt4(DX[i]);
        const f32x4 gm = ld4f(F + Cf::fGam + 16 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * i + 4 * g + j;
          const float dvv = DX[i][j];  // through a scalar (see the d = 64 kernel)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dvv), rdv, r * H * D * 4 + 4 * c,
                                                t0 * H * D * 4, 0);
          const float zu = Z[i][j] * U[i][j];
          zsum += zu;
          dgr[i][j] -= gm[j] * KS[i][j] * dvv + zu;
        }
      }
    }
    {
      const u32x4 x01 = pair(dxb[0], dxb[1]), x23 = pair(dxb[2], dxb[3]);
      const u32x4 u01 = pair(ub[0], ub[1]), u23 = pair(ub[2], ub[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 t = mma32(*blob(1, i, 1), x23, mma32(*blob(1, i, 0), x01, zero4()));
        const f32x4 rr = mma32(*blob(2, i, 1), u23, mma32(*blob(2, i, 0), u01, zero4()));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * i + 4 * g + j;
          const float db = row16_sum((dU[i][j] - t[j]) * (X[i][j] - rr[j]));
          const float dg = row16_sum(dgr[i][j]);
          if (c == 0) {
            F[Cf::fDB + 64 * w + r] = db;
            F[Cf::fDG + 64 * w + r] = dg;
          }
        }
      }
      zsum = lane::wave_sum(zsum);
      if (l == 0) F[Cf::fZS + w] = zsum;
    }
  }
  __syncthreads();  // V and dO are dead: U and dX go through their space to the workspace
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st_acc<D>(M(Cf::cV), 16 * i, cw, g, c, U[i]);
    st_acc<D>(M(Cf::cO), 16 * i, cw, g, c, DX[i]);
  }
  __syncthreads();
  {
    u32x4* const uw = reinterpret_cast<u32x4*>(a.Uw + ck * 64 * D);
    u32x4* const xw = reinterpret_cast<u32x4*>(a.Xw + ck * 64 * D);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int unit = tid + 512 * u, row = unit >> 4, pc = unit & 15;
      uw[unit] = *reinterpret_cast<const u32x4*>(M(Cf::cV) + row_off<D>(row, 8 * pc));
      xw[unit] = *reinterpret_cast<const u32x4*>(M(Cf::cO) + row_off<D>(row, 8 * pc));
    }
  }
  if (w == 0) {
    const int t = l;
    float dg = 0.f, db = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      dg += F[Cf::fDG + 64 * v + t];
      db += F[Cf::fDB + 64 * v + t];
    }
    if (t == 63) {
      float ss = 0.f, zt = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        ss += F[Cf::fSS + v];
        zt += F[Cf::fZS + v];
      }
      dg += __builtin_amdgcn_exp2f(gC) * ss + zt;
    }
    a.dgA[ck * 64 + t] = dg;
    const uint32_t spanG = span_bytes((size_t)T * H * 4, (size_t)h * 4);
    const __amdgpu_buffer_rsrc_t rdb = make_rsrc(a.dbeta + tokbase, spanG);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, db), rdb, t * H * 4, t0 * H * 4, 0);
  }
}

__global__ __launch_bounds__(256, 1) void grad_rows_kernel(GradArgs a) {
  using Cf = Grad128Cfg;
  constexpr int D = Cf::D;
  __shared__ __attribute__((aligned(16))) char smem[Cf::rBytes];
  float* const F = reinterpret_cast<float*>(smem + Cf::rF);
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, nch = a.nch;
  const int id = blockIdx.x;
  const int h = id % H, bn = id / H, n = bn % nch, b = bn / nch;
  const int chain = b * H + h, t0 = n * 64;
  const size_t tokbase = (size_t)b * T * H + h, ck = (size_t)chain * nch + n;
  const int rowB = H * D * 2;
  const uint32_t spanR = span_bytes((size_t)T * H * D * 2, (size_t)h * D * 2);
  const char* const rec = a.rec + ck * kRecBytes;
  auto M = [&](int off) { return reinterpret_cast<__bf16*>(smem + off); };

  // ---- loads: K, Q, dO rows; U and dX from the cols launch; its dg terms
  {
    const __bf16* src[3] = {a.k, a.q, a.dO};
    const int dst[3] = {Cf::rK, Cf::rQ, Cf::rO};
    u32x4 x[3][4], y[2][4];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(src[m] + tokbase * D, spanR);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int unit = tid + 256 * u, row = unit >> 4, pc = unit & 15;
        x[m][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, row * rowB + 16 * pc, t0 * rowB, 0));
      }
    }
    const u32x4* hw[2] = {reinterpret_cast<const u32x4*>(a.Uw + ck * 64 * D),
                          reinterpret_cast<const u32x4*>(a.Xw + ck * 64 * D)};
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) y[m][u] = hw[m][tid + 256 * u];
    if (w == 0) {
      const float gl = reinterpret_cast<const float*>(rec + kRecG)[l];
      gate_tables(F, gl, l, Cf::hG, Cf::hGam, Cf::hLam, Cf::hFs, Cf::hGe);
      F[Cf::hDA + l] = a.dgA[ck * 64 + l];
    }
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int unit = tid + 256 * u, row = unit >> 4, pc = unit & 15;
        *reinterpret_cast<u32x4*>(M(dst[m]) + row_off<D>(row, 8 * pc)) = x[m][u];
      }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int unit = tid + 256 * u, row = unit >> 4, pc = unit & 15;
        *reinterpret_cast<u32x4*>(M(m == 0 ? Cf::rU : Cf::rX) + row_off<D>(row, 8 * pc)) = y[m][u];
      }
  }
  __syncthreads();

  const __bf16* const mK = M(Cf::rK);
  const __bf16* const mQ = M(Cf::rQ);
  const __bf16* const mO = M(Cf::rO);
  const __bf16* const mU = M(Cf::rU);
  const __bf16* const mX = M(Cf::rX);
  const float* const gt = F + Cf::hG;

  // ---- phase 2: token rows 16I .. 16I + 15, I = w
  {
    const int I = w;
    __bf16* const mD1 = M(Cf::rD1);
    __bf16* const mM2 = M(Cf::rM2);
    u32x4 oR[4], xR[4], qI[4], kI[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      oR[p] = rowp<D>(mO, 16 * I + c, 32 * p + 8 * g);
      xR[p] = rowp<D>(mX, 16 * I + c, 32 * p + 8 * g);
      qI[p] = rowp<D>(mQ, 16 * I + c, 32 * p + 8 * g);
      kI[p] = rowp<D>(mK, 16 * I + c, 32 * p + 8 * g);
    }
    const f32x4 gI = ld4f(gt + 16 * I + 4 * g);
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > I) {
        st_acc<64>(mD1, 16 * I, 16 * J, g, c, zero4());
        if (g == 0) F[Cf::hCP + 64 * w + 16 * J + c] = 0.f;
        continue;
      }
      f32x4 dP = zero4(), dG = zero4(), P = zero4(), G = zero4();
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const u32x4 uJ = rowp<D>(mU, 16 * J + c, 32 * p + 8 * g);
        const u32x4 kJ = rowp<D>(mK, 16 * J + c, 32 * p + 8 * g);
        dP = mma32(oR[p], uJ, dP);
        dG = mma32(xR[p], uJ, dG);
        P = mma32(qI[p], kJ, P);
        G = mma32(kI[p], kJ, G);
      }
      const float gu = gt[16 * J + c];
      f32x4 d1, d2;
      float cs = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ti = 16 * I + 4 * g + r, uj = 16 * J + c;
        const float m = I > J ? cross_decay(F + Cf::hGe, F + Cf::hFs, J, ti, uj)
                              : __builtin_amdgcn_exp2f(ti >= uj ? gI[r] - gu : -INFINITY);
        const float ms = ti > uj ? m : 0.f;
        d1[r] = dP[r] * m;
        d2[r] = -dG[r] * ms;
        const float e = d1[r] * P[r] + d2[r] * G[r];
        rs[r] += e;
        cs += e;
      }
      cs = col4_sum(cs);
      if (g == 0) F[Cf::hCP + 64 * w + 16 * J + c] = cs;
      st_acc<64>(mD1, 16 * I, 16 * J, g, c, d1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ti = 16 * I + 4 * g + r, uj = 16 * J + c;
        const __bf16 val = __builtin_bit_cast(__bf16, (unsigned short)(cvt2(d2[r], 0.f) & 0xffffu));
        if (J < I || ti > uj) {
          mM2[row_off<64>(ti, uj)] = val;
          mM2[row_off<64>(uj, ti)] = val;
        } else if (ti == uj) {
          mM2[row_off<64>(ti, uj)] = __builtin_bit_cast(__bf16, (unsigned short)0);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = row16_sum(rs[r]);
      if (c == 0) F[Cf::hRP + 16 * I + 4 * g + r] = v;
    }
  }
  __syncthreads();

  // ---- phase 3: key columns 32w .. 32w + 31, two 16-column blocks
  {
    const __bf16* const mD1 = M(Cf::rD1);
    const __bf16* const mM2 = M(Cf::rM2);
    const __bf16* const Sg = a.Sck + ck * D * D;
    const __bf16* const dSg = a.dSck + ck * D * D;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kw = 32 * w + 16 * kb;
      u32x4 kB[2], qB[2], sR[4], dsR[4];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        kB[p] = colp<D>(mK, 32 * p + 8 * g, kw, c);
        qB[p] = colp<D>(mQ, 32 * p + 8 * g, kw, c);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // rows kw + c of S and dS', value columns 32p + 8g .. + 7
        sR[p] = *reinterpret_cast<const u32x4*>(Sg + (size_t)(kw + c) * D + 32 * p + 8 * g);
        dsR[p] = *reinterpret_cast<const u32x4*>(dSg + (size_t)(kw + c) * D + 32 * p + 8 * g);
      }
      const __amdgpu_buffer_rsrc_t rdq =
          make_rsrc(a.dq + tokbase * D + kw, span_bytes((size_t)T * H * D * 4, ((size_t)h * D + kw) * 4));
      const __amdgpu_buffer_rsrc_t rdk =
          make_rsrc(a.dk + tokbase * D + kw, span_bytes((size_t)T * H * D * 4, ((size_t)h * D + kw) * 4));
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 q1 = zero4(), q2 = zero4(), k1 = zero4(), k3 = zero4(), k4 = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          q1 = mma32(rowp<64>(mD1, 16 * I + c, 32 * p + 8 * g), kB[p], q1);
          k1 = mma32(colp<64>(mD1, 32 * p + 8 * g, 16 * I, c), qB[p], k1);
          k1 = mma32(rowp<64>(mM2, 16 * I + c, 32 * p + 8 * g), kB[p], k1);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          q2 = mma32(rowp<D>(mO, 16 * I + c, 32 * p + 8 * g), sR[p], q2);
          k3 = mma32(rowp<D>(mU, 16 * I + c, 32 * p + 8 * g), dsR[p], k3);
          k4 = mma32(rowp<D>(mX, 16 * I + c, 32 * p + 8 * g), sR[p], k4);
        }
        const f32x4 gm = ld4f(F + Cf::hGam + 16 * I + 4 * g), lm = ld4f(F + Cf::hLam + 16 * I + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * I + 4 * g + j;
          const float dqv = q1[j] + gm[j] * q2[j];
          const float dkv = k1[j] + lm[j] * k3[j] - gm[j] * k4[j];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dqv), rdq, r * H * D * 4 + 4 * c,
                                                t0 * H * D * 4, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dkv), rdk, r * H * D * 4 + 4 * c,
                                                t0 * H * D * 4, 0);
        }
      }
    }
  }

  // ---- phase 4: dg, d ln alpha as suffix sums, dalpha
  __syncthreads();
  if (w == 0) {
    const int t = l;
    float dg = F[Cf::hDA + t] + F[Cf::hRP + t];
#pragma unroll
    for (int v = 0; v < 4; ++v) dg -= F[Cf::hCP + 64 * v + t];
    const float pre = wave_prefix_sum(dg);
    const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pre), 63));
    const float dla = tot - pre + dg;
    const uint32_t spanG = span_bytes((size_t)T * H * 4, (size_t)h * 4);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.alpha + tokbase, spanG);
    const float al = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, t * H * 4, t0 * H * 4, 0));
    const __amdgpu_buffer_rsrc_t rda = make_rsrc(a.dalpha + tokbase, spanG);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, dla / al), rda, t * H * 4, t0 * H * 4, 0);
  }
}

}  // namespace grad

// Workspace of the matrix-core gradient path: the forward's two-launch
// workspace (records, and the segment maps when it segments), then the Tb^T
// records, the chunk start states and the chunk end gradients (bf16, D x D);
// at D = 128 also U, dX and the value-side dg terms for the second half of the
// gradient pass.
struct GradLayout {
  size_t fwd, recT, sck, dsck, uw, xw, dga, total;
};

static GradLayout grad_layout(int B, int T, int H, int D) {
  ChunkArgs f{};
  f.B = B;
  f.T = T;
  f.H = H;
  f.dk = D;
  f.dv = D;
  f.dtype = kDtBF16;
  const size_t chains = (size_t)B * H, nch = (size_t)(T + 63) / 64, cn = chains * nch;
  GradLayout L;
  L.fwd = (chunk_two_workspace_bytes(f) + 255) & ~(size_t)255;
  L.recT = L.fwd;
  L.sck = L.recT + cn * pipe::kRecBytes;
  L.dsck = L.sck + cn * D * D * 2;
  L.uw = L.dsck + cn * D * D * 2;
  L.xw = L.uw + (D == 128 ? cn * 64 * D * 2 : 0);
  L.dga = L.xw + (D == 128 ? cn * 64 * D * 2 : 0);
  L.total = L.dga + (D == 128 ? cn * 64 * 4 : 0);
  return L;
}

size_t chunk_grad_workspace_bytes(int B, int T, int H, int D) { return T > 0 ? grad_layout(B, T, H, D).total : 0; }

namespace grad {
// T = 0: dS0 = dS_T (or zero).  One thread per element.
__global__ void copy_or_zero_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}
}  // namespace grad

hipError_t launch_chunk_grad(const BwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const int D = a.D;
  const long chains = (long)a.B * a.H;
  if (a.T == 0) {
    if (!a.dS0) return hipSuccess;
    const size_t n = (size_t)chains * D * D;
    return launch_kernel(grad::copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, a.dS_final,
                         a.dS0, n);
  }
  const GradLayout L = grad_layout(a.B, a.T, a.H, D);
  char* const ws = static_cast<char*>(a.workspace);
  const int nch = (a.T + 63) / 64;
  ChunkArgs f{};
  f.q = a.q;
  f.k = a.k;
  f.v = a.v;
  f.alpha = a.alpha;
  f.beta = a.beta;
  f.S0 = a.S0;
  f.out = nullptr;
  f.S_final = nullptr;
  f.B = a.B;
  f.T = a.T;
  f.H = a.H;
  f.dk = D;
  f.dv = D;
  f.dtype = kDtBF16;
  f.stream = a.stream;
  hipError_t e = launch_chunk_two_states(f, ws, ws + L.recT, ws + L.sck);
  if (e != hipSuccess) return e;
  grad::AdjArgs j{};
  j.q = static_cast<const __bf16*>(a.q);
  j.k = static_cast<const __bf16*>(a.k);
  j.dO = static_cast<const __bf16*>(a.dout);
  j.recT = ws + L.recT;
  j.dSf = a.dS_final;
  j.dSck = reinterpret_cast<__bf16*>(ws + L.dsck);
  j.dS0 = a.dS0;
  j.T = a.T;
  j.H = a.H;
  j.DV = D;
  j.nch = nch;
  if (D == 64) {
    using ACf = grad::AdjCfg<64, 2>;
    e = launch_kernel(grad::adj_kernel<64, 2>, dim3((unsigned)(chains * (D / ACf::NV))), dim3(ACf::kThreads), st, j);
  } else {
    using ACf = grad::AdjCfg<128, 1>;
    e = launch_kernel(grad::adj_kernel<128, 1>, dim3((unsigned)(chains * (D / ACf::NV))), dim3(ACf::kThreads), st, j);
  }
  if (e != hipSuccess) return e;
  grad::GradArgs gr{};
  gr.q = static_cast<const __bf16*>(a.q);
  gr.k = static_cast<const __bf16*>(a.k);
  gr.v = static_cast<const __bf16*>(a.v);
  gr.dO = static_cast<const __bf16*>(a.dout);
  gr.alpha = a.alpha;
  gr.beta = a.beta;
  gr.rec = ws;
  gr.recT = ws + L.recT;
  gr.Sck = reinterpret_cast<const __bf16*>(ws + L.sck);
  gr.dSck = reinterpret_cast<const __bf16*>(ws + L.dsck);
  gr.dq = a.dq;
  gr.dk = a.dk;
  gr.dv = a.dv;
  gr.dalpha = a.dalpha;
  gr.dbeta = a.dbeta;
  gr.T = a.T;
  gr.H = a.H;
  gr.nch = nch;
  const dim3 grid((unsigned)(chains * nch));
  if (D == 64) return launch_kernel(grad::grad_kernel, grid, dim3(256), st, gr);
  gr.Uw = reinterpret_cast<__bf16*>(ws + L.uw);
  gr.Xw = reinterpret_cast<__bf16*>(ws + L.xw);
  gr.dgA = reinterpret_cast<float*>(ws + L.dga);
  e = launch_kernel(grad::grad_cols_kernel, grid, dim3(512), st, gr);
  if (e != hipSuccess) return e;
  return launch_kernel(grad::grad_rows_kernel, grid, dim3(256), st, gr);
}

}  // namespace gdn
