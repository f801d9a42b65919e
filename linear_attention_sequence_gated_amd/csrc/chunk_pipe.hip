// chunk_pipe.hip -- warp-specialised, software-pipelined chunkwise gated
// delta-rule forward for bf16 inputs on gfx950.
//
// Same method as the fused kernel (chunkwise WY / UT transform of the gated
// delta rule: Sykra 0.3.3 README, "Architectural Highlights"; DeltaPhase README,
// section 1 "Fast Triangular Solve" and section 5 "Exact Chunkwise-Parallel
// Scan"), organised so that the three limited resources of a CU -- LDS
// bandwidth, vector-ALU issue (a wave64 instruction occupies its SIMD for four
// cycles) and matrix-core issue -- are spread over the four SIMDs.
//
// The three-stage kernel below (namespace pipe3) runs bf16 at d = 64 with
// enough chains to fill the CUs, and the fused input prologue.  Namespace pipe
// holds its configuration, the consumer waves' state and the decayed-tile and
// output helpers.
//
// With S the state at the chunk start, g the within-chunk prefix sum of
// log alpha, gamma_r = exp(g_r), lambda_r = exp(g_C - g_r), Gamma_rs =
// exp(g_r - g_s) (r >= s), Gt = strict_lower(K K^T * Gamma) and T_ii =
// (I + diag(beta_i) Gt_ii)^{-1}, block row i of
// Ut = (I + A)^{-1} (diag(beta) V - diag(beta gamma) K S) is
//     Ut_i = T_ii diag(beta_i) (V_i - gamma_i * (K S)_i - sum_{j<i} Gt_ij Ut_j),
// so beta only enters through the producer-built factors T_ii diag(beta_i);
//     O  = gamma * (Q S) + lower(Q K^T * Gamma) Ut,
//     S <- gamma_C S + K^T (lambda * Ut).
// Diagonal blocks are inverted by row-owner forward substitution (each
// finished row broadcast along the 16-lane rows with DPP row_newbcast).
//
// Global traffic uses buffer loads/stores whose range check implements the
// ragged tail (rows >= T read as zero and are never written).  Decay factors
// are exp(g_r - g_s) with r >= s only (masked before the exponential), so no
// factor above one is ever formed.  Packed bf16 values are handled as 32-bit
// words throughout (two values per word), which keeps every conversion a
// paired v_cvt_pk_bf16_f32.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "gdn_pipe.hpp"

namespace gdn {
namespace pipe {

template <int DK> struct Cfg {
  // Value columns per workgroup: 32 at d = 64 (two consumer waves).
  static constexpr int NV = DK == 64 ? 32 : 16;
  static constexpr int NT = 1;               // 16-column tiles per consumer wave
  static constexpr int NCONS = NV / 16;      // consumer waves
  static constexpr int NVU = NV / 8;         // 16-byte units per V row
  static constexpr int kThreads = (NCONS + 5) * 64;  // consumers, 4 Gram waves, the V wave
  static constexpr int NDT = DK / 16, NKP = DK / 32;
  static constexpr int LDK = DK + 8, LDV = NV + 8, LD16 = 16 + 8;
  // bf16 element offsets inside one of the two stage buffers
  static constexpr int szTile = 16 * LD16;
  static constexpr int oK = 0, oQ = 64 * LDK, oV = 2 * 64 * LDK;
  static constexpr int oNG = oV + 64 * LDV;     // -Gt, the six sub-diagonal tiles
  static constexpr int oTP = oNG + 6 * szTile;  // T_ii diag(beta_i), four tiles
  static constexpr int oP = oTP + 4 * szTile;   // P, ten lower tiles
  static constexpr int szBuf = oP + 10 * szTile;
  static constexpr int fBase = ((2 * szBuf * 2 + 15) / 16) * 16;  // byte offset of the fp32 region
  // fp32 region (floats): per stage buffer gamma[64], lambda[64], gamma_C;
  // then one private gate table (g, beta per token) and one 16 x 20 block
  // scratch per Gram wave.
  static constexpr int szGate = 132, fGate = 0;
  static constexpr int fPGT = 2 * szGate, szPGT = 128;
  static constexpr int fDS = fPGT + 4 * szPGT, szDS = 16 * 20;
  static constexpr int nF = fDS + 4 * szDS;
  static constexpr int bytes = fBase + nF * 4;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

struct Ctx {
  const __bf16* qg;
  const __bf16* kg;
  const __bf16* vg;
  const float* alpha;
  const float* beta;
  const float* S0g;
  __bf16* outg;
  float* Sfg;
  int T, H, DV, b, h, chain, dv0, nchunks;
  float beta_scale;  // fused-prologue kernel only: beta = beta_scale * sigmoid(b)
};

// ---------------------------------------------------------------- producers
// Decay factors of diagonal block i: lane (g, c) gets Gamma[r][s] for r = 16i + c,
// s = 16i + 4g + j, masked to 0 for s > r before the exponential.
__device__ __forceinline__ f32x4 diag_gamma(const float* PGT, int i, int g, int c) {
  const float gr = PGT[16 * i + c];
  const f32x4 gs = *reinterpret_cast<const f32x4*>(PGT + 16 * i + 4 * g);
  f32x4 gm;
#pragma unroll
  for (int j = 0; j < 4; ++j) gm[j] = __builtin_amdgcn_exp2f(c >= 4 * g + j ? gr - gs[j] : -INFINITY);
  return gm;
}

// Decayed Gram tile (row block i, column block j < i, so every r > s):
// -Gt from the K K^T accumulator and P from the Q K^T accumulator.
template <int DK>
__device__ __forceinline__ void offdiag_tiles(const f32x4& G, const f32x4& P, const float* PGT, int i, int j, int g,
                                              int c, __bf16* R) {
  using Cf = Cfg<DK>;
  const float gr = PGT[16 * i + c];
  const f32x4 gs = *reinterpret_cast<const f32x4*>(PGT + 16 * j + 4 * g);
  f32x4 ng, pv;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float gm = __builtin_amdgcn_exp2f(gr - gs[jj]);
    ng[jj] = -gm * G[jj];
    pv[jj] = gm * P[jj];
  }
  *reinterpret_cast<u32x2*>(R + Cf::oNG + stri(i, j) * Cf::szTile + c * Cf::LD16 + 4 * g) = cvt4(ng);
  *reinterpret_cast<u32x2*>(R + Cf::oP + tri(i, j) * Cf::szTile + c * Cf::LD16 + 4 * g) = cvt4(pv);
}

// Decayed diagonal tile of P (gm from diag_gamma, zero above the diagonal).
template <int DK>
__device__ __forceinline__ void diag_p_tile(const f32x4& P, const f32x4& gm, int i, int g, int c, __bf16* R) {
  using Cf = Cfg<DK>;
  const f32x4 pv{gm[0] * P[0], gm[1] * P[1], gm[2] * P[2], gm[3] * P[3]};
  *reinterpret_cast<u32x2*>(R + Cf::oP + tri(i, i) * Cf::szTile + c * Cf::LD16 + 4 * g) = cvt4(pv);
}

// ---------------------------------------------------------------- output
// The output is computed transposed, so that each lane holds four consecutive
// value columns of one token:
//   O_i^T = (S^T Q_i^T) diag(gamma_i) + sum_{j <= i} Ut_j^T P_ij^T.
// For one 16-column tile, lane (g, c) gets token 16 i + c, columns 4g .. 4g + 3.
// First term: s = the state's bf16 operands for the tile (2 NKP sub-blocks, in
// key_row order), qr = keys 32p + 8g .. + 7 of Q row 16i + c, gm = gamma of
// the lane's token.
template <int NKP>
__device__ __forceinline__ f32x4 out_qs(const u32x2* s, const u32x4 (&qr)[NKP], float gm) {
  f32x4 o = zero4();
#pragma unroll
  for (int p = 0; p < NKP; ++p) o = mma32(pair(s[2 * p], s[2 * p + 1]), qr[p], o);
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] *= gm;
  return o;
}

// Second term, added to o: X[j][t] = Ut_j for the tile, Pm the ten lower P tiles.
template <int NTT>
__device__ __forceinline__ f32x4 out_pu(f32x4 o, int i, int t, const u32x2 (&X)[4][NTT], const u32x2 (&Pm)[10]) {
  if (i == 0) o = mma1(X[0][t], Pm[tri(0, 0)], o);
  if (i == 1) o = mma2(X[0][t], X[1][t], Pm[tri(1, 0)], Pm[tri(1, 1)], o);
  if (i == 2) {
    o = mma2(X[0][t], X[1][t], Pm[tri(2, 0)], Pm[tri(2, 1)], o);
    o = mma2(X[2][t], z4(), Pm[tri(2, 2)], z4(), o);
  }
  if (i == 3) {
    o = mma2(X[0][t], X[1][t], Pm[tri(3, 0)], Pm[tri(3, 1)], o);
    o = mma2(X[2][t], X[3][t], Pm[tri(3, 2)], Pm[tri(3, 3)], o);
  }
  return o;
}

// ---------------------------------------------------------------- consumers

// A consumer wave owns value columns 16 NT w .. 16 NT (w + 1) - 1 of the
// workgroup's slice, as NT 16-column tiles t.  The state lives in MFMA
// accumulators: S[t][d] holds rows key_row(d, g, j) of column 16t + c.
template <int DK>
struct Consumer {
  using Cf = Cfg<DK>;
  static constexpr int NDT = Cf::NDT, NKP = Cf::NKP, LDK = Cf::LDK, LDV = Cf::LDV, LD16 = Cf::LD16, NT = Cf::NT;
  f32x4 S[NT][NDT];
  int g, c, w, rowO, vofO, offRow, offTrK, offTrV, offT16;
  __amdgpu_buffer_rsrc_t ro;
  // Carried from begin() to chunk(): the state and K S of the chunk's start
  // state, and the chunk's V and decay operands.
  u32x2 sfr[NT][NDT], vv[4][NT];
  f32x4 acc[4][NT], gg[4];

  __device__ __forceinline__ void init(const Ctx& x, int w_, int l) {
    w = w_;
    g = l >> 4;
    c = l & 15;
    const int H = x.H, T = x.T, DV = x.DV;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = x.dv0 + 16 * NT * w + 16 * t + c;
#pragma unroll
      for (int d = 0; d < NDT; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          S[t][d][j] = x.S0g ? x.S0g[((size_t)x.chain * DK + key_row(d, g, j)) * DV + col] : 0.f;
    }
    // Output: lane (g, c) writes token c of each 16-token block, value columns
    // 16 NT w + 16t + 4g .. + 3 (one 8-byte store).
    const size_t obase = ((size_t)x.b * T * H + x.h) * DV + x.dv0;
    ro = make_rsrc(x.outg + obase, span_bytes((size_t)T * H * DV * 2, ((size_t)x.h * DV + x.dv0) * 2));
    rowO = H * DV * 2;
    vofO = c * rowO + (16 * NT * w + 4 * g) * 2;
    offRow = c * LDK + 8 * g;                                       // row c, keys 8g .. 8g + 7
    offTrK = (4 * g + (c >> 2)) * LDK + 8 * (c & 3);                // transposed K reads (key_row order)
    offTrV = (4 * g + (c >> 2)) * LDV + 16 * NT * w + 4 * (c & 3);  // transposed V reads
    offT16 = c * LD16 + 4 * g;                                      // 16x16 tiles
  }

  // First half of a chunk, which needs only operands published a step earlier:
  // V and gamma from stage buffer R / gate table G, and K S for the current
  // state.  With `pub` set, lane l also writes the state's bf16 operands
  // sfr[t][d] to pub[2 ((t NDT + d) 64 + l)] for a wave that forms the output.
  __device__ __forceinline__ void begin(const __bf16* R, const float* G, unsigned* pub = nullptr) {
    u32x4 kr[4][NKP];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int p = 0; p < NKP; ++p) kr[i][p] = *reinterpret_cast<const u32x4*>(R + Cf::oK + 16 * i * LDK + 32 * p + offRow);
#pragma unroll
      for (int t = 0; t < NT; ++t) vv[i][t] = ld4_tr(R + Cf::oV + 16 * i * LDV + 16 * t + offTrV);
      gg[i] = *reinterpret_cast<const f32x4*>(G + 16 * i + 4 * g);
    }
    issue_fence();
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        sfr[t][d] = cvt4(S[t][d]);
        if (pub) *reinterpret_cast<u32x2*>(pub + 2 * ((t * NDT + d) * 64 + 16 * g + c)) = sfr[t][d];
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[i][t] = zero4();
#pragma unroll
        for (int p = 0; p < NKP; ++p)
          acc[i][t] = mma32(kr[i][p], pair(sfr[t][2 * p], sfr[t][2 * p + 1]), acc[i][t]);
      }
  }

  // Operands of the state update, loaded with the diagonal factors so that
  // they are in flight during the substitution.
  struct Upd {
    u32x2 kt[NDT][4];
    f32x4 lm[4];
    float gC;
  };
  // Ut = (I + A)^{-1} (diag(beta) V - diag(beta gamma) K S) of the chunk in
  // stage buffer R, block rows in order (after begin() on the same buffer):
  // Xf = Ut and XL = lambda * Ut as bf16 operands.  G holds gamma (G[0..63])
  // and lambda (G[64..127]) per token and gamma_C at G[gCoff].  With `pub`
  // set, lane l also writes Xf[i][t] to pub[2 ((i NT + t) 64 + l)] for a wave
  // that forms the output.
  __device__ __forceinline__ void solve(const __bf16* R, const float* G, int gCoff, Upd& u, u32x2 (&Xf)[4][NT],
                                        u32x2 (&XL)[4][NT], unsigned* pub) {
    auto tile = [&](int o) { return ld4(R + o + offT16); };
    u32x2 TP[4], NG[6];
#pragma unroll
    for (int i = 0; i < 4; ++i) TP[i] = tile(Cf::oTP + i * Cf::szTile);
#pragma unroll
    for (int e = 0; e < 6; ++e) NG[e] = tile(Cf::oNG + e * Cf::szTile);
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) u.kt[d][i] = ld4_tr(R + Cf::oK + 16 * i * LDK + 32 * (d / 2) + 4 * (d % 2) + offTrK);
#pragma unroll
    for (int i = 0; i < 4; ++i) u.lm[i] = *reinterpret_cast<const f32x4*>(G + 64 + 16 * i + 4 * g);
    u.gC = G[gCoff];
    issue_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 y;
        const u32x2 v = vv[i][t];
        y[0] = lo_f(v[0]) - gg[i][0] * acc[i][t][0];
        y[1] = hi_f(v[0]) - gg[i][1] * acc[i][t][1];
        y[2] = lo_f(v[1]) - gg[i][2] * acc[i][t][2];
        y[3] = hi_f(v[1]) - gg[i][3] * acc[i][t][3];
        // y -= sum_{j < i} Gt_ij Ut_j   (the tiles hold -Gt)
        if (i == 1) y = mma1(NG[stri(1, 0)], Xf[0][t], y);
        if (i == 2) y = mma2(NG[stri(2, 0)], NG[stri(2, 1)], Xf[0][t], Xf[1][t], y);
        if (i == 3) {
          y = mma2(NG[stri(3, 0)], NG[stri(3, 1)], Xf[0][t], Xf[1][t], y);
          y = mma2(NG[stri(3, 2)], z4(), Xf[2][t], z4(), y);
        }
        const f32x4 X = mma1(TP[i], cvt4(y), zero4());
        Xf[i][t] = cvt4(X);
        if (pub) *reinterpret_cast<u32x2*>(pub + 2 * ((i * NT + t) * 64 + 16 * g + c)) = Xf[i][t];
        f32x4 xl;
#pragma unroll
        for (int j = 0; j < 4; ++j) xl[j] = X[j] * u.lm[i][j];
        XL[i][t] = cvt4(xl);
      }
  }

  // S <- gamma_C S + K^T (lambda * Ut)
  __device__ __forceinline__ void update(const Upd& u, const u32x2 (&XL)[4][NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        f32x4 sd = S[t][d];
#pragma unroll
        for (int j = 0; j < 4; ++j) sd[j] *= u.gC;
        sd = mma2(u.kt[d][0], u.kt[d][1], XL[0][t], XL[1][t], sd);
        sd = mma2(u.kt[d][2], u.kt[d][3], XL[2][t], XL[3][t], sd);
        S[t][d] = sd;
      }
  }

  __device__ __forceinline__ void finish(const Ctx& x) {
    if (!x.Sfg) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = x.dv0 + 16 * NT * w + 16 * t + c;
#pragma unroll
      for (int d = 0; d < NDT; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) x.Sfg[((size_t)x.chain * DK + key_row(d, g, j)) * x.DV + col] = S[t][d][j];
    }
  }
};

}  // namespace pipe

// ============================================================================
// Three-stage variant (dk = 64).  Per step k of the loop (one barrier each):
//   Gram waves 2, 3 and wave 5 build chunk k + 2 (K/Q rows, V tile, decayed
//   Gram tiles of row blocks 0..1 / 2..3 on and next to the diagonal, and the
//   fp32 rows of the four diagonal blocks of A); waves 3 and 2 also write
//   chunk k + 3's gate table from alpha and beta (one each);
//   Gram waves 4, 5 add chunk k + 1's remaining tiles from the published rows;
//   the inverse wave 7 turns chunk k + 1's diagonal blocks into T_ii diag(beta_i);
//   the consumer waves 0, 1 run chunk k (the substitution and the state
//   update) and hand Ut and their start-of-chunk state to the output wave 6,
//   which forms chunk k's Q S term and chunk k - 1's P Ut term and output.
// Stage buffers rotate over three slots (chunk m uses slot m % 3); the
// diagonal-block rows and the hand-off buffers over two (m & 1).  Taking the
// inverses and the output off the chain waves shortens their steps, and the
// inverse wave does all four blocks at once in a row-per-lane layout that
// skips the zero upper triangle (120 fused DPP FMAs per chunk instead of 240).
namespace pipe3 {
using namespace pipe;

struct Cfg3 {
  using B = Cfg<64>;
  static constexpr int NBUF = 3;
  static constexpr int fBase = ((NBUF * B::szBuf * 2 + 15) / 16) * 16;  // byte offset of the fp32 region
  // fp32 region (floats): a ring of NGATE gate tables (chunk m uses table
  // m % NGATE), each gamma[64], lambda[64], g[64] (log2 prefix of alpha),
  // beta[64], gamma_C (padded), and for the fused prologue gamma / |k|,
  // lambda / |k| and 1 / |k| per token [64 each]; two
  // slots of diagonal-block rows (4 blocks x 16 rows, row stride 20); the
  // 16 x 16 identity (row stride 20).
  // Then, as 32-bit words, two slots (by chunk parity) of the consumers' Ut
  // and two of their start-of-chunk states, both as bf16 MFMA operands in
  // lane order (4 operands of 64 lanes x 2 words per consumer wave), for the
  // wave that forms the output.
  // Gate tables are written one step before the K/Q rows of their chunk, so
  // the ring is one deeper than the stage slots.
  static constexpr int NGATE = 4;
  static constexpr int fGate = 0, oLam = 64, oG = 128, oBeta = 192, oGC = 256;
  static constexpr int oGk = 260, oLk = 324, oIk = 388, szGate = 452;
  static constexpr int szDS = 4 * 16 * 20, fDS = NGATE * szGate;
  static constexpr int fEye = fDS + 2 * szDS;
  static constexpr int szHand = 4 * 64 * 2, szHand2 = 2 * szHand;  // one consumer / both consumers
  static constexpr int fXU = fEye + 16 * 20, fXS = fXU + 2 * szHand2;
  static constexpr int nF = fXS + 2 * szHand2;
  static constexpr int bytes = fBase + nF * 4;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(oBeta == oG + 64, "g and beta adjacent: the Gram code reads them as one table");
  static_assert((oGk * 4) % 16 == 0 && (oLk * 4) % 16 == 0 && (oIk * 4) % 16 == 0,
                "per-token tables are read as 16-byte vectors");
  static_assert((szGate * 4) % 16 == 0 && (fDS * 4) % 16 == 0 && (fEye * 4) % 16 == 0 &&
                    (fXU * 4) % 16 == 0,
                "fp32 tables must be 16-byte aligned");
  static_assert(B::NT == 1 && B::NDT == 4, "one 16-column tile and four 16-row blocks per consumer wave");
};
constexpr int kThreads3 = 8 * 64;

// Gate table of chunk m.
__device__ __forceinline__ float* gate_table(char* smem, int m) {
  return reinterpret_cast<float*>(smem + Cfg3::fBase) + Cfg3::fGate + (m & (Cfg3::NGATE - 1)) * Cfg3::szGate;
}
__device__ __forceinline__ const float* gate_table(const char* smem, int m) {
  return reinterpret_cast<const float*>(smem + Cfg3::fBase) + Cfg3::fGate + (m & (Cfg3::NGATE - 1)) * Cfg3::szGate;
}

// Runs one barrier (after the gate table of chunk 0 is written), then
// step(phase, k) for k = -2, -1, ..., each followed by the barrier, with
// phase = (k + 2) % 3 known at compile time: chunk k + 2 (built in this step)
// uses stage slot and register set `phase`, chunk k + 1 slot (phase + 2) % 3
// and chunk k slot (phase + 1) % 3.  Steps come in whole triples (up to two
// trailing steps have nothing to do: every role skips chunks outside
// [0, nch)), so every wave executes the same barriers and the loop body has no
// conditional paths that would make the compiler's wait counts conservative.
template <class Step>
__device__ __forceinline__ void run_steps(int nch, Step&& step) {
  // T >= 0 (checked on the host), so the first triple always runs.  Without
  // this the loop gets an entry test, and the prologue's loads are sunk past it
  // and regrouped by address; the loop's static wait counts must also hold on
  // entry from the prologue, so every later iteration would then wait for
  // loads issued one step earlier instead of three.
  __builtin_assume(nch >= 0);
  stage_barrier();  // the gate table of chunk 0 is written before the loop
  for (int k = -2; k < nch; k += 3) {
    step(ic<0>{}, k);
    stage_barrier();
    step(ic<1>{}, k + 1);
    stage_barrier();
    step(ic<2>{}, k + 2);
    stage_barrier();
  }
}

// The output of chunk n is finished in step n + 1.  run_steps ends with step
// 3 ceil((nch + 2) / 3) - 3, which is nch - 1 when nch = 1 (mod 3); then
// every wave runs one more barrier and the output wave finishes the last
// chunk after it.
__device__ __forceinline__ bool needs_tail_step(int nch) { return 3 * ((nch + 4) / 3) - 3 < nch; }

// Fp32 rows of -A for a diagonal block: lane (g, c) writes -A[c][4g .. 4g + 3].
__device__ __forceinline__ void diag_rows(const f32x4& G, const f32x4& gm, const float* PGT, int i, int g, int c,
                                          float* dst) {
  const float br = PGT[64 + 16 * i + c];
  f32x4 na;
#pragma unroll
  for (int j = 0; j < 4; ++j) na[j] = c > 4 * g + j ? -br * gm[j] * G[j] : 0.f;
  *reinterpret_cast<f32x4*>(dst + c * 20 + 4 * g) = na;
}

// Loads are issued unconditionally (chunk index clamped; buffer loads are
// range-checked) so that every path through the loop has the same number of
// loads in flight and the compiler's wait counts stay three steps deep.  The
// clamped index is kept scalar.
__device__ __forceinline__ int clamp_chunk(int m, int nch) {
  return __builtin_amdgcn_readfirstlane(max(0, min(m, nch - 1)));
}

// The 64 x 32 V tile of chunk k + 2 in step k, from registers loaded three
// steps ahead.
struct VStage {
  using Cf = Cfg<64>;
  __amdgpu_buffer_rsrc_t rv;
  int rowV, nch, vof[4], lof[4];
  u32x4 st[3][4];

  __device__ __forceinline__ void init(const Ctx& x, int l) {
    nch = x.nchunks;
    const size_t tokbase = (size_t)x.b * x.T * x.H + x.h;
    rv = make_rsrc(x.vg + tokbase * x.DV + x.dv0,
                   span_bytes((size_t)x.T * x.H * x.DV * 2, ((size_t)x.h * x.DV + x.dv0) * 2));
    rowV = x.H * x.DV * 2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int unit = l + 64 * u, row = unit / 4, cu = unit % 4;
      vof[u] = row * rowV + cu * 16;
      lof[u] = row * Cf::LDV + cu * 8;
    }
  }
  template <int s> __device__ __forceinline__ void load(int m) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      st[s][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vof[u], m * 64 * rowV, 0));
  }
  __device__ __forceinline__ void prologue(char*) {
    load<0>(clamp_chunk(0, nch));
    issue_fence();
    load<1>(clamp_chunk(1, nch));
    issue_fence();
    load<2>(clamp_chunk(2, nch));
    issue_fence();
  }
  template <int ph> __device__ __forceinline__ void step(char* smem, int k) {
    if (k + 2 < nch) {
      __bf16* const R = reinterpret_cast<__bf16*>(smem) + ph * Cf::szBuf;  // slot (k + 2) % 3
#pragma unroll
      for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(R + Cf::oV + lof[u]) = st[ph][u];
    }
    issue_fence();
    load<ph>(clamp_chunk(k + 5, nch));  // the set just consumed; needed three steps later
  }
};

// The gate table of chunk k + 3 in step k, from alpha or beta loaded three
// steps ahead; chunk 0's before the loop.  With kAlpha the wave writes gamma,
// lambda, g and gamma_C; with kBeta it writes beta.  The two halves run on
// different waves: each strided 4-byte load touches 24 cache lines for 256
// bytes, which costs a loading wave several hundred cycles per step when the
// inputs come from HBM.
template <bool kAlpha, bool kBeta, bool kPro>
struct GateStage {
  __amdgpu_buffer_rsrc_t rs;
  int H, T, nch, l;
  float sv[3], bscale;

  __device__ __forceinline__ void init(const Ctx& x, int l_) {
    l = l_;
    H = x.H;
    T = x.T;
    nch = x.nchunks;
    bscale = x.beta_scale;
    const size_t tokbase = (size_t)x.b * T * H + x.h;
    rs = make_rsrc((kAlpha ? x.alpha : x.beta) + tokbase, span_bytes((size_t)T * H * 4, (size_t)x.h * 4));
  }
  template <int s> __device__ __forceinline__ void load(int m) {
    sv[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, l * H * 4, m * 64 * H * 4, 0));
  }
  // Gate table of chunk m from register set s (= m % 3).  g is the inclusive
  // prefix of log2 alpha (alpha = 1 on padding tokens; beta reads as 0 there).
  // With kPro the loads are logits: log2 alpha = -softplus(a) / ln 2 and
  // beta = bscale * sigmoid(b), both on padding tokens replaced as above.
  template <int s> __device__ __forceinline__ void gates(char* smem, int m) {
    float* const G = gate_table(smem, m);
    const bool live = m * 64 + l < T;
    if constexpr (kAlpha) {
      float la;
      if constexpr (kPro) {
        // softplus(a) / ln 2 = max(a, 0) log2(e) + log2(1 + 2^(-|a| log2(e)))
        const float u = sv[s] * 1.4426950408889634f;
        la = live ? -(fmaxf(u, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(u)))) : 0.f;
      } else {
        la = __builtin_amdgcn_logf(live ? sv[s] : 1.f);
      }
      const float xg = wave_prefix_sum(la);
      const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xg), 63));
      G[l] = __builtin_amdgcn_exp2f(xg);
      G[Cfg3::oLam + l] = __builtin_amdgcn_exp2f(gC - xg);
      G[Cfg3::oG + l] = xg;
      if (l == 63) G[Cfg3::oGC] = __builtin_amdgcn_exp2f(gC);
    }
    if constexpr (kBeta) {
      if constexpr (kPro)
        G[Cfg3::oBeta + l] = live ? bscale * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-sv[s] * 1.4426950408889634f)) : 0.f;
      else
        G[Cfg3::oBeta + l] = sv[s];
    }
  }
  // Sets hold chunks 0, 1, 2; chunk 0's table is written and set 0 refilled
  // with chunk 3, so step k finds chunk k + 3 in set (k + 3) % 3.
  __device__ __forceinline__ void prologue(char* smem) {
    load<0>(clamp_chunk(0, nch));
    issue_fence();
    load<1>(clamp_chunk(1, nch));
    issue_fence();
    load<2>(clamp_chunk(2, nch));
    issue_fence();
    if (nch > 0) gates<0>(smem, 0);
    issue_fence();
    load<0>(clamp_chunk(3, nch));
    issue_fence();
  }
  template <int ph> __device__ __forceinline__ void step(char* smem, int k) {
    constexpr int s = (ph + 1) % 3;  // (k + 3) % 3
    if (k + 3 < nch) gates<s>(smem, k + 3);
    issue_fence();
    load<s>(clamp_chunk(k + 6, nch));  // the set just consumed; needed three steps later
  }
};

// No extra work.
struct NoStage {
  __device__ __forceinline__ void init(const Ctx&, int) {}
  __device__ __forceinline__ void prologue(char*) {}
  template <int ph> __device__ __forceinline__ void step(char*, int) {}
};

// 1 / max(|x|, 1e-12) from |x|^2, as the layer's L2 normalisation divides.
__device__ __forceinline__ float inv_norm(float sq) { return __builtin_amdgcn_rsqf(fmaxf(sq, 1e-24f)); }

// Element c & 3 of v (lane (g, c) with g = c / 4 holds diagonal entry c of a
// 16 x 16 accumulator tile there).
__device__ __forceinline__ float diag_pick(const f32x4& v, int c) {
  const int j = c & 3;
  return j == 0 ? v[0] : j == 1 ? v[1] : j == 2 ? v[2] : v[3];
}

// x of lane `src` (0..63), through the cross-lane permute.
__device__ __forceinline__ float lane_read(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, x)));
}

// Orders this wave's LDS writes before its later LDS reads in every lane.
// Without it, lanes of one wave that exchange values through LDS may have a
// read placed before another lane's write: the compiler sees each lane as a
// thread of its own, and with a divergent write it splits the code into an
// if / else whose else side (the reads) can run first.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Waves 2 and 3: row blocks b0 and b0 + 1 (b0 = 0 or 2).  They also write the
// gate tables (Extra = GateStage): wave 2 beta, wave 3 the rest.  With kPro
// (fused prologue: raw q and k) they also find 1/|k_r| of their 32 rows from
// the diagonal of the K K^T tiles they form anyway, scale their K K^T tiles
// by it on both sides and their P tiles on the key side, and write it and
// gamma / |k|, lambda / |k| to the chunk's gate table.  (The output wave
// applies 1/|q|.)  Normalising the rows themselves would cost every row wave
// about a thousand cycles of vector work per step.
template <class Extra, bool kPro>
__device__ __forceinline__ void gram_rows(const Ctx& x, char* smem, int b0, int l) {
  using Cf = Cfg<64>;
  constexpr int NKP = Cf::NKP, LDK = Cf::LDK;
  __bf16* const sb = reinterpret_cast<__bf16*>(smem);
  float* const sf = reinterpret_cast<float*>(smem + Cfg3::fBase);
  const int g = l >> 4, c = l & 15, H = x.H, T = x.T, nch = x.nchunks;
  const size_t tokbase = (size_t)x.b * T * H + x.h;
  const uint32_t spanK = span_bytes((size_t)T * H * 64 * 2, (size_t)x.h * 64 * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(x.qg + tokbase * 64, spanK);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(x.kg + tokbase * 64, spanK);
  const int rowK = H * 64 * 2;
  // Loads read whole 128-byte rows: load (e, p) gives lane l 16 bytes of row
  // 16 (b0 + e) + 8 p + l / 8.  Per-CU load throughput scales with the number
  // of cache lines an instruction touches, and MFMA operand order (16 rows of
  // 64 bytes per instruction) would touch twice as many.  The rows go to LDS
  // row-major, and the operands are read back from there.
  int vofs[2][NKP], lofs[2][NKP];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int p = 0; p < NKP; ++p) {
      const int row = 16 * (b0 + e) + 8 * p + (l >> 3);
      vofs[e][p] = row * rowK + 16 * (l & 7);
      lofs[e][p] = row * LDK + 8 * (l & 7);
    }
  static_assert(NKP == 2, "two 8-row loads per 16-row block");
  struct Set {
    u32x4 k[2][NKP], q[2][NKP];
  };
  Set st[3];
  auto load = [&](auto sc, int m) {
    constexpr int s = decltype(sc)::value;
    const int c0 = m * 64;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        st[s].k[e][p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, vofs[e][p], c0 * rowK, 0));
        st[s].q[e][p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, vofs[e][p], c0 * rowK, 0));
      }
  };
  auto process = [&](auto sc, int m) {
    constexpr int s = decltype(sc)::value;
    const Set& S = st[s];
    __bf16* const R = sb + s * Cf::szBuf;  // slot m % 3 == s
    float* const D = sf + Cfg3::fDS + (m & 1) * Cfg3::szDS;
    const float* const PGT = gate_table(smem, m) + Cfg3::oG;  // g[64], then beta[64]
    // K and Q rows for this wave, the lower Gram waves and the consumers
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        *reinterpret_cast<u32x4*>(R + Cf::oK + lofs[e][p]) = S.k[e][p];
        *reinterpret_cast<u32x4*>(R + Cf::oQ + lofs[e][p]) = S.q[e][p];
      }
    // The operands below come from rows other lanes of this wave just wrote.
    wave_sync();
    u32x4 kk[2][NKP], qq[2][NKP];  // MFMA operands: lane (g, c) holds row c, k = 32 p + 8 g .. + 7
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        const int o = (16 * (b0 + e) + c) * LDK + 32 * p + 8 * g;
        kk[e][p] = *reinterpret_cast<const u32x4*>(R + Cf::oK + o);
        qq[e][p] = *reinterpret_cast<const u32x4*>(R + Cf::oQ + o);
      }
    f32x4 G0 = zero4(), P0 = zero4(), Go = zero4(), Po = zero4(), G1 = zero4(), P1 = zero4();
#pragma unroll
    for (int p = 0; p < NKP; ++p) {
      G0 = mma32(kk[0][p], kk[0][p], G0);
      P0 = mma32(kk[0][p], qq[0][p], P0);
      Go = mma32(kk[0][p], kk[1][p], Go);
      Po = mma32(kk[0][p], qq[1][p], Po);
      G1 = mma32(kk[1][p], kk[1][p], G1);
      P1 = mma32(kk[1][p], qq[1][p], P1);
    }
    if constexpr (kPro) {
      // Lane (g, c) holds [s = 16b + 4g + j][r = 16b' + c] of each tile, and
      // lane (c / 4, c) the diagonal entry of row c.  The diagonal lanes write
      // 1/|k| to the table; every lane then reads row c's and rows 4g .. 4g + 3's.
      float* const Gt = gate_table(smem, m);
      if (g == (c >> 2)) {
        Gt[Cfg3::oIk + 16 * b0 + c] = inv_norm(diag_pick(G0, c));
        Gt[Cfg3::oIk + 16 * (b0 + 1) + c] = inv_norm(diag_pick(G1, c));
      }
      wave_sync();
      const float ik0 = Gt[Cfg3::oIk + 16 * b0 + c], ik1 = Gt[Cfg3::oIk + 16 * (b0 + 1) + c];
      const f32x4 is0 = *reinterpret_cast<const f32x4*>(Gt + Cfg3::oIk + 16 * b0 + 4 * g);
      const f32x4 is1 = *reinterpret_cast<const f32x4*>(Gt + Cfg3::oIk + 16 * (b0 + 1) + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        G0[j] *= ik0 * is0[j];
        P0[j] *= is0[j];
        Go[j] *= ik1 * is0[j];
        Po[j] *= is0[j];
        G1[j] *= ik1 * is1[j];
        P1[j] *= is1[j];
      }
      if (l < 32) {  // row 16 b0 + l: lane (g, c) with g = 0 / 1 holds block b0 / b0 + 1's row c
        const int r = 16 * b0 + l;
        const float ik = l < 16 ? ik0 : ik1;
        Gt[Cfg3::oGk + r] = Gt[r] * ik;
        Gt[Cfg3::oLk + r] = Gt[Cfg3::oLam + r] * ik;
      }
    }
    offdiag_tiles<64>(Go, Po, PGT, b0 + 1, b0, g, c, R);
    const f32x4 gm0 = diag_gamma(PGT, b0, g, c), gm1 = diag_gamma(PGT, b0 + 1, g, c);
    diag_p_tile<64>(P0, gm0, b0, g, c, R);
    diag_p_tile<64>(P1, gm1, b0 + 1, g, c, R);
    diag_rows(G0, gm0, PGT, b0, g, c, D + b0 * 320);
    diag_rows(G1, gm1, PGT, b0 + 1, g, c, D + (b0 + 1) * 320);
  };
  // Loads are issued unconditionally (chunk index clamped; buffer loads are
  // range-checked) so that every path through the loop has the same number of
  // loads in flight and the compiler's wait counts stay three steps deep.
  // Clamped chunk index, kept in a scalar register: buffer-load offsets the
  // compiler cannot prove uniform become per-lane loops.
  auto clampc = [&](int m) { return __builtin_amdgcn_readfirstlane(max(0, min(m, nch - 1))); };
  Extra ex;  // first, so that its prologue waits only for its own first loads
  ex.init(x, l);
  ex.prologue(smem);
  load(ic<0>{}, clampc(0));
  issue_fence();
  load(ic<1>{}, clampc(1));
  issue_fence();
  load(ic<2>{}, clampc(2));
  issue_fence();
  run_steps(nch, [&](auto pc, int k) {
    constexpr int ph = decltype(pc)::value;
    if (k + 2 < nch) process(ic<ph>{}, k + 2);
    issue_fence();
    load(ic<ph>{}, clampc(k + 5));  // the set just consumed; needed three steps later
    issue_fence();
    ex.template step<ph>(smem, k);
  });
}

// Waves 4 and 5: row block i = 2 / 3, tiles (i, 0) and (i, 1).  They run one
// step behind the row waves and read K and Q of the chunk from the stage slot
// the row waves published (row-major), and g from the gate table.
// Wave 5 also writes the V tiles (Extra = VStage).  With kPro the K K^T tiles
// are scaled on both sides, the P tiles on the key side, by the 1/|k| the
// row waves wrote a step earlier.
template <class Extra, bool kPro>
__device__ __forceinline__ void gram_lower(const Ctx& x, char* smem, int i, int l) {
  using Cf = Cfg<64>;
  constexpr int NKP = Cf::NKP, LDK = Cf::LDK;
  __bf16* const sb = reinterpret_cast<__bf16*>(smem);
  const int g = l >> 4, c = l & 15, nch = x.nchunks;
  Extra ex;
  ex.init(x, l);
  ex.prologue(smem);
  run_steps(nch, [&](auto pc, int k) {
    constexpr int ph = decltype(pc)::value;
    constexpr int slot = (ph + 2) % 3;  // chunk k + 1
    const int m = k + 1;
    if (m >= 0 && m < nch) {
      __bf16* const R = sb + slot * Cf::szBuf;
      const float* const gt = gate_table(smem, m) + Cfg3::oG;
      u32x4 k0[NKP], k1[NKP], ki[NKP], qi[NKP];
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        const int o = c * LDK + 32 * p + 8 * g;
        k0[p] = *reinterpret_cast<const u32x4*>(R + Cf::oK + o);
        k1[p] = *reinterpret_cast<const u32x4*>(R + Cf::oK + 16 * LDK + o);
        ki[p] = *reinterpret_cast<const u32x4*>(R + Cf::oK + 16 * i * LDK + o);
        qi[p] = *reinterpret_cast<const u32x4*>(R + Cf::oQ + 16 * i * LDK + o);
      }
      f32x4 G0 = zero4(), P0 = zero4(), G1 = zero4(), P1 = zero4();
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        G0 = mma32(k0[p], ki[p], G0);
        P0 = mma32(k0[p], qi[p], P0);
        G1 = mma32(k1[p], ki[p], G1);
        P1 = mma32(k1[p], qi[p], P1);
      }
      if constexpr (kPro) {  // lane (g, c): [s = 16 jb + 4g + j][r = 16i + c]
        const float* const Gt = gate_table(smem, m);
        const float ikr = Gt[Cfg3::oIk + 16 * i + c];
        const f32x4 is0 = *reinterpret_cast<const f32x4*>(Gt + Cfg3::oIk + 4 * g);
        const f32x4 is1 = *reinterpret_cast<const f32x4*>(Gt + Cfg3::oIk + 16 + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          G0[j] *= ikr * is0[j];
          P0[j] *= is0[j];
          G1[j] *= ikr * is1[j];
          P1[j] *= is1[j];
        }
      }
      offdiag_tiles<64>(G0, P0, gt, i, 0, g, c, R);
      offdiag_tiles<64>(G1, P1, gt, i, 1, g, c, R);
    }
    ex.template step<ph>(smem, k);
  });
}

// Wave 6: the output of both consumers' columns, one step behind them:
// chunk n's Q S term in step n from their start-of-chunk state, its P Ut term
// in step n + 1 from their Ut.  With kPro (raw queries; P tiles scaled on the
// key side only) it also finds 1/|q| of each token from the diagonal of
// Q Q^T, two products per 16-token block on the Q operands it holds, and
// scales the token's output row by it: o = (gamma Q S + P Ut) / |q|.
template <bool kPro>
__device__ __forceinline__ void out_wave(const Ctx& x, char* smem, int l) {
  using Cf = Cfg<64>;
  constexpr int LDK = Cf::LDK;
  const __bf16* const sb = reinterpret_cast<const __bf16*>(smem);
  const unsigned* const hand = reinterpret_cast<const unsigned*>(smem + Cfg3::fBase);
  const int H = x.H, T = x.T, DV = x.DV, nch = x.nchunks;
  const int g = l >> 4, c = l & 15;
  // Lane (g, c) writes token c of each 16-token block, value columns
  // 16t + 4g .. + 3 of the slice (one 8-byte store per tile t).
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(x.outg + ((size_t)x.b * T * H + x.h) * DV + x.dv0,
                                              span_bytes((size_t)T * H * DV * 2, ((size_t)x.h * DV + x.dv0) * 2));
  const int rowO = H * DV * 2, vofO = c * rowO + 8 * g;
  const int offRow = c * LDK + 8 * g, offT16 = c * Cf::LD16 + 4 * g;  // Q row c, keys 8g .. + 7
  f32x4 o[4][2];  // Q S term of the chunk in progress, per block row and tile
  u32x2 Pm[10];   // its P tiles
  [[maybe_unused]] float iq[4];  // with kPro: 1/|q| of token 16i + c
  auto out_start = [&](int n, const __bf16* R, const float* G) {
    const unsigned* const hs = hand + Cfg3::fXS + (n & 1) * Cfg3::szHand2;
    u32x2 st[2][4];
    u32x4 qr[4][2];
    float gm[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int d = 0; d < 4; ++d) st[t][d] = *reinterpret_cast<const u32x2*>(hs + t * Cfg3::szHand + 2 * (d * 64 + l));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int p = 0; p < 2; ++p) qr[i][p] = *reinterpret_cast<const u32x4*>(R + Cf::oQ + 16 * i * LDK + 32 * p + offRow);
      gm[i] = G[16 * i + c];  // gamma of token 16i + c
    }
    issue_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) o[i][t] = out_qs<2>(st[t], qr[i], gm[i]);
    if constexpr (kPro) {  // |q|^2 of row c: lane (c / 4, c) of Q_i Q_i^T
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 d = mma32(qr[i][1], qr[i][1], mma32(qr[i][0], qr[i][0], zero4()));
        iq[i] = lane_read(inv_norm(diag_pick(d, c)), 16 * (c >> 2) + c);
      }
    }
#pragma unroll
    for (int e = 0; e < 10; ++e) Pm[e] = ld4(R + Cf::oP + e * Cf::szTile + offT16);
  };
  auto out_finish = [&](int n) {
    const unsigned* const hu = hand + Cfg3::fXU + (n & 1) * Cfg3::szHand2;
    u32x2 X[4][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) X[i][t] = *reinterpret_cast<const u32x2*>(hu + t * Cfg3::szHand + 2 * (i * 64 + l));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 r = out_pu(o[i][t], i, t, X, Pm);
        if constexpr (kPro) {
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] *= iq[i];
        }
        __builtin_amdgcn_raw_buffer_store_b64(cvt4(r), ro, vofO + 32 * t, (n * 64 + 16 * i) * rowO, 0);
      }
  };
  run_steps(nch, [&](auto pc, int k) {
    constexpr int cur = (decltype(pc)::value + 1) % 3;  // stage slot of chunk k
    if (k >= 1 && k <= nch) out_finish(k - 1);
    if (k >= 0 && k < nch) out_start(k, sb + cur * Cf::szBuf, gate_table(smem, k));
  });
  if (needs_tail_step(nch)) {
    stage_barrier();
    out_finish(nch - 1);
  }
}

// One forward-substitution step for the row-per-lane inverse: columns s <= M
// of every row get t_s += row_bcast<M>(t_s) * (-A[c][M]).
#define GDN_ST(R, A, M) "v_fmac_f32_dpp %" #R ", %" #R ", %" #A " row_newbcast:" #M " row_mask:0xf bank_mask:0xf\n"

// Wave 7: T_ii diag(beta_i) for all four diagonal blocks of chunk m.  Lane
// (b, c) owns row c of block b: t starts as row c of the identity and, once
// row M of the block is final (after step M - 1), it is broadcast along the
// 16-lane row and added, scaled by -A[c][M], to every row; rows with c <= M
// have A[c][M] = 0.  Row M has no entries right of the diagonal, so step M only
// touches columns 0..M.  Wait states: a DPP source must be written two
// instructions earlier; step M + 1 reads column s M + 1 instructions after step
// M wrote it, so only steps 1 and 2 need padding.
__device__ __forceinline__ void inverter(const Ctx& x, char* smem, int l) {
  using Cf = Cfg<64>;
  __bf16* const sb = reinterpret_cast<__bf16*>(smem);
  float* const sf = reinterpret_cast<float*>(smem + Cfg3::fBase);
  const int b = l >> 4, c = l & 15, nch = x.nchunks;
  float* const eye = sf + Cfg3::fEye;
  if (l < 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(eye + l * 20 + 4 * q) =
          f32x4{l == 4 * q ? 1.f : 0.f, l == 4 * q + 1 ? 1.f : 0.f, l == 4 * q + 2 ? 1.f : 0.f,
                l == 4 * q + 3 ? 1.f : 0.f};
  }
  run_steps(nch, [&](auto pc, int k) {
    constexpr int slot = (decltype(pc)::value + 2) % 3;  // (k + 1) % 3
    const int m = k + 1;
    if (m < 0 || m >= nch) return;
    const float* rowA = sf + Cfg3::fDS + (m & 1) * Cfg3::szDS + b * 320 + c * 20;
    float a[16], t[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 va = *reinterpret_cast<const f32x4*>(rowA + 4 * q);
      const f32x4 vt = *reinterpret_cast<const f32x4*>(eye + c * 20 + 4 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[4 * q + j] = va[j];
        t[4 * q + j] = vt[j];
      }
    }
    asm volatile("s_nop 1\n"
                 GDN_ST(0, 8, 0) "s_nop 1\n"
                 GDN_ST(0, 9, 1) GDN_ST(1, 9, 1) "s_nop 0\n"
                 GDN_ST(0, 10, 2) GDN_ST(1, 10, 2) GDN_ST(2, 10, 2)
                 GDN_ST(0, 11, 3) GDN_ST(1, 11, 3) GDN_ST(2, 11, 3) GDN_ST(3, 11, 3)
                 GDN_ST(0, 12, 4) GDN_ST(1, 12, 4) GDN_ST(2, 12, 4) GDN_ST(3, 12, 4) GDN_ST(4, 12, 4)
                 GDN_ST(0, 13, 5) GDN_ST(1, 13, 5) GDN_ST(2, 13, 5) GDN_ST(3, 13, 5) GDN_ST(4, 13, 5)
                 GDN_ST(5, 13, 5)
                 GDN_ST(0, 14, 6) GDN_ST(1, 14, 6) GDN_ST(2, 14, 6) GDN_ST(3, 14, 6) GDN_ST(4, 14, 6)
                 GDN_ST(5, 14, 6) GDN_ST(6, 14, 6)
                 GDN_ST(0, 15, 7) GDN_ST(1, 15, 7) GDN_ST(2, 15, 7) GDN_ST(3, 15, 7) GDN_ST(4, 15, 7)
                 GDN_ST(5, 15, 7) GDN_ST(6, 15, 7) GDN_ST(7, 15, 7)
                 : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
    asm volatile("s_nop 1\n"
                 GDN_ST(0, 15, 8) GDN_ST(1, 15, 8) GDN_ST(2, 15, 8) GDN_ST(3, 15, 8) GDN_ST(4, 15, 8)
                 GDN_ST(5, 15, 8) GDN_ST(6, 15, 8) GDN_ST(7, 15, 8) GDN_ST(8, 15, 8)
                 GDN_ST(0, 16, 9) GDN_ST(1, 16, 9) GDN_ST(2, 16, 9) GDN_ST(3, 16, 9) GDN_ST(4, 16, 9)
                 GDN_ST(5, 16, 9) GDN_ST(6, 16, 9) GDN_ST(7, 16, 9) GDN_ST(8, 16, 9) GDN_ST(9, 16, 9)
                 GDN_ST(0, 17, 10) GDN_ST(1, 17, 10) GDN_ST(2, 17, 10) GDN_ST(3, 17, 10) GDN_ST(4, 17, 10)
                 GDN_ST(5, 17, 10) GDN_ST(6, 17, 10) GDN_ST(7, 17, 10) GDN_ST(8, 17, 10) GDN_ST(9, 17, 10)
                 GDN_ST(10, 17, 10)
                 GDN_ST(0, 18, 11) GDN_ST(1, 18, 11) GDN_ST(2, 18, 11) GDN_ST(3, 18, 11) GDN_ST(4, 18, 11)
                 GDN_ST(5, 18, 11) GDN_ST(6, 18, 11) GDN_ST(7, 18, 11) GDN_ST(8, 18, 11) GDN_ST(9, 18, 11)
                 GDN_ST(10, 18, 11) GDN_ST(11, 18, 11)
                 GDN_ST(0, 19, 12) GDN_ST(1, 19, 12) GDN_ST(2, 19, 12) GDN_ST(3, 19, 12) GDN_ST(4, 19, 12)
                 GDN_ST(5, 19, 12) GDN_ST(6, 19, 12) GDN_ST(7, 19, 12) GDN_ST(8, 19, 12) GDN_ST(9, 19, 12)
                 GDN_ST(10, 19, 12) GDN_ST(11, 19, 12) GDN_ST(12, 19, 12)
                 GDN_ST(0, 20, 13) GDN_ST(1, 20, 13) GDN_ST(2, 20, 13) GDN_ST(3, 20, 13) GDN_ST(4, 20, 13)
                 GDN_ST(5, 20, 13) GDN_ST(6, 20, 13) GDN_ST(7, 20, 13) GDN_ST(8, 20, 13) GDN_ST(9, 20, 13)
                 GDN_ST(10, 20, 13) GDN_ST(11, 20, 13) GDN_ST(12, 20, 13) GDN_ST(13, 20, 13)
                 GDN_ST(0, 21, 14) GDN_ST(1, 21, 14) GDN_ST(2, 21, 14) GDN_ST(3, 21, 14) GDN_ST(4, 21, 14)
                 GDN_ST(5, 21, 14) GDN_ST(6, 21, 14) GDN_ST(7, 21, 14) GDN_ST(8, 21, 14) GDN_ST(9, 21, 14)
                 GDN_ST(10, 21, 14) GDN_ST(11, 21, 14) GDN_ST(12, 21, 14) GDN_ST(13, 21, 14) GDN_ST(14, 21, 14)
                 : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]),
                   "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14])
                 : "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]));
    const float* G = gate_table(smem, m) + Cfg3::oBeta + 16 * b;  // beta of block b
    u32x4 w0, w1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 bq = *reinterpret_cast<const f32x4*>(G + 4 * q);
      const unsigned lo = cvt2(t[4 * q] * bq[0], t[4 * q + 1] * bq[1]);
      const unsigned hi = cvt2(t[4 * q + 2] * bq[2], t[4 * q + 3] * bq[3]);
      if (q < 2) {
        w0[2 * q] = lo;
        w0[2 * q + 1] = hi;
      } else {
        w1[2 * q - 4] = lo;
        w1[2 * q - 3] = hi;
      }
    }
    __bf16* dst = sb + slot * Cf::szBuf + Cf::oTP + b * Cf::szTile + c * Cf::LD16;
    *reinterpret_cast<u32x4*>(dst) = w0;
    *reinterpret_cast<u32x4*>(dst + 8) = w1;
  });
}
#undef GDN_ST

// Waves 0 and 1: consumers.  They hand Ut and the start-of-chunk state to the
// output wave.  With kPro the keys are raw, so K S and the update take
// gamma / |k| and lambda / |k| from the gate table in place of gamma and
// lambda: (K / |k|) S = diag(1 / |k|) (K S) and (K / |k|)^T (lambda Ut) =
// K^T (lambda / |k| * Ut).
template <bool kPro>
__device__ __forceinline__ void consume(const Ctx& x, char* smem, int w, int l) {
  using Cf = Cfg<64>;
  using Cs = Consumer<64>;
  const __bf16* const sb = reinterpret_cast<const __bf16*>(smem);
  unsigned* const hand = reinterpret_cast<unsigned*>(smem + Cfg3::fBase) + w * Cfg3::szHand;
  Cs cs;
  cs.init(x, w, l);
  // Step k finishes chunk k and, since the rows, V and gates of chunk k + 1
  // were published a step earlier, starts chunk k + 1 before the barrier.
  run_steps(x.nchunks, [&](auto pc, int k) {
    constexpr int slot = (decltype(pc)::value + 1) % 3;  // k % 3
    constexpr int next = (slot + 1) % 3;
    if (k >= 0 && k < x.nchunks) {
      Cs::Upd u;
      u32x2 Xf[4][1], XL[4][1];
      // solve() reads lambda at G + 64 and gamma_C at G[gCoff]
      constexpr int shift = kPro ? Cfg3::oLk - Cfg3::oLam : 0;
      cs.solve(sb + slot * Cf::szBuf, gate_table(smem, k) + shift, Cfg3::oGC - shift, u, Xf, XL,
               hand + Cfg3::fXU + (k & 1) * Cfg3::szHand2);
      cs.update(u, XL);
    }
    if (k >= -1 && k + 1 < x.nchunks)
      cs.begin(sb + next * Cf::szBuf, gate_table(smem, k + 1) + (kPro ? Cfg3::oGk : 0),
               hand + Cfg3::fXS + ((k + 1) & 1) * Cfg3::szHand2);
  });
  cs.finish(x);
}

// Cache warm-up on the CUs the chains leave idle.  The compute workgroups'
// own loads run three chunks ahead, but from HBM their row loads still cost
// the loading waves several hundred cycles per step.  A warm-up workgroup
// takes some of its XCD's chains (wave i the i-th of them, at most two) and
// touches every row of their q, k and v and every token of their gates (one
// dword per 128-byte row), kWarmLead chunks ahead of a pace of kWarmStep
// shader cycles per chunk, so the compute workgroups find those lines in the
// caches.  The loads go straight to LDS that nothing reads: no register
// waits for them, and the wave waits once at the end.  Rows past T fail the
// buffer range check and read nothing.  The pace is an estimate; being ahead
// or behind only changes how much the warm-up helps.
constexpr int kWarmLead = 8, kWarmStep = 2200;

__device__ __forceinline__ void warm_chains(const __bf16* qg, const __bf16* kg, const __bf16* vg, const float* alpha,
                                            const float* beta, int T, int H, int DV, int chain0, int nchain, int first,
                                            int stride, char* smem) {
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, c = first + stride * wv;
  if (wv >= 2 || c >= nchain) return;
  const int chain = chain0 + c, b = chain / H, h = chain % H, nch = (T + 63) >> 6;
  const size_t tokbase = (size_t)b * T * H + h;
  const uint32_t spanB = span_bytes((size_t)T * H * 64 * 2, (size_t)h * 64 * 2);
  const uint32_t spanF = span_bytes((size_t)T * H * 4, (size_t)h * 4);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + tokbase * 64, spanB), rq = make_rsrc(qg + tokbase * 64, spanB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + tokbase * DV, span_bytes((size_t)T * H * DV * 2, (size_t)h * DV * 2));
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(alpha + tokbase, spanF), rb = make_rsrc(beta + tokbase, spanF);
  auto* const sink = (__attribute__((address_space(3))) void*)(smem + 256 * wv);
  const long long t0 = clock64();
  for (int m = 0; m < nch; ++m) {
    if (m > kWarmLead) {
      const long long due = t0 + (long long)(m - kWarmLead) * kWarmStep;
      while (clock64() < due) __builtin_amdgcn_s_sleep(1);
    }
    const uint32_t t = (uint32_t)(m * 64 + l);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, sink, 4, t * H * 128, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, sink, 4, t * H * 128, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, sink, 4, t * H * DV * 2, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, sink, 4, t * H * 4, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, sink, 4, t * H * 4, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// kPro = false: q, k are used as given and alpha, beta are the gates.
// kPro = true (fused prologue): q, k are raw and normalised per row inside the
// arithmetic; alpha and beta point to the logits a, b, with alpha =
// exp(-softplus(a)) and beta = beta_scale * sigmoid(b).
template <bool kPro>
__global__ __launch_bounds__(kThreads3, 1) void chunk_pipe3_kernel(const __bf16* __restrict__ qg,
                                                                  const __bf16* __restrict__ kg,
                                                                  const __bf16* __restrict__ vg,
                                                                  const float* __restrict__ alpha,
                                                                  const float* __restrict__ beta, const float* S0g,
                                                                  __bf16* __restrict__ outg, float* Sfg, int T, int H,
                                                                  int DV, int nslices, float beta_scale, int nwarm) {
  __shared__ __attribute__((aligned(16))) char smem[Cfg3::bytes];
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);  // keep neighbours on one XCD
  if (nwarm > 0) {  // the last nwarm of each XCD's blocks warm the caches for that XCD's chains
    const int per = nblk >> 3, xcd = bid / per, j = bid % per, ncx = per - nwarm;
    if (j >= ncx) {
      warm_chains(qg, kg, vg, alpha, beta, T, H, DV, xcd * (ncx / nslices), ncx / nslices, j - ncx, nwarm, smem);
      return;
    }
    bid = xcd * ncx + j;
  }
  const int slice = bid % nslices, chain = bid / nslices;
  Ctx x;
  x.qg = qg;
  x.kg = kg;
  x.vg = vg;
  x.alpha = alpha;
  x.beta = beta;
  x.S0g = S0g;
  x.outg = outg;
  x.Sfg = Sfg;
  x.T = T;
  x.H = H;
  x.DV = DV;
  x.b = chain / H;
  x.h = chain % H;
  x.chain = chain;
  x.dv0 = slice * Cfg<64>::NV;
  x.nchunks = (T + 63) >> 6;
  x.beta_scale = beta_scale;
  // The wave index is uniform (scalar branches only: matrix-core instructions
  // do not honour the exec mask).
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  if (w == 6) {
    out_wave<kPro>(x, smem, l);  // runs the tail step itself
    return;
  }
  if (w < 2)
    consume<kPro>(x, smem, w, l);
  else if (w == 2)
    gram_rows<GateStage<false, true, kPro>, kPro>(x, smem, 0, l);
  else if (w == 3)
    gram_rows<GateStage<true, false, kPro>, kPro>(x, smem, 2, l);
  else if (w == 4)
    gram_lower<NoStage, kPro>(x, smem, 2, l);
  else if (w == 5)
    gram_lower<VStage, kPro>(x, smem, 3, l);
  else
    inverter(x, smem, l);
  if (needs_tail_step(x.nchunks)) stage_barrier();
}

}  // namespace pipe3

hipError_t launch_chunk_pipe(const ChunkArgs& a) {
  if (a.dtype == kDtBF16 && a.dk == 64) {
    const int nslices = a.dv / pipe::Cfg<64>::NV;
    long nblk = (long)a.B * a.H * nslices;
    // On a whole device (256 CUs in 8 XCDs) with at least four idle CUs per
    // XCD and whole chains on every XCD, the grid is filled to 256 workgroups
    // with cache warm-up workgroups (on fewer CUs they would queue behind the
    // chains and only add their paced loop).  Not with the prologue folded
    // in: there they cost more than they saved (B8 T2048 H12: 48.2 against
    // 47.0 us, where the plain call gained 42.9 -> 41.7).
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      ncu = 0;
    int nwarm = 0;
    if (!a.prologue && ncu == 256 && nblk % 8 == 0 && nblk <= 224 && (nblk / 8) % nslices == 0) {
      nwarm = 32 - (int)(nblk / 8);
      nblk = 256;
    }
    auto kern = a.prologue ? pipe3::chunk_pipe3_kernel<true> : pipe3::chunk_pipe3_kernel<false>;
    return launch_kernel(kern, dim3((unsigned)nblk), dim3(pipe3::kThreads3), (hipStream_t)a.stream, a.q, a.k, a.v,
                         a.alpha, a.beta, a.S0, a.out, a.S_final, a.T, a.H, a.dv, nslices, a.beta_scale, nwarm);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
