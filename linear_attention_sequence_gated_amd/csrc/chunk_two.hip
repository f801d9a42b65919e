// chunk_two.hip -- chunkwise gated delta-rule forward for bf16 inputs in two
// launches: a chunk-parallel factor pass and a sequential state pass.
//
// Method: the chunkwise-parallel WY / UT form of the gated delta rule (Sykra
// 0.3.3 README, "Architectural Highlights", chunkwise parallel training;
// DeltaPhase README, section 1 "Fast Triangular Solve", one unit-triangular
// solve per chunk; section 5, the decay factorised in log space).  Per chunk,
// with S the state at its start, g the within-chunk prefix of log2 alpha,
// gamma = 2^g, lambda = 2^(g_C - g), Gamma_rs = 2^(g_r - g_s) (r >= s):
//
//   A  = strict_lower(diag(beta) K K^T * Gamma),  Tb = (I + A)^{-1} diag(beta)
//   Ut = Tb (V - gamma * (K S))
//   O  = gamma * (Q S) + lower(Q K^T * Gamma) Ut
//   S <- gamma_C S + K^T (lambda * Ut)
//
// Tb depends on K, alpha and beta only.  The FACTOR pass forms it for every
// chunk of every chain at once, one wave per chunk: the lower Gram tiles on
// bf16 matrix cores, the four 16 x 16 diagonal blocks of (I + A)^{-1} by
// row-owner forward substitution in fp32, the six blocks below them by block
// substitution on fp32 matrix cores, and it writes Tb (rounded once to bf16,
// already in matrix-core operand order) and g to the caller's workspace.
// The STATE pass is then free of any solve on the chain that carries S from
// chunk to chunk: its consumer waves run K S, one product with Tb and the
// update; the P tiles and the output are formed by two other waves, and
// loader waves stage the next chunks' rows through LDS three steps ahead.
//
// The state pass also runs the segment-parallel two-level scan for long
// sequences with few chains (DeltaPhase README, section 5: the chunkwise scan
// is exact, so a segment's effect on the state is an affine map
// S_out = M S_in + B).  Its MAP mode runs a segment from the identity (for
// M, with V = 0) and from zero (for B) without writing any output; a small
// combine kernel chains the maps from segment to segment; its OUTPUT mode then
// runs every segment from its true start state at once.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "gdn_pipe.hpp"

namespace gdn {
namespace two {
using namespace pipe;

// Orders this wave's LDS writes before its later LDS reads in every lane (the
// compiler treats each lane as a thread; see the three-stage kernel).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// c += a b on fp32 matrix cores for one 16-wide k block: a in A order (lane
// (g, c) holds A[c][4g + j]), b in B order (lane (g, c) holds B[4g + j][c]).
__device__ __forceinline__ f32x4 mmaf(const f32x4& a, const f32x4& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ u32x4 cvt8(const f32x4& a, const f32x4& b) {
  return u32x4{cvt2(a[0], a[1]), cvt2(a[2], a[3]), cvt2(b[0], b[1]), cvt2(b[2], b[3])};
}

// Row c of (I + A)^{-1} for a unit lower-triangular 16 x 16 block, columns
// 4g .. 4g + 3 (lane (g, c)), given a[m] = -A[c][m].  Row-owner forward
// substitution: once row m is final it is broadcast along the lane's row of 16
// (DPP row_newbcast) and added, scaled by -A[c][m], to every later row.  The
// four column chains are interleaved, so each DPP source was written three
// instructions earlier (two wait states are required); the leading s_nop
// covers the instructions before the block.
#define GDN_TWO_STEP(M, A)                                                           \
  "v_fmac_f32_dpp %0, %0, %" #A " row_newbcast:" #M " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %1, %1, %" #A " row_newbcast:" #M " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %2, %2, %" #A " row_newbcast:" #M " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %3, %3, %" #A " row_newbcast:" #M " row_mask:0xf bank_mask:0xf\n"
__device__ __forceinline__ f32x4 unit_lower_inverse(const float (&a)[16], int g, int c) {
  float t0 = c == 4 * g ? 1.f : 0.f, t1 = c == 4 * g + 1 ? 1.f : 0.f;
  float t2 = c == 4 * g + 2 ? 1.f : 0.f, t3 = c == 4 * g + 3 ? 1.f : 0.f;
  asm volatile("s_nop 1\n"
               GDN_TWO_STEP(0, 4) GDN_TWO_STEP(1, 5) GDN_TWO_STEP(2, 6) GDN_TWO_STEP(3, 7) GDN_TWO_STEP(4, 8)
               GDN_TWO_STEP(5, 9) GDN_TWO_STEP(6, 10) GDN_TWO_STEP(7, 11) GDN_TWO_STEP(8, 12)
               GDN_TWO_STEP(9, 13) GDN_TWO_STEP(10, 14) GDN_TWO_STEP(11, 15) GDN_TWO_STEP(12, 16)
               GDN_TWO_STEP(13, 17) GDN_TWO_STEP(14, 18)
               : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3)
               : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
                 "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]));
  return f32x4{t0, t1, t2, t3};
}
#undef GDN_TWO_STEP

// ------------------------------------------------------------- factor pass
// One single-wave workgroup per (chain, chunk), 11.4 KB of LDS each, so a CU
// holds a dozen of them and their load latencies overlap.  Chunk ids run over
// (batch, chunk, head): neighbouring workgroups read neighbouring heads' gates
// from the same cache lines.
template <int DK>
struct FactorCfg {
  static constexpr int NKP = DK / 32;
  // per-wave fp32 scratch: g, beta, ten 16 x 17 transpose tiles (four for
  // the diagonal blocks, six for the blocks below them), and 1/|k| (fused
  // prologue).  The rows of -A of
  // the four diagonal blocks (16 x 20 each) share the last six tiles: they are
  // dead once the inverses are formed, before those tiles are written.
  static constexpr int fG = 0, fB = 64, fTR = 128, fDS = fTR + 4 * 272, fR = fTR + 10 * 272, szW = fR + 64;
  static_assert(fDS + 4 * 16 * 20 <= szW, "diagonal-block rows fit the shared tiles");
};

// PRO: the layer's input transforms are fused in.  k and q are raw: the
// inverse row norms r = 1 / max(|k|, 1e-12) scale the Gram tiles (K^ K^^T =
// diag(r) K K^T diag(r) for the normalised keys K^), and r goes to
// rpw[chunk][64] for the state pass, which folds it into its gates (the
// queries' norms are taken by the state pass's output wave, from the rows it
// reads anyway); alpha and beta hold the logits a and b,
// alpha = exp(-softplus(a)), beta = bscale * sigmoid(b).
template <int DK, bool PRO>
__global__ __launch_bounds__(64) void factor_kernel(const __bf16* __restrict__ kg, const float* __restrict__ alpha,
                                                    const float* __restrict__ beta, char* __restrict__ ws,
                                                    char* __restrict__ wsT, int T, int H, int nch, int total,
                                                    float bscale, float* __restrict__ rpw) {
  using Cf = FactorCfg<DK>;
  constexpr int NKP = Cf::NKP;
  __shared__ __attribute__((aligned(16))) float W[Cf::szW];
  const int l = threadIdx.x & 63, g = l >> 4, c = l & 15;
  const int id = blockIdx.x;
  const int h = id % H, bn = id / H, n = bn % nch, b = bn / nch;
  const int chain = b * H + h, t0 = n * 64;
  char* const rec = ws + ((size_t)chain * nch + n) * kRecBytes;
  const size_t tokbase = (size_t)b * T * H + h;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + tokbase * DK, span_bytes((size_t)T * H * DK * 2, (size_t)h * DK * 2));
  const uint32_t spanG = span_bytes((size_t)T * H * 4, (size_t)h * 4);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(alpha + tokbase, spanG), rb = make_rsrc(beta + tokbase, spanG);
  const int rowK = H * DK * 2;

  // The lane's four key rows 16 i + c, keys 32 p + 8 g .. + 7: operands of
  // both sides of the Gram products (rows past T read as zero).
  u32x4 kr[4][NKP];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < NKP; ++p)
      kr[i][p] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (16 * i + c) * rowK + 2 * (32 * p + 8 * g), t0 * rowK, 0));
  const float av = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, l * H * 4, t0 * H * 4, 0));
  const float bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, l * H * 4, t0 * H * 4, 0));
  const bool live = t0 + l < T;

  if constexpr (PRO) {
    // Inverse norms of the lane's four key rows 16 i + c: its pieces 4p + g
    // are summed over p here and over g across lanes (xor 16, xor 32).
    float* const rp = rpw + ((size_t)chain * nch + n) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sk = 0.f;
#pragma unroll
      for (int p = 0; p < NKP; ++p) sk += piece_sumsq(kr[i][p]);
      sk += __shfl_xor(sk, 16);
      sk += __shfl_xor(sk, 32);
      const float r = inv_row_norm(sk);
      if (g == 0) {
        W[Cf::fR + 16 * i + c] = r;
        rp[16 * i + c] = r;
      }
    }
  }

  // Gates: padding tokens take alpha = 1 and beta = 0.  From logits,
  // log2 alpha = -softplus(a) / ln 2 = -(max(u, 0) + log2(1 + 2^-|u|)) with
  // u = a log2(e), and beta = bscale / (1 + 2^(-b log2(e))).
  float la, bt;
  if constexpr (PRO) {
    const float u = av * 1.4426950408889634f;
    la = live ? -(fmaxf(u, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(u)))) : 0.f;
    bt = live ? bscale * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-bv * 1.4426950408889634f)) : 0.f;
  } else {
    la = __builtin_amdgcn_logf(live ? av : 1.f);
    bt = bv;
  }
  const float gl = wave_prefix_sum(la);
  W[Cf::fG + l] = gl;
  W[Cf::fB + l] = bt;
  reinterpret_cast<float*>(rec + kRecG)[l] = gl;

  // Lower Gram tiles: lane (g, c) of G[i][k] holds (K K^T)[16i + c][16k + 4g + j].
  f32x4 G[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k <= i; ++k) {
      G[i][k] = zero4();
#pragma unroll
      for (int p = 0; p < NKP; ++p) G[i][k] = mma32(kr[k][p], kr[i][p], G[i][k]);
    }
  wave_sync();
  if constexpr (PRO) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ri = W[Cf::fR + 16 * i + c];
#pragma unroll
      for (int k = 0; k <= i; ++k) {
        const f32x4 rs = *reinterpret_cast<const f32x4*>(W + Cf::fR + 16 * k + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) G[i][k][j] *= ri * rs[j];
      }
    }
  }

  // Rows of -A for the diagonal blocks, through LDS to the row owners.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float gr = W[Cf::fG + 16 * i + c], br = W[Cf::fB + 16 * i + c];
    const f32x4 gs = *reinterpret_cast<const f32x4*>(W + Cf::fG + 16 * i + 4 * g);
    f32x4 na;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      na[j] = -br * __builtin_amdgcn_exp2f(c > 4 * g + j ? gr - gs[j] : -INFINITY) * G[i][i][j];
    *reinterpret_cast<f32x4*>(W + Cf::fDS + i * 320 + c * 20 + 4 * g) = na;
  }
  wave_sync();
  // TP[i] = (I + A_ii)^{-1} diag(beta_i) = Tb_ii, A order (lane (g, c): row c, columns 4g + j).
  f32x4 TP[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(W + Cf::fDS + i * 320 + c * 20 + 4 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[4 * q + j] = v[j];
    }
    const f32x4 t = unit_lower_inverse(a, g, c);
    const f32x4 bs = *reinterpret_cast<const f32x4*>(W + Cf::fB + 16 * i + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) TP[i][j] = t[j] * bs[j];
  }
  // TP in B order (lane (g, c): TP[4g + j][c]) through LDS.
  float* const TR = W + Cf::fTR;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) TR[i * 272 + c * 17 + 4 * g + j] = TP[i][j];
  // Decayed Gram blocks below the diagonal, A order: Gt[16i + c][16k + 4g + j].
  f32x4 Gt[4][4];
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < i; ++k) {
      const float gr = W[Cf::fG + 16 * i + c];
      const f32x4 gs = *reinterpret_cast<const f32x4*>(W + Cf::fG + 16 * k + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) Gt[i][k][j] = __builtin_amdgcn_exp2f(gr - gs[j]) * G[i][k][j];
    }
  wave_sync();
  f32x4 TPb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) TPb[i][j] = TR[i * 272 + (4 * g + j) * 17 + c];

  // Block substitution: Tb_ij = -TP_i sum_{k=j}^{i-1} Gt_ik Tb_kj (i > j),
  // in B order (accumulators).
  f32x4 Tb[4][4];
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int j = i - 1; j >= 0; --j) {
      f32x4 X = mmaf(Gt[i][j], TPb[j], zero4());
#pragma unroll
      for (int k = j + 1; k < i; ++k) X = mmaf(Gt[i][k], Tb[k][j], X);
      const f32x4 Y = mmaf(TP[i], X, zero4());
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Tb[i][j][jj] = -Y[jj];
    }
  // ... and in A order through LDS.
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < i; ++j) {
      const int e = 4 + stri(i, j);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) TR[e * 272 + (4 * g + jj) * 17 + c] = Tb[i][j][jj];
    }
  wave_sync();
  f32x4 TA[4][4];
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < i; ++j) {
      const int e = 4 + stri(i, j);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) TA[i][j][jj] = TR[e * 272 + c * 17 + 4 * g + jj];
    }

  // The record, one 16-byte store per block and lane.
  u32x4* const tb = reinterpret_cast<u32x4*>(rec + kRecTb) + l;
  tb[64 * pblk(0, 0)] = cvt8(TP[0], zero4());
  tb[64 * pblk(1, 0)] = cvt8(TA[1][0], TP[1]);
  tb[64 * pblk(2, 0)] = cvt8(TA[2][0], TA[2][1]);
  tb[64 * pblk(2, 1)] = cvt8(TP[2], zero4());
  tb[64 * pblk(3, 0)] = cvt8(TA[3][0], TA[3][1]);
  tb[64 * pblk(3, 1)] = cvt8(TA[3][2], TP[3]);
  if (wsT) {
    // Tb^T: its A operand of block (i, k) is the B order of Tb block (k, i).
    char* const recT = wsT + ((size_t)chain * nch + n) * kRecBytes;
    u32x4* const tt = reinterpret_cast<u32x4*>(recT + kRecTb) + l;
    tt[64 * qblk(0, 0)] = cvt8(TPb[0], Tb[1][0]);
    tt[64 * qblk(0, 1)] = cvt8(Tb[2][0], Tb[3][0]);
    tt[64 * qblk(1, 0)] = cvt8(zero4(), TPb[1]);
    tt[64 * qblk(1, 1)] = cvt8(Tb[2][1], Tb[3][1]);
    tt[64 * qblk(2, 1)] = cvt8(TPb[2], Tb[3][2]);
    tt[64 * qblk(3, 1)] = cvt8(zero4(), TPb[3]);
    reinterpret_cast<float*>(recT + kRecG)[l] = gl;
  }
}

// -------------------------------------------------------------- state pass
// NOQ: a pass that forms no output (segment maps, or the chunk states alone)
// stages no Q rows and has no P ring or output hand-off, so at d = 64 two of
// its workgroups fit a CU.
template <int DK, int NC, bool NOQ = false>
struct StateCfg {
  static constexpr int NV = 16 * NC;              // value columns per workgroup
  static constexpr int NDT = DK / 16, NKP = DK / 32;
  static constexpr int LDV = NV + 8;
  // waves: NC consumers, the P wave, the output wave, then the loaders
  static constexpr int wP = NC, wO = NC + 1, wL = NC + 2;
  static constexpr int NLOAD = DK == 64 ? 2 : 3;  // (K and Q rows | V, Tb, g) or (K | Q | V, Tb, g)
  static constexpr int kThreads = (NC + 2 + NLOAD) * 64;
  // stage slot (bytes): K rows, Q rows, V tile, Tb blocks, gate table
  static constexpr int oK = 0, oQ = 64 * DK * 2, oV = (NOQ ? 1 : 2) * 64 * DK * 2, oTb = oV + 64 * LDV * 2,
                       oGt = oTb + 6 * 1024;
  // gate table (floats): gamma, lambda, g, fs (decay to the end of the
  // token's 16-block), ge[3][64] (decay from the end of block k to the
  // token), gamma_C, gamma for the output, and g - log2 r for the P tiles'
  // diagonal blocks.  With the prologue fused in, the inverse row norms r of
  // the keys (from the factor pass) are folded in here: the consumers' gamma
  // and lambda, fs and the P tiles' key side carry r, so no wave of the step
  // multiplies by them itself.  The queries' norms p scale whole output rows
  // (o_t = p_t (gamma_t q_t S + (P Ut)_t) for raw q), so the output wave
  // applies them last.
  static constexpr int gGam = 0, gLam = 64, gG = 128, gFs = 192, gGe = 256, gGC = 448, gGO = 452, gGk = 516,
                       szG = 580;
  static constexpr int szSlot = oGt + szG * 4;
  static constexpr int oP = 3 * szSlot, szP = NOQ ? 0 : 6 * 1024;  // P ring, two slots
  // hand-off to the output wave, two slots each: Ut (NC x 4 tiles) and the
  // start-of-chunk state (NC x NDT tiles), bf16 operands in lane order
  static constexpr int szHU = NOQ ? 0 : NC * 4 * 64 * 8, szHS = NOQ ? 0 : NC * NDT * 64 * 8;
  static constexpr int oHU = oP + 2 * szP, oHS = oHU + 2 * szHU;
  static constexpr int bytes = oHS + 2 * szHS;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(szSlot % 16 == 0 && oTb % 16 == 0 && oGt % 16 == 0, "16-byte alignment");
  static constexpr int kPerCU = bytes <= 80 * 1024 ? 2 : 1;  // workgroups per CU the LDS allows
};

enum Mode { kOut = 0, kMap = 1 };

struct StateArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const char* ws;      // chunk records
  const float* S0;     // [chains][DK][DV] or NULL
  __bf16* out;
  float* Sf;           // [chains][DK][DV] or NULL
  float* seg_state;    // segmented scan: start states [chains][G][DK][DV] (output mode) or
                       // maps [chains][G][DK][DK + DV] (map mode)
  __bf16* Sck;         // output mode, or NULL: every chunk's start state, bf16 [chains][nch][DK][DV]
  const float* rp;     // fused prologue: 1 / |k| per token, [chains][nch][64]
  int T, H, DV, nch;
  int G, SC;           // segments per chain and chunks per segment (G = 1: one segment)
  int nseg;            // segments per chain in this launch's grid (G, or G - 1 in map mode)
  int mode;
};

// Chunks of one segment and the role context.
struct Seg {
  int b, h, chain, seg, n0, nloc;  // chunks n0 .. n0 + nloc - 1 of the chain
  int dv0;                         // first value column of the workgroup's slice
  int c0;                          // its first column of [M | B] (map mode) or of V
  bool mcol;                       // map mode, identity columns (V reads as zero)
};

template <int DK, int NC, bool NOQ>
struct Consumer2 {
  using Cf = StateCfg<DK, NC, NOQ>;
  static constexpr int NDT = Cf::NDT, NKP = Cf::NKP;
  f32x4 S[NDT];
  u32x2 sfr[NDT];
  int g, c, w, l;

  __device__ __forceinline__ void init(const StateArgs& a, const Seg& sg, int w_, int l_) {
    w = w_;
    l = l_;
    g = l >> 4;
    c = l & 15;
    const int col = sg.dv0 + 16 * w + c;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = key_row(d, g, j);
        float s0 = 0.f;
        if (a.mode == kMap) {
          s0 = (sg.mcol && key == col) ? 1.f : 0.f;  // identity columns of M, zero for B
        } else if (a.G > 1) {
          // segmented: every segment's start state, the first one included, comes
          // from the combine kernel, so S_final may alias S0 although the last
          // segment writes it while the first one may not have started
          s0 = a.seg_state[(((size_t)sg.chain * a.G + sg.seg) * DK + key) * a.DV + col];
        } else if (a.S0) {
          s0 = a.S0[((size_t)sg.chain * DK + key) * a.DV + col];
        }
        S[d][j] = s0;
      }
  }

  // The state's bf16 operands, also handed to the output wave when hs is given.
  __device__ __forceinline__ void publish_state(unsigned* hs) {
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      sfr[d] = cvt4(S[d]);
      if (hs) *reinterpret_cast<u32x2*>(hs + 2 * ((w * NDT + d) * 64 + l)) = sfr[d];
    }
  }

  // One chunk from stage slot R; Ut goes to hu (when the output is formed).
  __device__ __forceinline__ void chunk(const char* R, unsigned* hu, bool mzero) {
    const __bf16* const Rb = reinterpret_cast<const __bf16*>(R);
    const float* const Gt = reinterpret_cast<const float*>(R + Cf::oGt);
    // At d = 128 the K rows are read one 16-row block at a time and half of the
    // update's K^T operands after the Tb product: with everything held at once
    // the consumer needs more than its 256 registers and spills every step.
    constexpr int KRB = DK == 128 ? 1 : 4;    // row blocks of K read ahead of the K S products
    constexpr int KTB = DK == 128 ? 4 : NDT;  // key blocks of K^T read ahead of the Tb product
    u32x4 kr[KRB][NKP];
    u32x2 vv[4];
    f32x4 gg[4];
    auto krow = [&](int i, u32x4 (&dst)[NKP]) {
#pragma unroll
      for (int p = 0; p < NKP; ++p)
        dst[p] = *reinterpret_cast<const u32x4*>(Rb + Cf::oK / 2 + row_off<DK>(16 * i + c, 32 * p + 8 * g));
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < KRB) krow(i, kr[i]);
      vv[i] = ld4_tr(Rb + Cf::oV / 2 + (16 * i + 4 * g + (c >> 2)) * Cf::LDV + 16 * w + 4 * (c & 3));
      gg[i] = *reinterpret_cast<const f32x4*>(Gt + Cf::gGam + 16 * i + 4 * g);
    }
    u32x4 tb[6];
#pragma unroll
    for (int e = 0; e < 6; ++e) tb[e] = *reinterpret_cast<const u32x4*>(R + Cf::oTb + e * 1024 + l * 16);
    issue_fence();
    // K S, then X = V - gamma * (K S) as bf16 B operands
    u32x2 xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 ki[NKP];
      if (i < KRB) {
#pragma unroll
        for (int p = 0; p < NKP; ++p) ki[p] = kr[i < KRB ? i : 0][p];
      } else {
        krow(i, ki);
      }
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < NKP; ++p) acc = mma32(ki[p], pair(sfr[2 * p], sfr[2 * p + 1]), acc);
      f32x4 x;
      const u32x2 v = vv[i];
      const float v0 = mzero ? 0.f : lo_f(v[0]), v1 = mzero ? 0.f : hi_f(v[0]);
      const float v2 = mzero ? 0.f : lo_f(v[1]), v3 = mzero ? 0.f : hi_f(v[1]);
      x[0] = v0 - gg[i][0] * acc[0];
      x[1] = v1 - gg[i][1] * acc[1];
      x[2] = v2 - gg[i][2] * acc[2];
      x[3] = v3 - gg[i][3] * acc[3];
      xb[i] = cvt4(x);
    }
    // Operands of the update, in flight during the Tb product.
    auto ktr = [&](int d, u32x2 (&dst)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = ld4_tr(Rb + Cf::oK / 2 +
                        row_off<DK>(16 * i + 4 * g + (c >> 2), 32 * (d / 2) + 4 * (d % 2) + 8 * (c & 3)));
    };
    u32x2 kt[KTB][4];
#pragma unroll
    for (int d = 0; d < KTB; ++d) ktr(d, kt[d]);
    f32x4 lm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lm[i] = *reinterpret_cast<const f32x4*>(Gt + Cf::gLam + 16 * i + 4 * g);
    const float gC = Gt[Cf::gGC];
    issue_fence();
    // Ut = Tb X: block row i sums k blocks 0 .. i in pairs
    const u32x4 x01 = pair(xb[0], xb[1]), x23 = pair(xb[2], xb[3]);
    f32x4 U[4];
    U[0] = mma32(tb[pblk(0, 0)], x01, zero4());
    U[1] = mma32(tb[pblk(1, 0)], x01, zero4());
    U[2] = mma32(tb[pblk(2, 1)], x23, mma32(tb[pblk(2, 0)], x01, zero4()));
    U[3] = mma32(tb[pblk(3, 1)], x23, mma32(tb[pblk(3, 0)], x01, zero4()));
    u32x2 XL[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (hu) *reinterpret_cast<u32x2*>(hu + 2 * ((w * 4 + i) * 64 + l)) = cvt4(U[i]);
      f32x4 xl;
#pragma unroll
      for (int j = 0; j < 4; ++j) xl[j] = U[i][j] * lm[i][j];
      XL[i] = cvt4(xl);
    }
    // S <- gamma_C S + K^T (lambda * Ut)
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      u32x2 kd[4];
      if (d < KTB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kd[i] = kt[d < KTB ? d : 0][i];
      } else {
        ktr(d, kd);
      }
      f32x4 sd = S[d];
#pragma unroll
      for (int j = 0; j < 4; ++j) sd[j] *= gC;
      sd = mma2(kd[0], kd[1], XL[0], XL[1], sd);
      sd = mma2(kd[2], kd[3], XL[2], XL[3], sd);
      S[d] = sd;
    }
  }

  // The state at the start of local chunk k (its bf16 operand copy) into the
  // chunk-state array, through a buffer resource with 32-bit offsets formed
  // here (64-bit per-element addresses held across the loop would spill).
  __device__ __forceinline__ void store_start(const StateArgs& a, const Seg& sg, int k) {
    const size_t base = ((size_t)sg.chain * a.nch + sg.n0 + k) * DK * a.DV + sg.dv0 + 16 * w;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.Sck + base, (uint32_t)(DK * a.DV * 2));
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned u = sfr[d][j >> 1];
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)((j & 1) ? u >> 16 : u), rs,
                                              (key_row(d, g, j) * a.DV + c) * 2, 0, 0);
      }
  }

  __device__ __forceinline__ void finish(const StateArgs& a, const Seg& sg) {
    float* dst = nullptr;
    size_t ld = a.DV, base = 0;
    int col = sg.c0 + 16 * w + c;
    if (a.mode == kMap) {  // [chains][G][DK][DK + DV]: M in columns 0 .. DK - 1, B after
      dst = a.seg_state;
      ld = DK + a.DV;
      base = ((size_t)sg.chain * a.G + sg.seg) * DK * ld;
    } else if (sg.seg == a.G - 1 && a.Sf) {
      dst = a.Sf;
      base = (size_t)sg.chain * DK * a.DV;
    }
    if (!dst) return;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[base + (size_t)key_row(d, g, j) * ld + col] = S[d][j];
  }
};

// Steps k = -2 .. nloc (inclusive) with one barrier after each, in whole
// triples; in step k the loaders publish chunk k + 2, the P wave and the
// consumers work on chunk k and the output wave finishes chunk k - 1 and
// starts chunk k.  step(phase, k) has phase = (k + 2) % 3 at compile time:
// chunk k + 2 uses stage slot and register set `phase`, chunk k slot
// (phase + 1) % 3.
template <class Step>
__device__ __forceinline__ void run_steps2(int nloc, Step&& step) {
  __builtin_assume(nloc >= 0);
  for (int k = -2; k <= nloc; k += 3) {
    step(ic<0>{}, k);
    stage_barrier();
    step(ic<1>{}, k + 1);
    stage_barrier();
    step(ic<2>{}, k + 2);
    stage_barrier();
  }
}

__device__ __forceinline__ int clampc(int m, int nloc) { return __builtin_amdgcn_readfirstlane(max(0, min(m, nloc - 1))); }

template <int DK, int NC, bool NOQ>
__device__ __forceinline__ void consumer_role(const StateArgs& a, const Seg& sg, char* smem, int w, int l) {
  using Cf = StateCfg<DK, NC, NOQ>;
  Consumer2<DK, NC, NOQ> cs;
  cs.init(a, sg, w, l);
  // Output mode without an output array (the gradient pass's forward, which
  // keeps only the chunk states): nothing is handed to the output wave.
  const bool out = a.mode == kOut, form = !NOQ && out && a.out;
  run_steps2(sg.nloc, [&](auto pc, int k) {
    constexpr int slot = (decltype(pc)::value + 1) % 3;  // k % 3
    if (k == -1) cs.publish_state(form ? reinterpret_cast<unsigned*>(smem + Cf::oHS) : nullptr);  // chunk 0's start
    if (k >= 0 && k < sg.nloc) {
      if (out && a.Sck) cs.store_start(a, sg, k);
      unsigned* hu = form ? reinterpret_cast<unsigned*>(smem + Cf::oHU + (k & 1) * Cf::szHU) : nullptr;
      cs.chunk(smem + slot * Cf::szSlot, hu, sg.mcol);
      cs.publish_state(form ? reinterpret_cast<unsigned*>(smem + Cf::oHS + ((k + 1) & 1) * Cf::szHS) : nullptr);
    }
  });
  cs.finish(a, sg);
}

// P tiles of chunk k: lane (g, c) of tile (i, kk) holds P[16i + c][16kk + 4g + j]
// = q_(16i+c) . k_(16kk+4g+j) Gamma, A order, written in pairs like Tb.
template <int DK, int NC, bool PRO>
__device__ __forceinline__ void p_role(const StateArgs& a, const Seg& sg, char* smem, int l) {
  using Cf = StateCfg<DK, NC>;
  constexpr int NKP = Cf::NKP;
  const int g = l >> 4, c = l & 15;
  const bool form = a.mode == kOut && a.out;
  run_steps2(sg.nloc, [&](auto pc, int k) {
    constexpr int slot = (decltype(pc)::value + 1) % 3;
    if (!form || k < 0 || k >= sg.nloc) return;
    const char* R = smem + slot * Cf::szSlot;
    const __bf16* const Rb = reinterpret_cast<const __bf16*>(R);
    const float* const Gt = reinterpret_cast<const float*>(R + Cf::oGt);
    u32x4 kk[4][NKP], qq[4][NKP];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        const int o = row_off<DK>(16 * i + c, 32 * p + 8 * g);
        kk[i][p] = *reinterpret_cast<const u32x4*>(Rb + Cf::oK / 2 + o);
        qq[i][p] = *reinterpret_cast<const u32x4*>(Rb + Cf::oQ / 2 + o);
      }
    float gr[4], ger[4][3];
    f32x4 gsv[4], fsv[4];
    constexpr int oGr = Cf::gG, oGs = PRO ? Cf::gGk : Cf::gG;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gr[i] = Gt[oGr + 16 * i + c];
      gsv[i] = *reinterpret_cast<const f32x4*>(Gt + oGs + 16 * i + 4 * g);
      fsv[i] = *reinterpret_cast<const f32x4*>(Gt + Cf::gFs + 16 * i + 4 * g);
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) ger[i][kb] = Gt[Cf::gGe + kb * 64 + 16 * i + c];
    }
    issue_fence();
    f32x4 P[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int kb = 0; kb <= i; ++kb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int p = 0; p < NKP; ++p) acc = mma32(kk[kb][p], qq[i][p], acc);
        if (kb == i) {  // diagonal block: decay per element, masked above the diagonal
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[j] *= __builtin_amdgcn_exp2f(c >= 4 * g + j ? gr[i] - gsv[i][j] : -INFINITY);
        } else {  // below: 2^(g_r - g_end(kb)) 2^(g_end(kb) - g_s), both at most one
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] *= ger[i][kb] * fsv[kb][j];
        }
        P[i][kb] = acc;
      }
    u32x4* const dst = reinterpret_cast<u32x4*>(smem + Cf::oP + (k & 1) * Cf::szP) + l;
    dst[64 * pblk(0, 0)] = cvt8(P[0][0], zero4());
    dst[64 * pblk(1, 0)] = cvt8(P[1][0], P[1][1]);
    dst[64 * pblk(2, 0)] = cvt8(P[2][0], P[2][1]);
    dst[64 * pblk(2, 1)] = cvt8(P[2][2], zero4());
    dst[64 * pblk(3, 0)] = cvt8(P[3][0], P[3][1]);
    dst[64 * pblk(3, 1)] = cvt8(P[3][2], P[3][3]);
  });
}

// Element c & 3 of v: lane (c / 4, c) holds diagonal entry c of a 16 x 16
// accumulator tile there.
__device__ __forceinline__ float diag_entry(const f32x4& v, int c) {
  const int j = c & 3;
  return j == 0 ? v[0] : j == 1 ? v[1] : j == 2 ? v[2] : v[3];
}

// x of lane `src` (0..63), through the cross-lane permute.
__device__ __forceinline__ float from_lane(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, x)));
}

// The output, transposed so that lane (g, c) holds token 16i + c and value
// columns 16t + 4g .. + 3 of consumer tile t (one 8-byte store):
//   O_i^T = (S^T Q_i^T) diag(gamma_i) + sum_{k <= i} Ut_k^T P_ik^T.
// In step k it finishes chunk k - 1 (the P Ut term) and starts chunk k (the
// Q S term, from the start state the consumers handed over).  With the
// prologue fused in, q is raw and the P tiles are formed from it, so both
// terms are scaled last by the row's inverse query norm p: |q|^2 is the
// diagonal of Q_i Q_i^T, formed on the matrix cores from the Q operands the
// wave holds (a vector-instruction sum of squares cost this wave more than
// its slack).
template <int DK, int NC, bool PRO>
__device__ __forceinline__ void out_role(const StateArgs& a, const Seg& sg, char* smem, int l) {
  using Cf = StateCfg<DK, NC>;
  constexpr int NKP = Cf::NKP, NDT = Cf::NDT;
  const int g = l >> 4, c = l & 15;
  if (a.mode != kOut || !a.out) {
    run_steps2(sg.nloc, [&](auto, int) {});
    return;
  }
  const int H = a.H, T = a.T, DV = a.DV;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + ((size_t)sg.b * T * H + sg.h) * DV + sg.dv0,
                                              span_bytes((size_t)T * H * DV * 2, ((size_t)sg.h * DV + sg.dv0) * 2));
  const int rowO = H * DV * 2, vofO = c * rowO + 8 * g;
  const int tok0 = sg.n0 * 64;
  f32x4 o[4][NC];
  float pn[4];  // fused prologue: 1 / |q| of the lane's four token rows, carried from start to finish
  auto start = [&](int k, const char* R) {
    const __bf16* const Rb = reinterpret_cast<const __bf16*>(R);
    const float* const Gt = reinterpret_cast<const float*>(R + Cf::oGt);
    const unsigned* const hs = reinterpret_cast<const unsigned*>(smem + Cf::oHS + (k & 1) * Cf::szHS);
    u32x2 st[NC][NDT];
    u32x4 qr[4][NKP];
    float gm[4];
#pragma unroll
    for (int t = 0; t < NC; ++t)
#pragma unroll
      for (int d = 0; d < NDT; ++d) st[t][d] = *reinterpret_cast<const u32x2*>(hs + 2 * ((t * NDT + d) * 64 + l));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int p = 0; p < NKP; ++p)
        qr[i][p] = *reinterpret_cast<const u32x4*>(Rb + Cf::oQ / 2 + row_off<DK>(16 * i + c, 32 * p + 8 * g));
      gm[i] = Gt[Cf::gGO + 16 * i + c];
    }
    issue_fence();
    if constexpr (PRO) {  // |q|^2 of row 16i + c: lane (c / 4, c) of Q_i Q_i^T, read by every lane of row c
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 d = zero4();
#pragma unroll
        for (int p = 0; p < NKP; ++p) d = mma32(qr[i][p], qr[i][p], d);
        pn[i] = from_lane(inv_row_norm(diag_entry(d, c)), 16 * (c >> 2) + c);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < NC; ++t) {
        f32x4 r = zero4();
#pragma unroll
        for (int p = 0; p < NKP; ++p) r = mma32(pair(st[t][2 * p], st[t][2 * p + 1]), qr[i][p], r);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] *= gm[i];
        o[i][t] = r;
      }
  };
  auto finish = [&](int k) {
    const unsigned* const hu = reinterpret_cast<const unsigned*>(smem + Cf::oHU + (k & 1) * Cf::szHU);
    const u32x4* const pp = reinterpret_cast<const u32x4*>(smem + Cf::oP + (k & 1) * Cf::szP) + l;
    u32x4 P[6];
#pragma unroll
    for (int e = 0; e < 6; ++e) P[e] = pp[64 * e];
    u32x2 X[NC][4];
#pragma unroll
    for (int t = 0; t < NC; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) X[t][i] = *reinterpret_cast<const u32x2*>(hu + 2 * ((t * 4 + i) * 64 + l));
    issue_fence();
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const u32x4 x01 = pair(X[t][0], X[t][1]), x23 = pair(X[t][2], X[t][3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 r = mma32(x01, P[pblk(i, 0)], o[i][t]);
        if (i >= 2) r = mma32(x23, P[pblk(i, 1)], r);
        if constexpr (PRO) {
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] *= pn[i];
        }
        __builtin_amdgcn_raw_buffer_store_b64(cvt4(r), ro, vofO + 32 * t, (tok0 + k * 64 + 16 * i) * rowO, 0);
      }
    }
  };
  run_steps2(sg.nloc, [&](auto pc, int k) {
    constexpr int slot = (decltype(pc)::value + 1) % 3;
    if (k >= 1 && k <= sg.nloc) finish(k - 1);
    if (k >= 0 && k < sg.nloc) start(k, smem + slot * Cf::szSlot);
  });
}

// Loader waves: stage chunk k + 2 in step k from registers loaded three steps
// earlier, then reload that register set with chunk k + 5.  Loads are
// unconditional (clamped chunk index; range-checked buffer loads read rows
// past T as zero), so the loop has one load path and the compiler's wait
// counts stay three steps deep.  NOQ: the launch forms no output (map mode,
// or the chunk states alone), so the Q rows are neither loaded nor staged.
template <int DK, int NC, int ROLE, bool PRO, bool NOQ>
__device__ __forceinline__ void load_role(const StateArgs& a, const Seg& sg, char* smem, int l) {
  using Cf = StateCfg<DK, NC, NOQ>;
  const int H = a.H, T = a.T, DV = a.DV, nloc = sg.nloc;
  const size_t tokbase = (size_t)sg.b * T * H + sg.h;
  const int tok0 = sg.n0 * 64;
  // Role 0: K rows (and Q rows at d = 64).  Role 1 at d = 128: Q rows.  Last
  // role: V tile, Tb record and g, and the chunk's gate table.
  constexpr bool kRows = ROLE < Cf::NLOAD - 1;
  if constexpr (NOQ && DK == 128 && ROLE == 1) {  // the Q rows loader has nothing to do
    run_steps2(nloc, [](auto, int) {});
    return;
  }
  constexpr int NROW = DK == 64 && !NOQ ? 2 : 1;  // row matrices per rows loader
  constexpr int NU = DK / 8;              // 16-byte pieces per row
  constexpr int NPL = 64 * NU / 64;       // pieces per lane per matrix
  constexpr int NVU = Cf::NV / 8;         // 16-byte units per V row
  constexpr int NVL = 64 * NVU / 64;
  if constexpr (kRows) {
    const uint32_t span = span_bytes((size_t)T * H * DK * 2, (size_t)sg.h * DK * 2);
    const __bf16* src[NROW];
    int ldst[NROW];
    if constexpr (DK == 64) {
      src[0] = a.k;
      ldst[0] = Cf::oK / 2;
      if constexpr (NROW > 1) {
        src[1] = a.q;
        ldst[1] = Cf::oQ / 2;
      }
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
          st[s][r][u] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[r], vof[u], (tok0 + m * 64) * rowK, 0));
    };
    load(ic<0>{}, clampc(0, nloc));
    issue_fence();
    load(ic<1>{}, clampc(1, nloc));
    issue_fence();
    load(ic<2>{}, clampc(2, nloc));
    issue_fence();
    run_steps2(nloc, [&](auto pc, int k) {
      constexpr int ph = decltype(pc)::value;
      if (k + 2 < nloc) {
        __bf16* const R = reinterpret_cast<__bf16*>(smem + ph * Cf::szSlot);
#pragma unroll
        for (int r = 0; r < NROW; ++r)
#pragma unroll
          for (int u = 0; u < NPL; ++u) *reinterpret_cast<u32x4*>(R + ldst[r] + lof[u]) = st[ph][r][u];
      }
      issue_fence();
      load(ic<ph>{}, clampc(k + 5, nloc));
    });
  } else {
    // The identity columns of a segment map take no V: an empty range makes
    // their V loads return zero without reading memory.
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(
        a.v + tokbase * DV + sg.dv0,
        sg.mcol ? 0u : span_bytes((size_t)T * H * DV * 2, ((size_t)sg.h * DV + sg.dv0) * 2));
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.ws + ((size_t)sg.chain * a.nch + sg.n0) * kRecBytes,
                                                (uint32_t)nloc * kRecBytes);
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
      float gv, rk;
    };
    // fused prologue: the factor pass's 1 / |k| and 1 / |q| per token of the segment's chunks
    const __amdgpu_buffer_rsrc_t rn =
        make_rsrc(PRO ? a.rp + ((size_t)sg.chain * a.nch + sg.n0) * 64 : nullptr, PRO ? (uint32_t)nloc * 256 : 0u);
    Set st[3];
    auto load = [&](auto sc, int m) {
      constexpr int s = decltype(sc)::value;
#pragma unroll
      for (int u = 0; u < NVL; ++u)
        st[s].v[u] = __builtin_bit_cast(u32x4,
                                        __builtin_amdgcn_raw_buffer_load_b128(rv, vof[u], (tok0 + m * 64) * rowV, 0));
#pragma unroll
      for (int e = 0; e < 6; ++e)
        st[s].tb[e] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, kRecTb + e * 1024 + l * 16, m * kRecBytes, 0));
      st[s].gv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, kRecG + 4 * l, m * kRecBytes, 0));
      if constexpr (PRO) {
        st[s].rk = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, 4 * l, m * 256, 0));
      }
    };
    load(ic<0>{}, clampc(0, nloc));
    issue_fence();
    load(ic<1>{}, clampc(1, nloc));
    issue_fence();
    load(ic<2>{}, clampc(2, nloc));
    issue_fence();
    run_steps2(nloc, [&](auto pc, int k) {
      constexpr int ph = decltype(pc)::value;
      if (k + 2 < nloc) {
        char* const R = smem + ph * Cf::szSlot;
        __bf16* const Rb = reinterpret_cast<__bf16*>(R);
        float* const Gt = reinterpret_cast<float*>(R + Cf::oGt);
#pragma unroll
        for (int u = 0; u < NVL; ++u) *reinterpret_cast<u32x4*>(Rb + Cf::oV / 2 + lof[u]) = st[ph].v[u];
#pragma unroll
        for (int e = 0; e < 6; ++e) *reinterpret_cast<u32x4*>(R + Cf::oTb + e * 1024 + l * 16) = st[ph].tb[e];
        // gate table: g is the lane's token prefix; block ends are lanes 15, 31, 47, 63
        const float gl = st[ph].gv;
        auto at = [&](int src) {
          return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), src));
        };
        const float e0 = at(15), e1 = at(31), e2 = at(47), gC = at(63);
        const int blk = l >> 4;
        const float gend = blk == 0 ? e0 : blk == 1 ? e1 : blk == 2 ? e2 : gC;
        const float gam = __builtin_amdgcn_exp2f(gl);
        const float rk = PRO ? st[ph].rk : 1.f;
        Gt[Cf::gGam + l] = gam * rk;
        Gt[Cf::gLam + l] = __builtin_amdgcn_exp2f(gC - gl) * rk;
        Gt[Cf::gGO + l] = gam;
        Gt[Cf::gG + l] = gl;
        Gt[Cf::gFs + l] = __builtin_amdgcn_exp2f(gend - gl) * rk;
        if constexpr (PRO) Gt[Cf::gGk + l] = gl - __builtin_amdgcn_logf(rk);
        Gt[Cf::gGe + l] = __builtin_amdgcn_exp2f(blk > 0 ? gl - e0 : -INFINITY);
        Gt[Cf::gGe + 64 + l] = __builtin_amdgcn_exp2f(blk > 1 ? gl - e1 : -INFINITY);
        Gt[Cf::gGe + 128 + l] = __builtin_amdgcn_exp2f(blk > 2 ? gl - e2 : -INFINITY);
        if (l == 63) Gt[Cf::gGC] = __builtin_amdgcn_exp2f(gC);
      }
      issue_fence();
      load(ic<ph>{}, clampc(k + 5, nloc));
    });
  }
}

template <int DK, int NC, bool PRO, bool NOQ>
__global__ __launch_bounds__((StateCfg<DK, NC>::kThreads), (StateCfg<DK, NC, NOQ>::kPerCU)) void state_kernel(
    StateArgs a) {
  using Cf = StateCfg<DK, NC, NOQ>;
  __shared__ __attribute__((aligned(16))) char smem[Cf::bytes];
  // Block order: slices of one (chain, segment) are neighbours, kept on one
  // XCD (the hardware deals consecutive blocks to the eight XCDs in turn), so
  // their shared rows and records are fetched once into that XCD's L2.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int ncol = a.mode == kMap ? DK + a.DV : a.DV;
  const int nsl = ncol / Cf::NV;
  const int slice = bid % nsl, cs = bid / nsl;
  Seg sg;
  sg.chain = cs / a.nseg;
  sg.seg = cs % a.nseg;
  sg.b = sg.chain / a.H;
  sg.h = sg.chain % a.H;
  sg.n0 = sg.seg * a.SC;
  sg.nloc = max(0, min(a.SC, a.nch - sg.n0));
  const int c0 = slice * Cf::NV;
  sg.c0 = c0;
  sg.mcol = a.mode == kMap && c0 < DK;
  sg.dv0 = a.mode == kMap && c0 >= DK ? c0 - DK : c0;
  // Uniform wave index: role branches are scalar branches (matrix-core
  // instructions ignore the exec mask).
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  if (w < NC)
    consumer_role<DK, NC, NOQ>(a, sg, smem, w, l);
  else if (w == Cf::wP || w == Cf::wO) {
    if constexpr (NOQ)  // no output: the P and output waves only keep the barrier count
      run_steps2(sg.nloc, [](auto, int) {});
    else if (w == Cf::wP)
      p_role<DK, NC, PRO>(a, sg, smem, l);
    else
      out_role<DK, NC, PRO>(a, sg, smem, l);
  } else if (w == Cf::wL)
    load_role<DK, NC, 0, PRO, NOQ>(a, sg, smem, l);
  else if (w == Cf::wL + 1)
    load_role<DK, NC, 1, PRO, NOQ>(a, sg, smem, l);
  else if constexpr (Cf::NLOAD > 2)
    load_role<DK, NC, 2, PRO, NOQ>(a, sg, smem, l);
}

// Start states of the segments: S_(s+1) = M_s S_s + B_s for s = 0 .. G - 2,
// with S_0 = S0 (or zero).  One workgroup per (chain, 16 value columns); the
// sixteen columns are carried through the segments in fp32, one thread per
// (key row, column) entry.  Each map's M block is staged in LDS with 16-byte
// loads, the next one loaded into registers while the current one is applied.
template <int DK>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ S0, const float* __restrict__ maps,
                                                      float* __restrict__ starts, int G, int DV) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int NF4 = DK * DK / 4 / 256;  // float4 of an M block per thread
  constexpr int NR = DK / 16;             // rows per thread
  __shared__ __attribute__((aligned(16))) float Ms[DK][DK + 4];
  __shared__ float cur[DK][17];
  const int nsl = DV / 16, chain = blockIdx.x / nsl, col0 = (blockIdx.x % nsl) * 16;
  const int tid = threadIdx.x, cc = tid & 15, r0 = tid >> 4;
  const int LD = DK + DV;
  for (int r = r0; r < DK; r += 16) {
    const float s = S0 ? S0[((size_t)chain * DK + r) * DV + col0 + cc] : 0.f;
    cur[r][cc] = s;
    starts[(((size_t)chain * G) * DK + r) * DV + col0 + cc] = s;
  }
  f4 m[NF4];
  float bc[NR];
  auto load_map = [&](int s) {
    const float* M = maps + ((size_t)chain * G + s) * DK * LD;
#pragma unroll
    for (int u = 0; u < NF4; ++u) {
      const int idx = tid + 256 * u, r = idx / (DK / 4), c4 = idx % (DK / 4);
      m[u] = *reinterpret_cast<const f4*>(M + (size_t)r * LD + 4 * c4);
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) bc[q] = M[(size_t)(r0 + 16 * q) * LD + DK + col0 + cc];  // B_s
  };
  if (G > 1) load_map(0);
  for (int s = 0; s + 1 < G; ++s) {
    __syncthreads();  // cur written, and the previous block's readers done
#pragma unroll
    for (int u = 0; u < NF4; ++u) {
      const int idx = tid + 256 * u, r = idx / (DK / 4), c4 = idx % (DK / 4);
      *reinterpret_cast<f4*>(&Ms[r][4 * c4]) = m[u];
    }
    float acc[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) acc[q] = bc[q];
    __syncthreads();
    if (s + 2 < G) load_map(s + 1);
#pragma unroll 8
    for (int e = 0; e < DK; ++e) {
      const float ce = cur[e][cc];
#pragma unroll
      for (int q = 0; q < NR; ++q) acc[q] += Ms[r0 + 16 * q][e] * ce;
    }
    __syncthreads();  // every thread has read cur
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int r = r0 + 16 * q;
      cur[r][cc] = acc[q];
      starts[(((size_t)chain * G + s + 1) * DK + r) * DV + col0 + cc] = acc[q];
    }
  }
}

}  // namespace two

// ------------------------------------------------------------------- launch
// Segments of the two-level scan.  With G segments a chain takes about
// 2 nch / G chunk steps (maps of segments 0 .. G - 2 at once, then every
// segment's output at once) instead of nch, at the cost of running the
// segments' maps (dk more columns) once more, and at d = 64 of the factor
// pass that the single-launch kernel does not need.  Every workgroup holds a
// CU of its own (LDS), so a launch of more than 256 workgroups runs in rounds.
// G (2 .. 16, at least 16 chunks per segment) minimises the modelled step
// count: chunks per segment x (rounds of the map launch + rounds of the output
// launch), plus the combine's G steps and the factor pass (about 235 chunks in
// one step time on the whole chip); it is taken only when it saves a fifth of
// the single-segment count.
int chunk_two_segments(const ChunkArgs& a) {
  const long nch = (a.T + 63) / 64, chains = (long)a.B * a.H;
  const long nv = a.dk == 64 ? 32 : 16;
  const long out_sl = a.dv / nv, map_sl = (a.dk + a.dv) / nv;
  constexpr long kCU = 256;
  auto rounds = [](long wg) { return (wg + kCU - 1) / kCU; };
  const long factor = a.dk == 64 ? chains * nch / 235 : 0;
  // the map launch forms no output: at d = 64 two of its workgroups share a CU
  const long map_per_cu = a.dk == 64 ? two::StateCfg<64, 2, true>::kPerCU : two::StateCfg<128, 1, true>::kPerCU;
  const long base = nch * rounds(chains * out_sl);
  long best_cost = base;
  int best = 1;
  for (int G = 2; G <= 16; ++G) {
    const long sc = (nch + G - 1) / G;
    if (sc < 16) break;
    const long cost = sc * (rounds((chains * (G - 1) * map_sl + map_per_cu - 1) / map_per_cu) + rounds(chains * G * out_sl)) +
                      G + factor;
    if (cost < best_cost) {
      best_cost = cost;
      best = G;
    }
  }
  return 5 * best_cost < 4 * base ? best : 1;
}

size_t chunk_two_workspace_bytes(const ChunkArgs& a) {
  const size_t nch = (a.T + 63) / 64, chains = (size_t)a.B * a.H;
  size_t b = chains * nch * two::kRecBytes;
  const int G = chunk_two_segments(a);
  if (G > 1) b += chains * G * ((size_t)a.dk * (a.dk + a.dv) + (size_t)a.dk * a.dv) * 4;
  return b;
}

size_t chunk_two_prologue_workspace_bytes(const ChunkArgs& a) {
  return chunk_two_workspace_bytes(a) + (size_t)a.B * a.H * ((a.T + 63) / 64) * 64 * 4;
}

template <int DK, int NC, bool PRO>
static hipError_t launch_two_dk(const ChunkArgs& a, void* workspace, char* wsT, __bf16* Sck) {
  // fused prologue: 1 / |k| per token after the records and segment maps
  float* const rp = PRO ? reinterpret_cast<float*>(static_cast<char*>(workspace) + chunk_two_workspace_bytes(a))
                        : nullptr;
  using Cf = two::StateCfg<DK, NC>;
  const int nch = (a.T + 63) / 64;
  const long chains = (long)a.B * a.H;
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = static_cast<char*>(workspace);
  const long total = chains * nch;
  if (total > 0) {
    const hipError_t e = launch_kernel(two::factor_kernel<DK, PRO>, dim3((unsigned)total), dim3(64), st,
                                       static_cast<const __bf16*>(a.k), a.alpha, a.beta, ws, wsT, a.T, a.H, nch,
                                       (int)total, a.beta_scale, rp);
    if (e != hipSuccess) return e;
  }
  two::StateArgs s{};
  s.q = static_cast<const __bf16*>(a.q);
  s.k = static_cast<const __bf16*>(a.k);
  s.v = static_cast<const __bf16*>(a.v);
  s.ws = ws;
  s.S0 = static_cast<const float*>(a.S0);
  s.out = static_cast<__bf16*>(a.out);
  s.Sf = static_cast<float*>(a.S_final);
  s.Sck = Sck;
  s.rp = rp;
  s.T = a.T;
  s.H = a.H;
  s.DV = a.dv;
  s.nch = nch;
  const int G = chunk_two_segments(a);
  s.G = G;
  s.SC = G > 1 ? (nch + G - 1) / G : max(nch, 1);
  if (G > 1) {
    float* maps = reinterpret_cast<float*>(ws + (size_t)chains * nch * two::kRecBytes);
    float* starts = maps + (size_t)chains * G * DK * (DK + a.dv);
    s.mode = two::kMap;
    s.nseg = G - 1;
    s.seg_state = maps;
    hipError_t e = launch_kernel(two::state_kernel<DK, NC, PRO, true>, dim3((unsigned)(chains * (G - 1) * ((DK + a.dv) / Cf::NV))),
                                 dim3(Cf::kThreads), st, s);
    if (e != hipSuccess) return e;
    e = launch_kernel(two::combine_kernel<DK>, dim3((unsigned)(chains * (a.dv / 16))), dim3(256), st,
                      static_cast<const float*>(a.S0), static_cast<const float*>(maps), starts, G, a.dv);
    if (e != hipSuccess) return e;
    s.seg_state = starts;
  }
  s.mode = two::kOut;
  s.nseg = G;
  const dim3 grid((unsigned)(chains * G * (a.dv / Cf::NV)));
  if (s.out == nullptr) return launch_kernel(two::state_kernel<DK, NC, PRO, true>, grid, dim3(Cf::kThreads), st, s);
  return launch_kernel(two::state_kernel<DK, NC, PRO, false>, grid, dim3(Cf::kThreads), st, s);
}

hipError_t launch_chunk_two(const ChunkArgs& a, void* workspace) {
  if (a.prologue) {
    if (a.dk == 64) return launch_two_dk<64, 2, true>(a, workspace, nullptr, nullptr);
    if (a.dk == 128) return launch_two_dk<128, 1, true>(a, workspace, nullptr, nullptr);
    return hipErrorInvalidValue;
  }
  if (a.dk == 64) return launch_two_dk<64, 2, false>(a, workspace, nullptr, nullptr);
  if (a.dk == 128) return launch_two_dk<128, 1, false>(a, workspace, nullptr, nullptr);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_two_states(const ChunkArgs& a, void* workspace, void* recT, void* Sck) {
  if (a.prologue) return hipErrorInvalidValue;
  if (a.dk == 64)
    return launch_two_dk<64, 2, false>(a, workspace, static_cast<char*>(recT), static_cast<__bf16*>(Sck));
  if (a.dk == 128)
    return launch_two_dk<128, 1, false>(a, workspace, static_cast<char*>(recT), static_cast<__bf16*>(Sck));
  return hipErrorInvalidValue;
}

}  // namespace gdn
