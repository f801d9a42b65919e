// channel_chunk.hip -- the per-output-channel decay forward in chunk form,
// bf16 inputs, d_k = d_v = 64.
//
// The rule (DeltaPhase README, section 2: LaplacePhaseCore's gated-decay
// variant, the error read from the undecayed memory; section 5: the decay
// diag(r_t) on the memory's output rows, one factor per value channel), for
// every value channel j of the state S [dk, dv]:
//   s_j <- r_j s_j + k beta (v_j - k^T s_j),   o_j = q^T s_j.
// Section 5's exact chunkwise scan: because the decay sits on the output side,
// the coupling between the tokens of a chunk is the plain Gram K K^T, and the
// decay between tokens u < t of channel j is the product of its factors in
// between, so each channel needs its own unit lower-triangular solve.  With
// S the state at the start of a sub-chunk of 16 tokens, w_t = beta_t e_t:
//   w_t = beta_t (v_t - g'_t (K S)_t) - beta_t sum_{u<t} G_tu D'_tu w_u,
//     G = K K^T, D'_tu = prod_{u<i<t} r_i, g'_t = prod_{i<t} r_i;
//   o_t = g_t (Q S)_t + sum_{u<=t} P_tu D_tu w_u,
//     P = Q K^T, D_tu = prod_{u<i<=t} r_i, g_t = prod_{i<=t} r_i;
//   S <- diag(g_15) S + K^T (lambda * w),  lambda_u = prod_{u<i<=15} r_i.
// The decay products are formed by Horner's rule inside the solves (each
// earlier term is multiplied by r_u as token u passes), never as a ratio or
// an exponential of a difference, so nothing overflows however small r is.
//
// The value channels are independent, so each (batch, head) chain runs as
// two workgroups of 32 channels: with one workgroup per chain, 96 chains would
// leave most of the 256 CUs idle.  The two are kept on one XCD so that the K
// and Q rows they both read are fetched once into its L2.  Seven waves per
// workgroup:
//   state waves  (two, 16 channels each) S [64 x 16] in matrix-core
//                accumulators (keys in the key_row order of gdn_pipe.hpp); per
//                sub-chunk n they apply the update of sub-chunk n - 1, then
//                form K_(n+1) S and Q_n S, and between them the 16 x 16 tiles
//                P_n (wave 0), G_(n+1) and C_(n+1) = K_(n+1) K_n^T (wave 1);
//   solver waves (two) a lane quad per value channel: K S_n = g_15 (K_n
//                S_(n-1)) + C_n (lambda * w)_(n-1) (the last term on the
//                matrix cores), then the channel's forward substitution for w,
//                lane h of the quad keeping the running sums of the tokens
//                t = h (mod 4);
//   output waves (two) a lane quad per channel: o of sub-chunk n - 1;
//   loader wave  K, Q rows and the slice's V, r and beta of sub-chunk n + 2,
//                through LDS.
// A wave issues one vector instruction per 4 cycles whatever its active
// lanes, so the per-channel substitution and sums, one lane per channel in
// one wave, were issue-bound; four lanes per channel split each lane's share.
// Tables read by a quad's own tokens are stored with each row's tokens in
// "quad order" (token t at position 4 (t mod 4) + t / 4), so a lane reads its
// four with one 16-byte load; the triangular G and P tables put a lane's four
// in reverse, so that the entries at or below the diagonal, the only ones a
// row's readers use, are a prefix of the lane's 16 bytes (tri_pos).
// Everything a role reads in step n was written in an earlier step; one
// barrier per step.  The solver's substitution is the chain that carries the
// state from sub-chunk to sub-chunk; the products that need only the old
// state run on the state wave beside it.
#include <hip/hip_bf16.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "gdn_pipe.hpp"

namespace gdn {
namespace chc {
using namespace pipe;

constexpr int D = 64, SC = 16;  // head dimension, tokens per sub-chunk
constexpr int NCH = 32;         // value channels per workgroup
constexpr int NSL = D / NCH;    // workgroups per chain
constexpr int LDK = D + 8;      // bf16 row stride of the staged K and Q rows
constexpr int LDT = SC + 4;     // fp32 stride of [channel][token] tables (16-byte rows, five 16-byte
                                // banks apart: a 16-lane group reading or writing 16 bytes each hits 16 banks)
constexpr int LDX = SC + 8;     // bf16 stride of the [channel][token] lambda * w table
constexpr int NSLOT = 4;        // input slots: sub-chunks n - 1 .. n + 2

struct Lay {
  // input slot (bytes): K rows, Q rows [16][LDK] bf16; V^T (quad order), r^T [NCH][LDT] fp32; beta[16] in
  // token order, then in quad order
  static constexpr int iK = 0, iQ = 16 * LDK * 2, iV = 2 * 16 * LDK * 2, iR = iV + NCH * LDT * 4,
                       iB = iR + NCH * LDT * 4, iBq = iB + 16 * 4;
  static constexpr int szIn = iBq + 16 * 4;
  // per-parity ring (bytes): Y^T = (K S)^T, QS^T [NCH][LDT] fp32 (quad order); beta G^T [16][LDT] fp32
  // (column u of beta_t G_tu, t > u); P^T [16][LDT] fp32 (t >= u) -- both with the tokens of row u in
  // triangular order (tri_pos); C as bf16 A operands, 64 lanes x 8 bytes; (lambda w)^T [NCH][LDX] bf16;
  // w^T [NCH][LDT] fp32 (token order); g_15 per channel [NCH] fp32
  static constexpr int rY = 0, rQS = rY + NCH * LDT * 4, rG = rQS + NCH * LDT * 4, rP = rG + 16 * LDT * 4,
                       rC = rP + 16 * LDT * 4, rXL = rC + 64 * 8, rW = rXL + NCH * LDX * 2, rGE = rW + NCH * LDT * 4;
  static constexpr int szRing = rGE + NCH * 4;
  static constexpr int oIn = 0, oRing = NSLOT * szIn, oCX = oRing + 2 * szRing;  // solver's own [NCH][LDT] scratch
  static constexpr int bytes = oCX + NCH * LDT * 4;
  static_assert(szIn % 16 == 0 && szRing % 16 == 0 && rC % 16 == 0 && rXL % 16 == 0 && rW % 16 == 0 &&
                    iV % 16 == 0 && iR % 16 == 0 && iBq % 16 == 0,
                "alignment");
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

struct Args {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* r;
  const float* beta;
  const float* S0;
  __bf16* out;
  float* Sf;
  int T, H, nsub;
};

// Orders this wave's LDS writes before its later LDS reads in every lane.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Last step: nsub or nsub + 1, so that the loader's loop runs whole pairs of
// steps (a loop with a conditional load path gets conservative wait counts).
__device__ __forceinline__ int last_step(int nsub) { return nsub | 1; }

// Steps n = -2 .. last_step(nsub), one barrier after each.
template <class Step>
__device__ __forceinline__ void run(int nsub, Step&& step) {
  __builtin_assume(nsub >= 0);
  const int last = last_step(nsub);
  for (int n = -2; n <= last; ++n) {
    step(n);
    stage_barrier();
  }
}

__device__ __forceinline__ void ld16(const float* p, float (&x)[SC]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = reinterpret_cast<const f32x4*>(p)[q];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[4 * q + j] = v[j];
  }
}

__device__ __forceinline__ char* in_slot(char* smem, int m) { return smem + Lay::oIn + (m & (NSLOT - 1)) * Lay::szIn; }
__device__ __forceinline__ char* ring(char* smem, int m) { return smem + Lay::oRing + (m & 1) * Lay::szRing; }

// Position of token t in a quad-ordered row: lane h of a quad finds its tokens
// t = 4 i + h at 4 h + i.
__device__ __forceinline__ int quad_pos(int t) { return 4 * (t & 3) + (t >> 2); }
// Position of token t in a row of the triangular G and P tables: lane h finds
// token 4 i + h at 4 h + 3 - i, so the entries a row holds for tokens at or
// after a block (i >= i0) are the first 4 - i0 floats of the lane's piece,
// and the lanes read only those.
__device__ __forceinline__ int tri_pos(int t) { return 4 * (t & 3) + 3 - (t >> 2); }

// dst[i] for i = I0 .. 3 from the lane's piece p of a triangular-table row
// (dst[i] = p[3 - i]); one 16-, 12-, 8- or 4-byte read.
template <int I0>
__device__ __forceinline__ void ld_tri(const float* p, float (&dst)[4]) {
  typedef float f32x3 __attribute__((ext_vector_type(3)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if constexpr (I0 == 0) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    dst[3] = x[0], dst[2] = x[1], dst[1] = x[2], dst[0] = x[3];
  } else if constexpr (I0 == 1) {
    const f32x3 x = *reinterpret_cast<const f32x3*>(p);
    dst[3] = x[0], dst[2] = x[1], dst[1] = x[2];
  } else if constexpr (I0 == 2) {
    const f32x2 x = *reinterpret_cast<const f32x2*>(p);
    dst[3] = x[0], dst[2] = x[1];
  } else {
    dst[3] = p[0];
  }
}

// ------------------------------------------------------------ state waves
// Wave sw owns channel tile sw of the slice (channels dv0 + 16 sw .. + 15).
__device__ void state_role(const Args& a, int chain, int dv0, char* smem, int l, int sw) {
  const int g = l >> 4, c = l & 15, chs = 16 * sw + c;  // chs: the lane's channel within the slice
  f32x4 S[4];  // [dk block d]; lane (g, c) holds keys key_row(d, g, j), channel chs
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) S[d][j] = a.S0 ? a.S0[((size_t)chain * D + key_row(d, g, j)) * D + dv0 + chs] : 0.f;
  u32x2 sfr[4];
  auto to_bf16 = [&]() {
#pragma unroll
    for (int d = 0; d < 4; ++d) sfr[d] = cvt4(S[d]);
  };
  // A operand: keys 32p + 8g .. + 7 of row c of a staged [16][LDK] matrix
  auto row_piece = [&](const char* base, int p) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(base) + c * LDK + 32 * p + 8 * g);
  };
  to_bf16();
  run(a.nsub, [&](int n) {
    if (n < -1) return;
    const bool upd = n >= 1 && n <= a.nsub;  // S_n from S_(n-1)
    const bool cur = n >= 0 && n < a.nsub;   // Q_n S_n and P_n
    const bool nxt = n + 1 < a.nsub;         // K_(n+1) S_n, G_(n+1), and C_(n+1) when n >= 0
    // Every LDS read of the step first (reads issued after the step's first
    // LDS write would each wait out the LDS latency).
    u32x2 kt[4], xl;
    float gs;
    if (upd) {
      const char* Rp = ring(smem, n - 1);
      const __bf16* Kp = reinterpret_cast<const __bf16*>(in_slot(smem, n - 1) + Lay::iK);
      const __bf16* XL = reinterpret_cast<const __bf16*>(Rp + Lay::rXL);
      const float* ge = reinterpret_cast<const float*>(Rp + Lay::rGE);
#pragma unroll
      for (int d = 0; d < 4; ++d)  // K^T rows in key_row order, tokens 4g .. 4g + 3
        kt[d] = ld4_tr(Kp + (4 * g + (c >> 2)) * LDK + 32 * (d / 2) + 4 * (d % 2) + 8 * (c & 3));
      xl = *reinterpret_cast<const u32x2*>(XL + chs * LDX + 4 * g);
      gs = ge[chs];
    }
    const char* In = in_slot(smem, n);
    const char* In1 = in_slot(smem, n + 1);
    u32x4 q0, q1, k0, k1, n0, n1;
    f32x4 bn;
    if (cur) {
      q0 = row_piece(In + Lay::iQ, 0);
      q1 = row_piece(In + Lay::iQ, 1);
      k0 = row_piece(In + Lay::iK, 0);
      k1 = row_piece(In + Lay::iK, 1);
    }
    if (nxt) {
      n0 = row_piece(In1 + Lay::iK, 0);
      n1 = row_piece(In1 + Lay::iK, 1);
      bn = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(In1 + Lay::iB) + 4 * g);
    }
    issue_fence();
    if (upd) {  // S <- diag(g_15) S + K_(n-1)^T (lambda * w)_(n-1)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        f32x4 sv = S[d];
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[j] *= gs;
        S[d] = mma2(kt[d], z4(), xl, z4(), sv);
      }
      to_bf16();
    }
    // [16 tokens x 64 keys] rows (pieces a0, a1) times S, lane (g, c): tokens 4g + j, channel chs
    auto times_state = [&](const u32x4& a0, const u32x4& a1) {
      return mma32(a1, pair(sfr[2], sfr[3]), mma32(a0, pair(sfr[0], sfr[1]), zero4()));
    };
    f32x4 qs, y, P, G, C;
    if (cur) {
      qs = times_state(q0, q1);
      if (sw == 0) P = mma32(k1, q1, mma32(k0, q0, zero4()));  // lane (g, c): k_(4g+j) . q_c = P[c][4g + j]
    }
    if (nxt) {
      y = times_state(n0, n1);
      if (sw == 1) {
        G = mma32(n1, n1, mma32(n0, n0, zero4()));  // lane (g, c): k_(4g+j) . k_c
        if (n >= 0) C = mma32(k1, n1, mma32(k0, n0, zero4()));  // lane (g, c): k_(n, 4g+j) . k_(n+1, c) = C[c][4g + j]
      }
    }
    // ... then the writes, all transposed to [channel][token] or [u][t], tokens in quad order
    // (token 4g + j at position 4j + g) or, in the G and P tables, triangular order
    if (cur) {
      char* const R = ring(smem, n);
      float* QS = reinterpret_cast<float*>(R + Lay::rQS) + chs * LDT;
#pragma unroll
      for (int j = 0; j < 4; ++j) QS[4 * j + g] = qs[j];
      if (sw == 0) {
        float* PT = reinterpret_cast<float*>(R + Lay::rP);  // P^T[u][t] = q_t . k_u for t >= u
#pragma unroll
        for (int j = 0; j < 4; ++j) PT[(4 * g + j) * LDT + tri_pos(c)] = c >= 4 * g + j ? P[j] : 0.f;
      }
    }
    if (nxt) {
      char* const R1 = ring(smem, n + 1);
      float* Y = reinterpret_cast<float*>(R1 + Lay::rY) + chs * LDT;
#pragma unroll
      for (int j = 0; j < 4; ++j) Y[4 * j + g] = y[j];
      if (sw == 1) {
        // beta G^T[u][t] = beta_t k_t . k_u for t > u (row u = c, tokens 4g + j)
        float* GT = reinterpret_cast<float*>(R1 + Lay::rG) + c * LDT;
#pragma unroll
        for (int j = 0; j < 4; ++j) GT[tri_pos(4 * g + j)] = 4 * g + j > c ? bn[j] * G[j] : 0.f;
        if (n >= 0) *reinterpret_cast<u32x2*>(R1 + Lay::rC + 8 * l) = cvt4(C);
      }
    }
  });
  if (a.Sf) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) a.Sf[((size_t)chain * D + key_row(d, g, j)) * D + dv0 + chs] = S[d][j];
  }
}

// Value of lane H of this lane's quad (DPP quad_perm [H, H, H, H]).
template <int H>
__device__ __forceinline__ float quad_lane(float x) {
  constexpr int kCtrl = H | (H << 2) | (H << 4) | (H << 6);
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, true));
}

template <int U, class F>
__device__ __forceinline__ void unroll16(F&& f) {
  if constexpr (U < SC) {
    f(ic<U>{});
    unroll16<U + 1>(f);
  }
}

__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// ----------------------------------------------------------- solver waves
// Wave sv: lanes 4 m + h hold channel 16 sv + m of the slice; lane h keeps the
// running sums of the tokens t = 4 i + h.
__device__ void solver_role(const Args& a, char* smem, int l, int sv) {
  float* const CX = reinterpret_cast<float*>(smem + Lay::oCX);
  const int ch = 16 * sv + (l >> 2), h = l & 3;
  float ge_prev = 1.f;  // g_15 of the previous sub-chunk (1 before the first)
  run(a.nsub, [&](int n) {
    if (n < 0 || n >= a.nsub) return;
    const char* In = in_slot(smem, n);
    char* const R = ring(smem, n);
    const int g = l >> 4, c = l & 15;
    // Every LDS read of the step first (the compiler keeps LDS reads below
    // earlier LDS writes it cannot tell apart, so reads issued late would each
    // wait out the LDS latency inside the substitution).  r in token order;
    // y = K S, v and beta for the lane's own tokens 4 i + h (quad order).
    float rr[SC], gt[SC - 1][4];
    ld16(reinterpret_cast<const float*>(In + Lay::iR) + ch * LDT, rr);
    const f32x4 yv = ld4f(reinterpret_cast<const float*>(R + Lay::rY) + ch * LDT + 4 * h);
    const f32x4 vv = ld4f(reinterpret_cast<const float*>(In + Lay::iV) + ch * LDT + 4 * h);
    const f32x4 bv = ld4f(reinterpret_cast<const float*>(In + Lay::iBq) + 4 * h);
    const float* GT = reinterpret_cast<const float*>(R + Lay::rG) + 4 * h;
    // row u of beta G, this lane's tokens after u (uniform over a quad position)
    unroll16<0>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < SC - 1) ld_tri<((u + 1) >> 2)>(GT + u * LDT, gt[u]);
    });
    f32x4 ks;
    // the cross term C_n (lambda w)_(n-1) on the matrix cores (this wave's channel tile), back through LDS
    // to the lane quads
    if (n >= 1) {
      const char* Rp = ring(smem, n - 1);
      const u32x2 cA = *reinterpret_cast<const u32x2*>(R + Lay::rC + 8 * l);
      const u32x2 xl =
          *reinterpret_cast<const u32x2*>(reinterpret_cast<const __bf16*>(Rp + Lay::rXL) + (16 * sv + c) * LDX + 4 * g);
      const f32x4 x = mma2(cA, z4(), xl, z4(), zero4());  // lane (g, c): tokens 4g + j, channel 16 sv + c
      float* const cxw = CX + (16 * sv + c) * LDT;
#pragma unroll
      for (int j = 0; j < 4; ++j) cxw[4 * j + g] = x[j];
      wave_sync_lds();
      const f32x4 cx = ld4f(CX + ch * LDT + 4 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) ks[i] = ge_prev * yv[i] + cx[i];
    } else {
      ks = yv;
    }
    // w_t = beta_t (v_t - g'_t (K S)_t) - sum_{u<t} beta_t G_tu D'_tu w_u, Horner over u.  The sum for
    // token t runs in lane h = t % 4 (local index t / 4); w_u comes from that lane to the whole quad.
    float w[SC], acc[4] = {0.f, 0.f, 0.f, 0.f};
    float gp = 1.f;  // g'_t
    unroll16<0>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const float mine = bv[u >> 2] * (vv[u >> 2] - gp * ks[u >> 2]) - acc[u >> 2];
      w[u] = quad_lane<(u & 3)>(mine);
      gp *= rr[u];
      // tokens 4 i + h > u (entries of tokens already solved may be updated: they are not read again)
      if constexpr (u < SC - 1) {
#pragma unroll
        for (int i = (u + 1) >> 2; i < 4; ++i) acc[i] = acc[i] * rr[u] + gt[u][i] * w[u];
      }
    });
    // lambda_u = prod_{u<i<=15} r_i; (lambda w) as bf16 B operands, w for the output, g_15; lane h
    // writes tokens 4 h .. 4 h + 3
    __bf16* XLn = reinterpret_cast<__bf16*>(R + Lay::rXL) + ch * LDX;
    float* Wn = reinterpret_cast<float*>(R + Lay::rW) + ch * LDT;
    float lam = 1.f, xl[SC];
#pragma unroll
    for (int u = SC - 1; u >= 0; --u) {
      xl[u] = lam * w[u];
      lam *= rr[u];
    }
    // the lane's block 4 h .. 4 h + 3, picked by masked sums (a store per
    // block under a lane condition compiles to branches on the execution
    // mask, and a chain of selects to an indexed private array)
    f32x4 xs, ws;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[j] = (h == 0 ? xl[j] : 0.f) + (h == 1 ? xl[4 + j] : 0.f) + (h == 2 ? xl[8 + j] : 0.f) +
              (h == 3 ? xl[12 + j] : 0.f);
      ws[j] = (h == 0 ? w[j] : 0.f) + (h == 1 ? w[4 + j] : 0.f) + (h == 2 ? w[8 + j] : 0.f) +
              (h == 3 ? w[12 + j] : 0.f);
    }
    *reinterpret_cast<u32x2*>(XLn + 4 * h) = cvt4(xs);
    *reinterpret_cast<f32x4*>(Wn + 4 * h) = ws;
    if (h == 0) reinterpret_cast<float*>(R + Lay::rGE)[ch] = lam;
    ge_prev = lam;
  });
}

// ----------------------------------------------------------- output waves
// Wave so: lanes 4 m + h hold channel 16 so + m of the slice and the tokens t = 4 i + h.
__device__ void output_role(const Args& a, int b, int h_, int dv0, char* smem, int l, int so) {
  const int H = a.H, T = a.T;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + ((size_t)b * T * H + h_) * D + dv0,
                                              span_bytes((size_t)T * H * D * 2, ((size_t)h_ * D + dv0) * 2));
  const int rowO = H * D * 2;
  const int ch = 16 * so + (l >> 2), h = l & 3;
  run(a.nsub, [&](int n) {
    const int m = n - 1;  // sub-chunk finished in this step
    if (m < 0 || m >= a.nsub) return;
    const char* In = in_slot(smem, m);
    const char* R = ring(smem, m);
    const float* PT = reinterpret_cast<const float*>(R + Lay::rP);
    float rr[SC], w[SC], y[4], pt[SC][4];
    ld16(reinterpret_cast<const float*>(In + Lay::iR) + ch * LDT, rr);
    ld16(reinterpret_cast<const float*>(R + Lay::rW) + ch * LDT, w);
    const f32x4 qs = ld4f(reinterpret_cast<const float*>(R + Lay::rQS) + ch * LDT + 4 * h);
    // row u of P^T, this lane's tokens from u's block on (uniform over a quad position)
    unroll16<0>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      ld_tri<(u >> 2)>(PT + 4 * h + u * LDT, pt[u]);
    });
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = 0.f;
    // y_t = sum_{u<=t} P_tu D_tu w_u, Horner over u, for this lane's tokens t = 4 i + h >= u: every token of
    // the blocks after u's, and in u's own block (i = u / 4) the lanes h >= u % 4
#pragma unroll
    for (int u = 0; u < SC; ++u) {
      const int i0 = u >> 2;
      const float nxt = y[i0] * rr[u] + pt[u][i0] * w[u];
      y[i0] = (u & 3) == 0 || h >= (u & 3) ? nxt : y[i0];
#pragma unroll
      for (int i = i0 + 1; i < 4; ++i) y[i] = y[i] * rr[u] + pt[u][i] * w[u];
    }
    // o_t = g_t (Q S)_t + y_t, g_t = prod_{i<=t} r_i
    float gc[SC];
    gc[0] = rr[0];
#pragma unroll
    for (int t = 1; t < SC; ++t) gc[t] = gc[t - 1] * rr[t];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // g of the lane's token 4 i + h, the products of gc in the same order
      // with factors of one past it (a select of gc entries on h compiles to
      // branches on the execution mask, or to an indexed private array)
      const float gt = gc[4 * i] * (h >= 1 ? rr[4 * i + 1] : 1.f) * (h >= 2 ? rr[4 * i + 2] : 1.f) *
                       (h >= 3 ? rr[4 * i + 3] : 1.f);
      const float o = gt * qs[i] + y[i];
      const unsigned short ob = __builtin_bit_cast(unsigned short, __float2bfloat16(o));
      __builtin_amdgcn_raw_buffer_store_b16(ob, ro, 2 * ch + (4 * i + h) * rowO, m * SC * rowO, 0);
    }
  });
}

// ----------------------------------------------------------- loader wave
// Sub-chunk m in step m - 2, from registers loaded two steps earlier.  Tokens past
// T read k = q = v = 0, r = 1, beta = 0: the identity step.
__device__ void loader_role(const Args& a, int b, int h, int dv0, char* smem, int l) {
  const int H = a.H, T = a.T;
  const size_t tokbase = (size_t)b * T * H + h;
  const uint32_t span = span_bytes((size_t)T * H * D * 2, (size_t)h * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + tokbase * D, span), rq = make_rsrc(a.q + tokbase * D, span);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(a.v + tokbase * D + dv0, span_bytes((size_t)T * H * D * 2, ((size_t)h * D + dv0) * 2));
  const __amdgpu_buffer_rsrc_t rr =
      make_rsrc(a.r + tokbase * D + dv0, span_bytes((size_t)T * H * D * 4, ((size_t)h * D + dv0) * 4));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + tokbase, span_bytes((size_t)T * H * 4, (size_t)h * 4));
  const int rowB = H * D * 2, rowF = H * D * 4;
  // lane l: token l / 4 of the sub-chunk; keys 16 (l % 4) .. + 15, the slice's channels 8 (l % 4) .. + 7
  const int tk = l >> 2, cq = 16 * (l & 3), cv = 8 * (l & 3);
  struct Set {
    u32x4 k[2], q[2], v;
    f32x4 r[2];
    float be;
  };
  Set st[2];
  auto load = [&](auto sc, int m) {
    constexpr int s = decltype(sc)::value;
    const int t0 = m * SC;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int off = tk * rowB + 2 * (cq + 8 * e);
      st[s].k[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, t0 * rowB, 0));
      st[s].q[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, t0 * rowB, 0));
    }
    st[s].v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, tk * rowB + 2 * cv, t0 * rowB, 0));
#pragma unroll
    for (int e = 0; e < 2; ++e)
      st[s].r[e] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, tk * rowF + 4 * (cv + 4 * e), t0 * rowF, 0));
    st[s].be = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (l & 15) * H * 4, t0 * H * 4, 0));
  };
  auto publish = [&](auto sc, int m) {
    constexpr int s = decltype(sc)::value;
    char* const In = in_slot(smem, m);
    const bool live = m * SC + tk < T;
    __bf16* K = reinterpret_cast<__bf16*>(In + Lay::iK);
    __bf16* Q = reinterpret_cast<__bf16*>(In + Lay::iQ);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      *reinterpret_cast<u32x4*>(K + tk * LDK + cq + 8 * e) = st[s].k[e];
      *reinterpret_cast<u32x4*>(Q + tk * LDK + cq + 8 * e) = st[s].q[e];
    }
    float* Vt = reinterpret_cast<float*>(In + Lay::iV);
    float* Rt = reinterpret_cast<float*>(In + Lay::iR);
    const int pv = quad_pos(tk);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const unsigned wv = st[s].v[x];
      Vt[(cv + 2 * x) * LDT + pv] = lo_f(wv);
      Vt[(cv + 2 * x + 1) * LDT + pv] = hi_f(wv);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int x = 0; x < 4; ++x) Rt[(cv + 4 * e + x) * LDT + tk] = live ? st[s].r[e][x] : 1.f;
    if (l < 16) {
      const float bl = m * SC + l < T ? st[s].be : 0.f;
      reinterpret_cast<float*>(In + Lay::iB)[l] = bl;
      reinterpret_cast<float*>(In + Lay::iBq)[quad_pos(l)] = bl;
    }
  };
  auto clampm = [&](int m) { return __builtin_amdgcn_readfirstlane(max(0, min(m, a.nsub - 1))); };
  load(ic<0>{}, clampm(0));
  issue_fence();
  load(ic<1>{}, clampm(1));
  issue_fence();
  // Step n publishes sub-chunk n + 2 from set n & 1 and refills it with
  // sub-chunk n + 4; whole pairs of steps (n = -2 .. last_step).
  __builtin_assume(a.nsub >= 0);
  const int last = last_step(a.nsub);
  for (int n = -2; n <= last; n += 2) {
    if (n + 2 < a.nsub) publish(ic<0>{}, n + 2);
    issue_fence();
    load(ic<0>{}, clampm(n + 4));
    issue_fence();
    stage_barrier();
    if (n + 3 < a.nsub) publish(ic<1>{}, n + 3);
    issue_fence();
    load(ic<1>{}, clampm(n + 5));
    issue_fence();
    stage_barrier();
  }
}

constexpr int kThreads = 7 * 64;

// Block order: the NSL slices of a chain are neighbours, kept on one XCD (the
// hardware deals consecutive blocks to the eight XCDs in turn).
__global__ __launch_bounds__(kThreads, 1) void channel_chunk_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char smem[Lay::bytes];
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int chain = bid / NSL, dv0 = (bid % NSL) * NCH, b = chain / a.H, h = chain % a.H;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  if (w < 2)
    state_role(a, chain, dv0, smem, l, w);
  else if (w < 4)
    solver_role(a, smem, l, w - 2);
  else if (w < 6)
    output_role(a, b, h, dv0, smem, l, w - 4);
  else
    loader_role(a, b, h, dv0, smem, l);
}

}  // namespace chc

hipError_t launch_channel_chunk(const ChannelArgs& a) {
  chc::Args x{};
  x.q = static_cast<const __bf16*>(a.q);
  x.k = static_cast<const __bf16*>(a.k);
  x.v = static_cast<const __bf16*>(a.v);
  x.r = a.r;
  x.beta = a.beta;
  x.S0 = a.S0;
  x.out = static_cast<__bf16*>(a.out);
  x.Sf = a.S_final;
  x.T = a.T;
  x.H = a.H;
  x.nsub = (a.T + chc::SC - 1) / chc::SC;
  return launch_kernel(chc::channel_chunk_kernel, dim3((unsigned)((long)a.B * a.H * chc::NSL)), dim3(chc::kThreads),
                       (hipStream_t)a.stream, x);
}

}  // namespace gdn
