// chunk_pipe.hip -- warp-specialised, software-pipelined chunkwise gated
// delta-rule forward for bf16 inputs on gfx950.
//
// Same method as the fused kernel (chunkwise WY / UT transform of the gated
// delta rule: Sykra 0.3.3 README, "Architectural Highlights"; DeltaPhase README,
// section 1 "Fast Triangular Solve" and section 5 "Exact Chunkwise-Parallel
// Scan"), reorganised so that no wave stalls on another's latency:
//
//   * 8 waves per workgroup (one workgroup per (batch, head, 64 value columns)).
//     Waves 4..7 are PRODUCERS: for chunk n+1 they stage the raw q/k/v tiles
//     into LDS, run the log-space gate scan, form the Gram tiles of K Kr^T and
//     K Qr^T on MFMA, apply the decay, and invert the four 16x16 diagonal blocks
//     of (I + A).  Waves 0..3 are CONSUMERS: each owns 16 value columns of the
//     state and runs the sequential part for chunk n.  Two barriers per chunk.
//   * The consumer never forms W or U.  With S the state at the chunk start,
//       R  = diag(beta) V - diag(beta gamma) Kr S,
//       Ut = (I + A)^{-1} R                (block forward substitution),
//       O  = diag(gamma) Qr S + P Ut,
//       S <- gamma_C S + K^T diag(lambda) Ut,   lambda_t = exp(g_C - g_t),
//     which is the same algebra as Ut = U - W S with U = T diag(beta) V,
//     W = T diag(beta)(Kr * gamma).  Every intermediate stays in MFMA
//     accumulators and is fed back as the next product's operand.
//   * Decay factors above the diagonal blocks are products of a per-row and a
//     per-column factor, each <= 1 (exp(g_r - g_m) exp(g_m - g_s) with m the
//     first row of the row block), so only the diagonal blocks need per-element
//     exponentials, masked before the exponential.
//   * Transposed operands (K^T for the state update, V in accumulator layout)
//     are read with ds_read_b64_tr_b16 straight from the row-major tiles.
//   * Global traffic uses buffer loads/stores whose range check implements the
//     ragged tail (rows >= T read as zero and are never written).
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace pipe {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ bf16x4 as_bf16x4(short4_t s) { return __builtin_bit_cast(bf16x4, s); }

// Four consecutive bf16 at p (8-byte aligned LDS).
__device__ __forceinline__ bf16x4 ld4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }

// Transposed sub-block of a row-major bf16 LDS matrix M (row stride ld):
// lane (g, c) receives M[row0 + 4g + j][col + c], j = 0..3.
__device__ __forceinline__ bf16x4 ld4_tr(const __bf16* M, int ld, int row0, int col) {
  const int l = lane_id(), g = l >> 4, i = l & 15;
  const __bf16* p = M + (row0 + 4 * g + (i >> 2)) * ld + col + 4 * (i & 3);
  return as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p)));
}

__device__ __forceinline__ bf16x4 cvt4(const f32x4& a) {
  bf16x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (__bf16)a[j];
  return r;
}

__device__ __forceinline__ f32x4 mfma(const bf16x4& a0, const bf16x4& a1, const bf16x4& b0, const bf16x4& b1,
                                      const f32x4& c) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = a0[j];
    a[4 + j] = a1[j];
    b[j] = b0[j];
    b[4 + j] = b1[j];
  }
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 z4() {
  bf16x4 z;
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ float bcast_quad(float x, int q) {
  // quad_perm [q, q, q, q]
  switch (q) {
    case 0: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x00, 0xf, 0xf, false));
    case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x55, 0xf, 0xf, false));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xAA, 0xf, 0xf, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xFF, 0xf, 0xf, false));
  }
}

__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }

template <int DK> struct Cfg {
  static constexpr int NV = 64;                 // value columns per workgroup
  static constexpr int NDT = DK / 16, NKP = DK / 32;
  static constexpr int LDK = DK + 8, LDV = NV + 8, LD16 = 16 + 8;
  // element offsets (bf16) of the double-buffered raw tiles and hand-off tiles
  static constexpr int szK = 64 * LDK, szV = 64 * LDV;
  static constexpr int oRK = 0, oRQ = szK, oRV = 2 * szK, szRaw = 2 * szK + szV;
  static constexpr int szTri = 10 * 16 * LD16, szTd = 4 * 16 * LD16;
  static constexpr int oHA = 0, oHP = szTri, oHT = 2 * szTri, szHand = 2 * szTri + szTd;
  static constexpr int nBf = 2 * szRaw + 2 * szHand;
  static constexpr int fBase = ((nBf * 2 + 15) / 16) * 16;  // byte offset of the fp32 region
  // fp32 region (floats): gates[2] = beta, beta*gamma, gamma, lambda (64 each) + gamma_C (pad 4)
  static constexpr int szGate = 4 * 64 + 4;
  static constexpr int fGate = 0;
  // producer-only: per-token g2, beta, rowf (64 each) and colf for row blocks 1..3 (3 x 64)
  static constexpr int fPG = 2 * szGate, szPG = 6 * 64;
  // producer diagonal-block scratch (fp32 16 x 20 per producer wave)
  static constexpr int fDS = fPG + szPG, szDS = 16 * 20;
  static constexpr int nF = fDS + 4 * szDS;
  static constexpr int bytes = fBase + nF * 4;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  // global geometry
  static constexpr int UPRK = DK * 2 / 16, UPRV = NV * 2 / 16;   // 16-byte units per row
  static constexpr int NUK = 64 * UPRK / 256, NUV = 64 * UPRV / 256;
};

template <int DK>
__global__ __launch_bounds__(512, 1) void chunk_pipe_kernel(const __bf16* __restrict__ qg, const __bf16* __restrict__ kg,
                                                            const __bf16* __restrict__ vg,
                                                            const float* __restrict__ alpha,
                                                            const float* __restrict__ beta, const float* S0g,
                                                            __bf16* __restrict__ outg, float* Sfg, int T, int H,
                                                            int DV, int nslices) {
  using Cf = Cfg<DK>;
  constexpr int NDT = Cf::NDT, NKP = Cf::NKP, LDK = Cf::LDK, LDV = Cf::LDV, LD16 = Cf::LD16;
  __shared__ __attribute__((aligned(16))) char smem[Cf::bytes];
  __bf16* const sb = reinterpret_cast<__bf16*>(smem);
  float* const sf = reinterpret_cast<float*>(smem + Cf::fBase);

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);  // keep neighbours on one XCD
  const int slice = bid % nslices, chain = bid / nslices;
  const int b = chain / H, h = chain % H, dv0 = slice * Cf::NV;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  const int nchunks = (T + 63) >> 6;

  auto raw = [&](int buf) { return sb + buf * Cf::szRaw; };
  auto hand = [&](int buf) { return sb + 2 * Cf::szRaw + buf * Cf::szHand; };
  auto gate = [&](int buf) { return sf + Cf::fGate + buf * Cf::szGate; };

  if (w >= 4) {
    // ======================================================== PRODUCERS
    const int pt = tid - 256, pw = w - 4;
    const size_t tokbase = (size_t)b * T * H + h;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + tokbase * DK, (uint32_t)((size_t)T * H * DK * 2 - (size_t)h * DK * 2));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + tokbase * DK, (uint32_t)((size_t)T * H * DK * 2 - (size_t)h * DK * 2));
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vg + tokbase * DV + dv0, (uint32_t)((size_t)T * H * DV * 2 - ((size_t)h * DV + dv0) * 2));
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(alpha + tokbase, (uint32_t)(((size_t)T * H - h) * 4));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(beta + tokbase, (uint32_t)(((size_t)T * H - h) * 4));
    const int rowK = H * DK * 2, rowV = H * DV * 2;  // bytes between tokens
    uint4 pk[Cf::NUK], pq[Cf::NUK], pv[Cf::NUV];
    float pa = 1.f, pb = 0.f;
    int vofK[Cf::NUK], vofV[Cf::NUV];
#pragma unroll
    for (int u = 0; u < Cf::NUK; ++u) {
      const int unit = pt + 256 * u;
      vofK[u] = (unit / Cf::UPRK) * rowK + (unit % Cf::UPRK) * 16;
    }
#pragma unroll
    for (int u = 0; u < Cf::NUV; ++u) {
      const int unit = pt + 256 * u;
      vofV[u] = (unit / Cf::UPRV) * rowV + (unit % Cf::UPRV) * 16;
    }
    auto prefetch = [&](int n) {
      const int c0 = n * 64;
#pragma unroll
      for (int u = 0; u < Cf::NUK; ++u) {
        pk[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, vofK[u], c0 * rowK, 0));
        pq[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, vofK[u], c0 * rowK, 0));
      }
#pragma unroll
      for (int u = 0; u < Cf::NUV; ++u)
        pv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vofV[u], c0 * rowV, 0));
      pa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, l * H * 4, c0 * H * 4, 0));
      pb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, l * H * 4, c0 * H * 4, 0));
      if (c0 + l >= T) pa = 1.f;  // padding token: alpha = 1 (beta reads as 0)
    };

    // Stage chunk n (from the prefetch registers) into raw buffer n & 1, run the
    // gate scan, publish gates for the consumers and decay factors for the Gram.
    auto stage = [&](int n) {
      __bf16* R = raw(n & 1);
#pragma unroll
      for (int u = 0; u < Cf::NUK; ++u) {
        const int unit = pt + 256 * u, row = unit / Cf::UPRK, col = (unit % Cf::UPRK) * 8;
        *reinterpret_cast<uint4*>(R + Cf::oRK + row * LDK + col) = pk[u];
        *reinterpret_cast<uint4*>(R + Cf::oRQ + row * LDK + col) = pq[u];
      }
#pragma unroll
      for (int u = 0; u < Cf::NUV; ++u) {
        const int unit = pt + 256 * u, row = unit / Cf::UPRV, col = (unit % Cf::UPRV) * 8;
        *reinterpret_cast<uint4*>(R + Cf::oRV + row * LDV + col) = pv[u];
      }
      if (pw == 0) {
        float x = log2f(pa);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off, 64);
          if (l >= off) x += y;
        }
        const float g63 = __shfl(x, 63, 64);
        const float gblk = __shfl(x, l & ~15, 64);
        const float gam = exp2f(x);
        float* G = gate(n & 1);
        G[l] = pb;
        G[64 + l] = pb * gam;
        G[128 + l] = gam;
        G[192 + l] = exp2f(g63 - x);
        if (l == 63) G[256] = gam;
        float* PG = sf + Cf::fPG;
        PG[l] = x;
        PG[64 + l] = pb;
        PG[128 + l] = exp2f(x - gblk);
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          const float gi = __shfl(x, 16 * i, 64);
          PG[128 + 64 * i + l] = exp2f(l < 16 * i ? gi - x : -INFINITY);
        }
      }
    };

    // Gram tiles, decay, and the inverse of this wave's diagonal block for chunk n.
    auto gram = [&](int n) {
      const __bf16* R = raw(n & 1);
      __bf16* Hd = hand(n & 1);
      const float* PG = sf + Cf::fPG;
      float* DS = sf + Cf::fDS + pw * Cf::szDS;
      auto tile = [&](int ti, int tj) {
        f32x4 aG = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NKP; ++p) {
          const bf16x4 a0 = ld4(R + Cf::oRK + (16 * tj + c) * LDK + 32 * p + 4 * g);
          const bf16x4 a1 = ld4(R + Cf::oRK + (16 * tj + c) * LDK + 32 * p + 16 + 4 * g);
          const bf16x4 k0 = ld4(R + Cf::oRK + (16 * ti + c) * LDK + 32 * p + 4 * g);
          const bf16x4 k1 = ld4(R + Cf::oRK + (16 * ti + c) * LDK + 32 * p + 16 + 4 * g);
          const bf16x4 q0 = ld4(R + Cf::oRQ + (16 * ti + c) * LDK + 32 * p + 4 * g);
          const bf16x4 q1 = ld4(R + Cf::oRQ + (16 * ti + c) * LDK + 32 * p + 16 + 4 * g);
          aG = mfma(a0, a1, k0, k1, aG);  // [s][r] = k_s . k_r
          aP = mfma(a0, a1, q0, q1, aP);  // [s][r] = k_s . q_r
        }
        const int r = 16 * ti + c;
        f32x4 va, vp;
        if (ti != tj) {
          const float rf = PG[128 + r], nb = -PG[64 + r] * rf;
          const f32x4 cf = *reinterpret_cast<const f32x4*>(PG + 128 + 64 * ti + 16 * tj + 4 * g);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            va[j] = aG[j] * (nb * cf[j]);
            vp[j] = aP[j] * (rf * cf[j]);
          }
        } else {
          const float gr = PG[r], br = PG[64 + r];
          const f32x4 gs = *reinterpret_cast<const f32x4*>(PG + 16 * tj + 4 * g);
          f32x4 ad;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int s = 16 * tj + 4 * g + j;
            const float gm = exp2f(r >= s ? gr - gs[j] : -INFINITY);
            ad[j] = r > s ? br * gm * aG[j] : 0.f;
            va[j] = -ad[j];
            vp[j] = gm * aP[j];
          }
          *reinterpret_cast<f32x4*>(DS + c * 20 + 4 * g) = ad;
        }
        *reinterpret_cast<bf16x4*>(Hd + Cf::oHA + tri(ti, tj) * 16 * LD16 + c * LD16 + 4 * g) = cvt4(va);
        *reinterpret_cast<bf16x4*>(Hd + Cf::oHP + tri(ti, tj) * 16 * LD16 + c * LD16 + 4 * g) = cvt4(vp);
      };
      tile(pw, pw);
      if (pw == 0) { tile(1, 0); tile(2, 0); }
      if (pw == 1) { tile(2, 1); tile(3, 0); }
      if (pw == 2) tile(3, 1);
      if (pw == 3) tile(3, 2);
      // (I + A_pw,pw)^{-1} by forward substitution: lane (q = l & 3, cc = l >> 2)
      // owns column cc, rows 4k + q.  Once row s is final its value is broadcast
      // inside the quad and subtracted from every later row.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int q = l & 3, cc = l >> 2;
      float a[4][16], t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(DS + (4 * k + q) * 20 + 4 * s4);
#pragma unroll
          for (int j = 0; j < 4; ++j) a[k][4 * s4 + j] = v[j];
        }
        t[k] = (4 * k + q == cc) ? 1.f : 0.f;
      }
#pragma unroll
      for (int s = 0; s < 15; ++s) {
        const float ts = bcast_quad(t[s >> 2], s & 3);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * k + 3 > s) t[k] -= a[k][s] * ts;  // a[k][s] = 0 unless row 4k+q > s
      }
      __bf16* Td = Hd + Cf::oHT + pw * 16 * LD16;
#pragma unroll
      for (int k = 0; k < 4; ++k) Td[(4 * k + q) * LD16 + cc] = (__bf16)t[k];
    };

    // prologue: chunk 0 staged and solved before the consumers start
    if (nchunks > 0) {
      prefetch(0);
      stage(0);
      if (nchunks > 1) prefetch(1);
    }
    lds_barrier();
    if (nchunks > 0) gram(0);
    lds_barrier();
    for (int n = 0; n < nchunks; ++n) {
      if (n + 1 < nchunks) {
        stage(n + 1);
        if (n + 2 < nchunks) prefetch(n + 2);
      }
      lds_barrier();
      if (n + 1 < nchunks) gram(n + 1);
      lds_barrier();
    }
  } else {
    // ======================================================== CONSUMERS
    f32x4 S[NDT];
    const int col = dv0 + 16 * w + c;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S[d][j] = S0g ? S0g[((size_t)chain * DK + 16 * d + 4 * g + j) * DV + col] : 0.f;

    const size_t obase = ((size_t)b * T * H + h) * DV + dv0;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(outg + obase, (uint32_t)((size_t)T * H * DV * 2 - ((size_t)h * DV + dv0) * 2));
    const int rowO = H * DV * 2;
    const int vofO = 4 * g * rowO + (16 * w + c) * 2;

    lds_barrier();  // prologue: chunk 0 staged
    lds_barrier();  // prologue: chunk 0 Gram and diagonal inverses ready
    for (int n = 0; n < nchunks; ++n) {
      const int buf = n & 1;
      const __bf16* R = raw(buf);
      const __bf16* Hd = hand(buf);
      const float* G = gate(buf);
      // ---- phase 1: Ut = (I + A)^{-1}(diag(beta) V - diag(beta gamma) K S); state update
      bf16x4 sfr[NDT];
#pragma unroll
      for (int d = 0; d < NDT; ++d) sfr[d] = cvt4(S[d]);
      f32x4 X[4];
      bf16x4 Xf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NKP; ++p) {
          const bf16x4 a0 = ld4(R + Cf::oRK + (16 * i + c) * LDK + 32 * p + 4 * g);
          const bf16x4 a1 = ld4(R + Cf::oRK + (16 * i + c) * LDK + 32 * p + 16 + 4 * g);
          acc = mfma(a0, a1, sfr[2 * p], sfr[2 * p + 1], acc);
        }
        const bf16x4 vv = ld4_tr(R + Cf::oRV, LDV, 16 * i, 16 * w);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(G + 16 * i + 4 * g);
        const f32x4 bg = *reinterpret_cast<const f32x4*>(G + 64 + 16 * i + 4 * g);
        f32x4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = bt[j] * (float)vv[j] - bg[j] * acc[j];
        // y -= sum_{i' < i} A_{i i'} X_{i'}   (the hand-off holds -A)
        if (i == 1) y = mfma(ld4(Hd + Cf::oHA + tri(1, 0) * 16 * LD16 + c * LD16 + 4 * g), z4(), Xf[0], z4(), y);
        if (i == 2)
          y = mfma(ld4(Hd + Cf::oHA + tri(2, 0) * 16 * LD16 + c * LD16 + 4 * g),
                   ld4(Hd + Cf::oHA + tri(2, 1) * 16 * LD16 + c * LD16 + 4 * g), Xf[0], Xf[1], y);
        if (i == 3) {
          y = mfma(ld4(Hd + Cf::oHA + tri(3, 0) * 16 * LD16 + c * LD16 + 4 * g),
                   ld4(Hd + Cf::oHA + tri(3, 1) * 16 * LD16 + c * LD16 + 4 * g), Xf[0], Xf[1], y);
          y = mfma(ld4(Hd + Cf::oHA + tri(3, 2) * 16 * LD16 + c * LD16 + 4 * g), z4(), Xf[2], z4(), y);
        }
        X[i] = mfma(ld4(Hd + Cf::oHT + i * 16 * LD16 + c * LD16 + 4 * g), z4(), cvt4(y), z4(),
                    f32x4{0.f, 0.f, 0.f, 0.f});
        Xf[i] = cvt4(X[i]);
      }
      // S <- gamma_C S + K^T diag(lambda) Ut
      bf16x4 XL[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 lm = *reinterpret_cast<const f32x4*>(G + 192 + 16 * i + 4 * g);
        f32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = X[i][j] * lm[j];
        XL[i] = cvt4(t);
      }
      const float gC = G[256];
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        f32x4 s = S[d];
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] *= gC;
        s = mfma(ld4_tr(R + Cf::oRK, LDK, 0, 16 * d), ld4_tr(R + Cf::oRK, LDK, 16, 16 * d), XL[0], XL[1], s);
        s = mfma(ld4_tr(R + Cf::oRK, LDK, 32, 16 * d), ld4_tr(R + Cf::oRK, LDK, 48, 16 * d), XL[2], XL[3], s);
        S[d] = s;
      }
      lds_barrier();
      // ---- phase 2: O = diag(gamma) Q S + P Ut
      const int c0 = n * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NKP; ++p) {
          const bf16x4 a0 = ld4(R + Cf::oRQ + (16 * i + c) * LDK + 32 * p + 4 * g);
          const bf16x4 a1 = ld4(R + Cf::oRQ + (16 * i + c) * LDK + 32 * p + 16 + 4 * g);
          o = mfma(a0, a1, sfr[2 * p], sfr[2 * p + 1], o);
        }
        const f32x4 gm = *reinterpret_cast<const f32x4*>(G + 128 + 16 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] *= gm[j];
        const __bf16* Pi = Hd + Cf::oHP;
        if (i == 0) o = mfma(ld4(Pi + tri(0, 0) * 16 * LD16 + c * LD16 + 4 * g), z4(), Xf[0], z4(), o);
        if (i == 1)
          o = mfma(ld4(Pi + tri(1, 0) * 16 * LD16 + c * LD16 + 4 * g), ld4(Pi + tri(1, 1) * 16 * LD16 + c * LD16 + 4 * g),
                   Xf[0], Xf[1], o);
        if (i == 2) {
          o = mfma(ld4(Pi + tri(2, 0) * 16 * LD16 + c * LD16 + 4 * g), ld4(Pi + tri(2, 1) * 16 * LD16 + c * LD16 + 4 * g),
                   Xf[0], Xf[1], o);
          o = mfma(ld4(Pi + tri(2, 2) * 16 * LD16 + c * LD16 + 4 * g), z4(), Xf[2], z4(), o);
        }
        if (i == 3) {
          o = mfma(ld4(Pi + tri(3, 0) * 16 * LD16 + c * LD16 + 4 * g), ld4(Pi + tri(3, 1) * 16 * LD16 + c * LD16 + 4 * g),
                   Xf[0], Xf[1], o);
          o = mfma(ld4(Pi + tri(3, 2) * 16 * LD16 + c * LD16 + 4 * g), ld4(Pi + tri(3, 3) * 16 * LD16 + c * LD16 + 4 * g),
                   Xf[2], Xf[3], o);
        }
        // Extract the four 16-bit results from the packed dwords with explicit
        // shifts (element extraction from a bf16 vector followed by a 16-bit
        // bit cast was observed to drop the upper halves).
        const uint2 ob = __builtin_bit_cast(uint2, cvt4(o));
        const unsigned short h16[4] = {(unsigned short)(ob.x & 0xffffu), (unsigned short)(ob.x >> 16),
                                       (unsigned short)(ob.y & 0xffffu), (unsigned short)(ob.y >> 16)};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_amdgcn_raw_buffer_store_b16(h16[j], ro, vofO, (c0 + 16 * i + j) * rowO, 0);
      }
      lds_barrier();
    }
    if (Sfg) {
#pragma unroll
      for (int d = 0; d < NDT; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sfg[((size_t)chain * DK + 16 * d + 4 * g + j) * DV + col] = S[d][j];
    }
  }
}

}  // namespace pipe

template <int DK>
static hipError_t launch_pipe_dk(const ChunkArgs& a) {
  const int nslices = a.dv / pipe::Cfg<DK>::NV;
  const long nblk = (long)a.B * a.H * nslices;
  hipLaunchKernelGGL((pipe::chunk_pipe_kernel<DK>), dim3((unsigned)nblk), dim3(512), 0, (hipStream_t)a.stream,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                     a.alpha, a.beta, static_cast<const float*>(a.S0), static_cast<__bf16*>(a.out),
                     static_cast<float*>(a.S_final), a.T, a.H, a.dv, nslices);
  return hipGetLastError();
}

hipError_t launch_chunk_pipe(const ChunkArgs& a) {
  if (a.dtype == kDtBF16 && a.dk == 64) return launch_pipe_dk<64>(a);
  if (a.dtype == kDtBF16 && a.dk == 128) return launch_pipe_dk<128>(a);
  return hipErrorInvalidValue;
}

}  // namespace gdn
