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
//   * Decay factors below the diagonal blocks are products of a per-row and a
//     per-column factor, each <= 1 (exp(g_r - g_m) exp(g_m - g_s) with m the
//     first row of the row block), so only the diagonal blocks need per-element
//     exponentials, masked before the exponential.
//   * Transposed operands (K^T for the state update, V in accumulator layout)
//     are read with ds_read_b64_tr_b16 straight from the row-major tiles.
//   * Global traffic uses buffer loads/stores whose range check implements the
//     ragged tail (rows >= T read as zero and are never written).
//   * The chunk loop is unrolled by two so that every LDS address is a per-lane
//     base plus a compile-time offset.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace pipe {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
template <int V> using ic = std::integral_constant<int, V>;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// Barrier between pipeline phases: waits for this wave's LDS traffic only (so
// global prefetches stay in flight) and stops the scheduler from moving any
// instruction across it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x4 ld4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }

// Transposed sub-block of a row-major bf16 LDS matrix M (row stride ld):
// lane (g, c) receives M[row0 + 4g + j][col + c], j = 0..3.  `p` must be the
// lane's address &M[row0 + 4g + (c >> 2)][col + 4 (c & 3)].
__device__ __forceinline__ bf16x4 ld4_tr(const __bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p)));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// fp32 -> bf16 (round to nearest even), converted in pairs (one v_cvt_pk_bf16_f32 each).
__device__ __forceinline__ bf16x4 cvt4(const f32x4& a) {
  const bf16x2 lo = __builtin_convertvector(f32x2{a[0], a[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector(f32x2{a[2], a[3]}, bf16x2);
  return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

// Keeps the loads issued above it from being moved below it.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Barrier for waves that only read LDS in the current buffer: no wait on their
// own outstanding LDS reads, so operand loads stay in flight across it.
__device__ __forceinline__ void reader_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts within
// rows of 16, then the row totals are broadcast into the following rows.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  auto shr = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                                 0xf, 0xf, true));
  };
  x += shr(x, std::integral_constant<int, 0x111>{});  // row_shr:1
  x += shr(x, std::integral_constant<int, 0x112>{});  // row_shr:2
  x += shr(x, std::integral_constant<int, 0x114>{});  // row_shr:4
  x += shr(x, std::integral_constant<int, 0x118>{});  // row_shr:8
  // row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return x;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// c += [a0 a1] [b0; b1]  (two 16-wide k sub-blocks, one 16x16x32 issue)
__device__ __forceinline__ f32x4 mma2(const bf16x4& a0, const bf16x4& a1, const bf16x4& b0, const bf16x4& b1,
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

// c += a b  (one 16-wide k sub-block).  Only used where c comes from VALU code
// or is zero: a 16x16x16 issue that reads as its accumulator the result of a
// 16x16x32 issue was observed to be scheduled without the wait states that
// mixed-shape dependency needs, so such chains use 16x16x32 with a zero half.
__device__ __forceinline__ f32x4 mma1(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int Q> __device__ __forceinline__ float bcast_quad(float x) {
  constexpr int ctrl = Q * 0x55;  // quad_perm [Q, Q, Q, Q]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
}

__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }

template <int DK> struct Cfg {
  static constexpr int NV = 64;  // value columns per workgroup
  static constexpr int NDT = DK / 16, NKP = DK / 32;
  static constexpr int LDK = DK + 8, LDV = NV + 8, LD16 = 16 + 8;
  // bf16 element offsets: double-buffered raw tiles and hand-off tiles
  static constexpr int szK = 64 * LDK, szV = 64 * LDV;
  static constexpr int oRK = 0, oRQ = szK, oRV = 2 * szK, szRaw = 2 * szK + szV;
  static constexpr int szTile = 16 * LD16, szTri = 10 * szTile, szTd = 4 * szTile;
  static constexpr int oHA = 0, oHP = szTri, oHT = 2 * szTri, szHand = 2 * szTri + szTd;
  static constexpr int oRaw0 = 0, oHand0 = 2 * szRaw;
  static constexpr int nBf = 2 * szRaw + 2 * szHand;
  static constexpr int fBase = ((nBf * 2 + 15) / 16) * 16;  // byte offset of the fp32 region
  // fp32 region (floats): gates[2] = beta, beta*gamma, gamma, lambda (64 each) + gamma_C (padded)
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
  static constexpr int UPRK = DK * 2 / 16, UPRV = NV * 2 / 16;  // 16-byte units per row
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
    const int rowK = H * DK * 2, rowV = H * DV * 2;  // bytes between consecutive tokens
    uint4 pk[Cf::NUK], pq[Cf::NUK], pv[Cf::NUV];
    float pa = 1.f, pb = 0.f;
    int vofK[Cf::NUK], vofV[Cf::NUV], ldsK[Cf::NUK], ldsV[Cf::NUV];
#pragma unroll
    for (int u = 0; u < Cf::NUK; ++u) {
      const int unit = pt + 256 * u, row = unit / Cf::UPRK, cu = unit % Cf::UPRK;
      vofK[u] = row * rowK + cu * 16;
      ldsK[u] = row * LDK + cu * 8;
    }
#pragma unroll
    for (int u = 0; u < Cf::NUV; ++u) {
      const int unit = pt + 256 * u, row = unit / Cf::UPRV, cu = unit % Cf::UPRV;
      vofV[u] = row * rowV + cu * 16;
      ldsV[u] = row * LDV + cu * 8;
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
    };

    // Stage chunk n (prefetched registers) into raw buffer BUF, run the gate
    // scan, publish gates for the consumers and decay factors for the Gram.
    auto stage = [&](auto bufc, int n) {
      constexpr int BUF = decltype(bufc)::value;
      __bf16* R = sb + Cf::oRaw0 + BUF * Cf::szRaw;
#pragma unroll
      for (int u = 0; u < Cf::NUK; ++u) {
        *reinterpret_cast<uint4*>(R + Cf::oRK + ldsK[u]) = pk[u];
        *reinterpret_cast<uint4*>(R + Cf::oRQ + ldsK[u]) = pq[u];
      }
#pragma unroll
      for (int u = 0; u < Cf::NUV; ++u) *reinterpret_cast<uint4*>(R + Cf::oRV + ldsV[u]) = pv[u];
      if (pw == 0) {
        const float a = (n * 64 + l < T) ? pa : 1.f;  // padding token: alpha = 1 (beta reads as 0)
        const float x = wave_prefix_sum(__builtin_amdgcn_logf(a));
        const float g63 = __shfl(x, 63, 64);
        const float gblk = __shfl(x, l & ~15, 64);
        const float gam = __builtin_amdgcn_exp2f(x);
        float* G = sf + Cf::fGate + BUF * Cf::szGate;
        G[l] = pb;
        G[64 + l] = pb * gam;
        G[128 + l] = gam;
        G[192 + l] = __builtin_amdgcn_exp2f(g63 - x);
        if (l == 63) G[256] = gam;
        float* PG = sf + Cf::fPG;
        PG[l] = x;
        PG[64 + l] = pb;
        PG[128 + l] = __builtin_amdgcn_exp2f(x - gblk);
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          const float gi = __shfl(x, 16 * i, 64);
          PG[128 + 64 * i + l] = __builtin_amdgcn_exp2f(l < 16 * i ? gi - x : -INFINITY);
        }
      }
    };

    float* const DS = sf + Cf::fDS + pw * Cf::szDS;
    // Operands of one Gram tile: K rows of the column block (A operand) and the
    // K and Q rows of the row block (B operands), NKP k-pairs each.
    struct TileOps {
      bf16x4 a[NKP][2], k[NKP][2], q[NKP][2];
    };
    auto load_tile = [&](const __bf16* R, int ti, int tj, TileOps& o) {
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        const __bf16* ra_ = R + Cf::oRK + (16 * tj + c) * LDK + 32 * p + 4 * g;
        const __bf16* rk_ = R + Cf::oRK + (16 * ti + c) * LDK + 32 * p + 4 * g;
        const __bf16* rq_ = R + Cf::oRQ + (16 * ti + c) * LDK + 32 * p + 4 * g;
        o.a[p][0] = ld4(ra_);
        o.a[p][1] = ld4(ra_ + 16);
        o.k[p][0] = ld4(rk_);
        o.k[p][1] = ld4(rk_ + 16);
        o.q[p][0] = ld4(rq_);
        o.q[p][1] = ld4(rq_ + 16);
      }
    };
    // accumulators [s][r] = k_s . k_r and k_s . q_r of one tile
    auto tile_mma = [&](const TileOps& o, f32x4& aG, f32x4& aP) {
      aG = zero4();
      aP = zero4();
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        aG = mma2(o.a[p][0], o.a[p][1], o.k[p][0], o.k[p][1], aG);
        aP = mma2(o.a[p][0], o.a[p][1], o.q[p][0], o.q[p][1], aP);
      }
    };
    auto store_tile = [&](__bf16* Hd, int t, const f32x4& va, const f32x4& vp) {
      *reinterpret_cast<bf16x4*>(Hd + Cf::oHA + t * Cf::szTile + c * LD16 + 4 * g) = cvt4(va);
      *reinterpret_cast<bf16x4*>(Hd + Cf::oHP + t * Cf::szTile + c * LD16 + 4 * g) = cvt4(vp);
    };

    // (I + A_pw,pw)^{-1} by forward substitution.  Lane (q = l & 3, cc = l >> 2)
    // owns column cc and rows 4k + q; once row s is final its value is
    // broadcast inside the quad and subtracted from every later row.
    auto solve = [&](__bf16* Hd) {
      __bf16* Td = Hd + Cf::oHT + pw * Cf::szTile;
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
      auto step = [&](auto sc) {
        constexpr int s = decltype(sc)::value;
        const float ts = bcast_quad<s & 3>(t[s >> 2]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * k + 3 > s) t[k] -= a[k][s] * ts;  // a[k][s] = 0 unless row 4k+q > s
      };
      step(ic<0>{}); step(ic<1>{}); step(ic<2>{}); step(ic<3>{}); step(ic<4>{});
      step(ic<5>{}); step(ic<6>{}); step(ic<7>{}); step(ic<8>{}); step(ic<9>{});
      step(ic<10>{}); step(ic<11>{}); step(ic<12>{}); step(ic<13>{}); step(ic<14>{});
#pragma unroll
      for (int k = 0; k < 4; ++k) Td[(4 * k + q) * LD16 + cc] = (__bf16)t[k];
    };

    // Tiles of this wave: its diagonal tile (pw, pw) and two tiles below the
    // diagonal.  The six sub-diagonal tiles are split two per wave over waves
    // 0..2; wave 3 recomputes wave 2's pair and does not store it, so every
    // wave runs the same straight-line code.
    const int o1i = pw == 0 ? 1 : pw == 1 ? 2 : 3, o1j = pw == 0 ? 0 : pw == 1 ? 1 : 2;
    const int o2i = pw == 0 ? 2 : 3, o2j = pw == 0 ? 0 : pw == 1 ? 0 : 1;
    const bool storeOff = pw < 3;
    auto gram = [&](auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
      const __bf16* R = sb + Cf::oRaw0 + BUF * Cf::szRaw;
      __bf16* Hd = sb + Cf::oHand0 + BUF * Cf::szHand;
      const float* PG = sf + Cf::fPG;
      TileOps od, o1, o2;
      load_tile(R, pw, pw, od);
      load_tile(R, o1i, o1j, o1);
      load_tile(R, o2i, o2j, o2);
      // decay factors: diagonal tile (g2 and beta of row r, g2 of columns s) and
      // the row / column factors of the two sub-diagonal tiles
      const int rd = 16 * pw + c, r1 = 16 * o1i + c, r2 = 16 * o2i + c;
      const float gr = PG[rd], br = PG[64 + rd];
      const f32x4 gs = *reinterpret_cast<const f32x4*>(PG + 16 * pw + 4 * g);
      const float rf1 = PG[128 + r1], nb1 = -PG[64 + r1] * rf1;
      const float rf2 = PG[128 + r2], nb2 = -PG[64 + r2] * rf2;
      const f32x4 cf1 = *reinterpret_cast<const f32x4*>(PG + 128 + 64 * o1i + 16 * o1j + 4 * g);
      const f32x4 cf2 = *reinterpret_cast<const f32x4*>(PG + 128 + 64 * o2i + 16 * o2j + 4 * g);
      issue_fence();
      f32x4 gD, pD, g1, p1, g2, p2;
      tile_mma(od, gD, pD);
      tile_mma(o1, g1, p1);
      tile_mma(o2, g2, p2);
      // diagonal tile: per-element decay, masked before the exponential
      f32x4 ad, va, vp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 16 * pw + 4 * g + j;
        const float gm = __builtin_amdgcn_exp2f(rd >= s ? gr - gs[j] : -INFINITY);
        ad[j] = rd > s ? br * gm * gD[j] : 0.f;
        va[j] = -ad[j];
        vp[j] = gm * pD[j];
      }
      *reinterpret_cast<f32x4*>(DS + c * 20 + 4 * g) = ad;
      store_tile(Hd, tri(pw, pw), va, vp);
      // sub-diagonal tiles: decay = row factor x column factor
      f32x4 va1, vp1, va2, vp2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        va1[j] = g1[j] * (nb1 * cf1[j]);
        vp1[j] = p1[j] * (rf1 * cf1[j]);
        va2[j] = g2[j] * (nb2 * cf2[j]);
        vp2[j] = p2[j] * (rf2 * cf2[j]);
      }
      if (storeOff) {
        store_tile(Hd, tri(o1i, o1j), va1, vp1);
        store_tile(Hd, tri(o2i, o2j), va2, vp2);
      }
      solve(Hd);
    };

    // prologue: chunk 0 staged and solved before the consumers start
    if (nchunks > 0) {
      prefetch(0);
      stage(ic<0>{}, 0);
      if (nchunks > 1) prefetch(1);
    }
    phase_barrier();
    if (nchunks > 0) gram(ic<0>{});
    phase_barrier();
    // iteration n: stage / solve chunk n+1 into buffer (n+1) & 1
    // iteration n: stage / solve chunk n+1 into buffer (n+1) & 1
    auto iter = [&](auto nbufc, int n) {
      if (n + 1 < nchunks) {
        stage(nbufc, n + 1);
        if (n + 2 < nchunks) prefetch(n + 2);
      }
      phase_barrier();
      if (n + 1 < nchunks) gram(nbufc);
      phase_barrier();
    };
    for (int n = 0; n < nchunks; n += 2) {
      iter(ic<1>{}, n);
      if (n + 1 < nchunks) iter(ic<0>{}, n + 1);
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

    // Output: lane (g, c) of wave w writes token c of each 16-token block,
    // value columns 16w + 4g .. 16w + 4g + 3 (one 8-byte store).
    const size_t obase = ((size_t)b * T * H + h) * DV + dv0;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(outg + obase, (uint32_t)((size_t)T * H * DV * 2 - ((size_t)h * DV + dv0) * 2));
    const int rowO = H * DV * 2;
    const int vofO = c * rowO + (16 * w + 4 * g) * 2;
    // per-lane LDS element offsets (relative to a raw / hand-off buffer)
    const int offRow = c * LDK + 4 * g;                                  // row c, k sub-block 4g
    const int offTrK = (4 * g + (c >> 2)) * LDK + 4 * (c & 3);           // transposed K reads
    const int offTrV = (4 * g + (c >> 2)) * LDV + 16 * w + 4 * (c & 3);  // transposed V reads
    const int offT16 = c * LD16 + 4 * g;                                 // 16x16 hand-off tiles

    auto body = [&](auto bufc, int n) {
      constexpr int BUF = decltype(bufc)::value;
      const __bf16* R = sb + Cf::oRaw0 + BUF * Cf::szRaw;
      const __bf16* Hd = sb + Cf::oHand0 + BUF * Cf::szHand;
      const float* G = sf + Cf::fGate + BUF * Cf::szGate;
      auto Atile = [&](int i, int j) { return ld4(Hd + Cf::oHA + tri(i, j) * Cf::szTile + offT16); };
      auto Ptile = [&](int i, int j) { return ld4(Hd + Cf::oHP + tri(i, j) * Cf::szTile + offT16); };
      // ---- phase 1: Ut = (I + A)^{-1}(diag(beta) V - diag(beta gamma) K S); state update.
      // Operand loads for the whole phase are issued first.
      bf16x4 kr[4][NKP][2], vv[4], Am[6], Tm[4];
      f32x4 bt[4], bg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int p = 0; p < NKP; ++p) {
          const __bf16* pr = R + Cf::oRK + 16 * i * LDK + 32 * p + offRow;
          kr[i][p][0] = ld4(pr);
          kr[i][p][1] = ld4(pr + 16);
        }
        vv[i] = ld4_tr(R + Cf::oRV + 16 * i * LDV + offTrV);
        bt[i] = *reinterpret_cast<const f32x4*>(G + 16 * i + 4 * g);
        bg[i] = *reinterpret_cast<const f32x4*>(G + 64 + 16 * i + 4 * g);
        Tm[i] = ld4(Hd + Cf::oHT + i * Cf::szTile + offT16);
      }
      Am[0] = Atile(1, 0); Am[1] = Atile(2, 0); Am[2] = Atile(2, 1);
      Am[3] = Atile(3, 0); Am[4] = Atile(3, 1); Am[5] = Atile(3, 2);
      issue_fence();
      bf16x4 sfr[NDT];
#pragma unroll
      for (int d = 0; d < NDT; ++d) sfr[d] = cvt4(S[d]);
      f32x4 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = zero4();
#pragma unroll
        for (int p = 0; p < NKP; ++p) acc[i] = mma2(kr[i][p][0], kr[i][p][1], sfr[2 * p], sfr[2 * p + 1], acc[i]);
      }
      // operands of the state update, in flight during the substitution
      bf16x4 kt[NDT][4];
      f32x4 lm[4];
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        const __bf16* pk = R + Cf::oRK + 16 * d + offTrK;
#pragma unroll
        for (int i = 0; i < 4; ++i) kt[d][i] = ld4_tr(pk + 16 * i * LDK);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) lm[i] = *reinterpret_cast<const f32x4*>(G + 192 + 16 * i + 4 * g);
      const float gC = G[256];
      issue_fence();
      f32x4 X[4];
      bf16x4 Xf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = bt[i][j] * (float)vv[i][j] - bg[i][j] * acc[i][j];
        // y -= sum_{i' < i} A_{i i'} X_{i'}   (the hand-off holds -A)
        if (i == 1) y = mma1(Am[0], Xf[0], y);
        if (i == 2) y = mma2(Am[1], Am[2], Xf[0], Xf[1], y);
        if (i == 3) {
          y = mma2(Am[3], Am[4], Xf[0], Xf[1], y);
          y = mma2(Am[5], z4(), Xf[2], z4(), y);
        }
        X[i] = mma1(Tm[i], cvt4(y), zero4());
        Xf[i] = cvt4(X[i]);
      }
      // S <- gamma_C S + K^T diag(lambda) Ut
      bf16x4 XL[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = X[i][j] * lm[i][j];
        XL[i] = cvt4(t);
      }
      // operands of the output, in flight during the state update
      bf16x4 qr[4][NKP][2], Pm[10];
      float gm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int p = 0; p < NKP; ++p) {
          const __bf16* pr = R + Cf::oRQ + 16 * i * LDK + 32 * p + offRow;
          qr[i][p][0] = ld4(pr);
          qr[i][p][1] = ld4(pr + 16);
        }
        gm[i] = G[128 + 16 * i + c];  // gamma of token 16i + c
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) Pm[tri(i, j)] = Ptile(i, j);
      issue_fence();
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        f32x4 sd = S[d];
#pragma unroll
        for (int j = 0; j < 4; ++j) sd[j] *= gC;
        sd = mma2(kt[d][0], kt[d][1], XL[0], XL[1], sd);
        sd = mma2(kt[d][2], kt[d][3], XL[2], XL[3], sd);
        S[d] = sd;
      }
      reader_barrier();
      // ---- phase 2: output, computed transposed so each lane holds four
      // consecutive value columns of one token:
      //   O_i^T = S^T Q_i^T diag(gamma_i) + sum_{i' <= i} Ut_{i'}^T P_{i i'}^T.
      // S^T and Ut^T in A-operand layout are exactly the accumulator layouts of
      // S and Ut; Q_i^T and P^T in B-operand layout are row-major reads.
      const int c0 = n * 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 o = zero4();
#pragma unroll
        for (int p = 0; p < NKP; ++p) o = mma2(sfr[2 * p], sfr[2 * p + 1], qr[i][p][0], qr[i][p][1], o);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] *= gm[i];
        if (i == 0) o = mma1(Xf[0], Pm[tri(0, 0)], o);
        if (i == 1) o = mma2(Xf[0], Xf[1], Pm[tri(1, 0)], Pm[tri(1, 1)], o);
        if (i == 2) {
          o = mma2(Xf[0], Xf[1], Pm[tri(2, 0)], Pm[tri(2, 1)], o);
          o = mma2(Xf[2], z4(), Pm[tri(2, 2)], z4(), o);
        }
        if (i == 3) {
          o = mma2(Xf[0], Xf[1], Pm[tri(3, 0)], Pm[tri(3, 1)], o);
          o = mma2(Xf[2], Xf[3], Pm[tri(3, 2)], Pm[tri(3, 3)], o);
        }
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, cvt4(o)), ro, vofO, (c0 + 16 * i) * rowO, 0);
      }
      phase_barrier();
    };

    phase_barrier();  // prologue: chunk 0 staged
    phase_barrier();  // prologue: chunk 0 Gram and diagonal inverses ready
    for (int n = 0; n < nchunks; n += 2) {
      body(ic<0>{}, n);
      if (n + 1 < nchunks) body(ic<1>{}, n + 1);
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
