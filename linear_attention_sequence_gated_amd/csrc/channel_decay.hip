// channel_decay.hip -- the delta rule with a per-output-channel decay, token
// by token: real data with d_k = d_v = 64 (fp32 or bf16 q, k, v; fp32 decay,
// beta and state) and complex data with d_k = d_v = 32 (complex64 q, k, v and
// state; real decay and beta).
//
// DeltaPhase README, section 2 (the gated-decay variant that LaplacePhaseCore
// implements) and section 5 (the decay diag(r_t) on the memory's output rows):
// the memory is read through the key before it decays, and the error is
// written along the key.  With the state S [dk, dv] the output rows of the
// memory are the columns of S, and column j evolves on its own:
//   e_j = v_j - k^T s_j,   s_j <- r_j s_j + beta k e_j,   o_j = q^T s_j.
// The real token loop serves fp32 inputs (bf16 takes the chunk form).  A
// lane quad holds one column: lane l of wave w owns column 16 w + l / 4 and
// rows 16 (l % 4) .. + 15.  k^T s_j and q^T s_j are 16-term in-lane sums and
// two DPP adds.  Keys and queries are read from global memory by every lane
// (16 consecutive elements each), eight tokens ahead of their use; there is no
// LDS and no barrier.  Waves are independent: one workgroup of one wave per
// (chain, 16-column slice).
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_lane.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace chd {

using lane::quad_sum;
using lane::Row;

constexpr int D = 64;  // head dimension
constexpr int R = 16;  // rows per lane

__device__ __forceinline__ float f32(float x) { return x; }
__device__ __forceinline__ float f32(__hip_bfloat16 x) { return __bfloat162float(x); }
__device__ __forceinline__ void st(float* p, float x) { *p = x; }
__device__ __forceinline__ void st(__hip_bfloat16* p, float x) { *p = __float2bfloat16(x); }

template <class IT>
__global__ __launch_bounds__(64) void channel_decay_kernel(const IT* __restrict__ q, const IT* __restrict__ k,
                                                           const IT* __restrict__ v, const float* __restrict__ r,
                                                           const float* __restrict__ beta,
                                                           const float* __restrict__ S0, IT* __restrict__ out,
                                                           float* __restrict__ Sf, int T, int H) {
  const int l = threadIdx.x, slice = blockIdx.x & 3, chain = blockIdx.x >> 2;
  const int b = chain / H, h = chain % H;
  const int c = 16 * slice + (l >> 2), rq = l & 3, i0 = R * rq;
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };

  float s[R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) s[ii] = S0 ? S0[((size_t)chain * D + i0 + ii) * D + c] : 0.f;

  // This lane's inputs of one token (t clamped into [0, T), valid when T > 0),
  // kept as stored until used so that loading the next token never waits.
  struct Tok {
    Row<IT> k, q;
    IT v;
    float r, be;
  };
  auto load = [&](int t) {
    Tok x;
    const size_t rt = tok(max(0, min(t, T - 1)));
    x.k.load(k + rt * D + i0);
    x.q.load(q + rt * D + i0);
    x.v = v[rt * D + c];
    x.r = r[rt * D + c];
    x.be = beta[rt];
    return x;
  };

  // One token on s; o is stored by the quad's first lane.
  auto step = [&](const Tok& x, int t) {
    float u = 0.f;
#pragma unroll
    for (int ii = 0; ii < R; ++ii) u += x.k[ii] * s[ii];
    u = quad_sum(u);
    const float y = x.be * (f32(x.v) - u);  // error from the undecayed state
    float o = 0.f;
#pragma unroll
    for (int ii = 0; ii < R; ++ii) {
      s[ii] = x.r * s[ii] + x.k[ii] * y;
      o += x.q[ii] * s[ii];
    }
    o = quad_sum(o);
    if (rq == 0) st(out + tok(t) * D + c, o);
  };

  // Inputs are loaded PF tokens ahead (a token takes well under a memory
  // latency), in a ring of registers indexed at compile time; the loads are
  // unconditional (clamped), so the compiler's in-order load counts are static.
  constexpr int PF = 8;
  if (T > 0) {  // T = 0: the input buffers may be empty
    Tok ring[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[p] = load(p);
    for (int t = 0; t < T; t += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        if (t + p < T) step(ring[p], t + p);
        ring[p] = load(t + p + PF);
      }
    }
  }
  if (Sf) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) Sf[((size_t)chain * D + i0 + ii) * D + c] = s[ii];
  }
}

// Complex data, d_k = d_v = 32 (LaplacePhaseCore's keys are complex,
// e^{s dt} with Re(s) <= 0; DeltaPhase README, section 5): the same rule with
// the read through the conjugated key and query,
//   e_j = v_j - sum_i conj(k_i) s_ij,   s_ij <- r_j s_ij + beta k_i e_j,
//   o_j = sum_i conj(q_i) s_ij,
// r real.  The columns are independent, so each chain runs as eight waves of
// 4 columns (one 64-thread workgroup each): lane l owns column 4 g + l / 16 of
// its group g and rows 2 (l % 16) .. + 1, as (re, im) pairs; the column sums
// are 2-term in-lane sums and a 16-lane DPP sum.  (A wave issues one vector
// instruction per 4 cycles, so a token step costs about the instructions of
// one lane: with 4 rows per lane, four waves per chain, it took a third longer.)
// Each wave stages its inputs in LDS a block of 8 tokens ahead (k and q rows,
// its columns of v and r, beta), so the memory latency hides behind the
// previous block's steps.
constexpr int DC = 32;
constexpr int CG = 4;    // columns per wave
constexpr int RC = 2;    // rows per lane
constexpr int LPC = DC / RC;  // lanes per column
constexpr int NGC = DC / CG;
constexpr int BT = 8;    // tokens per staged block
static_assert(LPC * CG == 64, "one column per 16-lane row");

// Sum over the 16 lanes of a column (one DPP row): xor 1, xor 2 (quad_perm),
// then the half-row mirror and the row mirror, each of which reads a partner
// whose partial sum covers the other half once the smaller groups agree.
// Every lane of the row ends with the same value.
template <int ctrl> __device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  return v + dpp_mov<0x140>(v);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct CxBlk {
  float k[BT][2 * DC], q[BT][2 * DC], v[BT][2 * CG], r[BT][CG], be[BT];
};

__global__ __launch_bounds__(64) void channel_decay_c64_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                               const float* __restrict__ v, const float* __restrict__ r,
                                                               const float* __restrict__ beta,
                                                               const float* __restrict__ S0, float* __restrict__ out,
                                                               float* __restrict__ Sf, int T, int H) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) CxBlk buf[2];
  const int l = threadIdx.x;
  // The hardware deals consecutive blocks to the eight XCDs in turn; remap so
  // that a chain's groups share an XCD and its k and q rows are fetched once
  // into that XCD's L2.
  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int grp = bid % NGC, chain = bid / NGC, b = chain / H, h = chain % H;
  const int cl = l / LPC, c = grp * CG + cl, i0 = RC * (l % LPC);
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };
  float sr[RC], si[RC];
#pragma unroll
  for (int ii = 0; ii < RC; ++ii) {
    const size_t e = ((size_t)chain * DC + i0 + ii) * DC + c;
    sr[ii] = S0 ? S0[2 * e] : 0.f;
    si[ii] = S0 ? S0[2 * e + 1] : 0.f;
  }
  // A block's inputs in registers: k and q rows (512 floats each: 2 float4 per
  // lane), v of the group's columns (64 floats: 1 per lane), r (32: lanes 0 ..
  // 31), beta (lanes 0 .. 7).  Tokens past T read token T - 1 (never used).
  struct Regs {
    f4 k[2], q[2];
    float v, r, be;
  };
  auto load_block = [&](int blk) {
    Regs x;
    const int t0 = blk * BT;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = (l + 64 * u) * 4, m = f / (2 * DC), e = f % (2 * DC);
      const size_t rt = tok(min(t0 + m, T - 1));
      x.k[u] = *reinterpret_cast<const f4*>(k + rt * 2 * DC + e);
      x.q[u] = *reinterpret_cast<const f4*>(q + rt * 2 * DC + e);
    }
    {
      const int m = l / (2 * CG), e = l % (2 * CG);
      x.v = v[tok(min(t0 + m, T - 1)) * 2 * DC + 2 * grp * CG + e];
    }
    {
      const int m = (l & 31) / CG, e = l % CG;
      x.r = r[tok(min(t0 + m, T - 1)) * DC + grp * CG + e];
    }
    x.be = beta[tok(min(t0 + (l & 7), T - 1))];
    return x;
  };
  auto store_block = [&](const Regs& x, CxBlk& B) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = (l + 64 * u) * 4, m = f / (2 * DC), e = f % (2 * DC);
      *reinterpret_cast<f4*>(&B.k[m][e]) = x.k[u];
      *reinterpret_cast<f4*>(&B.q[m][e]) = x.q[u];
    }
    B.v[l / (2 * CG)][l % (2 * CG)] = x.v;
    if (l < BT * CG) B.r[l / CG][l % CG] = x.r;
    if (l < BT) B.be[l] = x.be;
  };
  const int nblk = (T + BT - 1) / BT;
  if (nblk > 0) {
    Regs x = load_block(0);
    for (int blk = 0; blk < nblk; ++blk) {
      CxBlk& B = buf[blk & 1];
      wave_sync();  // the block two back has been read
      store_block(x, B);
      wave_sync();
      if (blk + 1 < nblk) x = load_block(blk + 1);
      // One token of the block.  Every lane of a column's 16 ends with the same sums (sum16), so all of
      // them store them: no per-lane branch splits the unrolled block, and the compiler can issue a token's
      // LDS reads during the previous token's arithmetic.
      auto token = [&](int m) {
        const f4 ka = *reinterpret_cast<const f4*>(&B.k[m][2 * i0]);
        const f4 qa = *reinterpret_cast<const f4*>(&B.q[m][2 * i0]);
        const float kr[RC] = {ka.x, ka.z}, ki[RC] = {ka.y, ka.w};
        const float qr[RC] = {qa.x, qa.z}, qi[RC] = {qa.y, qa.w};
        const float rr = B.r[m][cl], be = B.be[m];
        const float vr = B.v[m][2 * cl], vi = B.v[m][2 * cl + 1];
        float ur = 0.f, ui = 0.f;  // sum_i conj(k_i) s_i
#pragma unroll
        for (int ii = 0; ii < RC; ++ii) {
          ur += kr[ii] * sr[ii] + ki[ii] * si[ii];
          ui += kr[ii] * si[ii] - ki[ii] * sr[ii];
        }
        ur = sum16(ur);
        ui = sum16(ui);
        const float er = be * (vr - ur), ei = be * (vi - ui);  // beta e
        float orr = 0.f, oi = 0.f;
#pragma unroll
        for (int ii = 0; ii < RC; ++ii) {
          const float nr = rr * sr[ii] + (kr[ii] * er - ki[ii] * ei);
          const float ni = rr * si[ii] + (kr[ii] * ei + ki[ii] * er);
          sr[ii] = nr;
          si[ii] = ni;
          orr += qr[ii] * nr + qi[ii] * ni;  // conj(q) s
          oi += qr[ii] * ni - qi[ii] * nr;
        }
        orr = sum16(orr);
        oi = sum16(oi);
        *reinterpret_cast<float2*>(out + (tok(blk * BT + m) * DC + c) * 2) = float2{orr, oi};
      };
      if ((blk + 1) * BT <= T) {
#pragma unroll
        for (int m = 0; m < BT; ++m) token(m);
      } else {  // the ragged last block
        const int mend = T - blk * BT;
#pragma unroll
        for (int m = 0; m < BT; ++m)
          if (m < mend) token(m);
      }
    }
  }
  if (Sf) {
#pragma unroll
    for (int ii = 0; ii < RC; ++ii) {
      const size_t e = ((size_t)chain * DC + i0 + ii) * DC + c;
      Sf[2 * e] = sr[ii];
      Sf[2 * e + 1] = si[ii];
    }
  }
}

}  // namespace chd

hipError_t launch_channel_decay(const ChannelArgs& a) {
  if (a.dtype == kDtC64)
    return launch_kernel(chd::channel_decay_c64_kernel, dim3((unsigned)((long)a.B * a.H * chd::NGC)), dim3(64),
                         (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v, a.r, a.beta,
                         (const float*)a.S0, (float*)a.out, (float*)a.S_final, a.T, a.H);
  const dim3 grid((unsigned)((long)a.B * a.H * 4)), block(64);
  if (a.dtype == kDtBF16)
    return launch_kernel(chd::channel_decay_kernel<__hip_bfloat16>, grid, block, (hipStream_t)a.stream,
                         (const __hip_bfloat16*)a.q, (const __hip_bfloat16*)a.k, (const __hip_bfloat16*)a.v, a.r,
                         a.beta, a.S0, (__hip_bfloat16*)a.out, a.S_final, a.T, a.H);
  return launch_kernel(chd::channel_decay_kernel<float>, grid, block, (hipStream_t)a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, a.r, a.beta, a.S0, (float*)a.out, a.S_final, a.T, a.H);
}

}  // namespace gdn
