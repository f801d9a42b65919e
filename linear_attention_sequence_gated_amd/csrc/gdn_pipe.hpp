// gdn_pipe.hpp -- bf16 matrix-core helpers shared by the pipelined chunk
// kernels (chunk_pipe.hip, chunk_two.hip, chunk_grad.hip): buffer resources
// and range-checked loads, LDS barriers, fp32 <-> bf16 packing, 16x16x32 /
// 16x16x16 products, wave prefix sums and broadcasts, the key order of the
// state held in matrix-core accumulators, the chunk records of the two-launch
// forward and the swizzled LDS row layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdn_device.hpp"

namespace gdn {
namespace pipe {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;  // four bf16
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // eight bf16
template <int V> using ic = std::integral_constant<int, V>;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// Bytes from `begin` to `end` of a chain's data, or 0 when there is none
// (T = 0): with a zero range every buffer access is dropped by the range
// check, so loads issued for no chunk never touch memory.
__device__ __forceinline__ uint32_t span_bytes(size_t end, size_t begin) {
  return end > begin ? (uint32_t)(end - begin) : 0u;
}

// Barrier between pipeline stages: waits for this wave's LDS traffic only (so
// global prefetches stay in flight) and stops the scheduler from moving any
// instruction across it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Keeps the loads issued above it from being moved below it.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ u32x2 ld4(const __bf16* p) { return *reinterpret_cast<const u32x2*>(p); }

// Transposed sub-block of a row-major bf16 LDS matrix M (row stride ld):
// lane (g, c) receives M[row0 + 4g + j][col + c], j = 0..3.  `p` must be the
// lane's address &M[row0 + 4g + (c >> 2)][col + 4 (c & 3)].
__device__ __forceinline__ u32x2 ld4_tr(const __bf16* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p)));
}

// fp32 -> bf16 (round to nearest even), two values per v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned cvt2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ u32x2 cvt4(const f32x4& a) { return u32x2{cvt2(a[0], a[1]), cvt2(a[2], a[3])}; }

// bf16 halves of a 32-bit word as fp32.
__device__ __forceinline__ float lo_f(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float hi_f(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts within
// rows of 16, then the row totals are broadcast into the following rows.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  auto shr = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                                 0xf, 0xf, true));
  };
  x += shr(x, ic<0x111>{});  // row_shr:1
  x += shr(x, ic<0x112>{});  // row_shr:2
  x += shr(x, ic<0x114>{});  // row_shr:4
  x += shr(x, ic<0x118>{});  // row_shr:8
  // row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return x;
}

// Value of lane M of this lane's row of 16 (DPP row_newbcast:M; every lane
// has a valid source, so no old value is needed).
template <int M> __device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + M, 0xf, 0xf, true));
}

// Input transforms of a layer (L2 normalisation of query and key rows), for
// kernels that read the rows in 16-byte pieces of eight bf16 values: the
// squared norm of a piece (fp32 sum of squares), and the inverse norm
// 1 / max(|x|, 1e-12) from a row's squared norm.
__device__ __forceinline__ float piece_sumsq(const u32x4& p) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = lo_f(p[e]), b = hi_f(p[e]);
    s = __builtin_fmaf(a, a, s);
    s = __builtin_fmaf(b, b, s);
  }
  return s;
}
__device__ __forceinline__ float inv_row_norm(float sq) { return __builtin_amdgcn_rsqf(fmaxf(sq, 1e-24f)); }
// Sum over NU consecutive lanes (NU = 8 or 16, aligned) that hold the pieces
// of one row.  Lane partners by DPP: xor 1 and xor 2 (quad_perm), then the
// half-row mirror (lane i ^ 7) and the row mirror (lane i ^ 15); once the
// partial sums agree within quads (and half-rows), those mirrors read the same
// values as xor 4 (and xor 8), so every lane of the group ends with the same
// total.
template <int NU> __device__ __forceinline__ float row_piece_sum(float s) {
  static_assert(NU == 8 || NU == 16, "8 or 16 pieces per row");
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value, 0xf,
                                                              0xf, true));
  };
  s += dpp(s, ic<0xB1>{});   // quad_perm [1, 0, 3, 2]
  s += dpp(s, ic<0x4E>{});   // quad_perm [2, 3, 0, 1]
  s += dpp(s, ic<0x141>{});  // row_half_mirror
  if constexpr (NU == 16) s += dpp(s, ic<0x140>{});  // row_mirror
  return s;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ u32x2 z4() { return u32x2{0u, 0u}; }

// c += a b over one 32-wide k block (operands straight from 16-byte loads).
__device__ __forceinline__ f32x4 mma32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// c += [a0 a1] [b0; b1]  (two 16-wide k sub-blocks, one 16x16x32 issue)
__device__ __forceinline__ f32x4 mma2(const u32x2& a0, const u32x2& a1, const u32x2& b0, const u32x2& b1,
                                     const f32x4& c) {
  return mma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, u32x4{b0[0], b0[1], b1[0], b1[1]}, c);
}

// Two 4-element operand pieces as one 8-element 16x16x32 operand.
__device__ __forceinline__ u32x4 pair(const u32x2& a, const u32x2& b) { return u32x4{a[0], a[1], b[0], b[1]}; }

// c += a b  (one 16-wide k sub-block).  Only used where c comes from VALU code
// or is zero: a 16x16x16 issue that reads as its accumulator the result of a
// 16x16x32 issue was observed to be scheduled without the wait states that
// mixed-shape dependency needs, so such chains use 16x16x32 with a zero half.
__device__ __forceinline__ f32x4 mma1(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), c,
                                                   0, 0, 0);
}

__host__ __device__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }   // i >= j
__host__ __device__ constexpr int stri(int i, int j) { return i * (i - 1) / 2 + j; }  // i > j

// Key row of the state held by accumulator block d, lane group g, element j.
// The state update reads K^T with a per-lane address (the transposed LDS read
// takes one per lane), so its output rows can be any 4-row groups: blocks 2p
// and 2p + 1 give lane group g the 8 consecutive keys 32p + 8g .. 32p + 8g + 7.
// K S and Q S then read their K and Q operands as one 16-byte row piece.
__host__ __device__ constexpr int key_row(int d, int g, int j) { return 32 * (d / 2) + 8 * g + 4 * (d % 2) + j; }

// Chunk records of the two-launch forward, read again by the gradient pass.
// One record per (chain, chunk) in the workspace:
//   Tb as six 1 KB blocks of bf16 A operands of 16x16x32 products: block
//   (i, p) holds, in lane L = 16 g + c, the 8 values Tb[16i + c][32p + 4g + j]
//   and Tb[16i + c][32p + 16 + 4g + j] (j = 0..3), the k layout of mma32 with a
//   pair of accumulator tiles as the B operand.  Blocks exist for p <= i / 2;
//   their tiles above the diagonal block are zero.
//   g[64] fp32, the inclusive prefix of log2 alpha over the chunk.
constexpr int kRecTb = 0, kRecG = 6 * 1024, kRecBytes = kRecG + 64 * 4;
__host__ __device__ constexpr int pblk(int i, int p) { return i < 2 ? i : 2 * i - 2 + p; }
// The gradient pass also needs Tb^T, the upper-triangular transpose, as A
// operands: a second record of the same size holds its six blocks (i, p), p
// >= i / 2 (tiles left of the diagonal block zero), then the same g.
__host__ __device__ constexpr int qblk(int i, int p) { return i < 2 ? 2 * i + p : i + 2; }

// Key rows and query rows are staged in LDS unpadded, 16-byte pieces swizzled:
// piece u of row r sits at position u ^ sw(r).  Two read patterns must spread
// over the 64 banks: a 16-lane group reading one piece of sixteen consecutive
// rows (MFMA operands in row order), and the transposed reads of K, where a
// 16-lane group reads pieces 4m .. 4m + 3 (one 8-byte half each) of four
// consecutive rows 4g .. 4g + 3.  sw(r) rotates the bits of r so that both are
// free of conflicts within 16 lanes (at d = 64 two rows share a 256-byte bank
// window, told apart by r & 1).
template <int DK> __device__ __forceinline__ int row_off(int r, int e) {
  constexpr int NU = DK / 8;
  const int sw = DK == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
  return r * DK + (((e >> 3) ^ sw) & (NU - 1)) * 8 + (e & 7);
}

}  // namespace pipe
}  // namespace gdn
