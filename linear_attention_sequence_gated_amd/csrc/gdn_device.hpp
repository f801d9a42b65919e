// gdn_device.hpp -- gfx950 building blocks shared by the gated delta-rule kernels.
//
// Matrix-core products are written in terms of 16-wide k "sub-blocks".  In a
// 64-lane wave, lane l = 16*g + c (c = l % 16, g = l / 16) holds, for one
// sub-block, the 4 operand values at k = 4g + j (j = 0..3):
//   - an A operand (M x K) holds row m = c, columns k = 4g + j;
//   - a B operand (K x N) holds column n = c, rows k = 4g + j.
// This is exactly the row layout of a 16x16 fp32 accumulator tile (lane holds
// rows 4g + j of column c), so an accumulator of X can be fed back as the B
// operand of Y * X (or the A operand of X^T * Y) with no data movement.
//   bf16 engine: v_mfma_f32_16x16x32_bf16 consumes two sub-blocks per issue.
//   fp32 engine: v_mfma_f32_16x16x4f32 consumes one sub-block in 4 issues.
// Both engines accumulate in fp32.  Complex operands are carried as separate
// real and imaginary planes and multiplied with four real products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kDtF32 = 0, kDtBF16 = 1, kDtC64 = 2;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Barrier for LDS producer/consumer hand-off.  Waits only for this wave's LDS
// traffic, so global prefetches issued earlier stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- sub-blocks
template <class Op> struct SubT;
template <> struct SubT<__bf16> { typedef bf16x4 type; };
template <> struct SubT<float> { typedef f32x4 type; };
template <class Op> using Sub = typename SubT<Op>::type;

template <class Op> __device__ __forceinline__ Sub<Op> sub_zero() {
  Sub<Op> z;
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = (Op)0.0f;
  return z;
}

// Four consecutive values at p (p must be 8-byte aligned for bf16, 16 for fp32).
template <class Op> __device__ __forceinline__ Sub<Op> sub_load(const Op* p) {
  return *reinterpret_cast<const Sub<Op>*>(p);
}

template <class Op> __device__ __forceinline__ Sub<Op> sub_from_acc(const f32x4& a) {
  if constexpr (std::is_same_v<Op, float>) {
    return a;
  } else {
    Sub<Op> s;
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = (Op)a[j];
    return s;
  }
}

template <class Op> __device__ __forceinline__ Sub<Op> sub_neg(const Sub<Op>& a) {
  Sub<Op> s;
#pragma unroll
  for (int j = 0; j < 4; ++j) s[j] = -a[j];
  return s;
}

// c += sum_{s < n} a[s] * b[s] over n sub-blocks (n is a compile-time constant
// after unrolling at every call site).
template <class Op, int NMAX>
__device__ __forceinline__ void mma_sub(f32x4& c, const Sub<Op> (&a)[NMAX], const Sub<Op> (&b)[NMAX], int n) {
  if constexpr (std::is_same_v<Op, float>) {
#pragma unroll
    for (int s = 0; s < NMAX; ++s) {
      if (s < n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s][j], b[s][j], c, 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < (NMAX + 1) / 2; ++p) {
      if (2 * p < n) {
        bf16x8 fa, fb;
        const bool two = (2 * p + 1 < n) && (2 * p + 1 < NMAX);
        Sub<Op> a1 = two ? a[(2 * p + 1) < NMAX ? 2 * p + 1 : 0] : sub_zero<Op>();
        Sub<Op> b1 = two ? b[(2 * p + 1) < NMAX ? 2 * p + 1 : 0] : sub_zero<Op>();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fa[j] = a[2 * p][j];
          fb[j] = b[2 * p][j];
          fa[4 + j] = a1[j];
          fb[4 + j] = b1[j];
        }
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, c, 0, 0, 0);
      }
    }
  }
}

// ------------------------------------------------------ real / complex values
// A value of the field: one plane for real data, (re, im) planes for complex.
template <bool CX, class T> struct Fv {
  T v[CX ? 2 : 1];
};
template <bool CX> using Acc = Fv<CX, f32x4>;
template <bool CX, class Op> using CSub = Fv<CX, Sub<Op>>;

template <bool CX> __device__ __forceinline__ Acc<CX> acc_zero() {
  Acc<CX> a;
#pragma unroll
  for (int p = 0; p < (CX ? 2 : 1); ++p) a.v[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  return a;
}

template <bool CX, class Op> __device__ __forceinline__ CSub<CX, Op> csub_from_acc(const Acc<CX>& a) {
  CSub<CX, Op> s;
#pragma unroll
  for (int p = 0; p < (CX ? 2 : 1); ++p) s.v[p] = sub_from_acc<Op>(a.v[p]);
  return s;
}

template <bool CX, class Op> __device__ __forceinline__ CSub<CX, Op> csub_zero() {
  CSub<CX, Op> s;
#pragma unroll
  for (int p = 0; p < (CX ? 2 : 1); ++p) s.v[p] = sub_zero<Op>();
  return s;
}

// c += sum_s op(a[s]) * op(b[s]) over n sub-blocks, where op conjugates when
// CA / CB is set (complex only).
template <bool CX, class Op, bool CA, bool CB, int NMAX>
__device__ __forceinline__ void cmma(Acc<CX>& c, const CSub<CX, Op> (&a)[NMAX], const CSub<CX, Op> (&b)[NMAX], int n) {
  Sub<Op> ar[NMAX], br[NMAX];
#pragma unroll
  for (int s = 0; s < NMAX; ++s) { ar[s] = a[s].v[0]; br[s] = b[s].v[0]; }
  mma_sub<Op, NMAX>(c.v[0], ar, br, n);
  if constexpr (CX) {
    Sub<Op> ai[NMAX], bi[NMAX], ain[NMAX];
    // re += -(sa*sb) * ai*bi ;  im += sb * ar*bi + sa * ai*br  with sa = CA ? -1 : 1, sb likewise
#pragma unroll
    for (int s = 0; s < NMAX; ++s) {
      ai[s] = CA ? sub_neg<Op>(a[s].v[1]) : a[s].v[1];
      bi[s] = CB ? sub_neg<Op>(b[s].v[1]) : b[s].v[1];
      ain[s] = sub_neg<Op>(ai[s]);
    }
    mma_sub<Op, NMAX>(c.v[0], ain, bi, n);
    mma_sub<Op, NMAX>(c.v[1], ar, bi, n);
    mma_sub<Op, NMAX>(c.v[1], ai, br, n);
  }
}

// ----------------------------------------------------------- LDS matrix views
// Row-major matrix in LDS, one plane per real component.
template <bool CX, class Op> struct LdsMat {
  Op* base;
  int ld;      // row stride (elements)
  int pstride; // distance between planes (elements)
  __device__ __forceinline__ Op* at(int p, int r, int c) const { return base + p * pstride + r * ld + c; }
};

// Sub-block of the operand whose lane row is `row` (this lane's m or n) and
// whose k range starts at col16 (lane reads k = col16 + 4g + j).
template <bool CX, class Op>
__device__ __forceinline__ CSub<CX, Op> csub_rows(const LdsMat<CX, Op>& m, int row, int col16) {
  const int g = lane_id() >> 4;
  CSub<CX, Op> s;
#pragma unroll
  for (int p = 0; p < (CX ? 2 : 1); ++p) s.v[p] = sub_load<Op>(m.at(p, row, col16 + 4 * g));
  return s;
}

// ------------------------------------------------------------ element access
template <class T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

}  // namespace gdn
