// decode.hip -- single-token gated delta-rule step on many independent states.
//
// For each state S (dk x dv, row = key dim) and one token:
//   x = S^T kread,  y = S^T qread,  ut = beta (v - alpha x),
//   o = alpha y + (k^T qread) ut,   S <- alpha S + k ut^T,
// which equals S_t = alpha (I - beta k kread^T) S + beta k v^T followed by
// o = S_t^T qread (kread = conj(k), qread = conj(q) for complex data).  The
// fixed-size state with an O(d^2) step is the decode mode of the delta layers
// (Sykra 0.3.3 README, "Computational Complexity": inference step O(d^2) on a
// fixed d x d state).
//
// Memory-bound by design: each state is read once into registers with
// 16-byte coalesced loads, both matrix-vector products are reduced across the
// threads that share a column group (wave shuffles, plus LDS when a state spans
// several waves), and the new state is written once.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int DT> struct StepIn;
template <> struct StepIn<kDtF32> { typedef float el; };
template <> struct StepIn<kDtBF16> { typedef __bf16 el; };
template <> struct StepIn<kDtC64> { typedef float el; };

// Element e of a run of El values held as 32-bit words, as fp32 (bf16 halves
// are taken with shifts, never by extracting a 16-bit vector element).
template <class El> __device__ __forceinline__ float elem(const uint32_t* w, int e) {
  if constexpr (std::is_same_v<El, __bf16>) {
    const uint32_t u = w[e >> 1];
    return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
  } else {
    return __uint_as_float(w[e]);
  }
}

// TPS threads per state.  Each thread holds NP consecutive rows x one 16-byte
// column group, so its slices of k and q are contiguous 16-byte-aligned runs.
template <int DT, int D, int TPS>
__global__ __launch_bounds__(256) void decode_kernel(const void* __restrict__ qg, const void* __restrict__ kg,
                                                     const void* __restrict__ vg, const float* __restrict__ alpha,
                                                     const float* __restrict__ beta, float* __restrict__ S,
                                                     void* __restrict__ outg, int N) {
  constexpr bool CX = DT == kDtC64;
  using El = typename StepIn<DT>::el;
  constexpr int NC = CX ? 2 : 1;      // real components per element
  constexpr int VC = CX ? 2 : 4;      // state columns per 16-byte vector
  constexpr int LPR = D / VC;         // threads across one state row
  constexpr int RPP = TPS / LPR;      // rows covered per pass
  constexpr int NP = D / RPP;         // rows per thread
  constexpr int SPB = 256 / TPS;      // states per block
  constexpr int NRED = 2 * VC * NC + NC;  // x, y, kq components
  static_assert(RPP * LPR == TPS && NP * RPP == D, "layout");

  __shared__ float red[(TPS > 64) ? (TPS / 64) * 64 * NRED : 1];

  const int tid = threadIdx.x;
  const int st = blockIdx.x * SPB + tid / TPS;
  const int lt = tid % TPS;
  const int cg = lt % LPR, rg = lt / LPR;
  const bool live = st < N;
  const int sts = live ? st : 0;  // dead lanes compute on state 0 but never store

  const El* q = static_cast<const El*>(qg) + (size_t)sts * D * NC;
  const El* k = static_cast<const El*>(kg) + (size_t)sts * D * NC;
  const El* v = static_cast<const El*>(vg) + (size_t)sts * D * NC;
  float4* Sv = reinterpret_cast<float4*>(S + (size_t)sts * D * D * NC);
  const float a = alpha[sts], bt = beta[sts];
  const int row0 = NP * rg;  // this thread's rows row0 .. row0 + NP - 1

  // k and q over this thread's rows, and v over its columns, as 16-byte loads.
  constexpr int KW = NP * NC * (int)sizeof(El) / 4;  // 32-bit words
  static_assert(KW % 4 == 0, "row runs of k and q are whole 16-byte units");
  uint32_t kw[KW], qw[KW];
#pragma unroll
  for (int i = 0; i < KW / 4; ++i) {
    reinterpret_cast<uint4*>(kw)[i] = reinterpret_cast<const uint4*>(k + row0 * NC)[i];
    reinterpret_cast<uint4*>(qw)[i] = reinterpret_cast<const uint4*>(q + row0 * NC)[i];
  }
  constexpr int VW = VC * NC * (int)sizeof(El) / 4;
  uint32_t vw[VW];
  if constexpr (VW == 4) {
    *reinterpret_cast<uint4*>(vw) = *reinterpret_cast<const uint4*>(v + cg * VC * NC);
  } else {
    static_assert(VW == 2, "column group of v is 8 or 16 bytes");
    *reinterpret_cast<uint2*>(vw) = *reinterpret_cast<const uint2*>(v + cg * VC * NC);
  }

  float4 s[NP];
  float kr[NP][NC];
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    s[m] = Sv[((row0 + m) * D * NC) / 4 + cg];
#pragma unroll
    for (int p = 0; p < NC; ++p) kr[m][p] = elem<El>(kw, m * NC + p);
  }

  // partial reductions over this thread's rows
  float red_v[NRED];
#pragma unroll
  for (int i = 0; i < NRED; ++i) red_v[i] = 0.f;
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const float* sv = reinterpret_cast<const float*>(&s[m]);
    if constexpr (!CX) {
      const float qv = elem<El>(qw, m);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        red_v[e] += sv[e] * kr[m][0];
        red_v[4 + e] += sv[e] * qv;
      }
      red_v[8] += kr[m][0] * qv;
    } else {
      const float qre = elem<El>(qw, 2 * m), qim = elem<El>(qw, 2 * m + 1);
      const float kre = kr[m][0], kim = kr[m][1];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float sre = sv[2 * e], sim = sv[2 * e + 1];
        // x += S * conj(k), y += S * conj(q)
        red_v[2 * e] += sre * kre + sim * kim;
        red_v[2 * e + 1] += sim * kre - sre * kim;
        red_v[4 + 2 * e] += sre * qre + sim * qim;
        red_v[4 + 2 * e + 1] += sim * qre - sre * qim;
      }
      // kq += k * conj(q)
      red_v[8] += kre * qre + kim * qim;
      red_v[9] += kim * qre - kre * qim;
    }
  }
  // reduce across row groups: lanes that differ by multiples of LPR
#pragma unroll
  for (int off = LPR; off < 64 && off < TPS; off <<= 1)
#pragma unroll
    for (int i = 0; i < NRED; ++i) red_v[i] += __shfl_xor(red_v[i], off, 64);
  if constexpr (TPS > 64) {
    const int wv = lt / 64;  // wave within the state
    if ((lt % 64) < LPR) {
#pragma unroll
      for (int i = 0; i < NRED; ++i) red[(wv * 64 + cg) * NRED + i] = red_v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NRED; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < TPS / 64; ++ww) acc += red[(ww * 64 + cg) * NRED + i];
      red_v[i] = acc;
    }
  }

  // ut = beta (v - alpha x), o = alpha y + kq ut
  float ut[VC][NC], o[VC][NC];
#pragma unroll
  for (int e = 0; e < VC; ++e) {
#pragma unroll
    for (int p = 0; p < NC; ++p) {
      const float vv = elem<El>(vw, e * NC + p);
      ut[e][p] = bt * (vv - a * red_v[e * NC + p]);
    }
    if constexpr (!CX) {
      o[e][0] = a * red_v[4 + e] + red_v[8] * ut[e][0];
    } else {
      o[e][0] = a * red_v[4 + 2 * e] + (red_v[8] * ut[e][0] - red_v[9] * ut[e][1]);
      o[e][1] = a * red_v[4 + 2 * e + 1] + (red_v[8] * ut[e][1] + red_v[9] * ut[e][0]);
    }
  }

  if (!live) return;
  // S <- alpha S + k ut^T
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    float* sv = reinterpret_cast<float*>(&s[m]);
#pragma unroll
    for (int e = 0; e < VC; ++e) {
      if constexpr (!CX) {
        sv[e] = a * sv[e] + kr[m][0] * ut[e][0];
      } else {
        const float sre = sv[2 * e], sim = sv[2 * e + 1];
        sv[2 * e] = a * sre + (kr[m][0] * ut[e][0] - kr[m][1] * ut[e][1]);
        sv[2 * e + 1] = a * sim + (kr[m][0] * ut[e][1] + kr[m][1] * ut[e][0]);
      }
    }
    Sv[((row0 + m) * D * NC) / 4 + cg] = s[m];
  }
  if (rg == 0) {
    El* out = static_cast<El*>(outg) + (size_t)st * D * NC;
#pragma unroll
    for (int e = 0; e < VC; ++e)
#pragma unroll
      for (int p = 0; p < NC; ++p) out[(cg * VC + e) * NC + p] = static_cast<El>(o[e][p]);
  }
}

template <int DT, int D, int TPS>
static hipError_t launch_decode(const StepArgs& a) {
  constexpr int SPB = 256 / TPS;
  const long nblk = ((long)a.N + SPB - 1) / SPB;
  return launch_kernel(decode_kernel<DT, D, TPS>, dim3((unsigned)nblk), dim3(256), (hipStream_t)a.stream, a.q, a.k, a.v,
                       a.alpha, a.beta, a.S, a.out, a.N);
}

hipError_t launch_recurrent_step(const StepArgs& a) {
  if (a.dtype == kDtBF16 && a.dk == 64) return launch_decode<kDtBF16, 64, 64>(a);
  if (a.dtype == kDtBF16 && a.dk == 128) return launch_decode<kDtBF16, 128, 256>(a);
  if (a.dtype == kDtF32 && a.dk == 64) return launch_decode<kDtF32, 64, 64>(a);
  if (a.dtype == kDtF32 && a.dk == 128) return launch_decode<kDtF32, 128, 256>(a);
  if (a.dtype == kDtC64 && a.dk == 32) return launch_decode<kDtC64, 32, 64>(a);
  return hipErrorInvalidValue;
}

}  // namespace gdn
