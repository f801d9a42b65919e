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
// 16-byte coalesced non-temporal loads, both matrix-vector products are
// reduced across the threads that share a column group (wave shuffles, plus
// LDS when a state spans several waves), and the new state is written once.
// Each wave streams two states, so HBM reads of one overlap writes of the
// other.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// The state is streamed: read once and written once per step, so its loads and
// stores are non-temporal (they do not displace other data in the caches).
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_stream(float4* p, const float4& x) {
  __builtin_nontemporal_store(f32x4v{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4v*>(p));
}

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
// A workgroup handles NSEQ rounds of 256 / TPS consecutive states.  The loads
// of round r + 1 are issued before round r is reduced and stored, so every
// wave keeps a state in flight while it writes the previous one and HBM reads
// and writes overlap (a state cannot be written before all of its rows have
// been read, which would otherwise make the whole grid read first and write
// afterwards).
template <int DT, int D, int TPS, int NSEQ>
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
  constexpr int SPB = 256 / TPS;      // states per round
  constexpr int NRED = 2 * VC * NC + NC;  // x, y, kq components
  constexpr int KW = NP * NC * (int)sizeof(El) / 4;  // 32-bit words of k / q per thread
  constexpr int VW = VC * NC * (int)sizeof(El) / 4;  // 32-bit words of v per thread
  static_assert(RPP * LPR == TPS && NP * RPP == D, "layout");
  static_assert(KW % 4 == 0, "row runs of k and q are whole 16-byte units");
  static_assert(VW == 4 || VW == 2, "column group of v is 8 or 16 bytes");

  // per-round cross-wave partial sums (double-buffered by round parity)
  __shared__ float red[2][(TPS > 64) ? (TPS / 64) * 64 * NRED : 1];

  const int tid = threadIdx.x;
  const int lt = tid % TPS;
  const int cg = lt % LPR, rg = lt / LPR;
  const int row0 = NP * rg;  // this thread's rows row0 .. row0 + NP - 1

  struct Round {
    float4 s[NP];
    uint32_t kw[KW], qw[KW], vw[VW];
    float a, bt;
  };
  // Rounds past the last state load state N - 1 (always valid memory) and
  // store nothing, so every round issues the same loads.
  auto state_of = [&](int r) { return ((int)blockIdx.x * NSEQ + r) * SPB + tid / TPS; };
  auto load = [&](Round& R, int r) {
    const int st = min(state_of(r), N - 1);
    const El* q = static_cast<const El*>(qg) + (size_t)st * D * NC;
    const El* k = static_cast<const El*>(kg) + (size_t)st * D * NC;
    const El* v = static_cast<const El*>(vg) + (size_t)st * D * NC;
    const float4* Sv = reinterpret_cast<const float4*>(S + (size_t)st * D * D * NC);
#pragma unroll
    for (int m = 0; m < NP; ++m) R.s[m] = load_stream(Sv + ((row0 + m) * D * NC) / 4 + cg);
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      reinterpret_cast<uint4*>(R.kw)[i] = reinterpret_cast<const uint4*>(k + row0 * NC)[i];
      reinterpret_cast<uint4*>(R.qw)[i] = reinterpret_cast<const uint4*>(q + row0 * NC)[i];
    }
    if constexpr (VW == 4)
      *reinterpret_cast<uint4*>(R.vw) = *reinterpret_cast<const uint4*>(v + cg * VC * NC);
    else
      *reinterpret_cast<uint2*>(R.vw) = *reinterpret_cast<const uint2*>(v + cg * VC * NC);
    R.a = alpha[st];
    R.bt = beta[st];
  };
  auto process = [&](Round& R, int r) {
    const int st = state_of(r);
    const bool live = st < N;
    const float a = R.a, bt = R.bt;
    float kr[NP][NC];
#pragma unroll
    for (int m = 0; m < NP; ++m)
#pragma unroll
      for (int p = 0; p < NC; ++p) kr[m][p] = elem<El>(R.kw, m * NC + p);
    // partial reductions over this thread's rows
    float red_v[NRED];
#pragma unroll
    for (int i = 0; i < NRED; ++i) red_v[i] = 0.f;
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const float* sv = reinterpret_cast<const float*>(&R.s[m]);
      if constexpr (!CX) {
        const float qv = elem<El>(R.qw, m);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          red_v[e] += sv[e] * kr[m][0];
          red_v[4 + e] += sv[e] * qv;
        }
        red_v[8] += kr[m][0] * qv;
      } else {
        const float qre = elem<El>(R.qw, 2 * m), qim = elem<El>(R.qw, 2 * m + 1);
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
      float* const rb = red[r & 1];
      const int wv = lt / 64;  // wave within the state
      if ((lt % 64) < LPR) {
#pragma unroll
        for (int i = 0; i < NRED; ++i) rb[(wv * 64 + cg) * NRED + i] = red_v[i];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NRED; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < TPS / 64; ++ww) acc += rb[(ww * 64 + cg) * NRED + i];
        red_v[i] = acc;
      }
    }
    // ut = beta (v - alpha x), o = alpha y + kq ut
    float ut[VC][NC], o[VC][NC];
#pragma unroll
    for (int e = 0; e < VC; ++e) {
#pragma unroll
      for (int p = 0; p < NC; ++p) {
        const float vv = elem<El>(R.vw, e * NC + p);
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
    float4* Sv = reinterpret_cast<float4*>(S + (size_t)st * D * D * NC);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      float* sv = reinterpret_cast<float*>(&R.s[m]);
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
      store_stream(Sv + ((row0 + m) * D * NC) / 4 + cg, R.s[m]);
    }
    if (rg == 0) {
      El* out = static_cast<El*>(outg) + (size_t)st * D * NC;
#pragma unroll
      for (int e = 0; e < VC; ++e)
#pragma unroll
        for (int p = 0; p < NC; ++p) out[(cg * VC + e) * NC + p] = static_cast<El>(o[e][p]);
    }
  };
  Round A, B;
  load(A, 0);
  if constexpr (NSEQ > 1) load(B, 1);
#pragma unroll
  for (int r = 0; r < NSEQ; ++r) {
    Round& X = (r & 1) ? B : A;
    process(X, r);
    if (r + 2 < NSEQ) load(X, r + 2);
  }
}

// Two rounds per workgroup when that still leaves two workgroups per compute
// unit (measured on 4096 states of 64 x 64: 26.8 us against 31.1 us for one
// round and 28.9 us for four), one round below that.
template <int DT, int D, int TPS>
static hipError_t launch_decode(const StepArgs& a) {
  constexpr int SPB = 256 / TPS;
  const long groups = ((long)a.N + SPB - 1) / SPB;
  if (groups >= 2L * 2 * 256) {
    const long nblk = (groups + 1) / 2;
    return launch_kernel(decode_kernel<DT, D, TPS, 2>, dim3((unsigned)nblk), dim3(256), (hipStream_t)a.stream, a.q,
                         a.k, a.v, a.alpha, a.beta, a.S, a.out, a.N);
  }
  return launch_kernel(decode_kernel<DT, D, TPS, 1>, dim3((unsigned)groups), dim3(256), (hipStream_t)a.stream, a.q, a.k,
                       a.v, a.alpha, a.beta, a.S, a.out, a.N);
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
