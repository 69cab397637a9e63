// Executor kernels for rows of any width d = 64 m (m >= 1), for the shapes
// the register-resident kernels of execute.hip do not take: d not a power of
// two, or rows too long to hold in registers (token-centric form: more than
// 4 KiB; expert-centric form: d > 4096).  Pages: gist.science explainer §2.1
// (the atomic expert sigma(x . w_in) w_out, its two vectors rows of the global
// matrices W and V) and interactive explainer "Expert-Centric Scheduling".
//
// A row is taken in chunks of 64 VEC elements, VEC the largest power of two
// that divides m (at most 16 bytes per lane); the chunk count is a run-time
// value, so neither a row nor the y accumulators of a row have to fit in
// registers at once.  Element q of chunk c of a row sits in lane
// (q / VEC) mod 64 at c * 64 VEC + lane * VEC + q mod VEC: the layout of
// RowFrag<T, VEC>, so one chunk is one RowFrag.
//
// Two kernels serve both forms:
//   chunk_coef_kernel   64 tasks per wave; coef = g silu(x_t . W[e]) (gated
//                       variant: times x_t . U[e]), each dot product taken
//                       chunk by chunk with seven (task, chunk) items in
//                       flight.  Expert-centric form: the tasks in the
//                       schedule's sorted order, coef and e written at the
//                       task's flat id; token-centric form: the tasks in
//                       flatten order (the flattened selection).
//   chunk_gather_kernel one wave per (token, chunk of columns): y_t over the
//                       chunk = sum_k coef[t, k] V[e_tk], k in order, fp32
//                       accumulation, written once.
// Both forms compute every coefficient and every y element with the same
// operations in the same order, so they give bit-identical y.
#include "device.hpp"
#include "launch.hpp"
#include "rowfrag.hpp"

namespace omni {

constexpr int kChRing = 8;     // (task, chunk) items per wave: seven in flight
constexpr int kChMaxD = 16384; // widest row the chunked kernels take

// This lane's share of one chunk's dot product, added to p in element order.
template <int VEC>
__device__ __forceinline__ float chunk_dot(const RowFrag<uint16_t, VEC>& a,
                                           const RowFrag<uint16_t, VEC>& b, float p) {
  if constexpr (VEC == 1) {
    return fmaf(a.get(0), b.get(0), p);
  } else {
#pragma unroll
    for (int i = 0; i < RowFrag<uint16_t, VEC>::NW; ++i)
      p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w[i]),
                                          __builtin_bit_cast(bf16x2, b.w[i]), p, false);
    return p;
  }
}
template <int VEC>
__device__ __forceinline__ float chunk_dot(const RowFrag<float, VEC>& a,
                                           const RowFrag<float, VEC>& b, float p) {
#pragma unroll
  for (int q = 0; q < VEC; ++q) p = fmaf(a.f[q], b.f[q], p);
  return p;
}

// h_j = x[t_j] . M[e_j] for the n (1..64) tasks of a wave (token t_j and
// expert e_j in lane j); h_j ends in lane j (lanes from n on: unspecified).
// Item i is chunk i mod nch of task i / nch.  Every load is issued
// unconditionally (items past the last re-read it, and their sums land in no
// lane below n), so the compiler's wait counts keep kChRing - 1 items in
// flight on every path.
template <typename T, int VEC, bool NT>
__device__ __forceinline__ float chunk_dots(const T* __restrict__ x, const T* __restrict__ M,
                                            int my_t, int my_e, int n, int nch, int d, int l) {
  using Frag = RowFrag<T, VEC>;
  constexpr int CH = 64 * VEC;
  Frag fw[kChRing], fx[kChRing];
  int la = 0, lc = 0;  // the next item to load: task la, chunk lc (stays on the last one)
  auto issue = [&](Frag& w, Frag& xr) {
    const size_t off = static_cast<size_t>(lc) * CH;
    w.template fetch<NT>(M + static_cast<size_t>(rdlane(my_e, la)) * d + off, l);
    xr.load(x + static_cast<size_t>(rdlane(my_t, la)) * d + off, l);
    if (lc + 1 < nch) {
      ++lc;
    } else if (la + 1 < n) {
      lc = 0;
      ++la;
    }
  };
#pragma unroll
  for (int s = 0; s < kChRing - 1; ++s) issue(fw[s], fx[s]);
  float my_h = 0.f, p = 0.f;
  int ca = 0, cc = 0;  // the item being computed: task ca, chunk cc
  const int nit = n * nch;
  for (int i = 0; i < nit; i += kChRing) {
#pragma unroll
    for (int s = 0; s < kChRing; ++s) {
      issue(fw[(s + kChRing - 1) % kChRing], fx[(s + kChRing - 1) % kChRing]);
      p = chunk_dot<VEC>(fx[s], fw[s], p);
      if (++cc == nch) {  // uniform over the wave
        const float h = wave_sum(p);
        if (l == ca) my_h = h;
        p = 0.f;
        cc = 0;
        ++ca;
      }
    }
  }
  return my_h;
}

// FLAT: task m is the flattened selection's entry m (token m / K, expert
// texp[m], gate tgate[m]) and its coefficient goes to coef[m] (which may be
// tgate itself: each lane reads its gate before it writes); eflat is not
// written.  Otherwise the tasks are the schedule's (task_token, task_expert,
// task_gate) in sorted order, coef and e written at task_index.  Ids outside
// their range (only from a corrupted list) are mapped to 0.
template <typename T, int VEC, bool GLU, bool NT, bool FLAT>
__global__ __launch_bounds__(256) void chunk_coef_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const T* __restrict__ U,
    const int32_t* __restrict__ ttok, const int32_t* __restrict__ texp, const float* tgate,
    const int32_t* __restrict__ tidx, int M, int K, int d, int L, int N, float* coef,
    int32_t* __restrict__ eflat) {
  const int wv = threadIdx.x >> 6, l = lane();
  const long long m0ll = (static_cast<long long>(blockIdx.x) * 4 + wv) * 64;
  if (m0ll >= M) return;
  const int m0 = static_cast<int>(m0ll);
  const int n = min(64, M - m0);
  int my_t = 0, my_e = 0, my_i = 0;
  float my_g = 0.f;
  if (l < n) {
    const int m = m0 + l;
    if constexpr (FLAT) {
      my_t = m / K;
      my_i = m;
    } else {
      my_t = ttok[m];
      my_i = tidx[m];
    }
    my_e = texp[m];
    my_g = tgate[m];
  }
  my_t = static_cast<unsigned>(my_t) < static_cast<unsigned>(L) ? my_t : 0;
  my_e = static_cast<unsigned>(my_e) < static_cast<unsigned>(N) ? my_e : 0;
  const bool idx_ok = static_cast<unsigned>(my_i) < static_cast<unsigned>(M);
  const int nch = d / (64 * VEC);
  const float h = chunk_dots<T, VEC, NT>(x, W, my_t, my_e, n, nch, d, l);
  float c = my_g * (h / (1.f + __expf(-h)));
  if constexpr (GLU) c *= chunk_dots<T, VEC, NT>(x, U, my_t, my_e, n, nch, d, l);
  if (l < n && idx_ok) {
    coef[my_i] = c;
    if constexpr (!FLAT) eflat[my_i] = my_e;
  }
}

// Wave g: token g / nch, columns [(g mod nch) 64 VEC, +64 VEC).  coef and
// eidx in flatten order (t K + k).
template <typename T, int VEC, bool NT>
__global__ __launch_bounds__(256) void chunk_gather_kernel(
    const T* __restrict__ V, const float* __restrict__ coef, const int32_t* __restrict__ eidx,
    int L, int K, int d, int N, float* __restrict__ y, int accumulate) {
  constexpr int CH = 64 * VEC;
  const int nch = d / CH;
  const long long g = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (g >= static_cast<long long>(L) * nch) return;
  const int t = static_cast<int>(g / nch);
  const size_t col0 = static_cast<size_t>(g % nch) * CH;
  const int l = lane();
  float acc[VEC];
#pragma unroll
  for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
  RowFrag<T, VEC> f[kChRing];
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int n = min(64, K - k0);
    int my_e = 0;
    float my_c = 0.f;
    if (l < n) {
      const size_t o = static_cast<size_t>(t) * K + k0 + l;
      const int e = eidx[o];
      my_e = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
      my_c = coef[o];
    }
    // the rows' chunk: the base pointer moved to the chunk's first column
    token_gather<T, VEC, NT, kChRing, false>(V + col0, my_e, my_c, n, d, l, f, acc);
  }
  store_row<T, VEC, NT ? kStoreDevice : kStoreNT>(acc, y + static_cast<size_t>(t) * d + col0,
                                                  accumulate);
}

int chunk_vec(int bf16, int d) {
  const int m = d / 64, cap = bf16 ? 8 : 4;
  int v = 1;
  while (v < cap && m % (2 * v) == 0) v *= 2;
  return v;
}

bool chunked_supported(int d) { return d >= 64 && d % 64 == 0 && d <= kChMaxD; }

template <typename T, int VEC, bool NT>
static hipError_t chunked_run(int form, bool glu, int L, int d, int N, int K, const T* x, const T* w,
                        const T* u, const T* v, const int32_t* ttok, const int32_t* texp,
                        const float* tgate, const int32_t* tidx, const int32_t* fe,
                        const float* fg, float* y, int acc, void* ws, hipStream_t s) {
  const int M = L * K;
  const size_t half = atomic_forward_ws_bytes(L, K) / 2;
  int32_t* wa = static_cast<int32_t*>(ws);
  float* wb = reinterpret_cast<float*>(static_cast<char*>(ws) + half);
  const dim3 cgrid(static_cast<unsigned>((M + 255) / 256));
  const int32_t* eidx;
  const float* coef;
  if (form == 1) {  // schedule order: coef to wa, e to wb
    float* cf = reinterpret_cast<float*>(wa);
    int32_t* ef = reinterpret_cast<int32_t*>(wb);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(chunk_coef_kernel<T, VEC, false, NT, false>), cgrid,
                       dim3(256), 0, s, x, w, static_cast<const T*>(nullptr), ttok, texp, tgate,
                       tidx, M, K, d, L, N, cf, ef);
    coef = cf;
    eidx = ef;
  } else {  // flatten order: the caller's lists, or the schedule inverted into wa / wb
    if (!fe) {
      const hipError_t e = launch_unpermute(texp, tgate, tidx, M, N, wa, wb, s);
      if (e != hipSuccess) return e;
      fe = wa;
      fg = wb;
    }
    // coefficients to wb (over the inverted gates, each read before written)
    if (glu)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(chunk_coef_kernel<T, VEC, true, NT, true>), cgrid,
                         dim3(256), 0, s, x, w, u, static_cast<const int32_t*>(nullptr), fe, fg,
                         static_cast<const int32_t*>(nullptr), M, K, d, L, N, wb,
                         static_cast<int32_t*>(nullptr));
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(chunk_coef_kernel<T, VEC, false, NT, true>), cgrid,
                         dim3(256), 0, s, x, w, static_cast<const T*>(nullptr),
                         static_cast<const int32_t*>(nullptr), fe, fg,
                         static_cast<const int32_t*>(nullptr), M, K, d, L, N, wb,
                         static_cast<int32_t*>(nullptr));
    coef = wb;
    eidx = fe;
  }
  const long long waves = static_cast<long long>(L) * (d / (64 * VEC));
  hipLaunchKernelGGL(HIP_KERNEL_NAME(chunk_gather_kernel<T, VEC, NT>),
                     dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, s, v, coef, eidx,
                     L, K, d, N, y, acc);
  return hipGetLastError();
}

template <typename T, bool NT>
static hipError_t chunked_vec(int bf16, int form, bool glu, int L, int d, int N, int K, const T* x,
                        const T* w, const T* u, const T* v, const int32_t* ttok,
                        const int32_t* texp, const float* tgate, const int32_t* tidx,
                        const int32_t* fe, const float* fg, float* y, int acc, void* ws,
                        hipStream_t s) {
#define OMNI_CH(VEC_)                                                                          \
  return chunked_run<T, VEC_, NT>(form, glu, L, d, N, K, x, w, u, v, ttok, texp, tgate, tidx, \
                                  fe, fg, y, acc, ws, s)
  switch (chunk_vec(bf16, d)) {
    case 1: OMNI_CH(1);
    case 2: OMNI_CH(2);
    case 4: OMNI_CH(4);
    case 8:
      if constexpr (sizeof(T) == 2) OMNI_CH(8);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
#undef OMNI_CH
}

hipError_t launch_chunked(int bf16, int form, bool glu, int L, int d, int N, int K,
                          const void* x, const void* w, const void* u, const void* v,
                          const int32_t* task_token, const int32_t* task_expert,
                          const float* task_gate, const int32_t* task_index,
                          const int32_t* flat_expert, const float* flat_gate, float* y,
                          bool accumulate, void* ws, hipStream_t s) {
  if (!chunked_supported(d) || (glu && form != 2) || (form != 1 && form != 2))
    return hipErrorInvalidValue;
  const int M = L * K;
  const bool nt = stream_rows(M, N);
  const int acc = accumulate ? 1 : 0;
  if (bf16) {
    const auto* xb = static_cast<const uint16_t*>(x);
    const auto* wb = static_cast<const uint16_t*>(w);
    const auto* ub = static_cast<const uint16_t*>(u);
    const auto* vb = static_cast<const uint16_t*>(v);
    return nt ? chunked_vec<uint16_t, true>(1, form, glu, L, d, N, K, xb, wb, ub, vb,
                                            task_token, task_expert, task_gate, task_index,
                                            flat_expert, flat_gate, y, acc, ws, s)
              : chunked_vec<uint16_t, false>(1, form, glu, L, d, N, K, xb, wb, ub, vb,
                                             task_token, task_expert, task_gate, task_index,
                                             flat_expert, flat_gate, y, acc, ws, s);
  } else {
    const auto* xf = static_cast<const float*>(x);
    const auto* wf = static_cast<const float*>(w);
    const auto* uf = static_cast<const float*>(u);
    const auto* vf = static_cast<const float*>(v);
    return nt ? chunked_vec<float, true>(0, form, glu, L, d, N, K, xf, wf, uf, vf, task_token,
                                         task_expert, task_gate, task_index, flat_expert,
                                         flat_gate, y, acc, ws, s)
              : chunked_vec<float, false>(0, form, glu, L, d, N, K, xf, wf, uf, vf, task_token,
                                          task_expert, task_gate, task_index, flat_expert,
                                          flat_gate, y, acc, ws, s);
  }
}

}  // namespace omni
