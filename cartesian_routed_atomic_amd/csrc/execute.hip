// Expert-centric execution of the schedule.  Pages: gist.science explainer
// §2.1 (atomic expert E_i(x) = sigma(x . w_in) w_out; all experts live in the
// global matrices W, V in R^{N x d}) and interactive explainer
// "Expert-Centric Scheduling" (each group's parameters are loaded once and
// reused for every token assigned to the group; parameter traffic
// 2d * |E_active| instead of 2d * L * K).
//
// The kernel walks the task list in its (group, token) order.  Each wave
// owns a contiguous run of tasks; per task it streams W[e] and V[e] from HBM
// with 16-byte loads (the next task's rows are in flight while the current
// one is computed), forms h = x_t . W[e] with a wave reduction, and adds
// g * silu(h) * V[e] into a per-token register accumulator.  When the token
// changes (the end of a (group, token) run) the accumulator is added into
// y[t] with float32 atomics, 256 contiguous bytes per instruction after a
// small LDS transpose.  Workgroups are laid out XCD by XCD over the task
// list, so one group's tasks run on one XCD and an expert used by several
// tokens of the group is re-read from that XCD's L2, not from HBM.
#include "device.hpp"
#include "launch.hpp"

namespace omni {

// A row fragment of one lane: EPL elements held raw (as loaded) so a load
// can stay in flight until the first use; element q = c * VEC + j maps to
// row[c * 64 * VEC + lane * VEC + j].
template <typename T, int EPL> struct RowFrag;

template <int EPL> struct RowFrag<uint16_t, EPL> {  // bfloat16 bits
  static constexpr int VEC = EPL < 8 ? EPL : 8;
  static constexpr int NCH = EPL / VEC;
  static constexpr int NW = (EPL + 1) / 2;
  uint32_t w[NW];
  __device__ __forceinline__ void load(const uint16_t* row, int l) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint16_t* p = row + c * 64 * VEC + l * VEC;
      if constexpr (VEC == 8) *reinterpret_cast<uint4*>(&w[c * 4]) = *reinterpret_cast<const uint4*>(p);
      else if constexpr (VEC == 4) *reinterpret_cast<uint2*>(&w[c * 2]) = *reinterpret_cast<const uint2*>(p);
      else if constexpr (VEC == 2) w[c] = *reinterpret_cast<const uint32_t*>(p);
      else w[0] = static_cast<uint32_t>(*p);
    }
  }
  __device__ __forceinline__ float get(int q) const {
    if constexpr (VEC == 1) return bf_lo(w[0]);
    else return (q & 1) ? bf_hi(w[q >> 1]) : bf_lo(w[q >> 1]);
  }
};

template <int EPL> struct RowFrag<float, EPL> {
  static constexpr int VEC = EPL < 4 ? EPL : 4;
  static constexpr int NCH = EPL / VEC;
  float f[EPL];
  __device__ __forceinline__ void load(const float* row, int l) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float* p = row + c * 64 * VEC + l * VEC;
      if constexpr (VEC == 4) *reinterpret_cast<float4*>(&f[c * 4]) = *reinterpret_cast<const float4*>(p);
      else if constexpr (VEC == 2) *reinterpret_cast<float2*>(&f[c * 2]) = *reinterpret_cast<const float2*>(p);
      else f[0] = *p;
    }
  }
  __device__ __forceinline__ float get(int q) const { return f[q]; }
};

__device__ __forceinline__ int rdlane(int v, int i) { return __builtin_amdgcn_readlane(v, i); }
__device__ __forceinline__ float rdlane(float v, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
}

constexpr int kExecWaves = 4;  // waves per workgroup

template <typename T, int EPL>
__global__ __launch_bounds__(256) void atomic_forward_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const T* __restrict__ V,
    const int32_t* __restrict__ ttok, const int32_t* __restrict__ texp,
    const float* __restrict__ tgate, int M, int d, int L, int N, int chunk, int nblk,
    float* __restrict__ y) {
  using Frag = RowFrag<T, EPL>;
  constexpr int VEC = Frag::VEC, NCH = Frag::NCH;
  __shared__ float tr[kExecWaves][64 * VEC];

  const int wv = threadIdx.x >> 6, l = lane();
  // XCD-contiguous workgroup order (workgroup b runs on XCD b % 8)
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int logical = xcd * per + min(xcd, rem) + loc;
  const long long m0ll = (static_cast<long long>(logical) * kExecWaves + wv) * chunk;
  if (m0ll >= M) return;
  const int m0 = static_cast<int>(m0ll);
  const int n = min(chunk, M - m0);

  // task metadata of the run, one task per lane (chunk <= 64)
  // ids outside [0, L) / [0, N) (only from a corrupted schedule) are mapped
  // to 0 so every access stays in bounds
  int my_t = (l < n) ? ttok[m0 + l] : 0;
  int my_e = (l < n) ? texp[m0 + l] : 0;
  my_t = static_cast<unsigned>(my_t) < static_cast<unsigned>(L) ? my_t : 0;
  my_e = static_cast<unsigned>(my_e) < static_cast<unsigned>(N) ? my_e : 0;
  const float my_g = (l < n) ? tgate[m0 + l] : 0.f;

  float acc[EPL];
  float xf[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
  int cur = rdlane(my_t, 0);
  {
    Frag xr;
    xr.load(x + static_cast<size_t>(cur) * d, l);
#pragma unroll
    for (int q = 0; q < EPL; ++q) xf[q] = xr.get(q);
  }

  auto flush = [&](int t) {
    float* yt = y + static_cast<size_t>(t) * d;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) tr[wv][l * VEC + j] = acc[c * VEC + j];
      wave_lds_fence();
#pragma unroll
      for (int q = 0; q < VEC; ++q)
        unsafeAtomicAdd(yt + c * 64 * VEC + q * 64 + l, tr[wv][q * 64 + l]);
      wave_lds_fence();
    }
  };

  auto process = [&](int i, const Frag& wf, const Frag& vf) {
    const int t = rdlane(my_t, i);
    if (t != cur) {
      flush(cur);
#pragma unroll
      for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
      cur = t;
      Frag xr;
      xr.load(x + static_cast<size_t>(cur) * d, l);
#pragma unroll
      for (int q = 0; q < EPL; ++q) xf[q] = xr.get(q);
    }
    float p = 0.f;
#pragma unroll
    for (int q = 0; q < EPL; ++q) p = fmaf(xf[q], wf.get(q), p);
    const float h = wave_sum(p);
    const float c = rdlane(my_g, i) * (h / (1.f + __expf(-h)));
#pragma unroll
    for (int q = 0; q < EPL; ++q) acc[q] = fmaf(c, vf.get(q), acc[q]);
  };

  // two tasks in flight: while one is computed the other's rows load
  Frag wa, va, wb, vb;
  {
    const int e = rdlane(my_e, 0);
    wa.load(W + static_cast<size_t>(e) * d, l);
    va.load(V + static_cast<size_t>(e) * d, l);
  }
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) {
      const int e = rdlane(my_e, i + 1);
      wb.load(W + static_cast<size_t>(e) * d, l);
      vb.load(V + static_cast<size_t>(e) * d, l);
    }
    process(i, wa, va);
    if (i + 1 >= n) break;
    if (i + 2 < n) {
      const int e = rdlane(my_e, i + 2);
      wa.load(W + static_cast<size_t>(e) * d, l);
      va.load(V + static_cast<size_t>(e) * d, l);
    }
    process(i + 1, wb, vb);
  }
  flush(cur);
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* __restrict__ p, size_t n4) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename T, int EPL>
static void launch_exec_t(const T* x, const T* w, const T* v, const int32_t* tt,
                          const int32_t* te, const float* tg, int M, int d, int L, int N,
                          float* y, hipStream_t s) {
  // ~16 waves per CU over 256 CUs at full size, at most 64 tasks per wave
  int chunk = M / (256 * 16);
  chunk = chunk < 1 ? 1 : (chunk > 64 ? 64 : chunk);
  const long long waves = (static_cast<long long>(M) + chunk - 1) / chunk;
  const int nblk = static_cast<int>((waves + kExecWaves - 1) / kExecWaves);
  atomic_forward_kernel<T, EPL><<<nblk, 64 * kExecWaves, 0, s>>>(x, w, v, tt, te, tg, M, d, L,
                                                                 N, chunk, nblk, y);
}

template <typename T>
static bool dispatch_exec(const T* x, const T* w, const T* v, const int32_t* tt,
                          const int32_t* te, const float* tg, int M, int d, int L, int N,
                          float* y, hipStream_t s) {
  switch (d) {
    case 64: launch_exec_t<T, 1>(x, w, v, tt, te, tg, M, d, L, N, y, s); return true;
    case 128: launch_exec_t<T, 2>(x, w, v, tt, te, tg, M, d, L, N, y, s); return true;
    case 256: launch_exec_t<T, 4>(x, w, v, tt, te, tg, M, d, L, N, y, s); return true;
    case 512: launch_exec_t<T, 8>(x, w, v, tt, te, tg, M, d, L, N, y, s); return true;
    case 1024: launch_exec_t<T, 16>(x, w, v, tt, te, tg, M, d, L, N, y, s); return true;
    case 2048: launch_exec_t<T, 32>(x, w, v, tt, te, tg, M, d, L, N, y, s); return true;
    case 4096: launch_exec_t<T, 64>(x, w, v, tt, te, tg, M, d, L, N, y, s); return true;
    default: return false;
  }
}

hipError_t launch_atomic_forward(int bf16, int L, int d, int N, int M, const void* x, const void* w,
                                 const void* v, const int32_t* task_token,
                                 const int32_t* task_expert, const float* task_gate, float* y,
                                 bool accumulate, hipStream_t s) {
  if (L == 0) return hipSuccess;
  if (!accumulate) {
    const size_t n4 = static_cast<size_t>(L) * d / 4;
    zero_f32_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, s>>>(
        reinterpret_cast<float4*>(y), n4);
  }
  if (M == 0) return hipGetLastError();
  bool ok;
  if (bf16)
    ok = dispatch_exec<uint16_t>(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                                 static_cast<const uint16_t*>(v), task_token, task_expert,
                                 task_gate, M, d, L, N, y, s);
  else
    ok = dispatch_exec<float>(static_cast<const float*>(x), static_cast<const float*>(w),
                              static_cast<const float*>(v), task_token, task_expert, task_gate,
                              M, d, L, N, y, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace omni
