// Execution of the routed layer.  Pages: gist.science explainer §2.1 (atomic
// expert E_i(x) = sigma(x . w_in) w_out; all experts live in the global
// matrices W, V in R^{N x d}; per token the selected rows are assembled into
// one block) and interactive explainer "Expert-Centric Scheduling" (each
// group's parameters are loaded once and reused for every token assigned to
// the group; parameter traffic 2d * |E_active| instead of 2d * L * K).
//
// Expert-centric form, two kernels, no atomics:
//   phase 1 (in the schedule's (group, token) order): per task
//     h = x_t . W[e], coef = g * silu(h), written at the task's flat id
//     m = t*K + k together with e.  Each wave walks a contiguous run of the
//     sorted tasks with three tasks' rows in flight; x_t is fetched once per
//     (group, token) run.  Workgroups are laid out XCD by XCD over the task
//     list, so the W rows of a group are read by one XCD, and the tasks of a
//     group visit the tokens in increasing order, so at any moment the waves
//     of the chip read x rows from a narrow token window that stays in L2.
//     The bf16 dot product runs on v_dot2_f32_bf16 (two products per
//     instruction, float32 accumulation).
//   phase 2 (token-centric gather): y_t = sum_k coef[t,k] * V[e_tk], one wave
//     (or a few, splitting d) per token, y written once with plain stores.
// Scattering the V contributions in expert-centric order instead needs a
// float32 atomic add into y per task, which measured about twice as slow on
// MI355X as reading the repeated V rows again.
//
// Token-centric form (the Dynamic Expert Assembly view of §2.1), one kernel
// when the caller hands over the flattened selection (the token lists in
// flatten order), else one more that inverts the schedule's sorted order:
//   one wave per token holds x_t in registers, streams the token's K W rows
//   (pass A: h_k, coef_k) and then its K V rows (pass B: y_t += coef_k V[e]).
//   It reads every W and V row once per task, like phase 1 + phase 2 above,
//   but x once per token and no coefficient round trip.  When the tasks reuse
//   experts little (uniform routing over N = 2^20 experts: 1.28 tasks per
//   active expert) both forms are bound by the DRAM rate for random 4 KiB
//   rows, and this one does less other work.  Three kernels share its
//   passes: token_kernel (one token per wave), token_multi_kernel (from 8192
//   tokens: four tokens per wave, their y rows written together at the end)
//   and token_split_kernel (below 4096 tokens: each token's tasks and
//   columns split over several waves, so that few tokens still fill the
//   chip).  Every form sums y in the same order with the same per-element
//   operations, so they give bit-identical y.
//
// Cache hints: where the expert rows are rarely read twice (stream_rows)
// they are loaded with the nontemporal hint and y is stored with the sc1
// scope bit; elsewhere y carries the nontemporal hint (store_row policies).
#include "device.hpp"
#include "launch.hpp"
#include "rowfrag.hpp"

namespace omni {

constexpr int kRing = 4;  // task slots per wave: three in flight, one computed

// Phase 1.  Issue the loads of task i into ring slot S.  NT: stream the
// expert rows with the nontemporal hint (see stream_rows).
template <typename T, int EPL, bool NT>
__device__ __forceinline__ void coef_issue(int i, int n, const T* __restrict__ x,
                                           const T* __restrict__ W, int d, int my_t, int my_e,
                                           RowFrag<T, EPL>& wslot, RowFrag<T, EPL>& xslot) {
  if (i >= n) return;
  wslot.template fetch<NT>(W + static_cast<size_t>(rdlane(my_e, i)) * d, lane());
  const int t = rdlane(my_t, i);
  const int tp = i ? rdlane(my_t, i - 1) : -1;
  if (t != tp) xslot.load(x + static_cast<size_t>(t) * d, lane());  // first task of a run
}

template <typename T, int EPL, bool NT>
__global__ __launch_bounds__(256) void coef_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const int32_t* __restrict__ ttok,
    const int32_t* __restrict__ texp, const float* __restrict__ tgate,
    const int32_t* __restrict__ tidx, int M, int d, int L, int N, int chunk, int nblk,
    float* __restrict__ coef, int32_t* __restrict__ eflat) {
  using Frag = RowFrag<T, EPL>;
  const int wv = threadIdx.x >> 6, l = lane();
  // XCD-contiguous workgroup order (workgroup b runs on XCD b % 8)
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int logical = xcd * per + min(xcd, rem) + loc;
  const long long m0ll = (static_cast<long long>(logical) * 4 + wv) * chunk;
  if (m0ll >= M) return;
  const int m0 = static_cast<int>(m0ll);
  const int n = min(chunk, M - m0);

  // task metadata, one task per lane (chunk <= 64).  Ids outside their range
  // (only from a corrupted schedule) are mapped to 0 so every access stays
  // in bounds.
  int my_t = (l < n) ? ttok[m0 + l] : 0;
  int my_e = (l < n) ? texp[m0 + l] : 0;
  int my_i = (l < n) ? tidx[m0 + l] : 0;
  const float my_g = (l < n) ? tgate[m0 + l] : 0.f;
  my_t = static_cast<unsigned>(my_t) < static_cast<unsigned>(L) ? my_t : 0;
  my_e = static_cast<unsigned>(my_e) < static_cast<unsigned>(N) ? my_e : 0;
  const bool idx_ok = static_cast<unsigned>(my_i) < static_cast<unsigned>(M);

  Frag wr[kRing], xr[kRing], xc;
  int cur = -1;
  float my_c = 0.f;
#pragma unroll
  for (int s = 0; s < kRing - 1; ++s)
    coef_issue<T, EPL, NT>(s, n, x, W, d, my_t, my_e, wr[s], xr[s]);
  for (int i = 0; i < n; i += kRing) {
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      const int ii = i + s;
      if (ii >= n) break;
      coef_issue<T, EPL, NT>(ii + kRing - 1, n, x, W, d, my_t, my_e,
                             wr[(s + kRing - 1) % kRing], xr[(s + kRing - 1) % kRing]);
      const int t = rdlane(my_t, ii);
      if (t != cur) {
        xc = xr[s];
        cur = t;
      }
      const float h = wave_sum(frag_dot<EPL>(xc, wr[s]));
      const float c = rdlane(my_g, ii) * (h / (1.f + __expf(-h)));
      if (l == ii) my_c = c;
    }
  }
  if (l < n && idx_ok) {
    coef[my_i] = my_c;
    eflat[my_i] = my_e;
  }
}

// Phase 2.  Wave g serves token g / split, columns [s * 64 * EPL, +64 * EPL).
template <typename T, int EPL, bool NT>
__global__ __launch_bounds__(256) void gather_kernel(
    const T* __restrict__ V, const float* __restrict__ coef, const int32_t* __restrict__ eflat,
    int L, int K, int d, int N, int split, float* __restrict__ y, int accumulate) {
  using Frag = RowFrag<T, EPL>;
  const long long g = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int l = lane();
  if (g >= static_cast<long long>(L) * split) return;
  const int t = static_cast<int>(g / split);
  const int col0 = static_cast<int>(g - static_cast<long long>(t) * split) * 64 * EPL;
  float acc[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int n = min(64, K - k0);
    const size_t base = static_cast<size_t>(t) * K + k0;
    int my_e = (l < n) ? eflat[base + l] : 0;
    my_e = static_cast<unsigned>(my_e) < static_cast<unsigned>(N) ? my_e : 0;
    const float my_c = (l < n) ? coef[base + l] : 0.f;
    Frag f[kRing];
    token_gather<T, EPL, NT, kRing>(V + col0, my_e, my_c, n, d, l, f, acc);
  }
  store_row<T, EPL, NT ? kStoreDevice : kStoreNT>(acc, y + static_cast<size_t>(t) * d + col0,
                                                  accumulate);
}

// Inverse of the schedule's task permutation: each token's (expert, gate)
// list in flatten order m = t*K + k, into le / lg.  Ids outside their range
// (only from a corrupted schedule) are mapped to expert 0 so every later
// access stays in bounds.
__global__ __launch_bounds__(256) void unpermute_kernel(const int32_t* __restrict__ texp,
                                                        const float* __restrict__ tgate,
                                                        const int32_t* __restrict__ tidx, int M,
                                                        int N, int32_t* __restrict__ le,
                                                        float* __restrict__ lg) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const int i = tidx[m];
  if (static_cast<unsigned>(i) >= static_cast<unsigned>(M)) return;
  const int e = texp[m];
  le[i] = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
  lg[i] = tgate[m];
}

constexpr int kTokRing = 6;  // row slots per wave in the token-centric kernel: five in flight

// GLU: the SwiGLU-gated variant, coefficient g silu(x . W[e]) (x . U[e]).
// NT: the expert rows and x_t (each read once here) carry the nontemporal hint.
template <typename T, int EPL, bool GLU, bool NT>
__global__ __launch_bounds__(256, 3) void token_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const T* __restrict__ U,
    const T* __restrict__ V, const int32_t* __restrict__ le, const float* __restrict__ lg, int L,
    int K, int d, int N, float* __restrict__ y, int accumulate) {
  using Frag = RowFrag<T, EPL>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane();
  if (t >= L) return;
  Frag xf;
  xf.template fetch<NT>(x + static_cast<size_t>(t) * d, l);
  float acc[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
  Frag f[kTokRing];  // one ring for both passes keeps the register count down
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int n = min(64, K - k0);
    int my_e = 0;
    float my_g = 0.f;
    if (l < n) {
      const size_t o = static_cast<size_t>(t) * K + k0 + l;
      const int e = le[o];
      my_e = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
      my_g = lg[o];
    }
    // pass A: h_k = x_t . W[e_k]; h_k ends in lane k
    const float my_h = token_dots<T, EPL, NT, kTokRing>(xf, W, my_e, n, d, l, f);
    float my_c = my_g * (my_h / (1.f + __expf(-my_h)));
    // gated variant, pass A': the up factor x_t . U[e_k]
    if constexpr (GLU) my_c *= token_dots<T, EPL, NT, kTokRing>(xf, U, my_e, n, d, l, f);
    // pass B: y_t += coef_k * V[e_k]
    token_gather<T, EPL, NT, kTokRing>(V, my_e, my_c, n, d, l, f, acc);
  }
  store_row<T, EPL, NT ? kStoreDevice : kStoreNT>(acc, y + static_cast<size_t>(t) * d,
                                                  accumulate);
}

static inline int clampi(long long v, int lo, int hi) {
  return static_cast<int>(v < lo ? lo : (v > hi ? hi : v));
}

template <typename T, int EPL, bool NT>
static void launch_coef_t(const T* x, const T* w, const int32_t* tt, const int32_t* te,
                          const float* tg, const int32_t* ti, int M, int d, int L, int N,
                          float* coef, int32_t* eflat, hipStream_t s) {
  // ~16 waves per CU over 256 CUs at full size, at most 64 tasks per wave
  const int chunk = clampi(M / (256 * 16), 1, 64);
  const long long waves = (static_cast<long long>(M) + chunk - 1) / chunk;
  const int nblk = static_cast<int>((waves + 3) / 4);
  coef_kernel<T, EPL, NT><<<nblk, 256, 0, s>>>(x, w, tt, te, tg, ti, M, d, L, N, chunk, nblk,
                                               coef, eflat);
}

template <typename T, int EPL, bool NT>
static void launch_gather_t(const T* v, const float* coef, const int32_t* eflat, int L, int K,
                            int d, int N, int split, float* y, int accumulate, hipStream_t s) {
  const long long waves = static_cast<long long>(L) * split;
  gather_kernel<T, EPL, NT><<<static_cast<unsigned>((waves + 3) / 4), 256, 0, s>>>(
      v, coef, eflat, L, K, d, N, split, y, accumulate);
}

// Phase-2 column split: enough waves to cover the chip when L is small,
// never fewer than 512 columns (1 KiB of bf16) per wave and row.
static int gather_split(int L, int d) {
  int split = 1;
  while (static_cast<long long>(L) * split < 256 * 8 && d / (split * 2) >= 512) split *= 2;
  return split;
}

template <typename T, bool NT>
static bool dispatch_exec(const T* x, const T* w, const T* v, const int32_t* tt,
                          const int32_t* te, const float* tg, const int32_t* ti, int M, int d,
                          int L, int K, int N, float* coef, int32_t* eflat, float* y,
                          int accumulate, hipStream_t s) {
  switch (d) {
#define OMNI_COEF(D_, EPL_) case D_: launch_coef_t<T, EPL_, NT>(x, w, tt, te, tg, ti, M, d, L, N, coef, eflat, s); break;
    OMNI_COEF(64, 1) OMNI_COEF(128, 2) OMNI_COEF(256, 4) OMNI_COEF(512, 8)
    OMNI_COEF(1024, 16) OMNI_COEF(2048, 32) OMNI_COEF(4096, 64)
#undef OMNI_COEF
    default: return false;
  }
  const int split = gather_split(L, d);
  switch (d / split) {
#define OMNI_GATHER(D_, EPL_) case D_: launch_gather_t<T, EPL_, NT>(v, coef, eflat, L, K, d, N, split, y, accumulate, s); break;
    OMNI_GATHER(64, 1) OMNI_GATHER(128, 2) OMNI_GATHER(256, 4) OMNI_GATHER(512, 8)
    OMNI_GATHER(1024, 16) OMNI_GATHER(2048, 32) OMNI_GATHER(4096, 64)
#undef OMNI_GATHER
    default: return false;
  }
  return true;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* __restrict__ p, size_t n4) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

size_t atomic_forward_ws_bytes(int L, int K) {
  const size_t m = static_cast<size_t>(L) * static_cast<size_t>(K) * 4;
  return 2 * ((m + 255) & ~static_cast<size_t>(255));
}

constexpr int kMultiTokens = 4;  // tokens per wave in token_multi_kernel
constexpr int kMultiRing = 3;    // its row slots: two rows in flight per wave, 8 waves per CU

// Token-centric form with kMultiTokens tokens per wave: each wave runs
// token_kernel's passes for its tokens one after another and keeps their y
// rows in registers until the last one is done.  With every wave resident
// from the start (2 per SIMD) the y writes of the call come together at its
// end instead of being spread through the random-row read stream, where each
// write costs the HBM a read / write turnaround.  Every coefficient and y
// element goes through token_kernel's operations in the same order, so y is
// bit-identical to it.
template <typename T, int EPL, bool GLU, bool NT>
__global__ __launch_bounds__(256, 2) void token_multi_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const T* __restrict__ U,
    const T* __restrict__ V, const int32_t* __restrict__ le, const float* __restrict__ lg, int L,
    int K, int d, int N, float* __restrict__ y, int accumulate) {
  using Frag = RowFrag<T, EPL>;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane();
  const int t0 = wv * kMultiTokens;
  if (t0 >= L) return;
  float acc[kMultiTokens][EPL];
#pragma unroll
  for (int tt = 0; tt < kMultiTokens; ++tt)
#pragma unroll
    for (int q = 0; q < EPL; ++q) acc[tt][q] = 0.f;
  Frag f[kMultiRing];
#pragma unroll
  for (int tt = 0; tt < kMultiTokens; ++tt) {
    const int t = t0 + tt;
    if (t >= L) continue;  // uniform over the wave
    Frag xf;
    xf.template fetch<NT>(x + static_cast<size_t>(t) * d, l);
    for (int k0 = 0; k0 < K; k0 += 64) {
      const int n = min(64, K - k0);
      int my_e = 0;
      float my_g = 0.f;
      if (l < n) {
        const size_t o = static_cast<size_t>(t) * K + k0 + l;
        const int e = le[o];
        my_e = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
        my_g = lg[o];
      }
      const float my_h = token_dots<T, EPL, NT, kMultiRing>(xf, W, my_e, n, d, l, f);
      float my_c = my_g * (my_h / (1.f + __expf(-my_h)));
      if constexpr (GLU) my_c *= token_dots<T, EPL, NT, kMultiRing>(xf, U, my_e, n, d, l, f);
      token_gather<T, EPL, NT, kMultiRing>(V, my_e, my_c, n, d, l, f, acc[tt]);
    }
  }
#pragma unroll
  for (int tt = 0; tt < kMultiTokens; ++tt)
    if (t0 + tt < L)
      store_row<T, EPL, NT ? kStoreDevice : kStoreNT>(
          acc[tt], y + static_cast<size_t>(t0 + tt) * d, accumulate);
}

constexpr int kSplitRing = 8;  // pass-B row-slice slots per wave in token_split_kernel

// Token-centric form for few tokens: one workgroup of WS waves per token.
// Pass A splits the token's tasks over the waves; each wave computes whole-row
// dot products for its share exactly as token_kernel does (x_t in registers,
// the W rows through the ring).  The coefficients meet in LDS.  Pass B splits
// the columns of y over the waves; each wave sums all of the token's tasks
// over its columns in k order.  Every coefficient and every y element goes
// through the same operations in the same order as in token_kernel, so y is
// bit-identical to it; the split only gives the chip WS times more waves.
template <typename T, int EPL, int WS, bool GLU, bool NT>
__global__ __launch_bounds__(64 * WS) void token_split_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const T* __restrict__ U,
    const T* __restrict__ V, const int32_t* __restrict__ le, const float* __restrict__ lg, int L,
    int K, int d, int N, float* __restrict__ y, int accumulate) {
  static_assert(EPL % WS == 0, "every wave needs at least one element per lane");
  constexpr int EPLB = EPL / WS;  // pass-B elements per lane
  using Frag = RowFrag<T, EPL>;
  using FragB = RowFrag<T, EPLB>;
  __shared__ float sc[64];
  __shared__ int se[64];
  const int t = blockIdx.x;
  const int w = threadIdx.x >> 6, l = lane();
  if (t >= L) return;  // the whole workgroup leaves together
  Frag xf;
  xf.template fetch<NT>(x + static_cast<size_t>(t) * d, l);
  const int col0 = w * 64 * EPLB;
  float acc[EPLB];
#pragma unroll
  for (int q = 0; q < EPLB; ++q) acc[q] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int n = min(64, K - k0);
    const int per = (n + WS - 1) / WS;
    const int a0 = w * per;
    const int na = max(0, min(per, n - a0));  // this wave's tasks: [a0, a0 + na)
    if (na > 0) {  // uniform over the wave
      int my_e = 0;
      float my_g = 0.f;
      if (l < na) {
        const size_t o = static_cast<size_t>(t) * K + k0 + a0 + l;
        const int e = le[o];
        my_e = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
        my_g = lg[o];
      }
      Frag f[kTokRing];
      const float my_h = token_dots<T, EPL, NT, kTokRing>(xf, W, my_e, na, d, l, f);
      float my_c = my_g * (my_h / (1.f + __expf(-my_h)));
      if constexpr (GLU) my_c *= token_dots<T, EPL, NT, kTokRing>(xf, U, my_e, na, d, l, f);
      if (l < na) {
        sc[a0 + l] = my_c;
        se[a0 + l] = my_e;
      }
    }
    __syncthreads();
    const int my_e = l < n ? se[l] : 0;
    const float my_c = l < n ? sc[l] : 0.f;
    FragB g[kSplitRing];
    token_gather<T, EPLB, NT, kSplitRing>(V + col0, my_e, my_c, n, d, l, g, acc);
    __syncthreads();  // the next chunk's coefficients overwrite sc / se
  }
  store_row<T, EPLB, NT ? kStoreDevice : kStoreNT>(acc, y + static_cast<size_t>(t) * d + col0,
                                                   accumulate);
}

// From 8192 tokens up the token-centric form runs kMultiTokens tokens per
// wave (token_multi_kernel).  Measured at L = 8192, d = 2048, N = 2^20:
// 702 us with one token per wave, 690 / 677 us with two (ring of 4 / 6 rows),
// 658 us with four (ring of 3 or 4).
static bool token_multi_tokens(int L) { return L >= 8192; }

// Waves per token for the token-centric form: 1 (token_kernel) from 4096
// tokens up; below, enough for about 8192 waves, at most 8, and at most one
// per 64 columns.  Measured (token form, us per call): decode (L = 256,
// d = 2048) 33.9 / 25.2 / 23.6 / 22.2 with 1 / 2 / 4 / 8 waves per token;
// small (L = 4096, d = 1024) 74.1 / 75.3 / 73.9 / 79.4; mid and large lose
// 4-95 % with any split.
static int token_split_waves(int L, int d) {
  if (L >= 4096) return 1;
  int ws = 1;
  while (ws < 8 && static_cast<long long>(L) * ws < 8192 && d / (64 * ws * 2) >= 1) ws *= 2;
  return ws;
}

// The token lists: the caller's flattened selection (fe, fg) when given,
// else the schedule inverted into the workspace (ws: M ids, then M gates).
template <typename T, bool GLU, bool NT>
static bool dispatch_token(const T* x, const T* w, const T* u, const T* v, const int32_t* te,
                           const float* tg, const int32_t* ti, const int32_t* fe,
                           const float* fg, int M, int d, int L, int K, int N, void* ws, float* y,
                           int accumulate, hipStream_t s) {
  if (!fe) {
    int32_t* le = static_cast<int32_t*>(ws);
    float* lg = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         atomic_forward_ws_bytes(L, K) / 2);
    unpermute_kernel<<<static_cast<unsigned>((M + 255) / 256), 256, 0, s>>>(te, tg, ti, M, N, le,
                                                                            lg);
    fe = le;
    fg = lg;
  }
  const int nw = token_split_waves(L, d);
  if (nw > 1) {
    const unsigned grid = static_cast<unsigned>(L);
#define OMNI_SPLIT(EPL_, WS_)                                                                   \
  token_split_kernel<T, EPL_, WS_, GLU, NT><<<grid, 64 * WS_, 0, s>>>(x, w, u, v, fe, fg, L, K, \
                                                                       d, N, y, accumulate)
#define OMNI_SPLIT_WS(EPL_)                                                                     \
  if (nw == 2) { if constexpr (EPL_ >= 2) OMNI_SPLIT(EPL_, 2); }                                \
  else if (nw == 4) { if constexpr (EPL_ >= 4) OMNI_SPLIT(EPL_, 4); }                           \
  else { if constexpr (EPL_ >= 8) OMNI_SPLIT(EPL_, 8); }
    switch (d) {
      case 128: OMNI_SPLIT_WS(2) break;
      case 256: OMNI_SPLIT_WS(4) break;
      case 512: OMNI_SPLIT_WS(8) break;
      case 1024: OMNI_SPLIT_WS(16) break;
      case 2048:
        if constexpr (sizeof(T) == 2) {
          OMNI_SPLIT_WS(32)
          break;
        }
        return false;
      default: return false;
    }
#undef OMNI_SPLIT_WS
#undef OMNI_SPLIT
    return true;
  }
  const bool multi = token_multi_tokens(L);
  const unsigned nblk = static_cast<unsigned>((L + 3) / 4);
  const unsigned mblk = static_cast<unsigned>((L + 4 * kMultiTokens - 1) / (4 * kMultiTokens));
  // rows of at most 4 KiB: d <= 2048 for bf16, d <= 1024 for float32
#define OMNI_TOK(EPL_)                                                                         \
  if (multi)                                                                                   \
    token_multi_kernel<T, EPL_, GLU, NT><<<mblk, 256, 0, s>>>(x, w, u, v, fe, fg, L, K, d, N,  \
                                                              y, accumulate);                  \
  else                                                                                         \
    token_kernel<T, EPL_, GLU, NT><<<nblk, 256, 0, s>>>(x, w, u, v, fe, fg, L, K, d, N, y,     \
                                                        accumulate);
  switch (d) {
    case 64: OMNI_TOK(1) break;
    case 128: OMNI_TOK(2) break;
    case 256: OMNI_TOK(4) break;
    case 512: OMNI_TOK(8) break;
    case 1024: OMNI_TOK(16) break;
    case 2048:
      if constexpr (sizeof(T) == 2) {
        OMNI_TOK(32)
        break;
      }
      return false;
    default: return false;
  }
#undef OMNI_TOK
  return true;
}

bool token_rows_in_registers(int bf16, int d) {
  const long long row_bytes = static_cast<long long>(d) * (bf16 ? 2 : 4);
  return row_bytes <= 4096 && d >= 64 && (d & (d - 1)) == 0;
}

// The expert-centric kernels above hold a row per wave for d = 64 .. 4096, a
// power of two; other widths run the chunked kernels (chunked.hip).
static bool expert_rows_in_registers(int d) { return d >= 64 && d <= 4096 && (d & (d - 1)) == 0; }

hipError_t launch_unpermute(const int32_t* texp, const float* tgate, const int32_t* tidx, int M,
                            int N, int32_t* le, float* lg, hipStream_t s) {
  unpermute_kernel<<<static_cast<unsigned>((M + 255) / 256), 256, 0, s>>>(texp, tgate, tidx, M,
                                                                          N, le, lg);
  return hipGetLastError();
}

bool stream_rows(long long M, long long N) {
  // Expert rows are streamed with the nontemporal hint when few are read
  // twice (no more tasks than experts) and the call is long enough to be
  // bound by bandwidth (at least 2^18 tasks).  Measured: the token kernel at
  // L = 8192, d = 2048, N = 2^20 (524,288 tasks) gains 4 %; with heavy reuse
  // (Zipf routing, 4 tasks per expert) it runs 2.6 x slower, and with few
  // tasks (decode, 16,384) the expert-centric form 14 % slower.
  return M >= (1ll << 18) && M <= N;
}

size_t exec_ws_bytes(int mode, int L, int d, int N, int K) {
  // the per-task lists (8 bytes per task) of every form; the grouped form's
  // counts, hot set and gathered V_H^T follow
  size_t n = atomic_forward_ws_bytes(L, K);
  if (mode == 3) n += grouped_ws_bytes(L, K, d, N);
  return n;
}

int auto_exec_mode(int bf16, int L, int d, int N, int K) {
  (void)N;
  (void)K;
  // One wave per token keeps 3072 waves resident (3 per SIMD); it beat the
  // two-kernel form from L = 8192 tokens of d = 2048 up (2.7 resident rounds)
  // and lost at L = 4096, d = 1024.  Below 4096 tokens each token is split
  // over several waves (token_split_kernel), which beat the two-kernel form
  // at L = 256, d = 2048 (22 against 27 us) and L = 64, d = 128 (12.5
  // against 15 us).
  if (!token_rows_in_registers(bf16, d)) return 1;
  if ((L >= 8192 && d >= 1024) || L < 4096) return 2;
  return 1;
}

hipError_t launch_atomic_forward(int bf16, int mode, int L, int d, int N, int K, const void* x,
                                 const void* w, const void* v, const int32_t* task_token,
                                 const int32_t* task_expert, const float* task_gate,
                                 const int32_t* task_index, const int32_t* flat_expert,
                                 const float* flat_gate, float* y, bool accumulate, void* ws,
                                 hipStream_t s) {
  if (L == 0) return hipSuccess;
  const int M = L * K;
  if (M == 0) {  // no tasks: the routed output is zero
    if (!accumulate) {
      const size_t n4 = static_cast<size_t>(L) * d / 4;
      zero_f32_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, s>>>(
          reinterpret_cast<float4*>(y), n4);
    }
    return hipGetLastError();
  }
  if ((mode == 2 && !token_rows_in_registers(bf16, d)) ||
      (mode == 1 && !expert_rows_in_registers(d)))
    return launch_chunked(bf16, mode, false, L, d, N, K, x, w, nullptr, v, task_token,
                          task_expert, task_gate, task_index, flat_expert, flat_gate, y,
                          accumulate, ws, s);
  const int acc = accumulate ? 1 : 0;
  const bool nt = stream_rows(M, N);
  bool ok;
  if (mode == 3) {  // grouped, bf16 only (checked by the caller)
    const int32_t* fe = flat_expert;
    const float* fg = flat_gate;
    if (!fe) {
      int32_t* le = static_cast<int32_t*>(ws);
      float* lg = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                           atomic_forward_ws_bytes(L, K) / 2);
      unpermute_kernel<<<static_cast<unsigned>((M + 255) / 256), 256, 0, s>>>(
          task_expert, task_gate, task_index, M, N, le, lg);
      fe = le;
      fg = lg;
    }
    return launch_grouped(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                          static_cast<const uint16_t*>(v), task_expert, fe,
                          fg, L, K, d, N, y, acc, static_cast<char*>(ws) + atomic_forward_ws_bytes(L, K),
                          s);
  } else if (mode == 2) {
    if (bf16) {
      const auto* xb = static_cast<const uint16_t*>(x);
      const auto* wb = static_cast<const uint16_t*>(w);
      const auto* vb = static_cast<const uint16_t*>(v);
      ok = nt ? dispatch_token<uint16_t, false, true>(xb, wb, nullptr, vb, task_expert, task_gate,
                                                      task_index, flat_expert, flat_gate, M, d, L,
                                                      K, N, ws, y, acc, s)
              : dispatch_token<uint16_t, false, false>(xb, wb, nullptr, vb, task_expert,
                                                       task_gate, task_index, flat_expert,
                                                       flat_gate, M, d, L, K, N, ws, y, acc, s);
    } else {
      const auto* xf = static_cast<const float*>(x);
      const auto* wf = static_cast<const float*>(w);
      const auto* vf = static_cast<const float*>(v);
      ok = nt ? dispatch_token<float, false, true>(xf, wf, nullptr, vf, task_expert, task_gate,
                                                   task_index, flat_expert, flat_gate, M, d, L, K,
                                                   N, ws, y, acc, s)
              : dispatch_token<float, false, false>(xf, wf, nullptr, vf, task_expert, task_gate,
                                                    task_index, flat_expert, flat_gate, M, d, L,
                                                    K, N, ws, y, acc, s);
    }
  } else {
    float* coef = static_cast<float*>(ws);
    int32_t* eflat = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                atomic_forward_ws_bytes(L, K) / 2);
    if (bf16) {
      const auto* xb = static_cast<const uint16_t*>(x);
      const auto* wb = static_cast<const uint16_t*>(w);
      const auto* vb = static_cast<const uint16_t*>(v);
      ok = nt ? dispatch_exec<uint16_t, true>(xb, wb, vb, task_token, task_expert, task_gate,
                                              task_index, M, d, L, K, N, coef, eflat, y, acc, s)
              : dispatch_exec<uint16_t, false>(xb, wb, vb, task_token, task_expert, task_gate,
                                               task_index, M, d, L, K, N, coef, eflat, y, acc, s);
    } else {
      const auto* xf = static_cast<const float*>(x);
      const auto* wf = static_cast<const float*>(w);
      const auto* vf = static_cast<const float*>(v);
      ok = nt ? dispatch_exec<float, true>(xf, wf, vf, task_token, task_expert, task_gate,
                                           task_index, M, d, L, K, N, coef, eflat, y, acc, s)
              : dispatch_exec<float, false>(xf, wf, vf, task_token, task_expert, task_gate,
                                            task_index, M, d, L, K, N, coef, eflat, y, acc, s);
    }
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// SwiGLU-gated variant: token-centric form only (the token's K tasks need
// both of their input rows before the V pass).
hipError_t launch_atomic_forward_glu(int bf16, int L, int d, int N, int K, const void* x,
                                     const void* w, const void* u, const void* v,
                                     const int32_t* task_expert, const float* task_gate,
                                     const int32_t* task_index, const int32_t* flat_expert,
                                     const float* flat_gate, float* y, bool accumulate,
                                     void* ws, hipStream_t s) {
  if (L == 0) return hipSuccess;
  const int M = L * K;
  if (M == 0) {
    if (!accumulate) {
      const size_t n4 = static_cast<size_t>(L) * d / 4;
      zero_f32_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, s>>>(
          reinterpret_cast<float4*>(y), n4);
    }
    return hipGetLastError();
  }
  if (!token_rows_in_registers(bf16, d))
    return launch_chunked(bf16, 2, true, L, d, N, K, x, w, u, v, nullptr, task_expert, task_gate,
                          task_index, flat_expert, flat_gate, y, accumulate, ws, s);
  const int acc = accumulate ? 1 : 0;
  const bool nt = stream_rows(M, N);
  bool ok;
  if (bf16) {
    const auto* xb = static_cast<const uint16_t*>(x);
    const auto* wb = static_cast<const uint16_t*>(w);
    const auto* ub = static_cast<const uint16_t*>(u);
    const auto* vb = static_cast<const uint16_t*>(v);
    ok = nt ? dispatch_token<uint16_t, true, true>(xb, wb, ub, vb, task_expert, task_gate,
                                                   task_index, flat_expert, flat_gate, M, d, L, K,
                                                   N, ws, y, acc, s)
            : dispatch_token<uint16_t, true, false>(xb, wb, ub, vb, task_expert, task_gate,
                                                    task_index, flat_expert, flat_gate, M, d, L,
                                                    K, N, ws, y, acc, s);
  } else {
    const auto* xf = static_cast<const float*>(x);
    const auto* wf = static_cast<const float*>(w);
    const auto* uf = static_cast<const float*>(u);
    const auto* vf = static_cast<const float*>(v);
    ok = nt ? dispatch_token<float, true, true>(xf, wf, uf, vf, task_expert, task_gate,
                                                task_index, flat_expert, flat_gate, M, d, L, K, N,
                                                ws, y, acc, s)
            : dispatch_token<float, true, false>(xf, wf, uf, vf, task_expert, task_gate,
                                                 task_index, flat_expert, flat_gate, M, d, L, K,
                                                 N, ws, y, acc, s);
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace omni
