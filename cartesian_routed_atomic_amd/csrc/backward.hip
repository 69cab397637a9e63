// Backward pass of the routed layer.  The pages train models with this layer
// but print no backward; the gradients follow from the forward by the chain
// rule (the expert selection is piecewise constant and passes no gradient):
//   u_k = dy_t . V[e],  h_k = x_t . W[e],  s = silu(h_k),  c_k = g_k s
//   dV[e] += c_k dy_t,   dg_k = s u_k,   dh_k = g_k silu'(h_k) u_k
//   dW[e] += dh_k x_t,   dx_t += dh_k W[e]
//   dS_k = g_k (dg_k - sum_j g_j dg_j)           (gate = softmax of the scores)
//   dz_r[i_k] += dS_k, dz_c[j_k] += dS_k          (S_k = a[i_k] + b[j_k])
//   dx_t += dz_r Wr + dz_c Wc,  dWr = dz_r^T x,  dWc = dz_c^T x, bias = column sums
// The log-softmax backward dz = da - softmax(z) sum(da) reduces to dz = da
// because sum_k dS_k = 0 exactly: the logit gradient is nonzero only on the
// rows and columns of the selected experts, which is what makes the router
// part a gather (dx) and a segmented reduction (dWr, dWc) instead of dense
// GEMMs.
//
// Two kinds of kernels:
//   bwd_token_kernel: one wave per token (x_t and dy_t in registers) walks the
//     token's V rows (u_k), W rows (h_k -> dh_k, dg_k, c_k; dx += dh_k W[e])
//     and router rows (dx += dS_k (Wr[i_k] + Wc[j_k])); writes dx_t and the
//     per-task c, dh, dS, dg at the flat task id.
//   seg_reduce_kernel + seg_fixup_kernel: out[row] = sum_task w_task src[token]
//     over a task list sorted by output row (expert-major for dW and dV, by
//     grid row / column for dWr and dWc).  The sorted lists are schedules with
//     groups of one (B = 1) built by the forward's scheduling code.  Each wave
//     takes 64 consecutive tasks; rows whose tasks all lie in its chunk are
//     written directly, rows that cross a chunk edge leave partial sums that a
//     second kernel adds in chunk order, so every result is deterministic.
#include "device.hpp"
#include "launch.hpp"
#include "rowfrag.hpp"

namespace omni {

// A float32 row in the element layout of RowFrag<T, EPL> (so it pairs
// element by element with a row fragment of T).
template <typename T, int EPL>
__device__ __forceinline__ void load_f32_as(const float* __restrict__ row, int l,
                                            float (&out)[EPL]) {
  constexpr int VEC = RowFrag<T, EPL>::VEC, NCH = RowFrag<T, EPL>::NCH;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const float* p = row + c * 64 * VEC + l * VEC;
    if constexpr (VEC % 4 == 0) {
#pragma unroll
      for (int j = 0; j < VEC; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + j);
        out[c * VEC + j] = v.x;
        out[c * VEC + j + 1] = v.y;
        out[c * VEC + j + 2] = v.z;
        out[c * VEC + j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < VEC; ++j) out[c * VEC + j] = p[j];
    }
  }
}

constexpr int kBwdRing = 4;  // row slots per wave: three in flight

template <typename T, int EPL>
__global__ __launch_bounds__(256, 3) void bwd_token_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const T* __restrict__ V,
    const T* __restrict__ wr, const T* __restrict__ wc, const int32_t* __restrict__ expert_idx,
    const float* __restrict__ gate, const float* __restrict__ dy, int L, int K, int d, int N,
    int Nr, int Nc, float* __restrict__ dx, float* __restrict__ coef, float* __restrict__ dh_out,
    float* __restrict__ ds_out, float* __restrict__ dgate) {
  using Frag = RowFrag<T, EPL>;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane();
  if (t >= L) return;
  const size_t tb = static_cast<size_t>(t) * K;
  int my_e = 0;
  float my_g = 0.f;
  if (l < K) {
    const int e = expert_idx[tb + l];
    my_e = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
    my_g = gate[tb + l];
  }
  float dyr[EPL];
  load_f32_as<T, EPL>(dy + static_cast<size_t>(t) * d, l, dyr);
  Frag xf;
  xf.load(x + static_cast<size_t>(t) * d, l);
  Frag f[kBwdRing];

  // pass 1: u_k = dy_t . V[e_k]
  float my_u = 0.f;
#pragma unroll
  for (int s = 0; s < kBwdRing - 1; ++s)
    if (s < K) f[s].load(V + static_cast<size_t>(rdlane(my_e, s)) * d, l);
  for (int i = 0; i < K; i += kBwdRing) {
#pragma unroll
    for (int s = 0; s < kBwdRing; ++s) {
      const int k = i + s;
      if (k >= K) break;
      if (k + kBwdRing - 1 < K)
        f[(s + kBwdRing - 1) % kBwdRing].load(
            V + static_cast<size_t>(rdlane(my_e, k + kBwdRing - 1)) * d, l);
      float p = 0.f;
#pragma unroll
      for (int q = 0; q < EPL; ++q) p = fmaf(dyr[q], f[s].get(q), p);
      const float u = wave_sum(p);
      if (l == k) my_u = u;
    }
  }

  // pass 2: h_k = x_t . W[e_k]; the task's scalars; dx += dh_k W[e_k]
  float acc[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
  float my_dh = 0.f, my_dg = 0.f, my_c = 0.f;
#pragma unroll
  for (int s = 0; s < kBwdRing - 1; ++s)
    if (s < K) f[s].load(W + static_cast<size_t>(rdlane(my_e, s)) * d, l);
  for (int i = 0; i < K; i += kBwdRing) {
#pragma unroll
    for (int s = 0; s < kBwdRing; ++s) {
      const int k = i + s;
      if (k >= K) break;
      if (k + kBwdRing - 1 < K)
        f[(s + kBwdRing - 1) % kBwdRing].load(
            W + static_cast<size_t>(rdlane(my_e, k + kBwdRing - 1)) * d, l);
      const float h = wave_sum(frag_dot<EPL>(xf, f[s]));
      const float g = rdlane(my_g, k), u = rdlane(my_u, k);
      const float sg = 1.f / (1.f + __expf(-h));
      const float sv = h * sg;
      const float dh = g * (sg * (1.f + h * (1.f - sg))) * u;
#pragma unroll
      for (int q = 0; q < EPL; ++q) acc[q] = fmaf(dh, f[s].get(q), acc[q]);
      if (l == k) {
        my_dh = dh;
        my_dg = sv * u;
        my_c = g * sv;
      }
    }
  }

  // gate softmax backward: dS_k = g_k (dg_k - sum_j g_j dg_j)
  const float gdg = wave_sum(l < K ? my_g * my_dg : 0.f);
  const float my_ds = my_g * (my_dg - gdg);

  // pass 3: dx += dS_k (Wr[i_k] + Wc[j_k]); rows 2k (Wr) and 2k+1 (Wc)
  const int n2 = 2 * K;
  const int my_ri = my_e / Nc, my_ci = my_e - (my_e / Nc) * Nc;
#pragma unroll
  for (int s = 0; s < kBwdRing - 1; ++s) {
    if (s < n2) {
      const int k = s >> 1;
      f[s].load((s & 1) ? wc + static_cast<size_t>(rdlane(my_ci, k)) * d
                        : wr + static_cast<size_t>(rdlane(my_ri, k)) * d, l);
    }
  }
  for (int i = 0; i < n2; i += kBwdRing) {
#pragma unroll
    for (int s = 0; s < kBwdRing; ++s) {
      const int q2 = i + s;
      if (q2 >= n2) break;
      const int qn = q2 + kBwdRing - 1;
      if (qn < n2) {
        const int k = qn >> 1;
        f[(s + kBwdRing - 1) % kBwdRing].load(
            (qn & 1) ? wc + static_cast<size_t>(rdlane(my_ci, k)) * d
                     : wr + static_cast<size_t>(rdlane(my_ri, k)) * d, l);
      }
      const float ds = rdlane(my_ds, q2 >> 1);
#pragma unroll
      for (int q = 0; q < EPL; ++q) acc[q] = fmaf(ds, f[s].get(q), acc[q]);
    }
  }
  store_row<T, EPL>(acc, dx + static_cast<size_t>(t) * d, 0);
  if (l < K) {
    coef[tb + l] = my_c;
    dh_out[tb + l] = my_dh;
    ds_out[tb + l] = my_ds;
    if (dgate) dgate[tb + l] = my_dg;
  }
  (void)Nr;
}

// Row id of each expert / grid row / grid column: e / Nc and e mod Nc.
__global__ __launch_bounds__(256) void split_ids_kernel(const int32_t* __restrict__ expert_idx,
                                                        int M, int N, int Nc,
                                                        int32_t* __restrict__ ri,
                                                        int32_t* __restrict__ ci) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  int e = expert_idx[m];
  e = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
  ri[m] = e / Nc;
  ci[m] = e - (e / Nc) * Nc;
}

__global__ __launch_bounds__(256) void zero_f32x4_kernel(float4* __restrict__ p, size_t n4) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}
__global__ __launch_bounds__(256) void zero_f32_kernel1(float* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ------------------------------------------------------------ reduction

// Output row of sorted task p: the expert's position among the active
// experts (rank != null) or the sorted id itself (grid rows / columns).
// Ids outside their range (only from a corrupted selection) are mapped to 0
// so every access stays in bounds.
__device__ __forceinline__ int out_row_of(const int32_t* __restrict__ te,
                                          const int32_t* __restrict__ rank, int p, int n_ids,
                                          int n_rows) {
  int r = te[p];
  r = static_cast<unsigned>(r) < static_cast<unsigned>(n_ids) ? r : 0;
  if (rank) r = rank[r];
  return static_cast<unsigned>(r) < static_cast<unsigned>(n_rows) ? r : 0;
}

// Wave w: sorted tasks [64 w, 64 w + 64).  out[row] = sum w_m src[token];
// osum[row] = sum w_m (if osum).  Partials of rows crossing a chunk edge go
// to part[(2 w + slot) * d]: slot 0 if the row began before the chunk, else
// slot 1 (the row begins here and continues).
template <typename S, int EPL>
__global__ __launch_bounds__(256) void seg_reduce_kernel(
    const int32_t* __restrict__ task_token, const int32_t* __restrict__ task_expert,
    const int32_t* __restrict__ task_index, const int32_t* __restrict__ rank,
    const float* __restrict__ wflat, const S* __restrict__ src, int M, int d, int L,
    int n_ids, int n_rows, float* __restrict__ out, float* __restrict__ osum, float* __restrict__ part,
    float* __restrict__ psum) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane();
  const int p0 = wv * 64;
  if (p0 >= M) return;
  const int n = min(64, M - p0);
  int my_t = 0, my_r = 0;
  float my_w = 0.f;
  if (l < n) {
    const int p = p0 + l;
    const int t = task_token[p];
    my_t = static_cast<unsigned>(t) < static_cast<unsigned>(L) ? t : 0;
    my_r = out_row_of(task_expert, rank, p, n_ids, n_rows);
    const int m = task_index[p];
    my_w = static_cast<unsigned>(m) < static_cast<unsigned>(M) ? wflat[m] : 0.f;
  }
  // does the first row begin before this chunk / the last row continue after it?
  const bool head = p0 > 0 && out_row_of(task_expert, rank, p0 - 1, n_ids, n_rows) == rdlane(my_r, 0);
  const bool tail = p0 + n < M && out_row_of(task_expert, rank, p0 + n, n_ids, n_rows) == rdlane(my_r, n - 1);
  constexpr int R = kBwdRing;
  using SF = RowFrag<S, EPL>;
  SF f[R];
  float acc[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
  float wsum = 0.f;
  int seg_start = 0;
#pragma unroll
  for (int s = 0; s < R - 1; ++s)
    if (s < n) f[s].load(src + static_cast<size_t>(rdlane(my_t, s)) * d, l);
  for (int i = 0; i < n; i += R) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int k = i + s;
      if (k >= n) break;
      if (k + R - 1 < n)
        f[(s + R - 1) % R].load(src + static_cast<size_t>(rdlane(my_t, k + R - 1)) * d, l);
      const float wk = rdlane(my_w, k);
#pragma unroll
      for (int q = 0; q < EPL; ++q) acc[q] = fmaf(wk, f[s].get(q), acc[q]);
      wsum += wk;
      const int row = rdlane(my_r, k);
      const bool last_of_row = k == n - 1 || rdlane(my_r, k + 1) != row;
      if (last_of_row) {
        const bool began_before = seg_start == 0 && head;
        const bool goes_on = k == n - 1 && tail;
        float* dst;
        float* dsum;
        if (!began_before && !goes_on) {
          dst = out + static_cast<size_t>(row) * d;
          dsum = osum ? osum + row : nullptr;
        } else {
          const int slot = began_before ? 0 : 1;
          dst = part + static_cast<size_t>(2 * wv + slot) * d;
          dsum = psum + 2 * wv + slot;
        }
        store_row<S, EPL>(acc, dst, 0);
        if (l == 0 && dsum) *dsum = wsum;
#pragma unroll
        for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
        wsum = 0.f;
        seg_start = k + 1;
      }
    }
  }
}

// Rows that cross chunk edges: the wave of the chunk where such a row begins
// (its slot-1 partial) adds the slot-0 partials of the following chunks, in
// order, for as long as the row continues.  S fixes the element layout of the
// partial rows (that of the reduction that wrote them).
template <typename S, int EPL>
__global__ __launch_bounds__(256) void seg_fixup_kernel(
    const int32_t* __restrict__ task_expert, const int32_t* __restrict__ rank, int M, int d,
    int n_ids, int n_rows, float* __restrict__ out, float* __restrict__ osum,
    const float* __restrict__ part, const float* __restrict__ psum) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane();
  const int p0 = wv * 64;
  if (p0 >= M) return;
  const int pe = min(p0 + 64, M);
  if (pe >= M) return;  // the last chunk has no successor
  const int row = out_row_of(task_expert, rank, pe - 1, n_ids, n_rows);
  if (out_row_of(task_expert, rank, pe, n_ids, n_rows) != row) return;  // no row crosses the end
  // rows are contiguous: the row began before this chunk only if it fills the
  // chunk and also holds the task before it; then an earlier chunk owns it
  if (out_row_of(task_expert, rank, p0, n_ids, n_rows) == row && p0 > 0 &&
      out_row_of(task_expert, rank, p0 - 1, n_ids, n_rows) == row)
    return;
  float acc[EPL];
  float tot[EPL];
  load_f32_as<S, EPL>(part + static_cast<size_t>(2 * wv + 1) * d, l, tot);
  float ws = psum[2 * wv + 1];
  for (int c = wv + 1;; ++c) {
    load_f32_as<S, EPL>(part + static_cast<size_t>(2 * c) * d, l, acc);
#pragma unroll
    for (int q = 0; q < EPL; ++q) tot[q] += acc[q];
    ws += psum[2 * c];
    const int ce = min((c + 1) * 64, M);
    if (ce >= M || out_row_of(task_expert, rank, ce, n_ids, n_rows) != row) break;
  }
  store_row<S, EPL>(tot, out + static_cast<size_t>(row) * d, 0);
  if (l == 0 && osum) osum[row] = ws;
}

// ------------------------------------------------------------ host side

static inline size_t a256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

namespace {
struct SchedBufs {  // a schedule with groups of one, in the backward workspace
  size_t cnt, act, off, tok, exp, gat, idx, ws;
  ScheduleWs lay;
};
}  // namespace

static SchedBufs sched_bufs(size_t& o, int L, int K, int N) {
  SchedBufs b{};
  const size_t M = static_cast<size_t>(L) * K;
  b.lay = schedule_ws_layout(L, K, N, 1);
  const size_t g = static_cast<size_t>(b.lay.max_groups);
  b.cnt = o; o = a256(o + 2 * 4);
  b.act = o; o = a256(o + (g > 0 ? g : 1) * 4);
  b.off = o; o = a256(o + (g + 1) * 4);
  b.tok = o; o = a256(o + (M > 0 ? M : 1) * 4);
  b.exp = o; o = a256(o + (M > 0 ? M : 1) * 4);
  b.gat = o; o = a256(o + (M > 0 ? M : 1) * 4);
  b.idx = o; o = a256(o + (M > 0 ? M : 1) * 4);
  b.ws = o;  o = a256(o + b.lay.bytes);
  return b;
}

namespace {
struct BwdLayout {
  size_t bytes, coef, dh, ds, ri, ci, part, psum;
  SchedBufs es, rs, cs;  // experts (the caller's counts / active), grid rows, grid columns
};
}  // namespace

static BwdLayout bwd_layout(int L, int d, int Nr, int Nc, int K) {
  BwdLayout w{};
  const size_t M = static_cast<size_t>(L) * K;
  const size_t m1 = M > 0 ? M : 1;
  size_t o = 0;
  w.coef = o; o = a256(o + m1 * 4);
  w.dh = o;   o = a256(o + m1 * 4);
  w.ds = o;   o = a256(o + m1 * 4);
  w.ri = o;   o = a256(o + m1 * 4);
  w.ci = o;   o = a256(o + m1 * 4);
  const size_t chunks = (m1 + 63) / 64;
  w.part = o; o = a256(o + chunks * 2 * static_cast<size_t>(d) * 4);
  w.psum = o; o = a256(o + chunks * 2 * 4);
  const long long N = static_cast<long long>(Nr) * Nc;
  w.es = sched_bufs(o, L, K, static_cast<int>(N));
  w.rs = sched_bufs(o, L, K, Nr);
  w.cs = sched_bufs(o, L, K, Nc);
  w.bytes = o;
  return w;
}

size_t routed_backward_ws_bytes(int L, int d, int Nr, int Nc, int K) {
  return bwd_layout(L, d, Nr, Nc, K).bytes;
}

template <typename T, int EPL>
static hipError_t launch_bwd_t(const T* x, const T* wr, const T* wc, const T* w, const T* v,
                         const int32_t* expert_idx, const float* gate, const float* dy,
                         float* dx, float* dwr, float* dwc, float* drb, float* dcb,
                         int32_t* counts, int32_t* active, float* dw, float* dv, float* dgate,
                         int L, int d, int Nr, int Nc, int K, char* ws, const BwdLayout& lay,
                         hipStream_t s) {
  const int N = Nr * Nc;
  const int M = L * K;
  float* coef = reinterpret_cast<float*>(ws + lay.coef);
  float* dh = reinterpret_cast<float*>(ws + lay.dh);
  float* ds = reinterpret_cast<float*>(ws + lay.ds);
  int32_t* ri = reinterpret_cast<int32_t*>(ws + lay.ri);
  int32_t* ci = reinterpret_cast<int32_t*>(ws + lay.ci);
  float* part = reinterpret_cast<float*>(ws + lay.part);
  float* psum = reinterpret_cast<float*>(ws + lay.psum);
  // dense router gradients: rows no task touches stay zero
  const size_t nr4 = static_cast<size_t>(Nr) * d / 4, nc4 = static_cast<size_t>(Nc) * d / 4;
  zero_f32x4_kernel<<<static_cast<unsigned>((nr4 + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<float4*>(dwr), nr4);
  zero_f32x4_kernel<<<static_cast<unsigned>((nc4 + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<float4*>(dwc), nc4);
  if (drb) zero_f32_kernel1<<<(Nr + 255) / 256, 256, 0, s>>>(drb, Nr);
  if (dcb) zero_f32_kernel1<<<(Nc + 255) / 256, 256, 0, s>>>(dcb, Nc);
  if (L > 0)
    bwd_token_kernel<T, EPL><<<static_cast<unsigned>((L + 3) / 4), 256, 0, s>>>(
        x, w, v, wr, wc, expert_idx, gate, dy, L, K, d, N, Nr, Nc, dx, coef, dh, ds, dgate);
  if (M > 0)
    split_ids_kernel<<<static_cast<unsigned>((M + 255) / 256), 256, 0, s>>>(expert_idx, M, N, Nc,
                                                                           ri, ci);
  auto I = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  // expert-major, grid-row-major and grid-column-major task lists
  hipError_t e = launch_schedule(L, K, N, 1, expert_idx, gate, counts, active, I(lay.es.off),
                                 I(lay.es.tok), I(lay.es.exp), F(lay.es.gat), I(lay.es.idx),
                                 ws + lay.es.ws, s);
  if (e != hipSuccess) return e;
  e = launch_schedule(L, K, Nr, 1, ri, gate, I(lay.rs.cnt), I(lay.rs.act), I(lay.rs.off),
                      I(lay.rs.tok), I(lay.rs.exp), F(lay.rs.gat), I(lay.rs.idx), ws + lay.rs.ws, s);
  if (e != hipSuccess) return e;
  e = launch_schedule(L, K, Nc, 1, ci, gate, I(lay.cs.cnt), I(lay.cs.act), I(lay.cs.off),
                      I(lay.cs.tok), I(lay.cs.exp), F(lay.cs.gat), I(lay.cs.idx), ws + lay.cs.ws, s);
  if (e != hipSuccess) return e;
  if (M == 0) return hipGetLastError();
  const unsigned nblk = static_cast<unsigned>((M + 255) / 256);  // 4 chunks of 64 per block
  const int32_t* rank = I(lay.es.ws + lay.es.lay.rank);
  const int n_exp = lay.es.lay.max_groups;
  // dV[i] = sum c dy_t, dW[i] = sum dh x_t over the tasks of active expert i
  seg_reduce_kernel<float, EPL><<<nblk, 256, 0, s>>>(I(lay.es.tok), I(lay.es.exp), I(lay.es.idx),
                                                     rank, coef, dy, M, d, L, N, n_exp, dv,
                                                     nullptr, part, psum);
  seg_fixup_kernel<float, EPL><<<nblk, 256, 0, s>>>(I(lay.es.exp), rank, M, d, N, n_exp, dv, nullptr,
                                                    part, psum);
  seg_reduce_kernel<T, EPL><<<nblk, 256, 0, s>>>(I(lay.es.tok), I(lay.es.exp), I(lay.es.idx), rank,
                                                 dh, x, M, d, L, N, n_exp, dw, nullptr, part, psum);
  seg_fixup_kernel<T, EPL><<<nblk, 256, 0, s>>>(I(lay.es.exp), rank, M, d, N, n_exp, dw, nullptr,
                                                part, psum);
  // dWr[i] = sum dS x_t over the tasks whose expert lies in grid row i; columns alike
  seg_reduce_kernel<T, EPL><<<nblk, 256, 0, s>>>(I(lay.rs.tok), I(lay.rs.exp), I(lay.rs.idx),
                                                 nullptr, ds, x, M, d, L, Nr, Nr, dwr, drb, part,
                                                 psum);
  seg_fixup_kernel<T, EPL><<<nblk, 256, 0, s>>>(I(lay.rs.exp), nullptr, M, d, Nr, Nr, dwr, drb, part,
                                                psum);
  seg_reduce_kernel<T, EPL><<<nblk, 256, 0, s>>>(I(lay.cs.tok), I(lay.cs.exp), I(lay.cs.idx),
                                                 nullptr, ds, x, M, d, L, Nc, Nc, dwc, dcb, part,
                                                 psum);
  seg_fixup_kernel<T, EPL><<<nblk, 256, 0, s>>>(I(lay.cs.exp), nullptr, M, d, Nc, Nc, dwc, dcb, part,
                                                psum);
  return hipGetLastError();
}

bool routed_backward_supported(int bf16, int d, int K) {
  const long long row_bytes = static_cast<long long>(d) * (bf16 ? 2 : 4);
  return row_bytes <= 4096 && d >= 64 && (d & (d - 1)) == 0 && K >= 1 && K <= 64;
}

hipError_t launch_routed_backward(int bf16, int L, int d, int Nr, int Nc, int K, const void* x,
                                  const void* wr, const void* wc, const void* w, const void* v,
                                  const int32_t* expert_idx, const float* gate, const float* dy,
                                  float* dx, float* dwr, float* dwc, float* drb, float* dcb,
                                  int32_t* counts, int32_t* active, float* dw, float* dv,
                                  float* dgate, void* ws, hipStream_t s) {
  const BwdLayout lay = bwd_layout(L, d, Nr, Nc, K);
  char* base = static_cast<char*>(ws);
#define OMNI_BWD(T_, D_, EPL_)                                                                  \
  case D_:                                                                                     \
    return launch_bwd_t<T_, EPL_>(static_cast<const T_*>(x), static_cast<const T_*>(wr),       \
                           static_cast<const T_*>(wc), static_cast<const T_*>(w),              \
                           static_cast<const T_*>(v), expert_idx, gate, dy, dx, dwr, dwc, drb, \
                           dcb, counts, active, dw, dv, dgate, L, d, Nr, Nc, K, base, lay, s);
  if (bf16) {
    switch (d) {
      OMNI_BWD(uint16_t, 64, 1) OMNI_BWD(uint16_t, 128, 2) OMNI_BWD(uint16_t, 256, 4)
      OMNI_BWD(uint16_t, 512, 8) OMNI_BWD(uint16_t, 1024, 16) OMNI_BWD(uint16_t, 2048, 32)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (d) {
      OMNI_BWD(float, 64, 1) OMNI_BWD(float, 128, 2) OMNI_BWD(float, 256, 4)
      OMNI_BWD(float, 512, 8) OMNI_BWD(float, 1024, 16)
      default: return hipErrorInvalidValue;
    }
  }
#undef OMNI_BWD
}

}  // namespace omni
