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
// rows and columns of the selected experts.  Both router products are dense
// MFMA GEMMs over that mostly-zero dz: dx += dz [Wr; Wc] and
// [dWr; dWc] = dz^T x (dense beats gathering 2K router rows per token: the
// two tables together outgrow one XCD's L2).
//
// Two kinds of kernels:
//   bwd_token_kernel: one wave per token (x_t and dy_t in registers) walks the
//     token's V rows (u_k) and W rows (h_k -> dh_k, dg_k, c_k; dx += dh_k W[e]);
//     writes dx_t, the per-task c, dh, dS, dg at the flat task id, and the
//     token's row of dz and column of dz^T.
//   seg_reduce_kernel + seg_fixup_kernel: dV[row] = sum c dy[token] and
//     dW[row] = sum dh x[token] over the expert-major task list, a schedule
//     with groups of one (B = 1) built by the forward's scheduling code.  Each wave
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

// float32 -> element type: bf16 by round to nearest even (finite values)
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
  const uint32_t u = __float_as_uint(v);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

constexpr int kBwdRing = 4;  // row slots per wave: three in flight
constexpr int kSegEpl = 16;  // row elements per lane in the dV / dW reduction

// NT: the W and V rows carry the nontemporal hint (stream_rows).
template <typename T, int EPL, bool NT>
__global__ __launch_bounds__(256, 3) void bwd_token_kernel(
    const T* __restrict__ x, const T* __restrict__ W, const T* __restrict__ V,
    const int32_t* __restrict__ expert_idx,
    const float* __restrict__ gate, const float* __restrict__ dy, int L, int K, int d, int N,
    int Nr, int Nc, float* __restrict__ dx, float* __restrict__ coef, float* __restrict__ dh_out,
    float* __restrict__ ds_out, float* __restrict__ dgate, float* __restrict__ dzt, int Lp,
    T* __restrict__ dz, int ldz) {
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
    if (s < K) f[s].template fetch<NT>(V + static_cast<size_t>(rdlane(my_e, s)) * d, l);
  for (int i = 0; i < K; i += kBwdRing) {
#pragma unroll
    for (int s = 0; s < kBwdRing; ++s) {
      const int k = i + s;
      if (k >= K) break;
      if (k + kBwdRing - 1 < K)
        f[(s + kBwdRing - 1) % kBwdRing].template fetch<NT>(
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
    if (s < K) f[s].template fetch<NT>(W + static_cast<size_t>(rdlane(my_e, s)) * d, l);
  for (int i = 0; i < K; i += kBwdRing) {
#pragma unroll
    for (int s = 0; s < kBwdRing; ++s) {
      const int k = i + s;
      if (k >= K) break;
      if (k + kBwdRing - 1 < K)
        f[(s + kBwdRing - 1) % kBwdRing].template fetch<NT>(
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

  const int my_ri = my_e / Nc, my_ci = my_e - (my_e / Nc) * Nc;
  store_row<T, EPL, kStorePlain>(acc, dx + static_cast<size_t>(t) * d, 0);
  // the token's logit gradients: dz_r[t, i] is the sum of dS over the token's
  // tasks in grid row i (summed in task order, stored by the first such task),
  // dz_c likewise; written to row t of dz (grid rows, then grid columns, for
  // the dx product) and to column t of dz^T (for the dWr, dWc product)
  float rsum = 0.f, csum = 0.f;
  bool rfirst = true, cfirst = true;
  for (int j = 0; j < K; ++j) {
    const float dj = rdlane(my_ds, j);
    if (rdlane(my_ri, j) == my_ri) {
      rsum += dj;
      rfirst = rfirst && j >= l;
    }
    if (rdlane(my_ci, j) == my_ci) {
      csum += dj;
      cfirst = cfirst && j >= l;
    }
  }
  if (l < K) {
    coef[tb + l] = my_c;
    dh_out[tb + l] = my_dh;
    ds_out[tb + l] = my_ds;
    if (dgate) dgate[tb + l] = my_dg;
    T* dzrow = dz + static_cast<size_t>(t) * ldz;
    if (rfirst) {
      dzt[static_cast<size_t>(my_ri) * Lp + t] = rsum;
      dzrow[my_ri] = from_f32<T>(rsum);
    }
    if (cfirst) {
      dzt[static_cast<size_t>(Nr + my_ci) * Lp + t] = csum;
      dzrow[Nr + my_ci] = from_f32<T>(csum);
    }
  }
}

// Row sums of the transposed logit gradients (the bias gradients) and their
// bf16 copy for the GEMM.  One wave per row (Lp a multiple of 64), four float4
// loads in flight per lane, lane partials added in a fixed order.
__device__ __forceinline__ uint32_t bf16_rne2(float lo, float hi) {
  // round to nearest even (finite values), two per word
  const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  return ((a + 0x7fffu + ((a >> 16) & 1u)) >> 16) |
         ((b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u);
}

__global__ __launch_bounds__(256) void dz_rows_kernel(const float* __restrict__ dzt, int rows,
                                                      int Lp, int Nr, uint16_t* __restrict__ dzt16,
                                                      float* __restrict__ drb,
                                                      float* __restrict__ dcb) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane();
  if (r >= rows) return;
  const float4* src = reinterpret_cast<const float4*>(dzt + static_cast<size_t>(r) * Lp);
  uint2* dst = dzt16 ? reinterpret_cast<uint2*>(dzt16 + static_cast<size_t>(r) * Lp) : nullptr;
  const int n4 = Lp >> 2;
  float sum = 0.f;
  for (int b = 0; b < n4; b += 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = b + u * 64 + l;
      v[u] = i < n4 ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = b + u * 64 + l;
      sum += (v[u].x + v[u].y) + (v[u].z + v[u].w);
      if (dst && i < n4) dst[i] = make_uint2(bf16_rne2(v[u].x, v[u].y), bf16_rne2(v[u].z, v[u].w));
    }
  }
  sum = wave_sum(sum);
  if (l == 0) {
    if (r < Nr) {
      if (drb) drb[r] = sum;
    } else if (dcb) {
      dcb[r - Nr] = sum;
    }
  }
}

// Transpose with zero padding of two stacked row blocks: the input rows are
// in0 [R0, d] followed by in1 [R1, d]; out[c][r] = row r, column c for
// r < R0 + R1 and 0 for R0 + R1 <= r < Lp (out [d, Lp]), through a 64 x 64
// LDS tile.
template <typename T>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const T* __restrict__ in0, int R0,
                                                            const T* __restrict__ in1, int R1,
                                                            int d, int Lp, T* __restrict__ out) {
  __shared__ T tile[64][65];
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 64; i += 4) {
    const int r = t0 + ty + i, c = c0 + tx;
    T v = T(0);
    if (c < d) {
      if (r < R0) v = in0[static_cast<size_t>(r) * d + c];
      else if (r < R0 + R1) v = in1[static_cast<size_t>(r - R0) * d + c];
    }
    tile[ty + i][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 64; i += 4) {
    const int c = c0 + ty + i, r = t0 + tx;
    if (c < d && r < Lp) out[static_cast<size_t>(c) * Lp + r] = tile[tx][ty + i];
  }
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

// Wave w of column block y: sorted tasks [64 w, 64 w + 64) and columns
// [64 EPL y, 64 EPL (y + 1)).  dV[row] = sum_m c_m dy[token_m] and
// dW[row] = sum_m dh_m x[token_m] over the tasks m of the row's expert, both
// from one walk of the task list.  Partials of rows crossing a chunk edge go
// to part[((2 w + slot) * 2 + o) * d] (o = 0 for dV, 1 for dW): slot 0 if the
// row began before the chunk, else slot 1 (the row begins here and continues).
template <typename T, int EPL>
__global__ __launch_bounds__(256) void seg_reduce_kernel(
    const int32_t* __restrict__ task_token, const int32_t* __restrict__ task_expert,
    const int32_t* __restrict__ task_index, const int32_t* __restrict__ rank,
    const float* __restrict__ coef, const float* __restrict__ dh, const float* __restrict__ dy,
    const T* __restrict__ x, int M, int d, int L, int n_ids, int n_rows, float* __restrict__ dv,
    float* __restrict__ dw, float* __restrict__ part) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane();
  const int p0 = wv * 64;
  if (p0 >= M) return;
  const int col0 = blockIdx.y * 64 * EPL;
  const int n = min(64, M - p0);
  int my_t = 0, my_r = 0;
  float my_c = 0.f, my_h = 0.f;
  if (l < n) {
    const int p = p0 + l;
    const int t = task_token[p];
    my_t = static_cast<unsigned>(t) < static_cast<unsigned>(L) ? t : 0;
    my_r = out_row_of(task_expert, rank, p, n_ids, n_rows);
    const int m = task_index[p];
    const bool ok = static_cast<unsigned>(m) < static_cast<unsigned>(M);
    my_c = ok ? coef[m] : 0.f;
    my_h = ok ? dh[m] : 0.f;
  }
  // does the first row begin before this chunk / the last row continue after it?
  const bool head = p0 > 0 && out_row_of(task_expert, rank, p0 - 1, n_ids, n_rows) == rdlane(my_r, 0);
  const bool tail = p0 + n < M && out_row_of(task_expert, rank, p0 + n, n_ids, n_rows) == rdlane(my_r, n - 1);
  constexpr int R = kBwdRing;
  RowFrag<float, EPL> fy[R];
  RowFrag<T, EPL> fx[R];
  const float* dyc = dy + col0;
  const T* xc = x + col0;
  float av[EPL], aw[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) av[q] = aw[q] = 0.f;
  int seg_start = 0;
#pragma unroll
  for (int s = 0; s < R - 1; ++s) {
    if (s < n) {
      const size_t o = static_cast<size_t>(rdlane(my_t, s)) * d;
      fy[s].load(dyc + o, l);
      fx[s].load(xc + o, l);
    }
  }
  for (int i = 0; i < n; i += R) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int k = i + s;
      if (k >= n) break;
      if (k + R - 1 < n) {
        const size_t o = static_cast<size_t>(rdlane(my_t, k + R - 1)) * d;
        fy[(s + R - 1) % R].load(dyc + o, l);
        fx[(s + R - 1) % R].load(xc + o, l);
      }
      const float ck = rdlane(my_c, k), hk = rdlane(my_h, k);
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        av[q] = fmaf(ck, fy[s].get(q), av[q]);
        aw[q] = fmaf(hk, fx[s].get(q), aw[q]);
      }
      const int row = rdlane(my_r, k);
      const bool last_of_row = k == n - 1 || rdlane(my_r, k + 1) != row;
      if (last_of_row) {
        const bool began_before = seg_start == 0 && head;
        const bool goes_on = k == n - 1 && tail;
        float* dst_v;
        float* dst_w;
        if (!began_before && !goes_on) {
          dst_v = dv + static_cast<size_t>(row) * d + col0;
          dst_w = dw + static_cast<size_t>(row) * d + col0;
        } else {
          const int slot = began_before ? 0 : 1;
          dst_v = part + static_cast<size_t>((2 * wv + slot) * 2) * d + col0;
          dst_w = dst_v + d;
        }
        store_row<float, EPL, kStorePlain>(av, dst_v, 0);
        store_row<T, EPL, kStorePlain>(aw, dst_w, 0);
#pragma unroll
        for (int q = 0; q < EPL; ++q) av[q] = aw[q] = 0.f;
        seg_start = k + 1;
      }
    }
  }
}

// Rows that cross chunk edges: the wave of the chunk where such a row begins
// (its slot-1 partials) adds the slot-0 partials of the following chunks, in
// order, for as long as the row continues.
template <typename T, int EPL>
__global__ __launch_bounds__(256) void seg_fixup_kernel(
    const int32_t* __restrict__ task_expert, const int32_t* __restrict__ rank, int M, int d,
    int n_ids, int n_rows, float* __restrict__ dv, float* __restrict__ dw,
    const float* __restrict__ part) {
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
  const int col0 = blockIdx.y * 64 * EPL;
  float tv[EPL], tw[EPL], a[EPL];
  const float* own = part + static_cast<size_t>((2 * wv + 1) * 2) * d + col0;
  load_f32_as<float, EPL>(own, l, tv);
  load_f32_as<T, EPL>(own + d, l, tw);
  for (int c = wv + 1;; ++c) {
    const float* pc = part + static_cast<size_t>(2 * c * 2) * d + col0;
    load_f32_as<float, EPL>(pc, l, a);
#pragma unroll
    for (int q = 0; q < EPL; ++q) tv[q] += a[q];
    load_f32_as<T, EPL>(pc + d, l, a);
#pragma unroll
    for (int q = 0; q < EPL; ++q) tw[q] += a[q];
    const int ce = min((c + 1) * 64, M);
    if (ce >= M || out_row_of(task_expert, rank, ce, n_ids, n_rows) != row) break;
  }
  store_row<float, EPL, kStorePlain>(tv, dv + static_cast<size_t>(row) * d + col0, 0);
  store_row<T, EPL, kStorePlain>(tw, dw + static_cast<size_t>(row) * d + col0, 0);
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
  b.lay = schedule_ws_layout(L, K, N, 1, 0);
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
  size_t bytes, coef, dh, ds, part, dzt, dzt16, xt, cgrad, dz, wrct, gpart;
  int Lp;        // tokens padded to a multiple of 64 (inner dimension of the dWr, dWc product)
  int Rp;        // grid rows + columns padded to a multiple of 64 (that of the dx product)
  SchedBufs es;  // experts, groups of one (the caller's counts / active)
};
}  // namespace

static BwdLayout bwd_layout(int L, int d, int Nr, int Nc, int K, int bf16) {
  BwdLayout w{};
  const size_t M = static_cast<size_t>(L) * K;
  const size_t m1 = M > 0 ? M : 1;
  const size_t es = bf16 ? 2 : 4;
  w.Lp = ((L > 0 ? L : 1) + 63) / 64 * 64;
  const size_t nrc = static_cast<size_t>(Nr) + Nc;
  size_t o = 0;
  w.coef = o;  o = a256(o + m1 * 4);
  w.dh = o;    o = a256(o + m1 * 4);
  w.ds = o;    o = a256(o + m1 * 4);
  const size_t chunks = (m1 + 63) / 64;
  w.part = o;  o = a256(o + chunks * 4 * static_cast<size_t>(d) * 4);
  w.dzt = o;   o = a256(o + nrc * w.Lp * 4);
  w.dzt16 = o; o = a256(o + (bf16 ? nrc * w.Lp * 2 : 0));
  w.xt = o;    o = a256(o + static_cast<size_t>(d) * w.Lp * es);
  w.cgrad = o; o = a256(o + nrc * static_cast<size_t>(d) * 4);
  w.Rp = static_cast<int>((nrc + 63) / 64 * 64);
  w.dz = o;    o = a256(o + static_cast<size_t>(L > 0 ? L : 1) * w.Rp * es);
  w.wrct = o;  o = a256(o + static_cast<size_t>(d) * w.Rp * es);
  // split-K partials of the two router products (they run one after the other)
  const size_t g1 = gemm_nt_ws_bytes(bf16, L, d, w.Rp);
  const size_t g2 = gemm_nt_ws_bytes(bf16, static_cast<int>(nrc), d, w.Lp);
  w.gpart = o; o = a256(o + (g1 > g2 ? g1 : g2));
  const long long N = static_cast<long long>(Nr) * Nc;
  w.es = sched_bufs(o, L, K, static_cast<int>(N));
  w.bytes = o;
  return w;
}

size_t routed_backward_ws_bytes(int bf16, int L, int d, int Nr, int Nc, int K) {
  return bwd_layout(L, d, Nr, Nc, K, bf16).bytes;
}

template <typename T, int EPL>
static hipError_t launch_bwd_t(const T* x, const T* wr, const T* wc, const T* w, const T* v,
                               const int32_t* expert_idx, const float* gate, const float* dy,
                               float* dx, float* dwr, float* dwc, float* drb, float* dcb,
                               int32_t* counts, int32_t* active, float* dw, float* dv,
                               float* dgate, int L, int d, int Nr, int Nc, int K, char* ws,
                               const BwdLayout& lay, hipStream_t s) {
  constexpr int bf16 = sizeof(T) == 2;
  const int N = Nr * Nc;
  const int M = L * K;
  const int NRC = Nr + Nc, Lp = lay.Lp;
  float* coef = reinterpret_cast<float*>(ws + lay.coef);
  float* dh = reinterpret_cast<float*>(ws + lay.dh);
  float* ds = reinterpret_cast<float*>(ws + lay.ds);
  float* part = reinterpret_cast<float*>(ws + lay.part);
  float* dzt = reinterpret_cast<float*>(ws + lay.dzt);
  uint16_t* dzt16 = bf16 ? reinterpret_cast<uint16_t*>(ws + lay.dzt16) : nullptr;
  T* xt = reinterpret_cast<T*>(ws + lay.xt);
  float* cgrad = reinterpret_cast<float*>(ws + lay.cgrad);
  T* dz = reinterpret_cast<T*>(ws + lay.dz);
  T* wrct = reinterpret_cast<T*>(ws + lay.wrct);
  const int Rp = lay.Rp;
  // logit gradients start at zero (a token writes only its own rows / columns)
  const size_t nz4 = static_cast<size_t>(NRC) * Lp / 4;
  zero_f32x4_kernel<<<static_cast<unsigned>((nz4 + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<float4*>(dzt), nz4);
  const size_t nzb = static_cast<size_t>(L) * Rp * sizeof(T) / 16;
  if (nzb > 0)
    zero_f32x4_kernel<<<static_cast<unsigned>((nzb + 255) / 256), 256, 0, s>>>(
        reinterpret_cast<float4*>(dz), nzb);
  // [Wr; Wc]^T, zero-padded to Rp columns: the right operand of the dx product
  transpose_pad_kernel<T><<<dim3(static_cast<unsigned>(Rp / 64),
                                 static_cast<unsigned>((d + 63) / 64)), 256, 0, s>>>(
      wr, Nr, wc, Nc, d, Rp, wrct);
  if (L > 0 && stream_rows(M, N))
    bwd_token_kernel<T, EPL, true><<<static_cast<unsigned>((L + 3) / 4), 256, 0, s>>>(
        x, w, v, expert_idx, gate, dy, L, K, d, N, Nr, Nc, dx, coef, dh, ds, dgate, dzt, Lp, dz,
        Rp);
  else if (L > 0)
    bwd_token_kernel<T, EPL, false><<<static_cast<unsigned>((L + 3) / 4), 256, 0, s>>>(
        x, w, v, expert_idx, gate, dy, L, K, d, N, Nr, Nc, dx, coef, dh, ds, dgate, dzt, Lp, dz,
        Rp);
  // router part of dx: dx += [dz_r dz_c] [Wr; Wc], one MFMA product
  void* gpart = ws + lay.gpart;
  hipError_t e = launch_gemm_nt(bf16, dz, wrct, dx, L, d, Rp, 1,
                                gemm_nt_ws_bytes(bf16, L, d, Rp) ? gpart : nullptr, s);
  if (e != hipSuccess) return e;
  // router weights: [dWr; dWc] = dz^T x, one MFMA product over the padded tokens
  dz_rows_kernel<<<static_cast<unsigned>((NRC + 3) / 4), 256, 0, s>>>(dzt, NRC, Lp, Nr, dzt16,
                                                                     drb, dcb);
  transpose_pad_kernel<T><<<dim3(static_cast<unsigned>(Lp / 64),
                                 static_cast<unsigned>((d + 63) / 64)), 256, 0, s>>>(
      x, L, nullptr, 0, d, Lp, xt);
  e = launch_gemm_nt(bf16, bf16 ? static_cast<const void*>(dzt16) : static_cast<const void*>(dzt),
                     xt, cgrad, NRC, d, Lp, 0,
                     gemm_nt_ws_bytes(bf16, NRC, d, Lp) ? gpart : nullptr, s);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(dwr, cgrad, static_cast<size_t>(Nr) * d * 4, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(dwc, cgrad + static_cast<size_t>(Nr) * d, static_cast<size_t>(Nc) * d * 4,
                     hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  // expert weights: dV[i] = sum c dy_t, dW[i] = sum dh x_t over the tasks of
  // active expert i, from the expert-major task list
  auto I = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  e = launch_schedule(L, K, N, 1, 0, expert_idx, gate, counts, active, I(lay.es.off), I(lay.es.tok),
                      I(lay.es.exp), F(lay.es.gat), I(lay.es.idx), ws + lay.es.ws, s);
  if (e != hipSuccess) return e;
  if (M == 0) return hipGetLastError();
  // columns in blocks of 64 * RE: more, smaller waves than one per whole row
  constexpr int RE = EPL < kSegEpl ? EPL : kSegEpl;
  const dim3 grid(static_cast<unsigned>((M + 255) / 256), EPL / RE);  // 4 chunks of 64 per block
  const int32_t* rank = I(lay.es.ws + lay.es.lay.rank);
  const int n_exp = lay.es.lay.max_groups;
  seg_reduce_kernel<T, RE><<<grid, 256, 0, s>>>(I(lay.es.tok), I(lay.es.exp), I(lay.es.idx), rank,
                                                coef, dh, dy, x, M, d, L, N, n_exp, dv, dw, part);
  seg_fixup_kernel<T, RE><<<grid, 256, 0, s>>>(I(lay.es.exp), rank, M, d, N, n_exp, dv, dw, part);
  (void)ds;
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
  const BwdLayout lay = bwd_layout(L, d, Nr, Nc, K, bf16);
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
