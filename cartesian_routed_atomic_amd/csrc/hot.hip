// Executor, hybrid form: the hot experts as two dense MFMA products, the
// rest per task.  Pages: interactive explainer "Expert-Centric Scheduling"
// (a group's expert parameters are loaded once and reused for all tokens
// assigned to it) and gist.science explainer §2.2 (grouped execution of the
// gathered tokens against a group's expert rows on matrix units).
//
// With skewed routing a few experts serve a large share of the tasks (Zipf
// routing with 16,384 tokens: 256 experts take three quarters of them).  For
// such an expert a dense product over all L tokens costs 4 L d flops on the
// matrix cores, while per-task evaluation re-reads its rows for every task.
// The hybrid form therefore splits the experts by task count:
//   * hot: at least max(2, ceil(L / kHotDensity)) tasks, that threshold
//     doubled until no more than kHotCap experts reach it.  Their
//     coefficients for every (token, hot expert) pair come from one bf16 MFMA
//     product H = x WH^T with the epilogue c = G * silu(H), where G holds the
//     gate of each task and 0 elsewhere; then y = C VH, a second MFMA
//     product, with c rounded to bf16 for it (fp32 accumulation);
//   * cold: every other task goes through the token-centric kernels, whose
//     per-token lists are compacted here, and is added onto that y.
// The hot list is sorted by expert id, so the result is deterministic.  The
// per-token lists must not repeat an expert (the top-K never does); repeats
// of a hot expert have their gates summed.
#include <climits>

#include "device.hpp"
#include "launch.hpp"

namespace omni {

// Hot slots are padded to a multiple of kHotPad (the column tiles of the
// products are 256 wide; their K steps 32).
constexpr int kHotPad = 128;

// info[0] = number of hot experts, info[1] = that rounded up to kHotPad (the
// padded width of the hot products), info[2] = whether the cold pass adds
// onto y (1) or overwrites it (0), info[8 + i] = experts with at least
// thr << i tasks (i < kLevels).
constexpr int kInfoInts = 64, kLevels = 16;

// Task counting: each workgroup aggregates a chunk of the tasks in an
// LDS hash table, then adds one count per distinct expert to memory, so a
// hot expert sees one atomic per chunk instead of one per task.
// Chunk c adds its counts to replica c % kCountReps, so the busiest
// experts' atomics spread over kCountReps addresses; readers sum the
// replicas.  After the sort, replica 0 marks hot expert e in slot s as
// -(s + 1) (a slot map for the split).
constexpr int kCountChunk = 2048, kCountSlots = 4096, kCountReps = 4;

size_t hot_threshold(int L, int K) {
  (void)K;
  const long long thr = (static_cast<long long>(L) + kHotDensity - 1) / kHotDensity;
  return static_cast<size_t>(thr > 2 ? thr : 2);
}

namespace {

constexpr size_t al256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

struct HotLayout {
  size_t ce, cg, kc, info, hot, g, cb, wh, vt, total;
  HotLayout(int L, int K, int d, int N) {
    const size_t M = static_cast<size_t>(L) * K;
    size_t o = 0;
    ce = o; o += al256(M * 4);
    cg = o; o += al256(M * 4);
    kc = o; o += al256(static_cast<size_t>(L) * 4);
    info = o; o += al256((kInfoInts + kCountReps * static_cast<size_t>(N) + 3) / 4 * 16);  // info, counts
    hot = o; o += al256(2 * kHotCap * 4);  // picked (any order), then sorted
    g = o; o += al256(static_cast<size_t>(L) * kHotCap * 4);
    cb = o; o += al256(static_cast<size_t>(L) * kHotCap * 2);
    wh = o; o += al256(static_cast<size_t>(kHotCap) * d * 2);
    vt = o; o += al256(static_cast<size_t>(d) * kHotCap * 2);
    total = o;
  }
};

__global__ __launch_bounds__(256) void hot_zero_kernel(int4* __restrict__ p, size_t n4) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_int4(0, 0, 0, 0);
}

// Tasks per expert (ids outside [0, N) count as expert 0, as the token
// kernels read them), over chunks of kCountChunk tasks of the sorted task
// list.  Sorted by group, a chunk spans few groups, so a hot expert is
// flushed by few chunks (Zipf routing, 2^20 tasks: 15 us with four count
// replicas, 41 us with one; over the token-major flattened selection every
// chunk holds the hot experts and their global atomics serialise: 149 us).
__global__ __launch_bounds__(256) void hot_count_kernel(const int32_t* __restrict__ te, int M,
                                                        int N, int32_t* __restrict__ cnt) {
  __shared__ int key[kCountSlots];
  __shared__ int num[kCountSlots];
  const int tid = threadIdx.x;
  for (int i = tid; i < kCountSlots; i += 256) {
    key[i] = -1;
    num[i] = 0;
  }
  __syncthreads();
  const int p0 = blockIdx.x * kCountChunk, p1 = min(M, p0 + kCountChunk);
  for (int p = p0 + tid; p < p1; p += 256) {
    const int e0 = te[p];
    const int e = static_cast<unsigned>(e0) < static_cast<unsigned>(N) ? e0 : 0;
    // at most kCountChunk distinct keys in a table of twice that: a free or
    // matching slot is always found
    unsigned h = (static_cast<unsigned>(e) * 2654435761u) >> 20;  // 12 bits
    for (;;) {
      const int k = atomicCAS(&key[h], -1, e);
      if (k == -1 || k == e) {
        atomicAdd(&num[h], 1);
        break;
      }
      h = (h + 1) & (kCountSlots - 1);
    }
  }
  __syncthreads();
  int32_t* rep = cnt + static_cast<size_t>(blockIdx.x % kCountReps) * N;
  for (int i = tid; i < kCountSlots; i += 256)
    if (key[i] >= 0) atomicAdd(&rep[key[i]], num[i]);
}

__device__ __forceinline__ int task_count(const int32_t* __restrict__ cnt, int N, int e) {
  int c = 0;
#pragma unroll
  for (int r = 0; r < kCountReps; ++r) c += cnt[static_cast<size_t>(r) * N + e];
  return c;
}

// info[8 + i] = experts with at least thr << i tasks (one atomic per wave
// and level).
__global__ __launch_bounds__(256) void hot_level_kernel(const int32_t* __restrict__ cnt, int N,
                                                        int thr, int32_t* __restrict__ info) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int c = e < N ? task_count(cnt, N, e) : 0;
  if (__ballot(c >= thr) == 0) return;  // uniform over the wave
  for (int i = 0; i < kLevels; ++i) {
    const int n = __popcll(__ballot(c >= (static_cast<long long>(thr) << i)));
    if (n == 0) break;
    if (lane() == 0) atomicAdd(&info[8 + i], n);
  }
}

// The hot experts: at least thr << i tasks for the least level i at which no
// more than kHotCap experts qualify; appended in any order (sorted next).
__global__ __launch_bounds__(256) void hot_pick_kernel(const int32_t* __restrict__ cnt, int N,
                                                       int thr, int32_t* __restrict__ hot,
                                                       int32_t* __restrict__ info) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= N) return;
  int lv = 0;
  while (lv < kLevels - 1 && info[8 + lv] > kHotCap) ++lv;
  if (task_count(cnt, N, e) < (static_cast<long long>(thr) << lv)) return;
  const int j = atomicAdd(&info[0], 1);
  if (j < kHotCap) hot[j] = e;
}

// The hot list in ascending id order (ids are distinct, so an id's place is
// the number of smaller ids): each of kSortBlocks workgroups loads every id
// and places kHotCap / kSortBlocks of them (the count is VALU work, spread
// over that many CUs); workgroup 0 also writes the sizes and the cold
// pass's accumulate flag (the capped count it stores gives every workgroup
// the same n).  The places go to a second list: hot itself is still being
// read by the other workgroups.
constexpr int kSortBlocks = 8, kSortThreads = kHotCap / kSortBlocks;
__global__ __launch_bounds__(kSortThreads) void hot_sort_kernel(
    const int32_t* __restrict__ hot_in, int32_t* __restrict__ hot, int32_t* __restrict__ info,
    int32_t* __restrict__ cnt, int accumulate) {
  __shared__ __attribute__((aligned(16))) int key[kHotCap];
  const int tid = threadIdx.x;
  const int n = min(info[0], kHotCap);
  const int n4 = (n + 3) / 4;
  for (int i = tid; i < 4 * n4; i += kSortThreads) key[i] = i < n ? hot_in[i] : INT_MAX;
  __syncthreads();
  {
    const int i = blockIdx.x * kSortThreads + tid;
    if (i < n) {
      const int k = key[i];
      int r = 0;
#pragma unroll 8
      for (int j = 0; j < n4; ++j) {  // pads are INT_MAX, never smaller
        const int4 v = reinterpret_cast<const int4*>(key)[j];
        r += (v.x < k) + (v.y < k) + (v.z < k) + (v.w < k);
      }
      hot[r] = k;
      cnt[k] = -(r + 1);  // replica 0 as the slot map
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    info[0] = n;
    info[1] = (n + kHotPad - 1) / kHotPad * kHotPad;
    info[2] = (n > 0 || accumulate) ? 1 : 0;
  }
}

// WH[s, :] = W[hot[s], :] and VT[:, s] = V[hot[s], :] for s < info[1] (zero
// for s >= info[0]).  Block: 64 hot slots x 64 columns; VT goes through an
// LDS transpose so both sides are written in 16-byte pieces.
__global__ __launch_bounds__(256) void hot_gather_kernel(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ hot, const int32_t* __restrict__ info, int d,
    uint16_t* __restrict__ WH, uint16_t* __restrict__ VT) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int nh = info[0], hp = info[1];
  const int s0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (s0 >= hp) return;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, r = c >> 3, ch = (c & 7) * 8;
    const int s = s0 + r;
    uint4 wv = make_uint4(0, 0, 0, 0), vv = wv;
    if (s < nh) {
      const size_t o = static_cast<size_t>(hot[s]) * d + c0 + ch;
      wv = *reinterpret_cast<const uint4*>(W + o);
      vv = *reinterpret_cast<const uint4*>(V + o);
    }
    *reinterpret_cast<uint4*>(WH + static_cast<size_t>(s) * d + c0 + ch) = wv;
    *reinterpret_cast<uint4*>(&tile[r][ch]) = vv;
  }
  __syncthreads();
  const int cc = tid >> 2, sb = (tid & 3) * 16;
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    pk[j] = static_cast<uint32_t>(tile[sb + 2 * j][cc]) |
            (static_cast<uint32_t>(tile[sb + 2 * j + 1][cc]) << 16);
  uint4* dst = reinterpret_cast<uint4*>(VT + static_cast<size_t>(c0 + cc) * kHotCap + s0 + sb);
  dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
}

// One wave per token: its hot tasks put their gates into row t of G (built
// in LDS, written whole), its cold tasks are compacted, in task order, into
// ce / cg[t K, t K + kc[t]).
__global__ __launch_bounds__(256) void hot_split_kernel(
    const int32_t* __restrict__ fe, const float* __restrict__ fg, const int32_t* __restrict__ slot_map,
    const int32_t* __restrict__ info, int L, int K, int N, float* __restrict__ G,
    int32_t* __restrict__ ce, float* __restrict__ cg, int32_t* __restrict__ kc) {
  __shared__ __attribute__((aligned(16))) float sg[4][kHotCap];
  const int w = threadIdx.x >> 6, l = lane();
  const int hp = info[1];
  for (int i = l; i < hp; i += 64) sg[w][i] = 0.f;
  __syncthreads();
  const int t = blockIdx.x * 4 + w;
  if (t < L) {
    int base = 0;
    for (int k0 = 0; k0 < K; k0 += 64) {
      const int n = min(64, K - k0);
      int e = 0, slot = -1;
      float g = 0.f;
      if (l < n) {
        const size_t o = static_cast<size_t>(t) * K + k0 + l;
        const int e0 = fe[o];
        e = static_cast<unsigned>(e0) < static_cast<unsigned>(N) ? e0 : 0;
        g = fg[o];
        const int m = slot_map[e];  // -(s + 1) for the hot expert in slot s
        slot = m < 0 ? -m - 1 : -1;
      }
      if (slot >= 0) atomicAdd(&sg[w][slot], g);
      const bool cold = l < n && slot < 0;
      const uint64_t mask = __ballot(cold);
      if (cold) {
        const size_t o = static_cast<size_t>(t) * K + base +
                         __popcll(mask & ((1ull << l) - 1ull));
        ce[o] = e;
        cg[o] = g;
      }
      base += __popcll(mask);
    }
    if (l == 0) kc[t] = base;
  }
  __syncthreads();
  if (t < L) {
    float* grow = G + static_cast<size_t>(t) * kHotCap;
    for (int i = l * 4; i < hp; i += 256)
      *reinterpret_cast<float4*>(grow + i) =
          make_float4(sg[w][i], sg[w][i + 1], sg[w][i + 2], sg[w][i + 3]);
  }
}

}  // namespace

size_t hot_ws_bytes(int L, int K, int d, int N) { return HotLayout(L, K, d, N).total; }

hipError_t launch_hot_part(const uint16_t* x, const uint16_t* w, const uint16_t* v,
                           const int32_t* task_expert, const int32_t* fe, const float* fg, int L,
                           int K, int d, int N, float* y, int accumulate, void* hws,
                           HotCold* out, hipStream_t s) {
  const HotLayout lay(L, K, d, N);
  char* base = static_cast<char*>(hws);
  int32_t* ce = reinterpret_cast<int32_t*>(base + lay.ce);
  float* cg = reinterpret_cast<float*>(base + lay.cg);
  int32_t* kc = reinterpret_cast<int32_t*>(base + lay.kc);
  int32_t* info = reinterpret_cast<int32_t*>(base + lay.info);
  int32_t* cnt = info + kInfoInts;
  int32_t* picked = reinterpret_cast<int32_t*>(base + lay.hot);
  int32_t* hot = picked + kHotCap;
  float* G = reinterpret_cast<float*>(base + lay.g);
  uint16_t* Cb = reinterpret_cast<uint16_t*>(base + lay.cb);
  uint16_t* WH = reinterpret_cast<uint16_t*>(base + lay.wh);
  uint16_t* VT = reinterpret_cast<uint16_t*>(base + lay.vt);
  const int M = L * K;
  const size_t n4 = (kInfoInts + kCountReps * static_cast<size_t>(N) + 3) / 4;
  hot_zero_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<int4*>(info), n4);
  const int thr = static_cast<int>(hot_threshold(L, K));
  hot_count_kernel<<<static_cast<unsigned>((M + kCountChunk - 1) / kCountChunk), 256, 0, s>>>(
      task_expert, M, N, cnt);
  const unsigned nb = static_cast<unsigned>((N + 255) / 256);
  hot_level_kernel<<<nb, 256, 0, s>>>(cnt, N, thr, info);
  hot_pick_kernel<<<nb, 256, 0, s>>>(cnt, N, thr, picked, info);
  hot_sort_kernel<<<kSortBlocks, kSortThreads, 0, s>>>(picked, hot, info, cnt, accumulate);
  hot_gather_kernel<<<dim3(kHotCap / 64, static_cast<unsigned>(d / 64)), 256, 0, s>>>(
      w, v, hot, info, d, WH, VT);
  hot_split_kernel<<<static_cast<unsigned>((L + 3) / 4), 256, 0, s>>>(fe, fg, cnt, info, L, K, N,
                                                                      G, ce, cg, kc);
  const hipError_t e = launch_hot_products(x, WH, VT, G, Cb, y, L, d, kHotCap, info + 0,
                                           accumulate, s);
  if (e != hipSuccess) return e;
  out->expert = ce;
  out->gate = cg;
  out->count = kc;
  out->accumulate = info + 2;
  return hipGetLastError();
}

}  // namespace omni
