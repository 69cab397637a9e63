// Expert-Centric Scheduling.  Pages: interactive explainer "Expert-Centric
// Scheduling" (flatten every (token, expert, weight) decision into M = L*K
// tasks; collect the unique active experts, sort them by id, cut them into
// groups of B; order the tasks by group first and token second) and
// gist.science explainer §2.2 (task collection, grouping and sorting).
//
// Device pipeline, no host synchronisation (n_active and n_groups stay on
// the device):
//   1. clear a byte flag per expert, then mark every expert some task uses
//      (plain byte stores of 1: without a read first the marking runs 3 us
//      faster at large and no slower under Zipf routing);
//   2. count flags per 4096-expert tile; each tile sums the counts of the
//      tiles before it, scans its own flags and writes rank[e] (position
//      among active experts) and the ascending active list;
//   3. stable LSD radix sort of the tasks by group g = rank[e] / B (or, in
//      the fixed-window variant, g = e / B: the id window): one pass of up
//      to 11 bits (up to 2048 groups), else passes of at most 8 bits.  Tasks
//      enter in flatten order m = t*K + k, which is already token-major, so
//      a stable sort by group alone yields (group, token) order with ties in
//      flatten order.  Each pass: per-tile digit histograms (the first pass
//      computes the group keys on the way), a parallel scan of each digit's
//      tile counts (with at most 32 tiles the scatter kernel sums them
//      itself), then a stable scatter ranked with one ballot per digit bit.
//      When several passes are
//      possible, passes beyond the digits that n_groups actually needs
//      return at once;
//   4. CSR group offsets: a single pass writes them from its digit bases
//      (the digit is the group); several passes take them from the group
//      boundaries of the sorted keys.
#include "device.hpp"
#include "launch.hpp"

namespace omni {

constexpr int kTile = 4096;   // experts per flag tile (256 threads x 16)
constexpr int kInlineCountTiles = 8;  // up to 32,768 experts: no separate tile-count launch
constexpr int kMaxDigitBits = 11;
constexpr int kMaxDigits = 1 << kMaxDigitBits;
constexpr int kSortWaves = 8;  // waves of a sort block (512 threads)
constexpr int kSortR = 4;  // tasks per lane: a sort tile is 2048 tasks
constexpr int kSTile = 512 * kSortR;
// Up to this many sort tiles the scatter kernel sums its digit rows of tile
// counts itself (no row-scan launch).
constexpr int kFuseTiles = 32;

static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

ScheduleWs schedule_ws_layout(int L, int K, int N, int B, int window) {
  ScheduleWs w{};
  const long long M = static_cast<long long>(L) * K;
  w.n_ftiles = static_cast<int>((static_cast<long long>(N) + kTile - 1) / kTile);
  w.n_ttiles = static_cast<int>((M + kSTile - 1) / kSTile);
  const long long mn = window ? N : (M < N ? M : N);  // every id window is a group
  w.max_groups = static_cast<int>((mn + B - 1) / B);
  int bits = 1;
  while (bits < 31 && (1ll << bits) < w.max_groups) ++bits;  // groups are < max_groups
  // One pass of up to 11 bits; beyond that passes of at most 8 bits, which
  // measured faster than fewer wider ones (the per-tile work grows with the
  // digit count: 3 x 7 bits 87 us, 2 x 10 bits 99 us for the B = 1 sort of
  // 524,288 tasks; 1 x 11 bits 56 us, 2 x 8 bits 65 us for B = 256).
  w.passes = bits <= kMaxDigitBits ? 1 : (bits + 7) / 8;
  w.dbits = (bits + w.passes - 1) / w.passes;
  const size_t nt = static_cast<size_t>(w.n_ttiles > 0 ? w.n_ttiles : 1);
  const size_t nd = static_cast<size_t>(1) << w.dbits;
  size_t o = 0;
  w.flags = o;    o = align256(o + static_cast<size_t>(w.n_ftiles) * kTile);
  w.tile_cnt = o; o = align256(o + static_cast<size_t>(w.n_ftiles) * 4);
  w.rank = o;     o = align256(o + static_cast<size_t>(N) * 4);
  w.key0 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.val0 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.key1 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.val1 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.hist = o;     o = align256(o + nd * nt * 4);
  w.dtot = o;     o = align256(o + nd * 4);
  w.bytes = o;
  return w;
}

// Passes that n_groups actually needs: max group id n_groups - 1 < 2^(db eff).
// counts == NULL: a single pass is all the layout has.
__device__ __forceinline__ int effective_passes(const int* counts, int db) {
  if (!counts) return 1;
  const long long n_groups = counts[1];
  int eff = 1;
  long long lim = 1ll << db;
  while (n_groups > lim && eff < 3) {
    ++eff;
    lim <<= db;
  }
  return eff;
}

// Group of a task whose expert is e.  Ids outside [0, N) go to group 0: the
// result is then unspecified but every access stays in bounds.
__device__ __forceinline__ int group_key(int e, const int* __restrict__ rank, int N, int B,
                                         int window) {
  return static_cast<unsigned>(e) < static_cast<unsigned>(N) ? (window ? e : rank[e]) / B : 0;
}

__global__ __launch_bounds__(256) void zero16_kernel(uint4* __restrict__ p, size_t n16) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
}

// Ids outside [0, N) are ignored here and sent to group 0 below.
__global__ __launch_bounds__(256) void mark_kernel(const int32_t* __restrict__ idx, int M, int N,
                                                   uint8_t* __restrict__ flags) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const int e = idx[m];
  if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) flags[e] = 1;
}

// block-wide sum over 256 threads (4 waves); red: 4 ints of LDS
__device__ __forceinline__ int block_sum256(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const int r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}

// popcount of a word whose bytes are each 0 or 1 = number of set flags
__device__ __forceinline__ int flag_count(uint4 v) {
  return __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
}

__global__ __launch_bounds__(256) void tile_count_kernel(const uint8_t* __restrict__ flags,
                                                         int* __restrict__ tile_cnt) {
  __shared__ int red[4];
  const uint4 v =
      reinterpret_cast<const uint4*>(flags + static_cast<size_t>(blockIdx.x) * kTile)[threadIdx.x];
  const int s = block_sum256(flag_count(v), red);
  if (threadIdx.x == 0) tile_cnt[blockIdx.x] = s;
}

// tile_cnt == NULL (few tiles): each block counts the flags of the tiles
// before it itself, in place of tile_count_kernel's per-tile counts.
__global__ __launch_bounds__(256) void rank_kernel(const uint8_t* __restrict__ flags, int N,
                                                   const int* __restrict__ tile_cnt, int n_tiles,
                                                   int B, int window, int* __restrict__ rank,
                                                   int* __restrict__ active,
                                                   int* __restrict__ counts) {
  __shared__ int red[4];
  __shared__ int wpre[4];
  const int b = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = lane();
  // this tile's flags, loaded before the counts of the tiles before it
  const uint4 v = reinterpret_cast<const uint4*>(flags + static_cast<size_t>(b) * kTile)[tid];
  int part = 0;
  if (tile_cnt) {
    for (int i = tid; i < b; i += 256) part += tile_cnt[i];
  } else {
    for (int i = 0; i < b; ++i)
      part += flag_count(
          reinterpret_cast<const uint4*>(flags + static_cast<size_t>(i) * kTile)[tid]);
  }
  const int off = block_sum256(part, red);
  const int c = flag_count(v);
  const int inc = wave_prefix_sum(c);
  if (l == 63) wpre[w] = inc;
  __syncthreads();
  int wbase = 0;
  for (int q = 0; q < w; ++q) wbase += wpre[q];
  int run = off + wbase + inc - c;
  const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if ((words[q >> 2] >> (8 * (q & 3))) & 0xff) {
      const int e = b * kTile + tid * 16 + q;
      rank[e] = run;
      active[run] = e;
      ++run;
    }
  }
  if (b == n_tiles - 1 && tid == 255) {
    counts[0] = run;
    counts[1] = window ? static_cast<int>((static_cast<long long>(N) + B - 1) / B)
                       : (run + B - 1) / B;
  }
}

// Exclusive scan of up to kMaxDigits values that a 512-thread block holds
// four per thread (thread t: digits 4t .. 4t + 3 in v, 0 past the digit
// count).  ex[j] = sum of the digits below digit 4t + j.  red: kSortWaves
// words of LDS.
__device__ __forceinline__ void block_scan_digits(const uint32_t (&v)[4], uint32_t (&ex)[4],
                                                  uint32_t* red) {
  const uint32_t s = v[0] + v[1] + v[2] + v[3];
  const uint32_t inc = wave_inclusive_scan(s);
  const int w = threadIdx.x >> 6;
  if (lane() == 63) red[w] = inc;
  __syncthreads();
  uint32_t run = inc - s;
  for (int q = 0; q < kSortWaves; ++q) run += q < w ? red[q] : 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ex[j] = run;
    run += v[j];
  }
}

// Stable rank of one wave's 64 elements among the elements of the same digit
// (db bits) this wave has ranked so far: lanes with equal digits find each
// other with db ballots, and the lowest of them advances the wave's count of
// that digit (whw: the wave's row of counts in LDS).
__device__ __forceinline__ uint32_t wave_rank_digit(uint32_t d, bool valid, int db,
                                                    uint16_t* whw) {
  const int l = lane();
  const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < kMaxDigitBits; ++bit) {
    if (bit < db) {
      const bool on = (d >> bit) & 1;
      const uint64_t bm = __ballot(valid && on);
      peers &= on ? bm : ~bm;
    }
  }
  const uint64_t below = peers & lt;
  const uint32_t before = whw[d];
  wave_lds_fence();
  if (valid && below == 0) whw[d] = static_cast<uint16_t>(before + __popcll(peers));
  wave_lds_fence();
  return before + static_cast<uint32_t>(__popcll(below));
}

// Per-tile digit histogram, digit-major (hist[digit * n_tt + tile]) or, with
// tmaj, tile-major (hist[tile * nd + digit]: each block writes its row
// whole, which pays with 2048 digits).  The first pass computes the group key
// of each task (kout) on the way.
__global__ __launch_bounds__(512) void radix_up_kernel(
    const int* __restrict__ kin, const int32_t* __restrict__ idx, const int* __restrict__ rank,
    int* __restrict__ kout, int M, int N, int B, int window, int pass, int db, int n_tt,
    int tmaj, const int* __restrict__ counts, int* __restrict__ hist) {
  if (pass >= effective_passes(counts, db)) return;
  __shared__ uint32_t h[kMaxDigits];
  const int nd = 1 << db;
  for (int i = threadIdx.x; i < nd; i += 512) h[i] = 0;
  const int shift = db * pass;
  const int base = blockIdx.x * kSTile;
  int key[kSortR];
  if (pass == 0) {
    int e[kSortR];
#pragma unroll
    for (int r = 0; r < kSortR; ++r) {
      const int i = base + r * 512 + threadIdx.x;
      e[r] = i < M ? idx[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < kSortR; ++r) key[r] = group_key(e[r], rank, N, B, window);
  } else {
#pragma unroll
    for (int r = 0; r < kSortR; ++r) {
      const int i = base + r * 512 + threadIdx.x;
      key[r] = i < M ? kin[i] : 0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortR; ++r) {
    const int i = base + r * 512 + threadIdx.x;
    if (i >= M) continue;
    if (pass == 0) kout[i] = key[r];
    atomicAdd(&h[(static_cast<uint32_t>(key[r]) >> shift) & (nd - 1)], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nd; i += 512)
    hist[tmaj ? static_cast<size_t>(blockIdx.x) * nd + i
              : static_cast<size_t>(i) * n_tt + blockIdx.x] = static_cast<int>(h[i]);
}

// Exclusive scan of each digit's row of tile counts; the row total goes to
// dtot[d].  One wave per digit.
__global__ __launch_bounds__(64) void radix_rowscan_kernel(int* __restrict__ hist, int n_tt,
                                                           int pass, int db,
                                                           const int* __restrict__ counts,
                                                           int* __restrict__ dtot) {
  if (pass >= effective_passes(counts, db)) return;
  int* row = hist + static_cast<size_t>(blockIdx.x) * n_tt;
  const int l = lane();
  uint32_t carry = 0;
  for (int b0 = 0; b0 < n_tt; b0 += 64) {
    const int b = b0 + l;
    const uint32_t v = b < n_tt ? static_cast<uint32_t>(row[b]) : 0u;
    const uint32_t inc = wave_inclusive_scan(v);
    if (b < n_tt) row[b] = static_cast<int>(carry + inc - v);
    carry += static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(inc), 63));
  }
  if (l == 0) dtot[blockIdx.x] = static_cast<int>(carry);
}

// Exclusive scan over the tiles of each digit's counts (a column of the
// tile-major histogram); the column total goes to dtot[d].  A workgroup takes
// 64 digits, one per lane, and its 16 waves a sixteenth of the tiles each:
// every load reads 64 consecutive counts of one tile row.
constexpr int kScanWaves = 16;
__global__ __launch_bounds__(1024) void radix_colscan_kernel(int* __restrict__ hist, int n_tt,
                                                             int pass, int db,
                                                             const int* __restrict__ counts,
                                                             int* __restrict__ dtot) {
  if (pass >= effective_passes(counts, db)) return;
  __shared__ uint32_t wsum[kScanWaves][64];
  const int nd = 1 << db;
  const int w = threadIdx.x >> 6, l = lane();
  const int dg = blockIdx.x * 64 + l;
  const bool ok = dg < nd;
  const int per = (n_tt + kScanWaves - 1) / kScanWaves;
  const int t0 = min(n_tt, w * per), t1 = min(n_tt, t0 + per);
  int* col = hist + (ok ? dg : 0);  // element t of this digit's column: col[t * nd]
  constexpr int U = 8, KEEP = 32;
  uint32_t run = 0;
  if (per <= KEEP) {  // the wave's counts stay in registers between the two steps
    uint32_t c[KEEP];
#pragma unroll
    for (int u = 0; u < KEEP; ++u)
      c[u] = (ok && t0 + u < t1) ? static_cast<uint32_t>(col[static_cast<size_t>(t0 + u) * nd]) : 0u;
    uint32_t s = 0;
#pragma unroll
    for (int u = 0; u < KEEP; ++u) s += c[u];
    wsum[w][l] = s;
    __syncthreads();
    for (int q = 0; q < w; ++q) run += wsum[q][l];
#pragma unroll
    for (int u = 0; u < KEEP; ++u) {
      if (ok && t0 + u < t1) col[static_cast<size_t>(t0 + u) * nd] = static_cast<int>(run);
      run += c[u];
    }
  } else {
    uint32_t s = 0;
    for (int t = t0; t < t1; t += U) {
      uint32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        c[u] = (ok && t + u < t1) ? static_cast<uint32_t>(col[static_cast<size_t>(t + u) * nd]) : 0u;
#pragma unroll
      for (int u = 0; u < U; ++u) s += c[u];
    }
    wsum[w][l] = s;
    __syncthreads();
    for (int q = 0; q < w; ++q) run += wsum[q][l];
    for (int t = t0; t < t1; t += U) {
      uint32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        c[u] = (ok && t + u < t1) ? static_cast<uint32_t>(col[static_cast<size_t>(t + u) * nd]) : 0u;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ok && t + u < t1) col[static_cast<size_t>(t + u) * nd] = static_cast<int>(run);
        run += c[u];
      }
    }
  }
  if (w == kScanWaves - 1 && ok) dtot[dg] = static_cast<int>(run);
}

// Stable scatter of one pass.  Wave w of a tile ranks its 256 consecutive
// elements 64 at a time.  The last effective pass writes the task arrays
// (and the keys only when write_keys: several passes, whose offsets come
// from the sorted keys); a single effective pass also writes the group
// offsets from its digit bases: off[g] = tasks in groups below g for
// g <= G (an empty group gets the start of the next non-empty one, groups
// past the last get M), spread over the blocks.
// fused != 0 (at most kFuseTiles tiles): hist holds the raw tile counts and
// each block sums its digits' counts itself; else hist holds the scanned
// counts and dtot the totals.  tmaj: the histogram's layout (as in
// radix_up_kernel).
__global__ __launch_bounds__(512) void radix_down_kernel(
    const int* __restrict__ kin, const int* __restrict__ vin, int M, int pass, int db, int n_tt,
    int tmaj, const int* __restrict__ hist, const int* __restrict__ dtot, int fused,
    const int* __restrict__ counts, int* __restrict__ kout, int* __restrict__ vout,
    int write_keys, int K, const int32_t* __restrict__ expert_idx,
    const float* __restrict__ gate, int32_t* __restrict__ task_token,
    int32_t* __restrict__ task_expert, float* __restrict__ task_gate,
    int32_t* __restrict__ task_index, int G, int32_t* __restrict__ group_offsets) {
  const int eff = effective_passes(counts, db);
  if (pass >= eff) return;
  const bool last = pass == eff - 1;
  __shared__ __attribute__((aligned(16))) uint16_t wh[kSortWaves][kMaxDigits];
  __shared__ uint32_t goff[kMaxDigits];
  __shared__ uint32_t red[kSortWaves];
  const int tid = threadIdx.x, w = tid >> 6, l = lane();
  const int nd = 1 << db;
  const int b = blockIdx.x;
  // this wave's elements, with their task data on the last pass (m = i on a
  // first pass, so those loads need not wait for vin)
  const int base = b * kSTile + w * (kSortR * 64);
  int kv[kSortR], vv[kSortR], ev[kSortR];
  float gv[kSortR];
#pragma unroll
  for (int r = 0; r < kSortR; ++r) {
    const int i = base + r * 64 + l;
    const bool valid = i < M;
    kv[r] = valid ? kin[i] : 0;
    vv[r] = valid ? (vin ? vin[i] : i) : 0;
  }
  if (last) {
#pragma unroll
    for (int r = 0; r < kSortR; ++r) {
      const bool valid = base + r * 64 + l < M;
      ev[r] = valid ? expert_idx[vv[r]] : 0;
      gv[r] = valid ? gate[vv[r]] : 0.f;
    }
  }
  if (nd >= 8) {  // 16-byte stores: nd / 8 per row of counts
    const int n8 = nd >> 3;
    for (int i = tid; i < kSortWaves * n8; i += 512)
      reinterpret_cast<uint4*>(wh[i / n8])[i % n8] = make_uint4(0u, 0u, 0u, 0u);
  } else {
    for (int i = tid; i < kSortWaves * nd; i += 512) wh[i >> db][i & (nd - 1)] = 0;
  }
  uint32_t v[4], ex[4], before[4];
  if (!fused && nd >= 4 && 4 * tid < nd) {  // four consecutive digits: 16-byte loads
    const int4 t4 = *reinterpret_cast<const int4*>(dtot + 4 * tid);
    v[0] = t4.x; v[1] = t4.y; v[2] = t4.z; v[3] = t4.w;
    if (tmaj) {
      const int4 h4 = *reinterpret_cast<const int4*>(hist + static_cast<size_t>(b) * nd + 4 * tid);
      before[0] = h4.x; before[1] = h4.y; before[2] = h4.z; before[3] = h4.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        before[j] = static_cast<uint32_t>(hist[static_cast<size_t>(4 * tid + j) * n_tt + b]);
    }
  } else if (fused) {
    // every tile's count of this thread's four digits (element t of digit
    // dj's counts is hist[base + t * step]), four tiles' loads in flight
    // before they are summed: a loop that summed each load as it came took
    // one memory latency per tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = 0u;
      before[j] = 0u;
    }
    for (int t0 = 0; t0 < n_tt; t0 += 4) {
      uint32_t c[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dj = 4 * tid + j;
        const size_t base = tmaj ? static_cast<size_t>(dj) : static_cast<size_t>(dj) * n_tt;
        const size_t step = tmaj ? static_cast<size_t>(nd) : 1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = t0 + u;
          c[j][u] = (dj < nd && t < n_tt) ? static_cast<uint32_t>(hist[base + t * step]) : 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[j] += c[j][u];
          before[j] += t0 + u < b ? c[j][u] : 0u;
        }
    }
  } else {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int dj = 4 * tid + j;
    v[j] = 0u;
    before[j] = 0u;
    if (dj < nd) {
      const size_t base = tmaj ? static_cast<size_t>(dj) : static_cast<size_t>(dj) * n_tt;
      const size_t step = tmaj ? static_cast<size_t>(nd) : 1;
      v[j] = static_cast<uint32_t>(dtot[dj]);
      before[j] = static_cast<uint32_t>(hist[base + b * step]);
    }
  }
  }
  block_scan_digits(v, ex, red);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * tid + j < nd) goff[4 * tid + j] = ex[j];
  __syncthreads();
  if (eff == 1) {
    for (long long g = static_cast<long long>(b) * 512 + tid; g <= G;
         g += static_cast<long long>(gridDim.x) * 512)
      group_offsets[g] = g < nd ? static_cast<int>(goff[g]) : M;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * tid + j < nd) goff[4 * tid + j] = ex[j] + before[j];
  __syncthreads();
  const int shift = db * pass;
  uint32_t dg[kSortR], lr[kSortR];
#pragma unroll
  for (int r = 0; r < kSortR; ++r) {
    const bool valid = base + r * 64 + l < M;
    dg[r] = (static_cast<uint32_t>(kv[r]) >> shift) & (nd - 1);
    lr[r] = wave_rank_digit(dg[r], valid, db, wh[w]);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortR; ++r) {
    const int i = base + r * 64 + l;
    if (i >= M) continue;
    // the element's digit in the waves before this one
    uint32_t wb = 0;
    for (int q = 0; q < w; ++q) wb += wh[q][dg[r]];
    const uint32_t pos = goff[dg[r]] + wb + lr[r];
    if (pos >= static_cast<uint32_t>(M)) continue;  // unreachable when counts agree
    if (!last) {
      kout[pos] = kv[r];
      vout[pos] = vv[r];
    } else {
      if (write_keys) kout[pos] = kv[r];
      task_token[pos] = vv[r] / K;
      task_expert[pos] = ev[r];
      task_gate[pos] = gv[r];
      if (task_index) task_index[pos] = vv[r];
    }
  }
}

// CSR offsets: off[g] = first sorted position of group g.  An empty group
// (only id windows can be empty) gets the position of the next non-empty
// one; entries past the last task's group, up to G, hold M.  The sorted keys
// are those of the last effective pass.
__global__ __launch_bounds__(256) void offsets_kernel(const int* __restrict__ skey_even,
                                                      const int* __restrict__ skey_odd, int M,
                                                      int G, int db,
                                                      const int* __restrict__ counts,
                                                      int* __restrict__ off) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int eff = effective_passes(counts, db);
  const int* skey = ((eff - 1) & 1) ? skey_odd : skey_even;
  if (i < M) {
    const int g = min(skey[i], G - 1);
    const int gp = i ? min(skey[i - 1], G - 1) : -1;
    for (int j = gp + 1; j <= g; ++j) off[j] = i;
  }
  if (i <= G && i > min(skey[M - 1], G - 1)) off[i] = M;
}

// No tasks: no active expert; every group (only id windows exist without
// tasks) is empty.
__global__ __launch_bounds__(256) void empty_schedule_kernel(int* counts, int* off, int n_groups,
                                                             int G) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) {
    counts[0] = 0;
    counts[1] = n_groups;
  }
  if (i <= G) off[i] = 0;
}

static inline unsigned blocks_for(long long n, int per) {
  return static_cast<unsigned>((n + per - 1) / per);
}

static void launch_sort(const ScheduleWs& lay, int M, int N, int B, int window, int K,
                        const int32_t* expert_idx, const float* gate, const int* rank,
                        int32_t* counts, int32_t* group_offsets, int32_t* task_token,
                        int32_t* task_expert, float* task_gate, int32_t* task_index, char* base,
                        hipStream_t s) {
  int* key0 = reinterpret_cast<int*>(base + lay.key0);
  int* val0 = reinterpret_cast<int*>(base + lay.val0);
  int* key1 = reinterpret_cast<int*>(base + lay.key1);
  int* val1 = reinterpret_cast<int*>(base + lay.val1);
  int* hist = reinterpret_cast<int*>(base + lay.hist);
  int* dtot = reinterpret_cast<int*>(base + lay.dtot);
  // a single pass needs no device-side pass count
  const int* cnt = lay.passes > 1 ? counts : nullptr;
  const int fused = lay.n_ttiles <= kFuseTiles ? 1 : 0;
  // pass p reads (key, val) from buffer p & 1 and writes buffer (p + 1) & 1;
  // pass 0 reads the group keys it computes itself (key0) and identity values
  int* kb[2] = {key0, key1};
  int* vb[2] = {val0, val1};
  const int write_keys = lay.passes > 1 ? 1 : 0;
  // 2048-digit histograms are kept tile-major (rows written and read whole by
  // the blocks, columns scanned); narrower ones digit-major (measured: large
  // 56.1 -> 52.9 us and mid 52.5 -> 46.4 us tile-major at 11 bits, but the
  // 7-bit passes of the B = 1 sort 83 -> 87 us)
  const int tmaj = lay.dbits >= 10 ? 1 : 0;
  for (int p = 0; p < lay.passes; ++p) {
    int* kin = kb[p & 1];
    const int* vin = p == 0 ? nullptr : vb[p & 1];
    hipLaunchKernelGGL(radix_up_kernel, dim3(lay.n_ttiles), dim3(512), 0, s, kin, expert_idx,
                       rank, key0, M, N, B, window, p, lay.dbits, lay.n_ttiles, tmaj, cnt, hist);
    if (!fused && tmaj)
      hipLaunchKernelGGL(radix_colscan_kernel, dim3(((1u << lay.dbits) + 63) / 64),
                         dim3(64 * kScanWaves), 0, s, hist, lay.n_ttiles, p, lay.dbits, cnt,
                         dtot);
    else if (!fused)
      hipLaunchKernelGGL(radix_rowscan_kernel, dim3(1u << lay.dbits), dim3(64), 0, s, hist,
                         lay.n_ttiles, p, lay.dbits, cnt, dtot);
    hipLaunchKernelGGL(radix_down_kernel, dim3(lay.n_ttiles), dim3(512), 0, s, kin, vin, M, p,
                       lay.dbits, lay.n_ttiles, tmaj, hist, dtot, fused, cnt, kb[(p + 1) & 1],
                       vb[(p + 1) & 1], write_keys, K, expert_idx, gate, task_token, task_expert,
                       task_gate, task_index, lay.max_groups, group_offsets);
  }
  // Several possible passes: the offsets come from the sorted keys (the last
  // effective pass p leaves them in kb[(p + 1) & 1]); a single effective
  // pass has written the same offsets already.
  if (lay.passes > 1) {
    const long long nthr = M > lay.max_groups + 1 ? M : lay.max_groups + 1;
    hipLaunchKernelGGL(offsets_kernel, dim3(blocks_for(nthr, 256)), dim3(256), 0, s, key1, key0,
                       M, lay.max_groups, lay.dbits, cnt, group_offsets);
  }
}

hipError_t launch_schedule(int L, int K, int N, int B, int window, const int32_t* expert_idx,
                           const float* gate, int32_t* counts, int32_t* active,
                           int32_t* group_offsets, int32_t* task_token, int32_t* task_expert,
                           float* task_gate, int32_t* task_index, void* ws, hipStream_t s) {
  const int M = L * K;
  const ScheduleWs lay = schedule_ws_layout(L, K, N, B, window);
  if (M == 0) {
    const int ng = window ? lay.max_groups : 0;
    hipLaunchKernelGGL(empty_schedule_kernel,
                       dim3(blocks_for(static_cast<long long>(lay.max_groups) + 1, 256)),
                       dim3(256), 0, s, counts, group_offsets, ng, lay.max_groups);
    return hipGetLastError();
  }
  char* base = static_cast<char*>(ws);
  uint8_t* flags = reinterpret_cast<uint8_t*>(base + lay.flags);
  int* tile_cnt = reinterpret_cast<int*>(base + lay.tile_cnt);
  int* rank = reinterpret_cast<int*>(base + lay.rank);

  const size_t n16 = static_cast<size_t>(lay.n_ftiles) * kTile / 16;
  hipLaunchKernelGGL(zero16_kernel, dim3(blocks_for(static_cast<long long>(n16), 256)),
                     dim3(256), 0, s, reinterpret_cast<uint4*>(flags), n16);
  hipLaunchKernelGGL(mark_kernel, dim3(blocks_for(M, 256)), dim3(256), 0, s, expert_idx, M, N,
                     flags);
  // few expert tiles: rank_kernel counts the flags before its tile itself
  const bool count_inline = lay.n_ftiles <= kInlineCountTiles;
  if (!count_inline)
    hipLaunchKernelGGL(tile_count_kernel, dim3(lay.n_ftiles), dim3(256), 0, s, flags, tile_cnt);
  hipLaunchKernelGGL(rank_kernel, dim3(lay.n_ftiles), dim3(256), 0, s, flags, N,
                     count_inline ? static_cast<const int*>(nullptr) : tile_cnt, lay.n_ftiles, B,
                     window, rank, active, counts);
  launch_sort(lay, M, N, B, window, K, expert_idx, gate, rank, counts, group_offsets, task_token,
              task_expert, task_gate, task_index, base, s);
  return hipGetLastError();
}

}  // namespace omni
