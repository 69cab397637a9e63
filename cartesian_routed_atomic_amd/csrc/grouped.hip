// Grouped execution of the schedule: the heavily shared experts of every
// token tile on the matrix cores, the rest per task.  Pages: interactive
// explainer "Expert-Centric Scheduling" (tasks are grouped by expert, each
// group's parameters are loaded once and reused by every token assigned to
// it, which turns the memory-bound gather into compute-bound work when tokens
// share experts) and gist.science explainer §2.2 (grouped execution on the
// matrix units).
//
// What is grouped, and why by tile.  The result y_t = sum_k g_tk silu(x_t .
// W[e_tk]) V[e_tk] is a sum over a token's K tasks; walking the schedule group
// by group makes every (group, token) pair add a float32 y row into y, which
// costs more traffic than it saves whenever a token's tasks spread over many
// groups.  So the reuse is organised per token tile instead: the executor
// takes from the schedule the number of tasks of every active expert and
// groups the experts it reuses most, the hot set H (at most kGfHot, in id
// order), into one block of expert rows.  Then
//   gf_cold_kernel runs every token's other (cold) tasks as the token-centric
//     form does, one token per wave, x_t in registers and the cold W then V
//     rows streamed whole, and writes every row of y;
//   gf_tile_kernel, one workgroup per tile of 64 consecutive tokens,
//   1. scatters the gates of the tile's hot tasks into a dense 64 x |H|
//      gate tile in LDS;
//   2. S = x_tile . W_H^T on MFMA (v_mfma_f32_16x16x32_bf16, float32
//      accumulation), the hot rows of W read once per tile;
//   3. C = bf16(G * silu(S)) in LDS (zero where a token has no task on that
//      expert);
//   4. y_tile^T += V_H^T . C^T on MFMA, 64 output columns at a time.
// The hot rows of W and V are thus read once per tile (256 times per call at
// L = 16384) instead of once per task.  The cold rows are read whole, a row
// per wave at a time: read in 64-column slices by the MFMA layout, 16 rows
// per load instruction, they cost 2-3 times as much; and in a kernel of
// their own they run at three waves per SIMD instead of the tile kernel's
// two (its LDS holds one workgroup per CU).
//
// The hot set comes from the schedule: gf_count_kernel walks the sorted tasks
// (contiguous id ranges of active experts) and counts the tasks of every
// expert with LDS counters; the hot set is the experts with at least tau
// tasks, tau = max(2, ceil(L / 64)) doubled until at most kGfHot remain.
// gf_level_kernel finds it in one parallel pass over the counts: for every
// level tau0 * 2^j how many experts reach it and the first kGfHot of them;
// gf_select_kernel (one workgroup) then picks the level and sorts that list
// (each id placed at the count of smaller ids).  gf_pack_kernel gathers the
// hot rows of W into one contiguous block
// (W_H, [kGfHot, d]) and those of V transposed (V_H^T, [d, kGfHot]), so both
// MFMA operands are K-contiguous and the tiles' loads touch a few pages
// instead of one per hot expert.
//
// Precision: hot coefficients are rounded to bf16 for the second product
// (float32 accumulation); cold tasks stay float32 throughout.  Deterministic:
// every sum has a fixed order.
#include <limits.h>

#include "device.hpp"
#include "launch.hpp"
#include "rowfrag.hpp"

namespace omni {

typedef __bf16 gf_bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGfHot = 512;        // hot experts at most
constexpr int kGfHotDiv = 64;      // hot from ceil(L / kGfHotDiv) tasks up (then doubled)
constexpr int kGfCS = kGfHot + 8;  // bf16 row stride of the C tile (16-byte pad)
constexpr int kGfMaxK = 64;        // tasks per token the tile kernel holds
constexpr int kGfCntChunk = 4096;  // sorted tasks per counting workgroup
constexpr int kGfCntLds = 4096;    // expert ids a counting workgroup counts in LDS
constexpr int kGfMisc = 64;        // ints: [1] |H|, [2] tau, [16 + j] level j counts
constexpr int kGfLevels = 16;      // thresholds tau0 * 2^j, j < kGfLevels
constexpr int kGfLvl = 16;         // misc index of the level counts

// --------------------------------------------------------------- workspace

struct GfWsLayout {
  size_t cnt, misc, lvl, hot, vtf, whf, bytes;
};

static size_t gf_align(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static GfWsLayout gf_layout(int L, int K, int d, int N) {
  (void)L;
  (void)K;
  GfWsLayout w;
  w.cnt = 0;  // tasks per expert id, N entries
  w.misc = gf_align(static_cast<size_t>(N) * 4);
  w.lvl = w.misc + gf_align(kGfMisc * 4);  // per level, the first kGfHot experts to reach it
  w.hot = w.lvl + gf_align(static_cast<size_t>(kGfLevels) * kGfHot * 4);
  w.vtf = w.hot + gf_align(kGfHot * 4);
  w.whf = w.vtf + gf_align(static_cast<size_t>(d) * kGfHot * 2);
  w.bytes = w.whf + gf_align(static_cast<size_t>(d) * kGfHot * 2);
  return w;
}

size_t grouped_ws_bytes(int L, int K, int d, int N) { return gf_layout(L, K, d, N).bytes; }

bool grouped_supported(int bf16, int d, int K) {
  return bf16 && K >= 1 && K <= kGfMaxK && d >= 64 && d <= 2048 && (d & (d - 1)) == 0;
}

// --------------------------------------------------------------- counting

__global__ __launch_bounds__(256) void gf_zero_kernel(int4* __restrict__ p, size_t n4) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_int4(0, 0, 0, 0);
}

// First index i in [0, n) with a[i] >= v (n if none); a is a device pointer
// or an LDS array (n must not exceed its size).
template <typename P>
__device__ __forceinline__ int lower_bound_i32(P&& a, int n, int v) {
  int lo = 0;
  while (n > 0) {
    const int h = n >> 1;
    if (a[lo + h] < v) {
      lo += h + 1;
      n -= h + 1;
    } else {
      n = h;
    }
  }
  return lo;
}


struct GfCntLds {
  int32_t cnt[kGfCntLds];
  int32_t mm[2][4];
};

// Tasks per expert id, counted over the schedule's sorted tasks.  A
// workgroup takes kGfCntChunk consecutive sorted tasks; the tasks are grouped
// by contiguous id ranges, so their ids usually span fewer than kGfCntLds ids
// and are counted in LDS first, one global atomic per distinct id (hot
// experts then cost one atomic per workgroup, not one per task).
__global__ __launch_bounds__(256) void gf_count_kernel(const int32_t* __restrict__ texp, int M,
                                                       int N, int32_t* __restrict__ cnt) {
  __shared__ GfCntLds S;
  constexpr int R = kGfCntChunk / 256;  // tasks per thread, held in registers
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kGfCntChunk;
  int ev[R];
  int emin = INT_MAX, emax = INT_MIN;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int m = m0 + r * 256 + tid;
    const int e = m < M ? texp[m] : -1;
    ev[r] = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : -1;
    if (ev[r] >= 0) {
      emin = min(emin, e);
      emax = max(emax, e);
    }
  }
  {
    // wave min / max of order-preserving keys (sign bit flipped), then across waves
    uint32_t wmin = static_cast<uint32_t>(emin) ^ 0x80000000u;
    uint32_t wmax = static_cast<uint32_t>(emax) ^ 0x80000000u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t a = static_cast<uint32_t>(__shfl_xor(static_cast<int>(wmin), o));
      const uint32_t b = static_cast<uint32_t>(__shfl_xor(static_cast<int>(wmax), o));
      wmin = a < wmin ? a : wmin;
      wmax = b > wmax ? b : wmax;
    }
    if (lane() == 0) {
      S.mm[0][tid >> 6] = static_cast<int32_t>(wmin ^ 0x80000000u);
      S.mm[1][tid >> 6] = static_cast<int32_t>(wmax ^ 0x80000000u);
    }
    __syncthreads();
    emin = min(min(S.mm[0][0], S.mm[0][1]), min(S.mm[0][2], S.mm[0][3]));
    emax = max(max(S.mm[1][0], S.mm[1][1]), max(S.mm[1][2], S.mm[1][3]));
    __syncthreads();
  }
  if (emin > emax) return;  // no valid id in the chunk
  const long long span = static_cast<long long>(emax) - emin + 1;
  if (span <= kGfCntLds) {
    const int ns = static_cast<int>(span);
    for (int i = tid; i < ns; i += 256) S.cnt[i] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (ev[r] >= 0) atomicAdd(&S.cnt[ev[r] - emin], 1);
    __syncthreads();
    for (int i = tid; i < ns; i += 256)
      if (S.cnt[i]) atomicAdd(&cnt[emin + i], S.cnt[i]);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (ev[r] >= 0) atomicAdd(&cnt[ev[r]], 1);
  }
}

constexpr int kGfLevelBlocks = 128;  // workgroups of the level pass (each walks N / 128 ids)
constexpr int kGfLevelCap = 4096;    // experts a workgroup may stage: at most L K / tau0 <= 64 K reach tau0

struct GfLevelLds {
  int32_t lc[kGfLevels];      // staged experts at each level
  int32_t lbase[kGfLevels];   // their first position in the level's list
  int32_t lpos[kGfLevels];    // positions handed out so far
  int32_t nq;
  int32_t q[kGfLevelCap];     // staged experts
  int8_t qtop[kGfLevelCap];   // the highest level each reaches
};

// For every level tau0 * 2^j (tau0 = max(2, ceil(L / 64)), j < kGfLevels):
// how many experts have at least that many tasks, and the first kGfHot of
// them in a list.  A workgroup stages the experts of its id stride that reach
// tau0 (no more than L K / tau0 in all), then reserves its range of each
// level's list with one atomic per level.
__global__ __launch_bounds__(256) void gf_level_kernel(const int32_t* __restrict__ cnt, int N,
                                                       int L, int32_t* __restrict__ misc,
                                                       int32_t* __restrict__ lvl) {
  __shared__ GfLevelLds S;
  const int tid = threadIdx.x;
  const long long tau0 = max(2, (L + kGfHotDiv - 1) / kGfHotDiv);
  if (tid < kGfLevels) S.lc[tid] = S.lpos[tid] = 0;
  if (tid == 0) S.nq = 0;
  __syncthreads();
  for (int e = blockIdx.x * 256 + tid; e < N; e += gridDim.x * 256) {
    const long long c = cnt[e];
    if (c < tau0) continue;
    int top = 0;  // the highest level this expert reaches
    while (top + 1 < kGfLevels && c >= (tau0 << (top + 1))) ++top;
    for (int j = 0; j <= top; ++j) atomicAdd(&S.lc[j], 1);
    const int i = atomicAdd(&S.nq, 1);
    if (i < kGfLevelCap) {  // always: the total is bounded as stated above
      S.q[i] = e;
      S.qtop[i] = static_cast<int8_t>(top);
    }
  }
  __syncthreads();
  if (tid < kGfLevels) S.lbase[tid] = S.lc[tid] ? atomicAdd(&misc[kGfLvl + tid], S.lc[tid]) : 0;
  __syncthreads();
  const int nq = min(S.nq, kGfLevelCap);
  for (int i = tid; i < nq; i += 256) {
    const int top = S.qtop[i];
    for (int j = 0; j <= top; ++j) {
      const int pos = S.lbase[j] + atomicAdd(&S.lpos[j], 1);
      if (pos < kGfHot) lvl[j * kGfHot + pos] = S.q[i];
    }
  }
}

// One workgroup, after the level pass: the lowest level that at most kGfHot
// experts reach (the top level, tau0 * 2^15 > L, only with a token listing an
// expert more than once), its list sorted by id: the hot ids, |H| and tau.
__global__ __launch_bounds__(256) void gf_select_kernel(int L, int32_t* __restrict__ misc,
                                                        const int32_t* __restrict__ lvl,
                                                        int32_t* __restrict__ hot_ids) {
  __shared__ int32_t ids[kGfHot];
  __shared__ int32_t pick[2];
  const int tid = threadIdx.x;
  const long long tau0 = max(2, (L + kGfHotDiv - 1) / kGfHotDiv);
  if (tid < 64) {  // the lowest level at most kGfHot experts reach (the last if none)
    const int c = tid < kGfLevels ? misc[kGfLvl + tid] : 0;
    const uint64_t ok = __ballot(tid < kGfLevels && c <= kGfHot);
    const int js = ok ? __builtin_ctzll(ok) : kGfLevels - 1;
    if (tid == js) {
      pick[0] = js;
      pick[1] = min(c, kGfHot);
    }
  }
  __syncthreads();
  const int js = pick[0], H = pick[1];
  for (int i = tid; i < kGfHot; i += 256) ids[i] = i < H ? lvl[js * kGfHot + i] : INT_MAX;
  __syncthreads();
  // ascending by id: each id's position is the number of smaller ids (the ids
  // are distinct; the slots past H hold INT_MAX and count for none)
  for (int i = tid; i < H; i += 256) {
    const int mine = ids[i];
    int r = 0;
    for (int j = 0; j < H; j += 4) {
      const int4 q = *reinterpret_cast<const int4*>(&ids[j]);
      r += (q.x < mine) + (q.y < mine) + (q.z < mine) + (q.w < mine);
    }
    hot_ids[r] = mine;
  }
  if (tid == 0) {
    misc[1] = H;
    misc[2] = static_cast<int>(tau0 << js);
  }
}

// The hot rows in the order the MFMA operands are read, so that every operand
// load of the tile kernel is one contiguous 1 KiB read per wave (64 lanes x
// 16 bytes), lane l = fr + 16 fq holding 8 consecutive K values:
//   whf (first product, B operand): tile ct of 16 hot slots, K step ks of 32
//     columns: element i of lane l is W[hot[16 ct + fr], 32 ks + 8 fq + i],
//     at ((ct * d / 32 + ks) * 64 + l) * 8;
//   vtf (second product, A operand): tile cc of 16 columns, K step kk of 32
//     hot slots: element i of lane l is V[hot[32 kk + 8 fq + i], 16 cc + fr],
//     at ((cc * kGfHot / 32 + kk) * 64 + l) * 8.
// Slots from |H| up to |H| rounded up to 64 hold zeros.  One workgroup per
// 64 columns x 64 slots.
__global__ __launch_bounds__(256) void gf_pack_kernel(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ V, int d,
                                                      const int32_t* __restrict__ misc,
                                                      const int32_t* __restrict__ hot_ids,
                                                      uint16_t* __restrict__ whf,
                                                      uint16_t* __restrict__ vtf) {
  __shared__ uint16_t tile[64][64 + 8];  // V[hot[s0 + r], c0 + c]
  const int H = min(max(misc[1], 0), kGfHot);
  const int Hp = (H + 63) & ~63;
  const int s0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (s0 >= Hp) return;
  const int tid = threadIdx.x, nks = d / 32;
  for (int i = tid; i < 64 * 8; i += 256) {
    const int r = i >> 3, ch = i & 7;
    const int sl = s0 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (sl < H) v = *reinterpret_cast<const uint4*>(V + static_cast<size_t>(hot_ids[sl]) * d +
                                                    c0 + ch * 8);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[r][ch * 8 + 2 * q] = static_cast<uint16_t>(u[q] & 0xffffu);
      tile[r][ch * 8 + 2 * q + 1] = static_cast<uint16_t>(u[q] >> 16);
    }
  }
  // whf: 4 slot tiles x 2 K steps x 64 lanes, straight from W
  for (int i = tid; i < 512; i += 256) {
    const int ctl = i >> 7, ksl = (i >> 6) & 1, l = i & 63;
    const int sl = s0 + 16 * ctl + (l & 15);
    const int k = c0 + 32 * ksl + 8 * (l >> 4);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (sl < H) v = *reinterpret_cast<const uint4*>(W + static_cast<size_t>(hot_ids[sl]) * d + k);
    const size_t o = (static_cast<size_t>(s0 / 16 + ctl) * nks + c0 / 32 + ksl) * 64 + l;
    *reinterpret_cast<uint4*>(whf + o * 8) = v;
  }
  __syncthreads();
  // vtf: 4 column tiles x 2 slot steps x 64 lanes, from the tile
  for (int i = tid; i < 512; i += 256) {
    const int ccl = i >> 7, kkl = (i >> 6) & 1, l = i & 63;
    const int c = 16 * ccl + (l & 15), r0 = 32 * kkl + 8 * (l >> 4);
    uint32_t u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      u[q] = static_cast<uint32_t>(tile[r0 + 2 * q][c]) |
             (static_cast<uint32_t>(tile[r0 + 2 * q + 1][c]) << 16);
    const size_t o =
        (static_cast<size_t>(c0 / 16 + ccl) * (kGfHot / 32) + s0 / 32 + kkl) * 64 + l;
    *reinterpret_cast<uint4*>(vtf + o * 8) = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// --------------------------------------------------------------- the tile kernel

constexpr int kGfXS = 64 + 8;  // bf16 row stride of the staged x chunk (16-byte pad)

template <int TT>
struct GfTileLds {
  int32_t hot[kGfHot];        // the hot expert ids, ascending
  uint16_t xs[2][TT][kGfXS];  // step 2: two x chunks of 64 columns
  union {
    float g[TT][kGfHot];      // steps 1-3: gates of the hot tasks (0 = no task)
    uint16_t c[TT][kGfCS];    // steps 3-4: C tile (bf16 bits)
  } u;
};

// Position of e in the hot list, or -1.
__device__ __forceinline__ int gf_find_hot(const int32_t (&hot)[kGfHot], int H, int e) {
  const int i = lower_bound_i32(hot, H, e);
  return (i < H && hot[i] == e) ? i : -1;
}

__device__ __forceinline__ uint16_t gf_bf16(float v) {  // round to nearest even (finite)
  const uint32_t b = __float_as_uint(v);
  return static_cast<uint16_t>((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}

constexpr int kGfStages = 4;  // register stages of the MFMA operand rings: three K steps in flight
constexpr int kGfXRing = 4;   // x chunks (64 columns) in registers: three in flight

// S = x_tile . W_H^T: this wave's NJ hot column tiles (tile wv + 8 j) over the
// tile's MT row tiles.  The x tile goes through LDS 64 columns at a time
// (every wave of the workgroup takes part, NJ = 0 included): each thread
// loads one 16-byte piece of a chunk kGfXRing - 1 chunks ahead, stores it
// when the chunk is due, and the waves read their A fragments from LDS.  The
// B fragments stream from whf, one contiguous 1 KiB load per tile and K step,
// kGfStages - 1 steps ahead.  NKC = d / 64 is a compile-time constant, so
// every ring index is static.
template <int NKC, int TT, int NJ>
__device__ __forceinline__ void gf_gemm1(const uint16_t* __restrict__ x, int t0, int L,
                                         const uint16_t* __restrict__ whf, int wv, int l,
                                         int tid, uint16_t (&xs)[2][TT][kGfXS],
                                         f32x4 (&acc)[4][4]) {
  constexpr int MT = TT / 16, NKS = 2 * NKC, P = kGfStages;
  constexpr int XR = NKC < kGfXRing ? NKC : kGfXRing;  // divides NKC (both powers of two)
  static_assert(XR == 1 || (2 * XR) % P == 0, "ring slots must repeat every XR chunks");
  constexpr int d = 64 * NKC;
  const int fr = l & 15, fq = l >> 4;
  // x pieces: thread tid takes row tid / 8 (mod TT), 16 bytes at (tid % 8) * 8;
  // with TT < 64 several threads load the same piece and one stores it
  const int xrow = (tid >> 3) % TT, xq = tid & 7;
  const bool xst = tid < TT * 8;
  const uint16_t* xsrc = x + static_cast<size_t>(min(t0 + xrow, L - 1)) * d + xq * 8;
  u32x4 xr[XR];  // a native vector type: an array of uint4 structs stays in scratch
#pragma unroll
  for (int c = 0; c < XR - 1; ++c) xr[c] = *reinterpret_cast<const u32x4*>(xsrc + c * 64);
  gf_bf16x8 b[P][NJ > 0 ? NJ : 1];
  const uint16_t* bp[NJ > 0 ? NJ : 1];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    bp[j] = whf + (static_cast<size_t>(wv + 8 * j) * NKS * 64 + l) * 8;
#pragma unroll
    for (int u = 0; u < P - 1; ++u)
      b[u][j] = *reinterpret_cast<const gf_bf16x8*>(bp[j] + min(u, NKS - 1) * 512);
  }
  // Loads are unconditional (positions past the end re-read the last chunk
  // or step), so the compiler's wait counts follow the rings exactly.
  for (int kc0 = 0; kc0 < NKC; kc0 += XR) {
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      const int kc = kc0 + u;
      // chunk kc + XR - 1 is requested (with XR = 1 that is chunk kc itself),
      // then chunk kc enters LDS (the barrier also ends every read of the
      // buffer it overwrites, chunk kc - 2)
      xr[(u + XR - 1) % XR] =
          *reinterpret_cast<const u32x4*>(xsrc + min(kc + XR - 1, NKC - 1) * 64);
      if (xst) *reinterpret_cast<u32x4*>(&xs[u & 1][xrow][xq * 8]) = xr[u];
      __syncthreads();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ks = 2 * kc + h, slot = (2 * u + h) % P;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          b[(slot + P - 1) % P][j] =
              *reinterpret_cast<const gf_bf16x8*>(bp[j] + min(ks + P - 1, NKS - 1) * 512);
        if constexpr (NJ > 0) {
          gf_bf16x8 a[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            a[mt] = *reinterpret_cast<const gf_bf16x8*>(&xs[u & 1][mt * 16 + fr][h * 32 + 8 * fq]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[slot][j],
                                                                   acc[mt][j], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();  // the last chunk's reads before LDS is reused
}

// y_tile^T (64 columns) = V_H^T . C^T over the hot slots [0, Hp): the A
// fragments stream from vtf (one contiguous 1 KiB load per column tile and K
// step) kGfStages - 1 steps ahead; the main loop takes whole groups of
// kGfStages steps with no condition in it (loads past the end re-read the
// last step), so the compiler's wait counts follow the ring exactly; C (the B
// operand) from LDS.
template <int TT>
__device__ __forceinline__ void gf_gemm2_step(const gf_bf16x8 (&av)[4],
                                              const uint16_t (&c)[TT][kGfCS], int kk, int fr,
                                              int fq, f32x4 (&a2)[4][4]) {
  constexpr int MT = TT / 16;
  gf_bf16x8 bv[MT];
#pragma unroll
  for (int nt = 0; nt < MT; ++nt)
    bv[nt] = *reinterpret_cast<const gf_bf16x8*>(&c[nt * 16 + fr][kk * 32 + 8 * fq]);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < MT; ++nt)
      a2[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv[nt], a2[mt][nt], 0, 0, 0);
}

template <int TT>
__device__ __forceinline__ void gf_gemm2(const uint16_t* const (&vrow)[4],
                                         const uint16_t (&c)[TT][kGfCS], int Hp, int fr, int fq,
                                         f32x4 (&a2)[4][4]) {
  constexpr int P = kGfStages;
  gf_bf16x8 av[P][4];
  const int nk = Hp / 32, last = nk - 1;
#pragma unroll
  for (int u = 0; u < P - 1; ++u)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      av[u][mt] = *reinterpret_cast<const gf_bf16x8*>(vrow[mt] + min(u, last) * 512);
  int k0 = 0;
  for (; k0 + P <= nk; k0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        av[(u + P - 1) % P][mt] =
            *reinterpret_cast<const gf_bf16x8*>(vrow[mt] + min(k0 + u + P - 1, last) * 512);
      __builtin_amdgcn_sched_barrier(0);
      gf_gemm2_step<TT>(av[u], c, k0 + u, fr, fq, a2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < P - 1; ++u)
    if (u < nk - k0) gf_gemm2_step<TT>(av[u], c, k0 + u, fr, fq, a2);
}

constexpr int kGfRing = 4;  // row slots per wave of the cold kernel: three in flight (153 VGPRs, 3 waves / SIMD)

// The cold tasks (experts outside the hot set), one token per wave as the
// token-centric form runs its tasks: the token's cold tasks gathered into
// lanes 0 .. nc - 1 in k order, x_t in registers, the cold W rows then the
// cold V rows streamed whole through the ring, y_t written (added to y_t with
// accumulate; zero where the token has no cold task).  Every token's row is
// written here, so the tile kernel adds the hot product to all of them.
// NT: the rows carry the nontemporal hint (stream_rows).
template <int EPL, bool NT>
__global__ __launch_bounds__(256, 3) void gf_cold_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ fe,
    const float* __restrict__ fg, int L, int K, int d, int N, const int32_t* __restrict__ misc,
    const int32_t* __restrict__ hot_ids, float* __restrict__ y, int accumulate) {
  __shared__ int32_t hot[kGfHot];
  __shared__ int32_t ce[4][kGfMaxK];
  __shared__ float cg[4][kGfMaxK];
  const int tid = threadIdx.x, wv = tid >> 6, l = lane();
  const int H = min(max(misc[1], 0), kGfHot);
  for (int i = tid; i < H; i += 256) hot[i] = hot_ids[i];
  __syncthreads();
  const int tok = blockIdx.x * 4 + wv;
  if (tok >= L) return;
  int my_e = 0;
  float my_g = 0.f;
  bool cold = false;
  if (l < K) {
    const size_t m = static_cast<size_t>(tok) * K + l;
    const int e = fe[m];
    my_e = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? e : 0;
    my_g = fg[m];
    cold = H == 0 || gf_find_hot(hot, H, e) < 0;
  }
  const uint64_t cm = __ballot(cold);
  const int nc = __popcll(cm);
  float* yrow = y + static_cast<size_t>(tok) * d;
  if (nc == 0) {  // uniform over the wave: a zero row, or y0 as it stands
    if (!accumulate) {
      float z[EPL];
#pragma unroll
      for (int q = 0; q < EPL; ++q) z[q] = 0.f;
      store_row<uint16_t, EPL, kStorePlain>(z, yrow, 0);
    }
    return;
  }
  if (cold) {  // the cold tasks into lanes 0 .. nc - 1, in k order
    const int j = mbcnt(cm);
    ce[wv][j] = my_e;
    cg[wv][j] = my_g;
  }
  wave_lds_fence();
  my_e = l < nc ? ce[wv][l] : 0;
  my_g = l < nc ? cg[wv][l] : 0.f;
  RowFrag<uint16_t, EPL> xf;
  xf.template fetch<NT>(x + static_cast<size_t>(tok) * d, l);
  RowFrag<uint16_t, EPL> f[kGfRing];
  const float h = token_dots<uint16_t, EPL, NT, kGfRing, false>(xf, W, my_e, nc, d, l, f);
  const float my_c = my_g * (h / (1.f + __expf(-h)));
  float acc[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
  token_gather<uint16_t, EPL, NT, kGfRing, false>(V, my_e, my_c, nc, d, l, f, acc);
  store_row<uint16_t, EPL, kStorePlain>(acc, yrow, accumulate);
}

// A tile of TT = 16, 32 or 64 tokens per workgroup of 8 waves.
template <int EPL, int TT>
__global__ __launch_bounds__(512) void gf_tile_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ fe,
    const float* __restrict__ fg, int L, int K, int d, const int32_t* __restrict__ misc,
    const int32_t* __restrict__ hot_ids, const uint16_t* __restrict__ whf,
    const uint16_t* __restrict__ vtf, float* __restrict__ y) {
  constexpr int MT = TT / 16;
  __shared__ __attribute__((aligned(16))) GfTileLds<TT> S;
  const int tid = threadIdx.x, wv = tid >> 6, l = lane();
  const int t0 = blockIdx.x * TT;
  const int H = min(max(misc[1], 0), kGfHot);
  if (H == 0) return;  // nothing hot: gf_cold_kernel has written y (uniform over the grid)
  const int Hp = (H + 63) & ~63;
  const int fr = l & 15, fq = l >> 4;

  // ---- 1. hot ids and the gate tile of the hot tasks (each thread loads all
  // of its tasks first, then places them)
  constexpr int RB = TT * kGfMaxK / 512;  // tasks per thread at most
  const int ntask = min(TT, L - t0) * K;
  int tv[RB];
  float gv[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int i = tid + 512 * r;
    tv[r] = i < ntask ? fe[static_cast<size_t>(t0) * K + i] : -1;
    gv[r] = i < ntask ? fg[static_cast<size_t>(t0) * K + i] : 0.f;
  }
  for (int i = tid; i < H; i += 512) S.hot[i] = hot_ids[i];
  {
    float4* g4 = reinterpret_cast<float4*>(&S.u.g[0][0]);
    for (int i = tid; i < TT * kGfHot / 4; i += 512) g4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (tv[r] >= 0) {
      const int s = gf_find_hot(S.hot, H, tv[r]);
      // a token listing one expert twice gets the sum of its gates
      if (s >= 0) atomicAdd(&S.u.g[(tid + 512 * r) / K][s], gv[r]);
    }
  }
  __syncthreads();

  // ---- 2. S = x_tile . W_H^T and 3. C = bf16(G * silu(S))
  const int ntiles = Hp / 16;
  const int nj = max(0, min(4, (ntiles - wv + 7) / 8));
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  {  // every wave stages its share of x, nj = 0 included
    switch (nj) {
      case 0: gf_gemm1<EPL, TT, 0>(x, t0, L, whf, wv, l, tid, S.xs, acc); break;
      case 1: gf_gemm1<EPL, TT, 1>(x, t0, L, whf, wv, l, tid, S.xs, acc); break;
      case 2: gf_gemm1<EPL, TT, 2>(x, t0, L, whf, wv, l, tid, S.xs, acc); break;
      case 3: gf_gemm1<EPL, TT, 3>(x, t0, L, whf, wv, l, tid, S.xs, acc); break;
      default: gf_gemm1<EPL, TT, 4>(x, t0, L, whf, wv, l, tid, S.xs, acc); break;
    }
  }
  // accumulator layout: row (token) 4 * fq + q of M-tile mt, column (hot slot) fr of tile j
  float cv[MT][4][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cv[mt][j][q] = 0.f;
        if (j < nj) {
          const float g = S.u.g[mt * 16 + 4 * fq + q][(wv + 8 * j) * 16 + fr];
          const float h = acc[mt][j][q];
          cv[mt][j][q] = g * (h / (1.f + __expf(-h)));
        }
      }
  __syncthreads();  // every gate read before the C tile overwrites them
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nj)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          S.u.c[mt * 16 + 4 * fq + q][(wv + 8 * j) * 16 + fr] = gf_bf16(cv[mt][j][q]);

  __syncthreads();  // the C tile complete before the second product reads it

  // ---- 4. y_tile^T = V_H^T . C^T, 64 output columns per pass, added to y
  const int ncb = d / 64;
  for (int b = wv; b < ncb; b += 8) {
    const int c0 = b * 64;
    f32x4 a2[4][4];  // [mt: 16 columns][nt: 16 tokens]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) a2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* vrow[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      vrow[mt] = vtf + (static_cast<size_t>(c0 / 16 + mt) * (kGfHot / 32) * 64 + l) * 8;
    // accumulator layout: column c0 + mt * 16 + 4 * fq + q, token nt * 16 + fr;
    // the rows gf_cold_kernel wrote already hold y0 (with accumulate) plus the
    // token's cold tasks.  Their old values are loaded before the product, so
    // the loads run under it (rows past L re-read the tile's first row).
    float4 yo[MT][4];
#pragma unroll
    for (int nt = 0; nt < MT; ++nt) {
      const int tok = min(t0 + nt * 16 + fr, L - 1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        yo[nt][mt] = *reinterpret_cast<const float4*>(y + static_cast<size_t>(tok) * d + c0 +
                                                      mt * 16 + 4 * fq);
    }
    gf_gemm2<TT>(vrow, S.u.c, Hp, fr, fq, a2);
#pragma unroll
    for (int nt = 0; nt < MT; ++nt) {
      const int tok = t0 + nt * 16 + fr;
      if (tok >= L) continue;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float* p = y + static_cast<size_t>(tok) * d + c0 + mt * 16 + 4 * fq;
        const float4 o = yo[nt][mt];
        const float4 v = make_float4(a2[mt][nt][0] + o.x, a2[mt][nt][1] + o.y,
                                     a2[mt][nt][2] + o.z, a2[mt][nt][3] + o.w);
        *reinterpret_cast<float4*>(p) = v;
      }
    }
  }
}

// --------------------------------------------------------------- launch

hipError_t launch_grouped(const uint16_t* x, const uint16_t* w, const uint16_t* v,
                          const int32_t* task_expert, const int32_t* fe, const float* fg, int L,
                          int K, int d, int N, float* y, int accumulate, void* gws,
                          hipStream_t s) {
  if (!grouped_supported(1, d, K)) return hipErrorInvalidValue;
  const int M = L * K;
  const GfWsLayout ly = gf_layout(L, K, d, N);
  char* base = static_cast<char*>(gws);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + ly.cnt);
  int32_t* misc = reinterpret_cast<int32_t*>(base + ly.misc);
  int32_t* lvl = reinterpret_cast<int32_t*>(base + ly.lvl);
  int32_t* hot = reinterpret_cast<int32_t*>(base + ly.hot);
  uint16_t* vtf = reinterpret_cast<uint16_t*>(base + ly.vtf);
  uint16_t* whf = reinterpret_cast<uint16_t*>(base + ly.whf);
  // counters and the misc block (|H|, tau, level counts) start at zero
  const size_t n4 = ly.lvl / 16;
  hipLaunchKernelGGL(gf_zero_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0,
                     s, reinterpret_cast<int4*>(base), n4);
  hipLaunchKernelGGL(gf_count_kernel, dim3(static_cast<unsigned>((M + kGfCntChunk - 1) / kGfCntChunk)),
                     dim3(256), 0, s, task_expert, M, N, cnt);
  hipLaunchKernelGGL(gf_level_kernel, dim3(static_cast<unsigned>(min((N + 255) / 256, kGfLevelBlocks))),
                     dim3(256), 0, s, cnt, N, L, misc, lvl);
  hipLaunchKernelGGL(gf_select_kernel, dim3(1), dim3(256), 0, s, L, misc, lvl, hot);
  hipLaunchKernelGGL(gf_pack_kernel, dim3(static_cast<unsigned>(d / 64), kGfHot / 64),
                     dim3(256), 0, s, w, v, d, misc, hot, whf, vtf);
  // the cold tasks of every token first (they write every row of y), then the
  // hot product of every tile added onto those rows
  const bool nt = stream_rows(M, N);
  const dim3 cgrid(static_cast<unsigned>((L + 3) / 4));
  // tokens per tile: 64 where that still gives a tile per CU (the hot rows are
  // read once per tile), fewer for smaller batches
  const int tt = L >= 256 * 64 ? 64 : (L >= 256 * 32 ? 32 : 16);
  const dim3 grid(static_cast<unsigned>((L + tt - 1) / tt));
#define OMNI_GF_TT(EPL_, TT_)                                                                   \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(gf_tile_kernel<EPL_, TT_>), grid, dim3(512), 0, s, x, fe,   \
                     fg, L, K, d, misc, hot, whf, vtf, y)
#define OMNI_GF(EPL_)                                                                           \
  if (nt)                                                                                       \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(gf_cold_kernel<EPL_, true>), cgrid, dim3(256), 0, s, x, w,  \
                       v, fe, fg, L, K, d, N, misc, hot, y, accumulate);                         \
  else                                                                                          \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(gf_cold_kernel<EPL_, false>), cgrid, dim3(256), 0, s, x, w, \
                       v, fe, fg, L, K, d, N, misc, hot, y, accumulate);                         \
  if (tt == 64) OMNI_GF_TT(EPL_, 64);                                                           \
  else if (tt == 32) OMNI_GF_TT(EPL_, 32);                                                      \
  else OMNI_GF_TT(EPL_, 16)
  switch (d) {
    case 64: OMNI_GF(1); break;
    case 128: OMNI_GF(2); break;
    case 256: OMNI_GF(4); break;
    case 512: OMNI_GF(8); break;
    case 1024: OMNI_GF(16); break;
    case 2048: OMNI_GF(32); break;
    default: return hipErrorInvalidValue;
  }
#undef OMNI_GF_TT
#undef OMNI_GF
  return hipGetLastError();
}

}  // namespace omni
