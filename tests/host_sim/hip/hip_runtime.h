// Host model of gfx950 wavefronts, for CPU tests of the kernels' index
// arithmetic.  Test infrastructure only: nothing of the library links it.
//
// A kernel source written for gfx950 is compiled for the x86 host against this
// header in place of the HIP runtime header.  A launch runs its workgroups one
// after another; inside a workgroup every work-item is a fiber (ucontext) on
// one OS thread, switched at every cross-lane operation and barrier.  The 64
// work-items of a wave meet at every cross-lane operation (ballot, shuffle,
// readlane, DPP, wave barrier): the operation is evaluated from the values of
// all live lanes at once, as the hardware evaluates it in lockstep, and every
// lane then continues with its own result.  __syncthreads() is a barrier over
// the workgroup's live work-items.  LDS (`__shared__`) is filled with a chosen
// byte before each workgroup, so a result that depends on LDS no lane wrote
// changes with that byte.
//
// Built with the address and array-bounds sanitizers, an index out of range
// of an LDS array (fixed-size arrays, also when passed by reference) or of a
// global buffer (exact-size host allocations) stops the run and names the
// source line.
//
// Limits of the model (it stops with a message rather than guess):
//   * cross-lane operations must sit in wave-uniform control flow; a wave
//     whose lanes wait at different cross-lane operations times out;
//   * DPP controls other than row_shr:1..15, row_bcast:15 and row_bcast:31
//     are not modelled;
//   * reading another lane's value from a lane that has returned is an error.
// Transcendental functions are the host's; sim::g_log_ulps shifts every
// __logf result by that many float32 ulps, to cover the hardware
// approximation's last-bit differences.
#pragma once
#if defined(__has_feature)
#if __has_feature(address_sanitizer)
#define OMNI_SIM_ASAN 1
#include <sanitizer/common_interface_defs.h>
#endif
#endif
#ifndef OMNI_SIM_ASAN
#define OMNI_SIM_ASAN 0
#endif
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <csetjmp>
#include <functional>
#include <memory>
#include <ucontext.h>
#include <type_traits>
#include <vector>

struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef struct sim_stream* hipStream_t;
inline hipError_t hipGetLastError() { return hipSuccess; }

struct alignas(16) ulonglong2 { unsigned long long x, y; };
struct alignas(16) float4 { float x, y, z, w; };
struct alignas(16) int4 { int x, y, z, w; };
struct alignas(16) uint4 { unsigned x, y, z, w; };
struct alignas(8) uint2 { unsigned x, y; };
inline float4 make_float4(float a, float b, float c, float d) { return float4{a, b, c, d}; }
inline int4 make_int4(int a, int b, int c, int d) { return int4{a, b, c, d}; }
inline uint4 make_uint4(unsigned a, unsigned b, unsigned c, unsigned d) { return uint4{a, b, c, d}; }
// Buffer resources exist for the parser only; the model stops if a kernel uses one.
typedef struct { void* p; } __amdgpu_buffer_rsrc_t;

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static __attribute__((section("omni_sim_lds")))
#define HIP_KERNEL_NAME(...) __VA_ARGS__

namespace sim {

[[noreturn]] inline void fail(const char* what) {
  std::fprintf(stderr, "wave model: %s\n", what);
  std::fflush(stderr);
  std::abort();
}

inline int g_log_ulps = 0;            // __logf results shifted by this many ulps
inline unsigned char g_lds_fill = 0;  // byte written over LDS before each workgroup
inline long long g_collectives = 0;   // cross-lane operations evaluated (statistics)

// Work-items run as fibers on one OS thread, switched at every cross-lane
// operation or barrier; the scheduler resumes them round robin.
enum LaneState { kRun = 0, kWait = 1, kDone = 2 };

struct Group {  // the live lanes of one wave, or the live threads of one workgroup
  int live = 0, arrived = 0;
  unsigned long long gen = 0;
  uint64_t val[64] = {}, snap[64] = {};
  bool present[64] = {}, snap_present[64] = {};
  std::vector<int> waiting;  // fibers parked until this group's operation completes
};

struct Fiber {
  ucontext_t ctx;    // first entry only
  jmp_buf jb;        // later switches (no signal-mask system call)
  char* stack = nullptr;
  bool started = false;
  int state = kRun;
  int lane = 0, wave = 0;
  dim3 tid;
};

struct Launch {
  std::vector<Fiber> fibers;
  std::vector<Group> waves;
  Group block;
  std::function<void()> body;
  ucontext_t sched;
  jmp_buf sched_jb;
  int cur = -1;
  const void* sched_stack_bottom = nullptr;
  size_t sched_stack_size = 0;
};
inline Launch* g_launch = nullptr;

inline int t_lane_get() { return g_launch->fibers[g_launch->cur].lane; }
#define OMNI_SIM_LANE (sim::t_lane_get())

inline void to_scheduler() {
  Launch& L = *g_launch;
  Fiber& me = L.fibers[L.cur];
#if OMNI_SIM_ASAN
  void* fs = nullptr;
  __sanitizer_start_switch_fiber(&fs, L.sched_stack_bottom, L.sched_stack_size);
#endif
  if (_setjmp(me.jb) == 0) _longjmp(L.sched_jb, 1);
#if OMNI_SIM_ASAN
  __sanitizer_finish_switch_fiber(fs, nullptr, nullptr);
#endif
}

inline void complete(Group& g) {  // every live member has arrived
  std::memcpy(g.snap, g.val, sizeof g.val);
  std::memcpy(g.snap_present, g.present, sizeof g.present);
  std::memset(g.present, 0, sizeof g.present);
  g.arrived = 0;
  ++g.gen;
  ++g_collectives;
  for (int f : g.waiting) g_launch->fibers[f].state = kRun;
  g.waiting.clear();
}

// Arrive at the group's current operation with payload v (slot `slot`) and
// park until every live member has arrived.
inline void arrive(Group& g, int slot, uint64_t v) {
  Launch& L = *g_launch;
  g.val[slot] = v;
  g.present[slot] = true;
  L.fibers[L.cur].state = kWait;
  g.waiting.push_back(L.cur);
  if (++g.arrived == g.live) complete(g);
  to_scheduler();
}

// Every live lane deposits v; returns with all lanes' values.
inline void exchange(uint64_t v, uint64_t (&all)[64], bool (&pres)[64]) {
  Launch& L = *g_launch;
  Fiber& me = L.fibers[L.cur];
  Group& g = L.waves[me.wave];
  arrive(g, me.lane, v);
  std::memcpy(all, g.snap, sizeof all);
  std::memcpy(pres, g.snap_present, sizeof pres);
}

inline void block_barrier() {
  Launch& L = *g_launch;
  arrive(L.block, 0, 0);
}

inline void leave(Group& g) {
  --g.live;
  if (g.live > 0 && g.arrived == g.live) complete(g);
}

template <class T> inline uint64_t to_bits(T v) {
  static_assert(sizeof(T) <= 8 && std::is_trivially_copyable<T>::value, "payload");
  uint64_t u = 0;
  std::memcpy(&u, &v, sizeof(T));
  return u;
}
template <class T> inline T from_bits(uint64_t u) {
  T v;
  std::memcpy(&v, &u, sizeof(T));
  return v;
}

template <class T> inline T lane_value(T v, int src) {
  uint64_t all[64];
  bool pres[64];
  exchange(to_bits(v), all, pres);
  if (src < 0 || src > 63) fail("lane index out of range");
  if (!pres[src]) fail("value read from a lane that is not active");
  return from_bits<T>(all[src]);
}

inline unsigned long long ballot(bool p) {
  uint64_t all[64];
  bool pres[64];
  exchange(p ? 1u : 0u, all, pres);
  unsigned long long m = 0;
  for (int i = 0; i < 64; ++i)
    if (pres[i] && all[i]) m |= 1ull << i;
  return m;
}

inline int update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl) {
  uint64_t all[64];
  bool pres[64];
  exchange(static_cast<uint32_t>(src), all, pres);
  const int l = OMNI_SIM_LANE, row = l >> 4, bank = (l & 15) >> 2;
  if (!((row_mask >> row) & 1) || !((bank_mask >> bank) & 1)) return old;
  int sl = -1;
  if (ctrl >= 0x111 && ctrl <= 0x11f) {  // row_shr:n
    const int n = ctrl - 0x110;
    if ((l & 15) >= n) sl = l - n;
  } else if (ctrl == 0x142) {  // row_bcast:15: lane 15 of the row below
    if (row >= 1) sl = row * 16 - 1;
  } else if (ctrl == 0x143) {  // row_bcast:31: lane 31 into rows 2 and 3
    if (row >= 2) sl = 31;
  } else {
    fail("DPP control not modelled");
  }
  if (sl < 0 || !pres[sl]) return bound_ctrl ? 0 : old;
  return static_cast<int>(static_cast<uint32_t>(all[sl]));
}

// Evaluate an operation whose per-lane payload is `bytes` long: every live
// lane deposits its bytes, and gets all lanes' payloads back.
template <int BYTES>
inline void exchange_bytes(const void* mine, unsigned char (&all)[64][BYTES], bool (&pres)[64]) {
  static_assert(BYTES % 8 == 0, "payload of whole 8-byte words");
  for (int w = 0; w < BYTES / 8; ++w) {
    uint64_t v, got[64];
    std::memcpy(&v, static_cast<const unsigned char*>(mine) + 8 * w, 8);
    exchange(v, got, pres);
    for (int i = 0; i < 64; ++i) std::memcpy(&all[i][8 * w], &got[i], 8);
  }
}

// v_mfma_f32_16x16x32_bf16: D = A B + C for a 16 x 16 x 32 block.  Lane l holds
// A[m = l % 16][k = 8 (l / 16) + i] and B[k = 8 (l / 16) + i][n = l % 16], i =
// 0..7, and C, D[m = 4 (l / 16) + q][n = l % 16], q = 0..3.  Products summed
// in float64 (the order of the hardware's float32 sums is not modelled).
template <class VB, class VF>
inline VF mfma_16x16x32_bf16(VB a, VB b, VF c) {
  struct P { VB a, b; VF c; } mine{a, b, c};
  static_assert(sizeof(P) == 48, "payload layout");
  unsigned char all[64][48];
  bool pres[64];
  exchange_bytes<48>(&mine, all, pres);
  for (int i = 0; i < 64; ++i)
    if (!pres[i]) fail("MFMA with inactive lanes");
  const int l = OMNI_SIM_LANE;
  VF d;
  for (int q = 0; q < 4; ++q) {
    const int m = 4 * (l / 16) + q, n = l % 16;
    double acc = 0.0;
    for (int kg = 0; kg < 4; ++kg) {
      P pa, pb;
      std::memcpy(&pa, all[kg * 16 + m], 48);
      std::memcpy(&pb, all[kg * 16 + n], 48);
      for (int i = 0; i < 8; ++i) acc += static_cast<double>(static_cast<float>(pa.a[i])) *
                                          static_cast<double>(static_cast<float>(pb.b[i]));
    }
    P pc;
    std::memcpy(&pc, all[l], 48);
    d[q] = static_cast<float>(acc + static_cast<double>(pc.c[q]));
  }
  return d;
}

inline uint64_t bits_below(int l) { return l >= 64 ? ~0ull : ((1ull << l) - 1ull); }

extern "C" char __start_omni_sim_lds[] __attribute__((weak));
extern "C" char __stop_omni_sim_lds[] __attribute__((weak));

__attribute__((no_sanitize("address"))) inline void fill_lds(unsigned char b) {
  if (!__start_omni_sim_lds || !__stop_omni_sim_lds) return;
  volatile char* p = __start_omni_sim_lds;
  for (; p < __stop_omni_sim_lds; ++p) *p = static_cast<char>(b);
}

}  // namespace sim

inline dim3 blockIdx, blockDim, gridDim;
#define threadIdx (sim::g_launch->fibers[sim::g_launch->cur].tid)

// ---- the device builtins the kernels use, on the model
#define __lane_id() (static_cast<unsigned>(OMNI_SIM_LANE))
#define __ballot(p) sim::ballot(static_cast<bool>(p))
#define __builtin_amdgcn_readlane(v, i) sim::lane_value<int>((v), (i))
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) \
  sim::update_dpp((old), (src), (ctrl), (rm), (bm), (bc))
#define __builtin_amdgcn_wave_barrier() sim::ballot(false)
#define __builtin_amdgcn_fence(...) std::atomic_thread_fence(std::memory_order_seq_cst)
// mbcnt: set bits of the mask in the lanes below this one (lo: lanes 0-31,
// hi: lanes 32-63), plus acc.
inline unsigned sim_mbcnt_lo(unsigned m, unsigned acc) {
  const int l = OMNI_SIM_LANE;
  return acc + static_cast<unsigned>(__builtin_popcountll(m & sim::bits_below(l < 32 ? l : 32)));
}
inline unsigned sim_mbcnt_hi(unsigned m, unsigned acc) {
  const int l = OMNI_SIM_LANE;
  return acc + (l < 32 ? 0u : static_cast<unsigned>(__builtin_popcountll(m & sim::bits_below(l - 32))));
}
#define __builtin_amdgcn_mbcnt_lo(m, acc) sim_mbcnt_lo(static_cast<unsigned>(m), static_cast<unsigned>(acc))
#define __builtin_amdgcn_mbcnt_hi(m, acc) sim_mbcnt_hi(static_cast<unsigned>(m), static_cast<unsigned>(acc))

inline void __syncthreads() { sim::block_barrier(); }
inline void __threadfence() { std::atomic_thread_fence(std::memory_order_seq_cst); }
#define __builtin_amdgcn_sched_barrier(m) ((void)0)
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x0, x1, x2) sim::mfma_16x16x32_bf16((a), (b), (c))
#define __builtin_amdgcn_fdot2_f32_bf16(a, b, c, clamp)                                  \
  ((c) + static_cast<float>((a)[0]) * static_cast<float>((b)[0]) +                      \
   static_cast<float>((a)[1]) * static_cast<float>((b)[1]))
#define __builtin_amdgcn_make_buffer_rsrc(...) (sim::fail("buffer resources are not modelled"), __amdgpu_buffer_rsrc_t{})
#define __builtin_amdgcn_raw_buffer_store_b128(...) sim::fail("buffer stores are not modelled")
#define __HIP_MEMORY_SCOPE_AGENT 3
#define __hip_atomic_load(p, order, scope) __atomic_load_n((p), __ATOMIC_RELAXED)
template <class T> inline T atomicAdd(T* p, T v) { T o = *p; *p = o + v; return o; }
template <class T> inline T atomicOr(T* p, T v) { T o = *p; *p = o | v; return o; }

template <class T> inline T __shfl(T v, int src, int width = 64) {
  const int base = OMNI_SIM_LANE & ~(width - 1);
  return sim::lane_value<T>(v, base + ((src % width) + width) % width);
}
template <class T> inline T __shfl_xor(T v, int mask, int width = 64) {
  const int base = OMNI_SIM_LANE & ~(width - 1);
  return sim::lane_value<T>(v, base + (((OMNI_SIM_LANE - base) ^ mask) & (width - 1)));
}

inline int __popcll(unsigned long long v) { return __builtin_popcountll(v); }
inline int __popc(unsigned v) { return __builtin_popcount(v); }
inline int __clz(int v) { return v ? __builtin_clz(static_cast<unsigned>(v)) : 32; }
inline int __clzll(long long v) {
  return v ? __builtin_clzll(static_cast<unsigned long long>(v)) : 64;
}
inline unsigned __float_as_uint(float f) { return __builtin_bit_cast(unsigned, f); }
inline float __uint_as_float(unsigned u) { return __builtin_bit_cast(float, u); }
inline int __float_as_int(float f) { return __builtin_bit_cast(int, f); }
inline float __int_as_float(int u) { return __builtin_bit_cast(float, u); }
inline float __expf(float x) { return std::exp(x); }
inline float __logf(float x) {
  float r = std::log(x);
  for (int i = 0; i < sim::g_log_ulps; ++i) r = std::nextafter(r, INFINITY);
  for (int i = 0; i > sim::g_log_ulps; --i) r = std::nextafter(r, -INFINITY);
  return r;
}
#include <math.h>




template <class A, class B> inline std::common_type_t<A, B> min(A a, B b) {
  return a < b ? a : b;
}
template <class A, class B> inline std::common_type_t<A, B> max(A a, B b) {
  return a < b ? b : a;
}

namespace sim {

constexpr size_t kFiberStack = 256 << 10;

// Fiber stacks, allocated once and reused by every workgroup.
inline char* fiber_stack(unsigned i) {
  static std::vector<std::unique_ptr<char[]>> pool;
  while (pool.size() <= i) pool.emplace_back(new char[kFiberStack]);
  return pool[i].get();
}

inline void fiber_entry() {
  Launch& L = *g_launch;
#if OMNI_SIM_ASAN
  __sanitizer_finish_switch_fiber(nullptr, &L.sched_stack_bottom, &L.sched_stack_size);
#endif
  L.body();
  Fiber& me = L.fibers[L.cur];
  me.state = kDone;
  leave(L.waves[me.wave]);
  leave(L.block);
#if OMNI_SIM_ASAN
  __sanitizer_start_switch_fiber(nullptr, L.sched_stack_bottom, L.sched_stack_size);
#endif
  _longjmp(L.sched_jb, 1);
}

// Runs `kernel` over the grid: workgroups in order, each as blockDim fibers.
template <class... P, class... A>
void launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t, hipStream_t, A... args) {
  const unsigned nthreads = block.x * block.y * block.z;
  if (nthreads == 0 || nthreads > 1024 || nthreads % 64 != 0)
    fail("workgroup size must be a multiple of 64 up to 1024");
  gridDim = grid;
  blockDim = block;
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        fill_lds(g_lds_fill);
        Launch L;
        g_launch = &L;
        blockIdx = dim3(bx, by, bz);
        L.body = [&] { kernel(static_cast<P>(args)...); };
        const unsigned nw = nthreads / 64;
        L.waves.resize(nw);
        for (auto& w : L.waves) w.live = 64;
        L.block.live = static_cast<int>(nthreads);
        L.fibers.resize(nthreads);
        for (unsigned i = 0; i < nthreads; ++i) {
          Fiber& f = L.fibers[i];
          f.lane = static_cast<int>(i % 64);
          f.wave = static_cast<int>(i / 64);
          f.tid = dim3(i % block.x, (i / block.x) % block.y, i / (block.x * block.y));
          f.stack = fiber_stack(i);
          getcontext(&f.ctx);
          f.ctx.uc_stack.ss_sp = f.stack;
          f.ctx.uc_stack.ss_size = kFiberStack;
          f.ctx.uc_link = nullptr;
          makecontext(&f.ctx, fiber_entry, 0);
        }
        for (;;) {
          bool ran = false, all_done = true;
          for (unsigned i = 0; i < nthreads; ++i) {
            if (L.fibers[i].state == kDone) continue;
            all_done = false;
            if (L.fibers[i].state != kRun) continue;
            ran = true;
            L.cur = static_cast<int>(i);
#if OMNI_SIM_ASAN
            void* fs = nullptr;
            __sanitizer_start_switch_fiber(&fs, L.fibers[i].stack, kFiberStack);
#endif
            if (_setjmp(L.sched_jb) == 0) {
              if (!L.fibers[i].started) {
                L.fibers[i].started = true;
                swapcontext(&L.sched, &L.fibers[i].ctx);
              } else {
                _longjmp(L.fibers[i].jb, 1);
              }
            }
#if OMNI_SIM_ASAN
            __sanitizer_finish_switch_fiber(fs, nullptr, nullptr);
#endif
          }
          if (all_done) break;
          if (!ran) fail("work-items wait at different cross-lane operations or barriers");
        }
        g_launch = nullptr;
      }
}

}  // namespace sim

#define hipLaunchKernelGGL(kernel, grid, block, shmem, stream, ...) \
  sim::launch(kernel, dim3(grid), dim3(block), (shmem), (stream), __VA_ARGS__)
