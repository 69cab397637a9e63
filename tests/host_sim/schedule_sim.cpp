// Runs Expert-Centric Scheduling (cartesian_routed_atomic_amd/csrc/schedule.hip,
// compiled for the host against the wave model in hip/hip_runtime.h) on one
// input file and writes every output, for tests/test_host_sim_schedule.py.
//
//   schedule_sim IN OUT LDS_FILL
//   IN:  int32 L, K, N, B, window; int32 expert_idx [L*K]; float32 gate [L*K]
//   OUT: int32 counts [2]; int32 active [min(L*K, N)]; int32 group_offsets [G+1];
//        int32 task_token, task_expert [L*K]; float32 task_gate [L*K];
//        int32 task_index [L*K]; int32 rank [N] (the workspace's rank array)
// Every buffer is an exact-size heap allocation, so the address sanitizer
// stops the run at the first access outside one.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "hip/hip_runtime.h"
#include "schedule.hip"

template <class T> static void rd(FILE* f, std::vector<T>& v) {
  if (std::fread(v.data(), sizeof(T), v.size(), f) != v.size()) sim::fail("short input file");
}
template <class T> static void wr(FILE* f, const T* p, size_t n) {
  if (std::fwrite(p, sizeof(T), n, f) != n) sim::fail("short write");
}

int main(int argc, char** argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: schedule_sim IN OUT LDS_FILL\n");
    return 2;
  }
  sim::g_lds_fill = static_cast<unsigned char>(std::atoi(argv[3]));
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) sim::fail("cannot open input");
  std::vector<int32_t> hdr(5);
  rd(f, hdr);
  const int L = hdr[0], K = hdr[1], N = hdr[2], B = hdr[3], window = hdr[4];
  const size_t M = static_cast<size_t>(L) * K;
  std::vector<int32_t> idx(M);
  std::vector<float> gate(M);
  rd(f, idx);
  rd(f, gate);
  std::fclose(f);
  const omni::ScheduleWs lay = omni::schedule_ws_layout(L, K, N, B, window);
  const size_t n_act = M < static_cast<size_t>(N) ? M : static_cast<size_t>(N);
  const size_t G = static_cast<size_t>(lay.max_groups);
  // outputs start as garbage: every entry the schedule defines must be written
  std::vector<int32_t> counts(2, -7), active(n_act > 0 ? n_act : 1, -7), off(G + 1, -7),
      tok(M, -7), exp_(M, -7), tidx(M, -7);
  std::vector<float> tg(M, -7.f);
  char* ws = static_cast<char*>(std::aligned_alloc(256, (lay.bytes + 255) / 256 * 256));
  std::memset(ws, 0xA5, lay.bytes);  // the kernels must not rely on any content
  const hipError_t e = omni::launch_schedule(L, K, N, B, window, idx.data(), gate.data(),
                                             counts.data(), active.data(), off.data(), tok.data(),
                                             exp_.data(), tg.data(), tidx.data(), ws, nullptr);
  if (e != hipSuccess) sim::fail("launch_schedule returned an error");
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) sim::fail("cannot open output");
  wr(o, counts.data(), 2);
  wr(o, active.data(), n_act);
  wr(o, off.data(), G + 1);
  wr(o, tok.data(), M);
  wr(o, exp_.data(), M);
  wr(o, tg.data(), M);
  wr(o, tidx.data(), M);
  wr(o, reinterpret_cast<const int32_t*>(ws + lay.rank), static_cast<size_t>(N));
  std::fclose(o);
  std::free(ws);
  return 0;
}
