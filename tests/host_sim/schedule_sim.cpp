// Runs the one-workgroup schedule (cartesian_routed_atomic_amd/csrc/
// schedule_small.hip, compiled for the host against the wave model in
// hip/hip_runtime.h) on one input file and writes its outputs, for
// tests/test_host_sim_schedule.py.
//
//   schedule_sim IN OUT LDS_FILL
//   IN:  int32 L, K, N, B, window, G; int32 expert_idx [L*K]; float32 gate [L*K]
//   OUT: int32 counts [2], active [min(N, L*K)], group_offsets [G + 1],
//        task_token, task_expert [L*K], float32 task_gate [L*K],
//        int32 task_index [L*K]
// Every buffer is an exact-size heap allocation, so the address sanitizer
// stops the run at the first access outside one.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "hip/hip_runtime.h"
#include "schedule_small.hip"

template <class T> static void rd(FILE* f, std::vector<T>& v) {
  if (std::fread(v.data(), sizeof(T), v.size(), f) != v.size()) sim::fail("short input file");
}
template <class T> static void wr(FILE* f, const std::vector<T>& v) {
  if (std::fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) sim::fail("short write");
}

int main(int argc, char** argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: schedule_sim IN OUT LDS_FILL\n");
    return 2;
  }
  sim::g_lds_fill = static_cast<unsigned char>(std::atoi(argv[3]));
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) sim::fail("cannot open input");
  std::vector<int32_t> hdr(6);
  rd(f, hdr);
  const int L = hdr[0], K = hdr[1], N = hdr[2], B = hdr[3], window = hdr[4], G = hdr[5];
  const size_t M = static_cast<size_t>(L) * K;
  std::vector<int32_t> idx(M);
  std::vector<float> gate(M);
  rd(f, idx);
  rd(f, gate);
  std::fclose(f);
  std::vector<int32_t> counts(2), active(M < static_cast<size_t>(N) ? M : N), off(G + 1), tt(M),
      te(M), ti(M);
  std::vector<float> tg(M);
  const hipError_t e = omni::launch_schedule_small(L, K, N, B, window, G, idx.data(), gate.data(),
                                                   counts.data(), active.data(), off.data(),
                                                   tt.data(), te.data(), tg.data(), ti.data(),
                                                   nullptr);
  if (e != hipSuccess) sim::fail("launch_schedule_small returned an error");
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) sim::fail("cannot open output");
  wr(o, counts);
  wr(o, active);
  wr(o, off);
  wr(o, tt);
  wr(o, te);
  wr(o, tg);
  wr(o, ti);
  std::fclose(o);
  return 0;
}
