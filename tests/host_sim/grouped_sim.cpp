// Runs the grouped executor form (cartesian_routed_atomic_amd/csrc/grouped.hip,
// compiled for the host against the wave model in hip/hip_runtime.h) on one
// input file and writes y, the hot-set summary and the hot ids, for
// tests/test_host_sim_grouped.py.
//
//   grouped_sim IN OUT LDS_FILL [NT]
//   IN:  int32 L, K, d, N, accumulate;
//        uint16 x [L, d], W [N, d], V [N, d] (bf16 bits);
//        int32 flat_expert [L*K]; float32 flat_gate [L*K];
//        int32 task_expert [L*K] (schedule order);
//        float32 y0 [L, d] (y before the call)
//   OUT: float32 y [L, d]; int32 misc [4]; int32 hot [512]
// Every buffer is an exact-size heap allocation, so the address sanitizer
// stops the run at the first access outside one.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "hip/hip_runtime.h"
#include "grouped.hip"

// stream_rows lives in execute.hip (whose kernels the wave model does not
// compile); here it is the run's NT argument, so both cold-kernel variants run.
static bool g_nt = false;
bool omni::stream_rows(long long, long long) { return g_nt; }

template <class T> static void rd(FILE* f, std::vector<T>& v) {
  if (std::fread(v.data(), sizeof(T), v.size(), f) != v.size()) sim::fail("short input file");
}
template <class T> static void wr(FILE* f, const T* p, size_t n) {
  if (std::fwrite(p, sizeof(T), n, f) != n) sim::fail("short write");
}

int main(int argc, char** argv) {
  if (argc != 4 && argc != 5) {
    std::fprintf(stderr, "usage: grouped_sim IN OUT LDS_FILL [NT]\n");
    return 2;
  }
  sim::g_lds_fill = static_cast<unsigned char>(std::atoi(argv[3]));
  g_nt = argc == 5 && std::atoi(argv[4]) != 0;
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) sim::fail("cannot open input");
  std::vector<int32_t> hdr(5);
  rd(f, hdr);
  const int L = hdr[0], K = hdr[1], d = hdr[2], N = hdr[3], acc = hdr[4];
  const size_t M = static_cast<size_t>(L) * K;
  std::vector<uint16_t> x(static_cast<size_t>(L) * d), W(static_cast<size_t>(N) * d),
      V(static_cast<size_t>(N) * d);
  std::vector<int32_t> fe(M), texp(M);
  std::vector<float> fg(M), y(static_cast<size_t>(L) * d);
  rd(f, x);
  rd(f, W);
  rd(f, V);
  rd(f, fe);
  rd(f, fg);
  rd(f, texp);
  rd(f, y);
  std::fclose(f);
  const size_t wsb = omni::grouped_ws_bytes(L, K, d, N);
  char* ws = static_cast<char*>(std::aligned_alloc(256, (wsb + 255) / 256 * 256));
  std::memset(ws, 0xA5, wsb);  // the kernels must not rely on any content
  const hipError_t e = omni::launch_grouped(x.data(), W.data(), V.data(), texp.data(),
                                            fe.data(), fg.data(), L, K,
                                            d, N, y.data(), acc, ws, nullptr);
  if (e != hipSuccess) sim::fail("launch_grouped returned an error");
  const omni::GfWsLayout ly = omni::gf_layout(L, K, d, N);
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) sim::fail("cannot open output");
  wr(o, y.data(), y.size());
  wr(o, reinterpret_cast<const int32_t*>(ws + ly.misc), 4);
  wr(o, reinterpret_cast<const int32_t*>(ws + ly.hot), 512);
  std::fclose(o);
  std::free(ws);
  return 0;
}
