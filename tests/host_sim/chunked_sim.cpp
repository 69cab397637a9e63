// Runs the chunked executor kernels (cartesian_routed_atomic_amd/csrc/
// chunked.hip, compiled for the host against the wave model in
// hip/hip_runtime.h) on one input file and writes y, for
// tests/test_host_sim_chunked.py.
//
//   chunked_sim IN OUT
//   IN:  int32 L, K, d, N, bf16, form, glu, accumulate, flat;
//        x [L, d], W [N, d], U [N, d] (glu only), V [N, d] (bf16 bits or
//        float32); int32 flat_expert [L*K]; float32 flat_gate [L*K];
//        int32 task_token, task_expert [L*K]; float32 task_gate [L*K];
//        int32 task_index [L*K] (the schedule's sorted order);
//        float32 y0 [L, d] (y before the call)
//   OUT: float32 y [L, d]
// flat = 0 hands the token-centric form no flattened selection, so it
// inverts the schedule first.  Every buffer is an exact-size heap
// allocation, so the address sanitizer stops the run at the first access
// outside one.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "hip/hip_runtime.h"
#include "chunked.hip"

// The three library functions chunked.hip calls that live in execute.hip
// (whose kernels the wave model does not compile): the workspace size the
// same way, no nontemporal rows (their sc1 buffer stores are not modelled),
// and the schedule inverted by a host loop.
namespace omni {
size_t atomic_forward_ws_bytes(int L, int K) {
  const size_t m = static_cast<size_t>(L) * static_cast<size_t>(K) * 4;
  return 2 * ((m + 255) & ~static_cast<size_t>(255));
}
bool stream_rows(long long, long long) { return false; }
hipError_t launch_unpermute(const int32_t* texp, const float* tgate, const int32_t* tidx, int M,
                            int N, int32_t* le, float* lg, hipStream_t) {
  for (int m = 0; m < M; ++m) {
    const int i = tidx[m];
    if (i < 0 || i >= M) continue;
    le[i] = texp[m] >= 0 && texp[m] < N ? texp[m] : 0;
    lg[i] = tgate[m];
  }
  return hipSuccess;
}
}  // namespace omni

template <class T> static void rd(FILE* f, std::vector<T>& v) {
  if (std::fread(v.data(), sizeof(T), v.size(), f) != v.size()) sim::fail("short input file");
}

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: chunked_sim IN OUT\n");
    return 2;
  }
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) sim::fail("cannot open input");
  std::vector<int32_t> hdr(9);
  rd(f, hdr);
  const int L = hdr[0], K = hdr[1], d = hdr[2], N = hdr[3], bf16 = hdr[4], form = hdr[5],
            glu = hdr[6], acc = hdr[7], flat = hdr[8];
  const size_t M = static_cast<size_t>(L) * K, es = bf16 ? 2 : 4;
  std::vector<unsigned char> x(L * d * es), W(N * d * es), U(glu ? N * d * es : 0),
      V(N * d * es);
  std::vector<int32_t> fe(M), tt(M), te(M), ti(M);
  std::vector<float> fg(M), tg(M), y(static_cast<size_t>(L) * d);
  rd(f, x);
  rd(f, W);
  if (glu) rd(f, U);
  rd(f, V);
  rd(f, fe);
  rd(f, fg);
  rd(f, tt);
  rd(f, te);
  rd(f, tg);
  rd(f, ti);
  rd(f, y);
  std::fclose(f);
  const size_t wsb = omni::atomic_forward_ws_bytes(L, K);
  char* ws = static_cast<char*>(std::aligned_alloc(256, wsb));
  std::memset(ws, 0xA5, wsb);  // the kernels must not rely on any content
  const hipError_t e = omni::launch_chunked(
      bf16, form, glu != 0, L, d, N, K, x.data(), W.data(), glu ? U.data() : nullptr, V.data(),
      tt.data(), te.data(), tg.data(), ti.data(), flat ? fe.data() : nullptr,
      flat ? fg.data() : nullptr, y.data(), acc != 0, ws, nullptr);
  if (e != hipSuccess) sim::fail("launch_chunked returned an error");
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) sim::fail("cannot open output");
  if (std::fwrite(y.data(), sizeof(float), y.size(), o) != y.size()) sim::fail("short write");
  std::fclose(o);
  std::free(ws);
  return 0;
}
