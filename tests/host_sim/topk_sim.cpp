// Runs the product top-K kernels (cartesian_routed_atomic_amd/csrc/topk.hip,
// compiled for the host against the wave model in hip/hip_runtime.h) on one
// input file and writes every output, for tests/test_host_sim_topk.py.
//
//   topk_sim IN OUT LDS_FILL LOG_ULPS
//   IN:  int32 L, Nr, Nc, kprime, K; float32 row_logits [L, Nr]; col_logits [L, Nc]
//   OUT: int32 expert_idx [L, K]; float32 score, gate [L, K];
//        float32 row_logp [L, Nr], col_logp [L, Nc]; int32 row_sel, col_sel [L, k'];
//        int32 tie_flag [L]; int64 cross-lane operations evaluated
// Every buffer is an exact-size heap allocation, so the address sanitizer
// stops the run at the first access outside one.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "hip/hip_runtime.h"
#include "topk.hip"

template <class T> static void rd(FILE* f, T* p, size_t n) {
  if (std::fread(p, sizeof(T), n, f) != n) sim::fail("short input file");
}
template <class T> static void wr(FILE* f, const std::vector<T>& v) {
  if (std::fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) sim::fail("short write");
}

int main(int argc, char** argv) {
  if (argc != 5) {
    std::fprintf(stderr, "usage: topk_sim IN OUT LDS_FILL LOG_ULPS\n");
    return 2;
  }
  sim::g_lds_fill = static_cast<unsigned char>(std::atoi(argv[3]));
  sim::g_log_ulps = std::atoi(argv[4]);
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) sim::fail("cannot open input");
  int hdr[5];
  rd(f, hdr, 5);
  const int L = hdr[0], Nr = hdr[1], Nc = hdr[2], kp = hdr[3], K = hdr[4];
  std::vector<float> zr(static_cast<size_t>(L) * Nr), zc(static_cast<size_t>(L) * Nc);
  rd(f, zr.data(), zr.size());
  rd(f, zc.data(), zc.size());
  std::fclose(f);

  std::vector<int32_t> idx(static_cast<size_t>(L) * K), rsel(static_cast<size_t>(L) * kp),
      csel(static_cast<size_t>(L) * kp), tie(L);
  std::vector<float> score(static_cast<size_t>(L) * K), gate(static_cast<size_t>(L) * K),
      ra(static_cast<size_t>(L) * Nr), cb(static_cast<size_t>(L) * Nc), lse(2 * static_cast<size_t>(L));
  const hipError_t e = omni::launch_product_topk(zr.data(), zc.data(), L, Nr, Nc, kp, K,
                                                 idx.data(), score.data(), gate.data(), ra.data(),
                                                 cb.data(), rsel.data(), csel.data(), tie.data(),
                                                 lse.data(), nullptr);
  if (e != hipSuccess) sim::fail("launch_product_topk returned an error");
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) sim::fail("cannot open output");
  wr(o, idx);
  wr(o, score);
  wr(o, gate);
  wr(o, ra);
  wr(o, cb);
  wr(o, rsel);
  wr(o, csel);
  wr(o, tie);
  const long long nc = sim::g_collectives;
  std::fwrite(&nc, sizeof nc, 1, o);
  std::fclose(o);
  return 0;
}
