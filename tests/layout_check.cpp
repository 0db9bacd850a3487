// Host-only check of the workspace layout of libspecverify (no GPU is touched):
// for every (B, K, N, V, mode) the zero region (counters + queue) ends at the same
// offset for a given (B, K), holds every unit one call can publish, and the whole
// layout fits in spec_workspace_bytes(B, K, N).
#include "spec_verify.hip"
#include <cstdio>

int main() {
  int bad = 0, checked = 0;
  const int Bs[] = {1, 3, 16, 64, 257};
  const int Ks[] = {1, 2, 5, 8, 20, 64};
  const int Ns[] = {1, 7, 21, 64};
  const int Vs[] = {1, 3, 7, 8, 9, 511, 513, 2048, 9000, 16384, 16385, 32000, 40000, 65536, 128256, 151936,
                    1000003, 1 << 20};
  for (int B : Bs)
    for (int K : Ks) {
      const size_t zero = spec_workspace_counter_bytes(B, K);
      for (int N : Ns) {
        const size_t total = spec_workspace_bytes(B, K, N);
        for (int V : Vs)
          for (int mode = 0; mode < 2; ++mode)
            for (int fused = 0; fused < 2; ++fused) {
              if (mode == MODE_VERIFY && (fused || N != 1)) continue;
              const Shape s = make_shape(B, K, N, V, mode, fused);
              const WsLayout L = ws_layout(s);
              ++checked;
              const bool ok = L.zero_end == zero && L.queue + 8 * static_cast<size_t>(s.n_dyn) <= L.zero_end &&
                              L.total <= total && L.stat_k >= L.zero_end && L.subsum >= L.stat_k &&
                              L.dec + 8 * static_cast<size_t>(B) * kDecWords <= L.total;
              if (!ok) {
                ++bad;
                if (bad < 10)
                  printf("layout violation B=%d K=%d N=%d V=%d mode=%d fused=%d zero_end=%zu/%zu total=%zu/%zu\n", B,
                         K, N, V, mode, fused, L.zero_end, zero, L.total, total);
              }
            }
      }
    }
  printf("checked %d layouts, %d violations\n", checked, bad);
  return bad ? 1 : 0;
}
