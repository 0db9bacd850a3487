// Host-only check of the workspace layout of libspecverify (no GPU is touched):
// for every (B, K, N, V, mode) the regions a call indexes with its own slice and
// sub-tile counts stay inside their region, the regions do not overlap, the
// fault word lies in the flags region, and the layout fits in
// spec_workspace_bytes(B, K, N), whatever V is.
#include "spec_verify.hip"
#include <cstdio>
#include <vector>

int main() {
  int bad = 0, checked = 0;
  const int Bs[] = {1, 3, 16, 64, 257};
  const int Ks[] = {1, 2, 5, 8, 20, 64};
  const int Ns[] = {1, 7, 21, 64};
  const int Vs[] = {1, 3, 7, 8, 9, 511, 513, 2048, 9000, 16384, 16385, 32000, 40000, 65536, 128256, 151936,
                    1000003, 1 << 20};
  for (int B : Bs)
    for (int K : Ks)
      for (int N : Ns) {
        const size_t total = spec_workspace_bytes(B, K, N);
        for (int V : Vs)
          for (int mode = 0; mode < 2; ++mode)
            for (int fused = 0; fused < 2; ++fused) {
              if (mode == MODE_VERIFY && (fused || N != 1)) continue;
              const Shape s = make_shape(B, K, N, V, mode, fused);
              const WsLayout L = ws_layout(s);
              ++checked;
              const size_t part_words = static_cast<size_t>(B) * s.R * s.S * kWaves;
              const size_t gpart_words = mode == MODE_GAMMA ? static_cast<size_t>(B) * K * N * s.S * kWaves : 0;
              const bool ok = L.flags == 0 && L.done >= 16 && L.done + 4 * static_cast<size_t>(B) <= L.part &&
                              L.part + 8 * part_words <= L.tot &&
                              L.tot + 8 * static_cast<size_t>(B) * kMaxSlices * kMaxSlices <= L.gpart &&
                              L.gpart + 8 * gpart_words <= L.cand && L.cand <= L.pstat &&
                              L.pstat + (mode == MODE_GAMMA ? 8 * static_cast<size_t>(kMaxGrid) * kWaves : 0) <= L.pdone &&
                              L.pdone + (mode == MODE_GAMMA ? 4 * static_cast<size_t>(kMaxGrid) : 0) <= L.selw &&
                              L.selw + (mode == MODE_GAMMA ? 8 * static_cast<size_t>(B) : 0) <= L.lrnw &&
                              L.lrnw + (mode == MODE_GAMMA ? 8 * static_cast<size_t>(B) : 0) <= L.total &&
                              L.total <= total && s.nsub <= kMaxSub && s.S <= kMaxSlices;
              if (!ok) {
                ++bad;
                if (bad < 10)
                  printf("layout violation B=%d K=%d N=%d V=%d mode=%d fused=%d total=%zu/%zu\n", B, K, N, V, mode,
                         fused, L.total, total);
              }
            }
      }
  // draft-tree calls: ticket per target row, target statistics words, slice records
  const int topks[] = {1, 2, 8, 33, 64};
  for (int B : Bs)
    for (int K : Ks)
      for (int N : Ns)
        for (int tk : topks) {
          for (int V : Vs) {
            const size_t total = spec_tree_workspace_bytes(B, K, N, V, tk);
            Shape s = make_shape(B, K, N, V, MODE_TREE, 0);
            s.topk = tk;
            const WsLayout L = ws_layout(s);
            ++checked;
            const size_t part_words = static_cast<size_t>(B) * s.R * s.S * kWaves;
            const size_t rec_words = static_cast<size_t>(B) * K * N * ((V + kPieceTok - 1) / kPieceTok) * tk;
            const bool ok = s.R == K && s.RT == K && s.total0 == static_cast<int64_t>(B) * K * s.S &&
                            L.done >= 16 && L.done + 4 * static_cast<size_t>(B) * K <= L.part &&
                            L.part + 8 * part_words <= L.tot && L.cand + 8 * rec_words <= L.total &&
                            L.total <= total && s.S <= kMaxSlices &&
                            (V < 2 || L.total >= ws_layout([&] { Shape t = make_shape(B, K, N, V / 2, MODE_TREE, 0); t.topk = tk; return t; }()).total);
            if (!ok) {
              ++bad;
              if (bad < 10) printf("tree layout violation B=%d K=%d N=%d V=%d topk=%d\n", B, K, N, V, tk);
            }
          }
        }
  printf("checked %d layouts, %d violations\n", checked, bad);
  // phase-0 schedule (slot-weighted, and the draft-tree calls' first-slot one):
  // every slice of the list is dealt exactly once, and a workgroup's list ends
  // for good at its first T0 (static_phase stops there)
  int sched_bad = 0, sched_checked = 0;
  const int Cs[] = {1, 3, 8, 256};
  const int T0s[] = {1, 2, 7, 100, 511, 512, 513, 5632, 24320, 100003};
  std::vector<int> seen;
  for (int P = 1; P <= kMaxSlots; ++P)
    for (int C : Cs)
      for (int dG = 0; dG < 2; ++dG)
        for (int T0 : T0s) {
          const int G = P * C - dG;  // dG = 1: a grid that is not all of the slots (no weighting)
          if (G < 1) continue;
          for (int tree = 0; tree < 2; ++tree) {
          const Split sp = tree ? tree_split(T0, C, P, G) : make_split(T0, C, P, G);
          seen.assign(T0, 0);
          bool ok = true;
          for (int g = 0; g < G && ok; ++g) {
            bool ended = false;
            for (int k = 0; k < T0 + 2; ++k) {
              const int s = static_slice(sp, k, g);
              if (s == T0) { ended = true; continue; }
              if (ended || s < 0 || s > T0) { ok = false; break; }
              ++seen[s];
            }
          }
          for (int i = 0; i < T0 && ok; ++i) ok = seen[i] == 1;
          ++sched_checked;
          if (!ok) {
            ++sched_bad;
            if (sched_bad < 10) printf("schedule violation P=%d C=%d G=%d T0=%d tree=%d\n", P, C, G, T0, tree);
          }
          }
        }
  printf("checked %d schedules, %d violations\n", sched_checked, sched_bad);
  // gamma row chunks: every row of every group is a regular job of exactly one
  // slot; a drafter row's target row comes earlier in the same slot's jobs; a
  // prefix job is the target row of the group its chunk starts inside; the
  // weights grow by each slot's share and weigh a slot by its last member
  int chunk_bad = 0, chunk_checked = 0;
  const int nGs[] = {1, 2, 5, 160, 512, 777};
  const int R1s[] = {2, 3, 8, 22, 65};
  const int Qs[] = {1, 2, 7, 51, 64, 300, 4096};
  // (members S, compute units, dispatch slots P)
  const int SPs[][3] = {{8, 256, 2}, {10, 256, 2}, {3, 7, 3}, {1, 1, 1}, {5, 64, 4}, {7, 256, 1}};
  std::vector<int> regular;
  for (const auto& sp3 : SPs) {
    const int S = sp3[0], ncu = sp3[1], P = sp3[2];
    for (int q = 0; q < 600; ++q) {
      const int c_last = std::min(P - 1, ((q + 1) * S - 1) / ncu);
      const int64_t want = P == 1 ? kShareDen : gamma_share(P, c_last);
      if (slot_weights(q + 1, S, ncu, P) - slot_weights(q, S, ncu, P) != want) {
        ++chunk_bad;
        if (chunk_bad < 10) printf("slot weight violation S=%d ncu=%d P=%d q=%d\n", S, ncu, P, q);
        break;
      }
    }
  }
  for (int skip0 = 0; skip0 < 2; ++skip0)
  for (const auto& sp3 : SPs)
  for (int nG : nGs)
    for (int R1 : R1s)
      for (int Q : Qs) {
        const int S = sp3[0], ncu = sp3[1], P = sp3[2];
        const int64_t J = static_cast<int64_t>(nG) * R1;
        regular.assign(J, 0);
        bool ok = true;
        // skip0 (fused HedgeSpec rounds, Q >= 2): slot 0 takes no rows
        if (skip0 && Q >= 2 && row_chunk(J, R1, Q, 0, S, ncu, P, true).njobs != 0) ok = false;
        for (int slot = 0; slot < Q && ok; ++slot) {
          const RowChunk c = row_chunk(J, R1, Q, slot, S, ncu, P, skip0 != 0);
          int have_target = -1;
          for (int n = 0; n < c.njobs && ok; ++n) {
            int q, r;
            bool priv;
            chunk_job(c, R1, nG, n, q, r, priv);
            if (q < 0 || q >= nG || r < 0 || r >= R1) { ok = false; break; }
            if (priv) {
              ok = n == 0 && r == 0 && c.prefix && q == c.j0 / R1;
            } else {
              ++regular[static_cast<int64_t>(q) * R1 + r];
            }
            if (r == 0) have_target = q;
            else if (have_target != q) ok = false;
          }
          int q, r;
          bool priv;
          chunk_job(c, R1, nG, c.njobs, q, r, priv);
          if (q != nG) ok = false;
        }
        for (int64_t j = 0; j < J && ok; ++j) ok = regular[j] == 1;
        ++chunk_checked;
        if (!ok) {
          ++chunk_bad;
          if (chunk_bad < 10) printf("row chunk violation nG=%d R1=%d Q=%d S=%d ncu=%d P=%d\n", nG, R1, Q, S, ncu, P);
        }
      }
  printf("checked %d row-chunk partitions, %d violations\n", chunk_checked, chunk_bad);
  return (bad || sched_bad || chunk_bad) ? 1 : 0;
}
