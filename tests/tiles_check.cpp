// Host-side exhaustive check of the key-tile schedule used by the scheduler and the attention
// kernels: every (query, key) pair a work item may attend within its key range lies in a
// visited tile, tiles are visited in increasing order and inside the range, the visit count
// matches the closed-form count(), and a tile reported as mask-free holds only visible pairs.
#include <cstdio>
#include <vector>

#include "../hybrid_sparse_full_elastic_amd/csrc/elastic_internal.hpp"

using namespace elastic;

static int failures = 0;
static void fail(const char* what, int mode, int t0, int t1, int BK, int kt) {
  if (failures++ < 20) std::printf("FAIL %s mode=%d t0=%d t1=%d BK=%d tile=%d\n", what, mode, t0, t1, BK, kt);
}

int main() {
  std::vector<Pattern> pats;
  const int SW[][2] = {{0, 1}, {4, 64}, {1, 1}, {70, 130}, {128, 1024}, {3, 40}, {0, 4096}, {64, 63}};
  for (auto& s : SW) pats.push_back(Pattern{ELASTIC_SPARSE_STREAMING, s[0], s[1], 64, 0, 0, 0});
  const int BL[][4] = {{64, 1, 2, 3}, {128, 1, 8, 16}, {128, 0, 1, 0}, {64, 0, 0, 0}, {64, 3, 1, 2}, {128, 2, 0, 1}};
  for (auto& b : BL) pats.push_back(Pattern{ELASTIC_SPARSE_BLOCK, 0, 1, b[0], b[1], b[2], b[3]});
  long checked = 0, steady = 0;
  for (int BK : {32, 64}) {
    for (int n : {1, 5, 63, 64, 65, 300, 1000, 1500}) {
      for (int BT : {1, 7, 16, 32, 36, 42, 51, 64, 85, 128, 256}) {
        for (size_t pi = 0; pi <= pats.size(); ++pi) {
          const bool full = pi == pats.size();
          const Pattern p = full ? pats[0] : pats[pi];
          const int mode = full ? MODE_FULL : p.kind;
          // key ranges [kb, ke) on the same axis as the queries: the whole sequence, a prefix,
          // an aligned suffix and an aligned middle piece (kb aligned to the tile and block)
          const int align = (mode == MODE_BLOCK && p.block > BK) ? p.block : BK;
          const int mid = (n / 2 / align) * align;
          const int ranges[][2] = {{0, n}, {0, n / 2 + 1}, {mid, n}, {mid, mid + n / 3 + 1}};
          for (auto& rg : ranges) {
            const int kb = rg[0], ke = rg[1] < n ? rg[1] : n;
            if (kb != 0 && kb == mid && mid == 0 && rg[1] == n) continue;  // duplicate of the first
            for (int t0 = 0; t0 < n; t0 += BT) {
              const int t1 = (t0 + BT < n ? t0 + BT : n) - 1;
              KeyTiles kt(mode, p, t0, t1, BK, kb, ke);
              std::vector<char> vis((n + BK - 1) / BK + 2, 0);
              int prev = -1, cnt = 0;
              for (int t = kt.next(0); t >= 0; t = kt.next(t + 1)) {
                if (t <= prev) fail("order", mode, t0, t1, BK, t);
                if (t >= (int)vis.size() || t * BK < kb || t * BK >= ke) { fail("range", mode, t0, t1, BK, t); break; }
                vis[t] = 1; prev = t; ++cnt;
                if (!kt.needs_mask(t)) {
                  for (int i = t0; i <= t1; ++i)
                    for (int j = t * BK; j < t * BK + BK; ++j)
                      if (j >= ke || !key_allowed(mode, p, i, j)) { fail("maskfree", mode, t0, t1, BK, t); i = t1 + 1; break; }
                }
              }
              if (cnt != kt.count()) fail("count", mode, t0, t1, BK, cnt);
              // steady pairs of full items: consecutive visited tiles, whole, mask-free
              for (int j = kt.next(0); j >= 0; j = kt.next(j + 1)) {
                if (!kt.steady_pair(j)) continue;
                ++steady;
                for (int i = 1; i <= 6; ++i)
                  if (kt.next(j + i) != j + i) fail("steady-next", mode, t0, t1, BK, j + i);
                if ((j + 6) * BK > ke) fail("steady-whole", mode, t0, t1, BK, j);
                if (kt.needs_mask(j + 1) || kt.needs_mask(j + 2)) fail("steady-mask", mode, t0, t1, BK, j);
              }
              // the compile-time-mode instances walk the same tiles
              for (int t = 0; t <= kt.diag + 1; ++t) {
                int a = -2, b = -2; bool ma = false, mb = false;
                if (mode == MODE_FULL) { KeyTilesT<MODE_FULL> s(mode, p, t0, t1, BK, kb, ke); a = s.next(t); if (a >= 0) ma = s.needs_mask(a); }
                else if (mode == MODE_STREAM) { KeyTilesT<MODE_STREAM> s(mode, p, t0, t1, BK, kb, ke); a = s.next(t); if (a >= 0) ma = s.needs_mask(a); }
                else { KeyTilesT<MODE_BLOCK> s(mode, p, t0, t1, BK, kb, ke); a = s.next(t); if (a >= 0) ma = s.needs_mask(a); }
                b = kt.next(t); if (b >= 0) mb = kt.needs_mask(b);
                if (a != b || ma != mb) { fail("static-mode", mode, t0, t1, BK, t); break; }
              }
              for (int i = t0; i <= t1; ++i)
                for (int j = kb; j <= i && j < ke; ++j)
                  if (key_allowed(mode, p, i, j) && !vis[j / BK]) { fail("missed", mode, t0, t1, BK, j / BK); i = t1 + 1; break; }
              if (kb == 0 && ke == n && !vis[t0 / BK]) fail("diag", mode, t0, t1, BK, t0 / BK);
              ++checked;
            }
          }
        }
      }
    }
  }
  std::printf("%ld items checked, %ld steady pairs verified, %d failures\n", checked, steady, failures);
  return failures ? 1 : 0;
}
