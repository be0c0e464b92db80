// Host check of the column score's row-chunk geometry (chunk_count,
// chunk_range, chunk_of): for every segment length and chunk size tried, the
// chunks tile [0, n) in order without gaps or overlaps, every token maps to
// the chunk that holds it, and a segment of at most RC tokens is one chunk.
#include <cstdio>

#include "internal.h"

int main() {
  using namespace tsel;
  long long checked = 0;
  const int rcs[] = {32, 64, 256, 512, 1024, 8192};
  for (int rc : rcs) {
    for (int split : {1, 2, 4, 8}) {
      const int rcf = rc / split;
      for (int n = 0; n <= 3 * rc + rcf + 7; n += (n < 2 * rc ? 1 : 3)) {
        const int cnt = chunk_count(n, rc, rcf);
        if (n == 0) {
          if (cnt != 0) { std::printf("FAIL n=0 count %d\n", cnt); return 1; }
          continue;
        }
        if (n <= rc && cnt != 1) { std::printf("FAIL short n=%d rc=%d count %d\n", n, rc, cnt); return 1; }
        int expect = 0;
        for (int r = 0; r < cnt; ++r) {
          int lo, hi;
          chunk_range(r, n, rc, rcf, lo, hi);
          if (lo != expect || hi <= lo || hi > n) {
            std::printf("FAIL n=%d rc=%d rcf=%d chunk %d [%d,%d) expected start %d\n", n, rc, rcf, r, lo, hi, expect);
            return 1;
          }
          if (hi - lo > (r < chunk_whole(n, rc) ? rc : rcf)) {
            std::printf("FAIL n=%d rc=%d rcf=%d chunk %d too long\n", n, rc, rcf, r);
            return 1;
          }
          for (int t = lo; t < hi; ++t)
            if (chunk_of(t, n, rc, rcf) != r) {
              std::printf("FAIL n=%d rc=%d rcf=%d token %d maps to %d not %d\n", n, rc, rcf, t,
                          chunk_of(t, n, rc, rcf), r);
              return 1;
            }
          expect = hi;
          ++checked;
        }
        if (expect != n) { std::printf("FAIL n=%d chunks end at %d\n", n, expect); return 1; }
      }
    }
  }
  std::printf("ok %lld chunks\n", checked);
  return 0;
}
