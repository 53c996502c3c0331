// Host check of the 64-row decode's slot walk (mla_slot_walk.h, the same
// header the kernel includes).  For random batches, block tables and
// partition ranges it walks every partition as the kernel does and checks:
//   - each block-table entry read (pages that hold tokens) lies inside the
//     sequence's used pages and inside its table row;
//   - no entry is read for a page without tokens (an empty sequence, or a
//     page past the end);
//   - every copy is sized to the slot's live tokens (0 .. 32), and the
//     copy of a slot that holds no tokens is empty;
//   - the walk visits exactly the partition's (sequence, page) items, two
//     halves each, in order.
// Prints "ok" and exits 0, or names the first failure and exits 1.
#include <cstdio>
#include <vector>

#include "mla_slot_walk.h"

using mla::SlotPos;

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;
static unsigned next_u32() {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return (unsigned)(rng_state >> 33);
}

// pages the schedule gives a sequence of L tokens (an empty one counts one),
// written here independently of the header
static int pages_of(int L) { return L == 0 ? 1 : (L + 63) / 64; }

static int fail(const char* what, int trial, int b, int j) {
  std::printf("FAIL trial %d: %s (sequence %d, page %d)\n", trial, what, b, j);
  return 1;
}

int main() {
  for (int trial = 0; trial < 20000; ++trial) {
    const int batch = 1 + (int)(next_u32() % 40);
    std::vector<int> L(batch);
    int max_pages = 1;
    for (int b = 0; b < batch; ++b) {
      const unsigned k = next_u32() % 8;
      L[b] = k == 0 ? 0 : (k == 1 ? 64 * (int)(next_u32() % 6) : (int)(next_u32() % 700));
      const int used = (L[b] + 63) / 64;
      if (used > max_pages) max_pages = used;
    }
    // the items of the whole batch, in order: every sequence's pages, an
    // empty sequence counting one
    std::vector<SlotPos> items;
    for (int b = 0; b < batch; ++b)
      for (int j = 0; j < pages_of(L[b]); ++j) items.push_back(SlotPos{b, j, 0});
    const int n = (int)items.size();
    // a partition: items [lo, hi), hi = n ends at (batch, 0)
    int lo = (int)(next_u32() % n);
    int hi = lo + 1 + (int)(next_u32() % (n - lo));
    const int eb = hi < n ? items[hi].b : batch;
    const int ej = hi < n ? items[hi].j : 0;
    SlotPos s = items[lo];
    int visited = 0;
    while (true) {
      // the slot's sequence and page must be an item of the range
      if (s.b >= batch) return fail("walked past the batch", trial, s.b, s.j);
      if (s.j >= pages_of(L[s.b])) return fail("page past the sequence", trial, s.b, s.j);
      const SlotPos want = items[lo + visited / 2];
      if (want.b != s.b || want.j != s.j || s.h != visited % 2)
        return fail("walk left the item order", trial, s.b, s.j);
      // the table entry the kernel reads for this slot's page
      if (mla::slot_page_used(s.j, L[s.b])) {
        if (s.j >= max_pages) return fail("entry past the table row", trial, s.b, s.j);
        if (s.j * 64 >= L[s.b]) return fail("entry of a page without tokens", trial, s.b, s.j);
      } else if (L[s.b] > s.j * 64) {
        return fail("a page with tokens left unread", trial, s.b, s.j);
      }
      const int live = mla::slot_live_tokens(s.j, s.h, L[s.b]);
      const int expect = L[s.b] - 64 * s.j - 32 * s.h;
      if (live < 0 || live > 32) return fail("copy size out of range", trial, s.b, s.j);
      if ((expect <= 0) != (live == 0)) return fail("copy of a slot without tokens", trial, s.b, s.j);
      if (expect > 0 && live != (expect < 32 ? expect : 32))
        return fail("copy size differs from the live tokens", trial, s.b, s.j);
      ++visited;
      // advance as the kernel does: the second half stays on its page; a new
      // page is valid while it is before the partition's end
      const SlotPos nx = mla::slot_next(s, L[s.b]);
      if (s.h == 0) {
        s = nx;
        continue;
      }
      if (!mla::slot_before(nx, eb, ej)) break;
      s = nx;
    }
    if (visited != 2 * (hi - lo)) return fail("walk did not cover the partition", trial, eb, ej);
  }
  std::printf("ok\n");
  return 0;
}
