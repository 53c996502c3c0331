// The 64-row decode walks its partition's key range in 32-token slots (half
// pages).  These are the walk's arithmetic, free of any device code, so that
// the same lines build into the kernel and into a host check of them.
// constexpr functions are callable from device code under HIP.
#pragma once

namespace mla {

constexpr int kSlotPage = 64;    // tokens per page
constexpr int kSlotHalf = 32;    // tokens per slot

// Half h of logical page j of sequence b.
struct SlotPos {
  int b, j, h;
};

// Pages a sequence of L tokens occupies in the schedule: an empty sequence
// still counts one (empty) page.
constexpr int slot_pages(int L) { return L > 0 ? (L + kSlotPage - 1) / kSlotPage : 1; }

// The slot after s, given the length L of sequence s.b: the second half of
// the same page, else the next page, else page 0 of the next sequence.
constexpr SlotPos slot_next(SlotPos s, int L) {
  if (s.h == 0) return SlotPos{s.b, s.j, 1};
  if (s.j + 1 < slot_pages(L)) return SlotPos{s.b, s.j + 1, 0};
  return SlotPos{s.b + 1, 0, 0};
}

// Whether page j of a sequence of L tokens holds tokens, i.e. whether its
// block-table entry is in use and may be read.
constexpr bool slot_page_used(int j, int L) { return j * kSlotPage < L; }

// Tokens of slot (j, h) that hold data (0 .. 32): the size of its copy.
constexpr int slot_live_tokens(int j, int h, int L) {
  const int live = L - j * kSlotPage - h * kSlotHalf;
  return live < 0 ? 0 : (live > kSlotHalf ? kSlotHalf : live);
}

// (b, j) before (eb, ej) in sequence-major order: the end of a partition.
constexpr bool slot_before(SlotPos s, int eb, int ej) { return s.b < eb || (s.b == eb && s.j < ej); }

}  // namespace mla
