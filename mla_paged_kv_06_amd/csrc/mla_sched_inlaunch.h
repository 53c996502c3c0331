// The split-KV schedule computed inside a decode launch.
//
// Same rule and same result as the separate scheduler (mla_sched.hip):
// sequence b costs c0 + max(1, ceil(L_b / 64)) units, the concatenation of
// all units is cut into `parts` equal shares of q = ceil(T / parts) units,
// partition p starts at unit p * q, and sequence b (pages at units
// [A_b, A_b + n_b), A_b = U_b + c0) is split at every multiple of q inside
// them.  Every workgroup computes it for itself at the start of the launch,
// so the step needs no schedule launch (FlashMLA release note: variable
// length sequences; the cut rule itself is our own).
//
// Each of the kNT threads holds kFusedMaxBatch / kNT consecutive sequences.
// Unit and split-count prefixes are wave scans by DPP row shifts plus lane
// reads (VALU only); one barrier joins the waves' unit totals, one more
// publishes the result.  The split prefix is kept per wave, with the waves'
// totals beside it, and added up by whoever reads it (split_of).  The
// thread whose sequence holds this partition's first unit also reads that
// page's block-table entry while the split counts are scanned, so the first
// copy needs no dependent load.  32-bit arithmetic: the caller keeps
// batch * (max_pages + 2) below 2^30, and page counts are clamped to the
// block-table row.
#pragma once

#include "mla_decode_common.h"

namespace mla {

constexpr int kFusedMaxBatch = 1024;

// Inclusive prefix sum over the 64 lanes of a wave, and the wave's total:
// Hillis-Steele inside each row of 16 lanes by DPP row shifts (lanes shifted
// in from outside the row add 0), then each row adds the totals of the rows
// before it, read from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int x, int lane, int* total) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
  const int row = lane >> 4;
  x += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  *total = (r0 + r1) + (r2 + r3);
  return x;
}

template <int kNT>
struct InLaunchShared {
  static constexpr int kW = kNT / 64;
  int split[kFusedMaxBatch];  // first split of each sequence, counted inside its wave
  int wt[kW];                 // the waves' split totals
  int wu[kW];                 // the waves' unit totals
  int pos[2][5];              // where partitions p and p + 1 start:
                              // (sequence, page, split, length, physical page)
};

struct InLaunchStart {
  Item cur;       // first (sequence, page) of the partition
  int eb, ej;     // first item past it
  int split_idx;  // index of the partition among those sharing sequence cur.b
  int L0, phys0;  // length of cur.b and the physical page of cur (if it holds tokens)
};

// First split of sequence b (b = batch: the number of slots used).
template <int kNT>
__device__ __forceinline__ int split_of(const InLaunchShared<kNT>& sh, int b, int nb) {
  constexpr int kPer = kFusedMaxBatch / kNT;
  const int wv = b / (64 * kPer);  // the wave that scanned b
  const int sv = sh.split[min(b, kFusedMaxBatch - 1)];
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) {
    const int x = sh.wt[w];
    tot += x;
    off += w < wv ? x : 0;
  }
  return b >= nb ? tot : sv + off;
}

// Called by every thread of the workgroup (it holds two barriers).  The
// workgroup with write_splits set also stores num_splits for the combine.
template <int kNT>
__device__ __forceinline__ InLaunchStart schedule_in_launch(
    InLaunchShared<kNT>& sh, int part, int num_parts, int nb, int c0, int max_pages,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ block_table,
    int32_t* __restrict__ splits, bool write_splits) {
  constexpr int kPer = kFusedMaxBatch / kNT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  // every argument used here, in one round of scalar loads
  asm volatile("" ::"s"(c0), "s"(nb), "s"(max_pages), "s"(num_parts), "s"(seqlens),
               "s"(splits), "s"(block_table));
  // all loads in flight at once: indexes past the batch read its last length
  // and are dropped (a branch per load would serialise them)
  int n[kPer], lv[kPer], c = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) lv[i] = seqlens[min(kPer * tid + i, nb - 1)];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    int x = (lv[i] + kPage - 1) >> 6;
    x = x < 1 ? 1 : (x > max_pages ? max_pages : x);
    x = (kPer * tid + i < nb) ? x : 0;
    c += x > 0 ? c0 + x : 0;
    n[i] = x;
  }
  int wt;
  int U = wave_incl_scan(c, lane, &wt) - c;  // exclusive, inside the wave
  if (lane == 0) sh.wu[wave] = wt;
  __syncthreads();
  int T = 0, before = 0;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) {
    const int x = sh.wu[w];
    T += x;
    before += w < wave ? x : 0;
  }
  U += before;
  const unsigned q = ((unsigned)T + num_parts - 1) / (unsigned)num_parts;
  const int u0 = part * (int)q;  // both below T + q < 2^31
  const int u1 = u0 + (int)q;
  // the sequence whose units [U_b, U_b + c0 + n_b) hold u0 (u1), if it is one
  // of this thread's: (b, page, split, length) and (b, page)
  int ns[kPer], nsum = 0;
  int pb = -1, pj = 0, pf = 0, pL = 0, qb = -1, qj = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = kPer * tid + i;
    const int A = U + c0;
    const int fa = (int)((unsigned)A / q);
    ns[i] = (b < nb) ? 1 + (int)((unsigned)(A + n[i] - 1) / q) - fa : 0;
    nsum += ns[i];
    const int Ue = A + n[i];
    const bool h0 = b < nb && U <= u0 && u0 < Ue;
    const bool h1 = b < nb && U <= u1 && u1 < Ue;
    pb = h0 ? b : pb;
    pj = h0 ? (u0 > A ? u0 - A : 0) : pj;
    pf = h0 ? (u0 > A ? part - fa : 0) : pf;
    pL = h0 ? lv[i] : pL;
    qb = h1 ? b : qb;
    qj = h1 ? (u1 > A ? u1 - A : 0) : qj;
    U += (b < nb) ? c0 + n[i] : 0;
  }
  // the first page's block-table entry, read while the split counts are
  // scanned (threads without it read entry 0 and drop it)
  const bool p_live = pb >= 0 && pj * kPage < pL;
  const int ph = block_table[p_live ? (size_t)pb * max_pages + pj : 0];
  int S = wave_incl_scan(nsum, lane, &wt) - nsum;  // exclusive, inside the wave
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = kPer * tid + i;
    if (b < nb) sh.split[b] = S;
    S += ns[i];
  }
  if (lane == 0) sh.wt[wave] = wt;
  if (pb >= 0) {
    sh.pos[0][0] = pb;
    sh.pos[0][1] = pj;
    sh.pos[0][2] = pf;
    sh.pos[0][3] = pL;
    sh.pos[0][4] = p_live ? ph : 0;
  }
  if (qb >= 0) {
    sh.pos[1][0] = qb;
    sh.pos[1][1] = qj;
  }
  if (tid == 0) {
    // a start at or past the last unit is the end of the batch
    if (u0 >= T) sh.pos[0][0] = nb, sh.pos[0][1] = 0, sh.pos[0][2] = 0, sh.pos[0][3] = 0;
    if (u1 >= T) sh.pos[1][0] = nb, sh.pos[1][1] = 0;
  }
  __syncthreads();
  if (write_splits) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (kPer * tid + i < nb) splits[kPer * tid + i] = split_of<kNT>(sh, kPer * tid + i, nb);
    if (tid == 0) splits[nb] = split_of<kNT>(sh, nb, nb);
  }
  InLaunchStart st;
  st.cur = Item{uni(sh.pos[0][0]), uni(sh.pos[0][1])};
  st.eb = uni(sh.pos[1][0]);
  st.ej = uni(sh.pos[1][1]);
  st.split_idx = uni(sh.pos[0][2]);
  st.L0 = uni(sh.pos[0][3]);
  st.phys0 = uni(sh.pos[0][4]);
  return st;
}

}  // namespace mla
