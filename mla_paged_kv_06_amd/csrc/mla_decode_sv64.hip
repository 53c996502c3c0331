// Paged MLA decode, 64 query rows per workgroup of 8 waves in two roles.
//
// What is computed, and the layouts shared with the other decode kernels,
// are described in mla_decode.hip (FlashMLA release note: MLA principles and
// the paged bf16 cache; DeepSeek-V3 summary: one latent shared by all heads).
//
// Every SIMD runs one score wave and one value wave, and the two work half a
// page apart, so one's softmax, LDS latency and copy issue overlap the
// other's matrix instructions:
//
//   score wave r (waves 0..3): rows 16 r .. 16 r + 15.  For each 32-token
//     slot: S^T = K Q^T over the slot's two 16-token tiles (36 MFMA
//     16x16x32), the masked row max, the lazy rescale decision and the bf16
//     weights, written to LDS already in the B-operand layout of the value
//     product, with the rescale factor of each row;
//   value wave c (waves 4..7): output columns 128 c .. 128 c + 127 of all 64
//     rows.  For the slot the score waves finished one step earlier: rescale
//     if any row asks for it, then O^T += V^T P^T (32 MFMA); and the copies
//     of the slot two steps ahead.
//
// The stream is cut into 32-token slots (half pages) kept in a ring of four
// 36 KiB LDS buffers.  Step i: score waves on slot i, value waves on slot
// i - 1 and copying slot i + 2 into the buffer slot i - 2 left; one barrier
// ends the step.  Weights and rescale factors are double-buffered.
//
// Value wave c copies 8-token block c of each slot (nine 1 KiB buffer loads
// straight into LDS, through a resource bounded by the slot's live tokens,
// so a partial or empty slot arrives zero-filled).  The copies are written
// in assembly, so the compiler does not track them and never waits for a
// slot still in flight; each value wave waits for its own copies of slot i
// (vmcnt: the newest nine, slot i + 1's, may stay in flight) before the
// barrier that opens step i.  Score waves issue no copies and write LDS;
// value waves only read it, so their barrier skips the LDS-count wait and a
// block-table load issued at the end of their step stays in flight.
//
// Each role runs its own loop; both take the same number of steps and meet
// at one barrier per step, so each role's registers are live only in its
// own loop (the value waves' 128 accumulators, the score waves' query rows).

#include "mla_decode_common.h"
#include "mla_sched_inlaunch.h"
#include "mla_slot_walk.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

namespace sv {
constexpr int kWavesSV = 8;
constexpr int kThreadsSV = 64 * kWavesSV;
constexpr int kRows = 64;
constexpr int kRT = 4;                               // 16-row tiles
constexpr int kCT = 8;                               // 16-column tiles per value wave
constexpr int kKS = kD / 32;                         // 18 k-steps of the score product
constexpr int kSlotTokens = 32;
constexpr int kSlotBytes = kSlotTokens * kRowBytes;  // 36864
constexpr int kRing = 4;
constexpr int kCopies = 9;                           // per value wave and slot
constexpr int kBlockBytes = 8 * kRowBytes;           // 9216: one 8-token block
}  // namespace sv

// One wave-wide copy HBM -> LDS, 16 bytes per lane: lane l's bytes at offset
// voff + soff of the resource go to LDS address lds + 16 l (reads past the
// resource's size return zero).  M0 carries the LDS base; no compiled code
// in this kernel uses M0.  The wait states after the M0 write cover SGPR
// operands that a VALU readfirstlane may have written just before.
__device__ __forceinline__ void sv_copy16(MLA_LDS char* lds, int voff, i32x4 rsrc, int soff) {
  const int m0 = uni((int)(size_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// Buffer resource over `bytes` bytes from `base` (wave-uniform).
__device__ __forceinline__ i32x4 sv_rsrc(const char* base, int bytes) {
  const unsigned long long a = (unsigned long long)base;
  return i32x4{uni((int)(unsigned)a), uni((int)((a >> 32) & 0xFFFF)), uni(bytes), kBufferFlags};
}

// s_waitcnt between compiler fences: the wait intrinsic alone does not keep
// the scheduler from moving LDS reads above it.
template <int kImm>
__device__ __forceinline__ void sv_fenced_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  asm volatile("" ::: "memory");
}

// A 32-token slot of the stream: half h of page j of sequence b.
struct SvSlot {
  int b, j, h;
  int L;     // length of sequence b
  int phys;  // physical page of (b, j) (value waves only)
  bool valid;
};

// kFused: no tile_metadata; every workgroup computes the schedule itself.
template <bool kFused>
__global__ void __launch_bounds__(sv::kThreadsSV, 1)
    decode_kernel_sv64(const DecodeParams prm, const uint16_t* q_ptr,
                       const uint16_t* __restrict__ kv_ptr,
                       const int32_t* __restrict__ block_table,
                       const int32_t* __restrict__ seqlens, const int32_t* __restrict__ meta,
                       int32_t* __restrict__ splits, uint16_t* __restrict__ out_ptr,
                       float* __restrict__ lse_ptr, uint16_t* __restrict__ o_acc,
                       float* __restrict__ lse_acc) {
  using namespace sv;
  __shared__ __attribute__((aligned(1024))) char ring_[kRing * kSlotBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][kRT][64];  // [step & 1][row tile][lane]
  __shared__ float alpha_buf[2][kRows];                            // [step & 1][row]
  __shared__ float stat_l[kRows];                                  // row sums at a segment end
  __shared__ std::conditional_t<kFused, InLaunchShared<kThreadsSV>, char> sched_sh;
  MLA_LDS char* ring = (MLA_LDS char*)ring_;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // XCD-aware mapping: the row groups of a partition share an XCD, so the
  // pages they all read are fetched from HBM once into that XCD's L2.  With
  // fewer than 8 partitions (thousands of rows) that would leave XCDs idle:
  // consecutive workgroups then take consecutive row groups instead.
  const int bid = blockIdx.x;
  int rg, part;
  if (prm.num_parts >= 8) {
    const int rr = bid >> 3;
    rg = rr % prm.row_groups;
    part = (rr / prm.row_groups) * 8 + (bid & 7);
  } else {
    rg = bid % prm.row_groups;
    part = bid / prm.row_groups;
  }
  rg = uni(rg);
  part = uni(part);
  if (part >= prm.num_parts) return;

  int eb, ej, b0, j0, split0, L0 = 0, phys0 = 0;
  if constexpr (kFused) {
    // the separate scheduler's cuts, computed by this workgroup
    const InLaunchStart st =
        schedule_in_launch<kThreadsSV>(sched_sh, part, prm.num_parts, prm.batch, prm.sched_c0,
                                       prm.max_pages, seqlens, block_table, splits,
                                       part == 0 && rg == 0);
    eb = st.eb;
    ej = st.ej;
    b0 = st.cur.b;
    j0 = st.cur.j;
    split0 = st.split_idx;
    L0 = st.L0;
    phys0 = st.phys0;
  } else {
    const int32_t* m = meta + part * kMetaInts;
    eb = uni(m[2]);
    ej = uni(m[3]);
    b0 = uni(m[0]);
    j0 = uni(m[1]);
    split0 = uni(m[4]);
  }
  if (!item_before(Item{b0, j0}, eb, ej)) return;
  // first split of sequence b (b = batch: slots used)
  auto split_at = [&](int b) __attribute__((always_inline)) -> int {
    if constexpr (kFused)
      return uni(split_of<kThreadsSV>(sched_sh, b, prm.batch));
    else
      return uni(splits[b]);
  };
  const int row0 = rg * kRows;
  const bool is_value = wave >= 4;

  // ---- slot stream (every wave runs the same bookkeeping on scalars)
  auto next_slot = [&](const SvSlot& s) __attribute__((always_inline)) -> SvSlot {
    SvSlot n = s;
    const SlotPos p = slot_next(SlotPos{s.b, s.j, s.h}, s.L);
    n.b = uni(p.b);
    n.j = uni(p.j);
    n.h = p.h;
    if (s.h == 0) return n;  // the same page: its length and entry stand
    n.valid = s.valid && slot_before(p, eb, ej);
    if (n.valid) {
      if (n.b != s.b) n.L = load_uniform(seqlens, n.b);
      // only pages that hold tokens have a block-table entry (an empty
      // sequence's single unit holds none); the others get page 0 and a
      // resource of zero bytes
      if (is_value)
        n.phys = slot_page_used(n.j, n.L)
                     ? load_uniform(block_table, (size_t)n.b * prm.max_pages + n.j)
                     : 0;
    }
    return n;
  };
  SvSlot s0;
  s0.b = b0;
  s0.j = j0;
  s0.h = 0;
  if constexpr (kFused) {  // read with the schedule
    s0.L = L0;
    s0.phys = is_value ? phys0 : 0;
  } else {
    s0.L = load_uniform(seqlens, b0);
    s0.phys = (is_value && slot_page_used(j0, s0.L))
                  ? load_uniform(block_table, (size_t)b0 * prm.max_pages + j0)
                  : 0;
  }
  s0.valid = true;

  if (!is_value) {
    // ================= score waves =================
    const int rt = wave;
    const int qk_row = row0 + 16 * rt + l16;  // the row this lane scores
    const bool live = qk_row < prm.R;
    // K fragment (A operand): token l16 (+16 for the second tile) of the
    // slot, logical chunk 4 ks + g at physical (4 ks + g) ^ (token & 7)
    const int sw = l16 & 7;
    const int k_lane = l16 * kRowBytes + 16 * (g ^ (sw & 3));
    const int k_even = k_lane + ((sw & 4) ? 64 : 0);
    const int k_odd = k_lane - ((sw & 4) ? 64 : 0);

    bf16x8 qf[kKS];
    float m_used = -INFINITY, l_part = 0.f;
    int n_vis = 0;
    int seg_s_lo = 0, seg_nsplit = 0, split_idx = split0;

    auto begin_segment = [&](int b, int L) __attribute__((always_inline)) {
      seg_s_lo = split_at(b);
      seg_nsplit = split_at(b + 1) - seg_s_lo;
      const uint16_t* qrow = q_ptr + ((size_t)b * prm.R + (live ? qk_row : 0)) * kD + 8 * g;
      static_for<0, kKS>([&](auto kc) __attribute__((always_inline)) {
        qf[decltype(kc)::value] = *(const bf16x8*)(qrow + 32 * decltype(kc)::value);
      });
      const int i = (live ? qk_row : 0) / prm.h_q;
      int n = prm.causal ? (L - prm.s_q + 1 + i) : L;
      n = n < 0 ? 0 : (n > L ? L : n);
      n_vis = live ? n : 0;
      m_used = -INFINITY;
      l_part = 0.f;
    };

    auto finish_segment = [&](int b) __attribute__((always_inline)) {
      const float lt = wave_sum_x4(l_part);
      if (g == 0) {
        stat_l[16 * rt + l16] = lt;
        if (live) {
          const float lse2 =
              lt > 0.f ? m_used * prm.scale_log2 + __builtin_amdgcn_logf(lt) : -INFINITY;
          if (seg_nsplit <= 1)
            lse_ptr[(size_t)b * prm.R + qk_row] = lse2 * kLn2;
          else
            lse_acc[(size_t)(seg_s_lo + split_idx) * prm.R + qk_row] = lse2;
        }
      }
      split_idx = 0;  // later sequences of this partition start at their page 0
    };

    // scores, softmax and weights of one slot
    auto score_slot = [&](MLA_LDS char* buf, int pos0, int pb) __attribute__((always_inline)) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
      auto load_k = [&](int ks, int tt) __attribute__((always_inline)) {
        return *(MLA_LDS bf16x8*)(buf + ((ks & 1) ? k_odd : k_even) + 64 * ks +
                                  tt * 16 * kRowBytes);
      };
      constexpr int DK = 4;  // k-steps of fragments in flight
      bf16x8 ka[DK + 1], kb[DK + 1];
      static_for<0, DK>([&](auto ic) __attribute__((always_inline)) {
        ka[decltype(ic)::value] = load_k(decltype(ic)::value, 0);
        kb[decltype(ic)::value] = load_k(decltype(ic)::value, 1);
      });
      static_for<0, kKS>([&](auto ksc) __attribute__((always_inline)) {
        constexpr int ks = decltype(ksc)::value;
        if constexpr (ks + DK < kKS) {
          ka[(ks + DK) % (DK + 1)] = load_k(ks + DK, 0);
          kb[(ks + DK) % (DK + 1)] = load_k(ks + DK, 1);
        }
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks % (DK + 1)], qf[ks], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks % (DK + 1)], qf[ks], sb, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      // ---- masked row max over the slot's 32 tokens (raw score units; the
      //      scale is positive)
      const int t0 = pos0 + 4 * g;
      float x[8];
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = (t0 + r < n_vis) ? sa[r] : -INFINITY;
        x[4 + r] = (t0 + 16 + r < n_vis) ? sb[r] : -INFINITY;
        mt = fmaxf(mt, fmaxf(x[r], x[4 + r]));
      }
      mt = wave_max_x4(mt);
      // ---- online softmax (log2 domain), one decision for the wave
      const bool upd = __builtin_amdgcn_ballot_w64((mt - m_used) * prm.scale_log2 >
                                                   kRescaleThreshold) != 0;
      const float mn = upd ? fmaxf(m_used, mt) : m_used;
      const float alpha = (upd && mn != -INFINITY)
                              ? __builtin_amdgcn_exp2f((m_used - mn) * prm.scale_log2)
                              : 1.f;
      m_used = mn;
      l_part *= alpha;
      const float nref = (mn == -INFINITY) ? 0.f : -mn * prm.scale_log2;
      float p[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], prm.scale_log2, nref));
        l_part += p[r];
      }
      // k-slot 8 g + i <-> token 4 g + i (i < 4) or 16 + 4 g + (i - 4)
      const bf16x2 a0 = to_bf16x2(p[0], p[1]);
      const bf16x2 a1 = to_bf16x2(p[2], p[3]);
      const bf16x2 a2 = to_bf16x2(p[4], p[5]);
      const bf16x2 a3 = to_bf16x2(p[6], p[7]);
      pbuf[pb][rt][lane] = bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      if (g == 0) alpha_buf[pb][16 * rt + l16] = alpha;
    };

    SvSlot sc = s0;
    SvSlot s1 = next_slot(sc);
    begin_segment(sc.b, sc.L);
    for (int step = 0;; ++step) {
      lds_barrier();  // slot `step` landed (value waves waited); weights of step - 1 read
      if (!sc.valid) break;
      score_slot(ring + (step & 3) * kSlotBytes, sc.j * kPage + sc.h * kSlotTokens, step & 1);
      const bool seg_end = sc.h == 1 && (!s1.valid || s1.b != sc.b);
      if (seg_end) {
        finish_segment(sc.b);
        if (s1.valid) begin_segment(s1.b, s1.L);
      }
      sc = s1;
      s1 = next_slot(s1);
    }
  } else {
    // ================= value waves =================
    const int c = wave - 4;
    const int col_base = c * (kDv / 4);
    // V^T fragment offsets for the transposed read (the value is the first
    // 512 values of the latent): lane (g, l16) reads token rows
    // 4 g + l16 / 4 and 16 + that, matching the weights' k-slot order
    const int vt = 4 * g + (l16 >> 2);
    const int vsw = swz(vt);
    const int ve = (l16 & 3) >> 1;
    int v_off[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      v_off[c4] = vt * kRowBytes + 16 * ((2 * c4 + ve) ^ vsw) + 8 * (l16 & 1);
    // copy k of this wave: LDS chunk 64 k + l of block c of a slot
    int coff[kCopies];
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const int pc = 64 * k + lane;
      const int t = pc / kChunksPerRow;
      const int p = pc - t * kChunksPerRow;
      coff[k] = t * kRowBytes + 16 * (p ^ swz(t));
    }
    const int blk = c * kBlockBytes;
    const char* kvbase = (const char*)kv_ptr;

    f32x4 o[kRT][kCT];  // O^T tiles: row 16 r2 + l16, columns col_base + 16 ct + 4 g + r
    static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
      static_for<0, kCT>([&](auto cc) __attribute__((always_inline)) {
        o[decltype(rc)::value][decltype(cc)::value] = f32x4{0.f, 0.f, 0.f, 0.f};
      });
    });
    int seg_s_lo = split_at(b0);
    int seg_nsplit = split_at(b0 + 1) - seg_s_lo;
    int split_idx = split0;

    // resource of a slot: its page's half h, bounded by the live tokens
    auto slot_rsrc = [&](const SvSlot& s) __attribute__((always_inline)) {
      const int live = slot_live_tokens(s.j, s.h, s.L);
      return sv_rsrc(kvbase + (size_t)s.phys * kTileBytes + s.h * kSlotBytes, live * kRowBytes);
    };
    auto copy_one = [&](MLA_LDS char* buf, i32x4 rs, int k) __attribute__((always_inline)) {
      sv_copy16(buf + blk + 1024 * k, coff[k], rs, blk);
    };

    auto load_v = [&](MLA_LDS char* buf, bf16x8& vf, int ct) __attribute__((always_inline)) {
      const int cta = col_base / 16 + ct;
      const int a = v_off[cta & 3] + 128 * (cta >> 2);
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(buf + a));
      i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(buf + a + 16 * kRowBytes));
      vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // value product of one slot; the nine copies of another go out first,
    // right after the barrier: the earlier they leave, the less of their
    // HBM latency is left to wait for two steps later
    auto value_slot = [&](MLA_LDS char* buf, int pb, MLA_LDS char* cbuf, i32x4 crs, bool cvalid)
                          __attribute__((always_inline)) {
      bf16x8 pw[kRT];
      float al[kRT];
      bool resc = false;
#pragma unroll
      for (int r2 = 0; r2 < kRT; ++r2) {
        pw[r2] = pbuf[pb][r2][lane];
        al[r2] = alpha_buf[pb][16 * r2 + l16];
        resc |= al[r2] != 1.f;
      }
      if (cvalid) {
#pragma unroll
        for (int k = 0; k < kCopies; ++k) copy_one(cbuf, crs, k);
      }
      // the rescale decision before the first value fragments are read: the
      // wait for the factors then covers only them and the weights, which
      // the copies above have given time to arrive
      if (__builtin_amdgcn_ballot_w64(resc) != 0) {
        static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
          constexpr int r2 = decltype(rc)::value;
          static_for<0, kCT>([&](auto cc) __attribute__((always_inline)) {
            o[r2][decltype(cc)::value] *= al[r2];
          });
        });
      }
      constexpr int DV = 3;
      bf16x8 vr[DV + 1];
      static_for<0, DV>([&](auto ic) __attribute__((always_inline)) {
        load_v(buf, vr[decltype(ic)::value], decltype(ic)::value);
      });
      static_for<0, kCT>([&](auto ctc) __attribute__((always_inline)) {
        constexpr int ct = decltype(ctc)::value;
        if constexpr (ct + DV < kCT) load_v(buf, vr[(ct + DV) % (DV + 1)], ct + DV);
        static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
          constexpr int r2 = decltype(rc)::value;
          o[r2][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[ct % (DV + 1)], pw[r2],
                                                              o[r2][ct], 0, 0, 0);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    auto finish_segment = [&](int b) __attribute__((always_inline)) {
      const bool direct = seg_nsplit <= 1;
      const int slot = seg_s_lo + split_idx;
      static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r2 = decltype(rc)::value;
        const int row = row0 + 16 * r2 + l16;
        const float lr = stat_l[16 * r2 + l16];
        const float inv = lr > 0.f ? 1.f / lr : 0.f;
        // tiles 2 p and 2 p + 1 of this row: a lane swap between 16-lane
        // groups leaves lane group g with 8 consecutive columns, 16 (2 p + (g
        // & 1)) + 8 (g >> 1) .. + 7, so each store covers 64 contiguous bytes
        // of a row
        uint16_t* orow = direct ? out_ptr + ((size_t)b * prm.R + row) * kDv + col_base
                                : o_acc + ((size_t)slot * prm.R + row) * kDv + col_base;
        typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
        static_for<0, kCT / 2>([&](auto pc) __attribute__((always_inline)) {
          constexpr int pp = decltype(pc)::value;
          const f32x4 v0 = o[r2][2 * pp] * inv;
          const f32x4 v1 = o[r2][2 * pp + 1] * inv;
          const u32x2 x0 = __builtin_bit_cast(u32x2, bf16x4{to_bf16x2(v0[0], v0[1])[0],
                                                            to_bf16x2(v0[0], v0[1])[1],
                                                            to_bf16x2(v0[2], v0[3])[0],
                                                            to_bf16x2(v0[2], v0[3])[1]});
          const u32x2 x1 = __builtin_bit_cast(u32x2, bf16x4{to_bf16x2(v1[0], v1[1])[0],
                                                            to_bf16x2(v1[0], v1[1])[1],
                                                            to_bf16x2(v1[2], v1[3])[0],
                                                            to_bf16x2(v1[2], v1[3])[1]});
          const u32x2 s0 = __builtin_amdgcn_permlane16_swap(x0[0], x1[0], false, false);
          const u32x2 s1 = __builtin_amdgcn_permlane16_swap(x0[1], x1[1], false, false);
          if (row < prm.R) {
            const int col = 16 * (2 * pp + (g & 1)) + 8 * (g >> 1);
            *(i32x4*)(orow + col) = i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
          }
        });
        static_for<0, kCT>([&](auto cc) __attribute__((always_inline)) {
          o[r2][decltype(cc)::value] = f32x4{0.f, 0.f, 0.f, 0.f};
        });
      });
      split_idx = 0;
    };

    SvSlot sp;  // slot of the value product (one behind the score waves)
    sp.valid = false;
    sp.b = b0;
    SvSlot sc = s0;
    SvSlot s1 = next_slot(sc);
    SvSlot s2 = next_slot(s1);
    SvSlot s3 = next_slot(s2);
    // the first two slots go out before the loop
    {
      const i32x4 r0 = slot_rsrc(sc);
#pragma unroll
      for (int k = 0; k < kCopies; ++k) copy_one(ring, r0, k);
      if (s1.valid) {
        const i32x4 r1 = slot_rsrc(s1);
#pragma unroll
        for (int k = 0; k < kCopies; ++k) copy_one(ring + kSlotBytes, r1, k);
      }
    }
    for (int step = 0;; ++step) {
      // this wave's copies of slot `step` landed (slot step + 1's may fly)
      if (s1.valid)
        sv_fenced_wait<kWaitVm9>();
      else
        sv_fenced_wait<kWaitVm0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (!sc.valid && !sp.valid) break;
      MLA_LDS char* cbuf = ring + ((step + 2) & 3) * kSlotBytes;
      const i32x4 crs = slot_rsrc(s2);
      if (sp.valid) {
        value_slot(ring + ((step - 1) & 3) * kSlotBytes, (step - 1) & 1, cbuf, crs, s2.valid);
        const bool seg_end = sp.h == 1 && (!sc.valid || sc.b != sp.b);
        if (seg_end) {
          finish_segment(sp.b);
          if (sc.valid) {
            seg_s_lo = split_at(sc.b);
            seg_nsplit = split_at(sc.b + 1) - seg_s_lo;
          }
        }
      } else if (s2.valid) {
#pragma unroll
        for (int k = 0; k < kCopies; ++k) copy_one(cbuf, crs, k);
      }
      if (!sc.valid) break;
      sp = sc;
      sc = s1;
      s1 = s2;
      s2 = s3;
      s3 = next_slot(s3);
    }
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_decode_sv64(const mla::DecodeParams* prm, hipStream_t stream) {
  using namespace mla;
  const int groups = (prm->num_parts + 7) / 8;
  const dim3 grid(prm->num_parts >= 8 ? groups * 8 * prm->row_groups
                                      : prm->num_parts * prm->row_groups);
  if (prm->meta)
    hipLaunchKernelGGL(decode_kernel_sv64<false>, grid, dim3(sv::kThreadsSV), 0, stream, *prm,
                       prm->q, prm->kv, prm->block_table, prm->seqlens, prm->meta, prm->splits,
                       prm->out, prm->lse, prm->o_acc, prm->lse_acc);
  else  // schedule inside the launch (batch <= kFusedMaxBatch, checked by the caller)
    hipLaunchKernelGGL(decode_kernel_sv64<true>, grid, dim3(sv::kThreadsSV), 0, stream, *prm,
                       prm->q, prm->kv, prm->block_table, prm->seqlens, prm->meta, prm->splits,
                       prm->out, prm->lse, prm->o_acc, prm->lse_acc);
  return hipGetLastError();
}
