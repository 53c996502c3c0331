// Paged MLA decode for gfx950, workgroups of at most 16 query rows (the
// memory-bound regime: few heads, one query token).
//
// What is computed, and the layouts shared with the other decode kernels,
// are described in mla_decode.hip (FlashMLA release note: MLA principles and
// the paged bf16 cache; DeepSeek-V3 summary: one latent shared by all heads).
//
// With 16 rows there is one row tile, so the four waves split the tokens:
// wave w scores token tile w (tokens 16 w .. 16 w + 15) of every 64-token
// page for all 16 rows (18 MFMA 16x16x32; every K byte of the page is read
// from LDS once).  The four tile maxima of each row meet in LDS, so every
// wave takes the same running max and the same rescale decision and applies
// it to its own accumulators; each wave writes its bf16 weights into its
// 8-byte half of the value product's B-operand slot, and then runs the value
// product of its 128 output columns over the whole page (16 MFMA).  Each
// wave sums its own tokens' weights; the four sums meet at the end.
//
// Page copies and their waits are those of the other 16/32-row kernel: the
// page is double-buffered, the next page's 18 copies per wave go out one per
// k-step of the score product, and the top of a page waits for this wave's
// copies, then a barrier.

#include "mla_decode_common.h"
#include "mla_sched_inlaunch.h"

namespace mla {


namespace t16 {
constexpr int kKS = kD / 32;  // 18 k-steps of the score product
constexpr int kCT = 8;        // 16-column tiles per wave (128 columns)
}  // namespace t16

// FP8 latent cache: per token 512 E4M3 codes, four float32 power-of-two
// scales (one per 128 latent values), the 64 rotary values in bf16.
constexpr int kF8TokenBytes = 656;
constexpr int kF8PageBytes = kPage * kF8TokenBytes;  // 41984 = 41 KiB
constexpr int kF8Copies = kF8PageBytes / 1024;       // 41 wave-wide copies per page

// FP8 page copy k (0 .. 40): a straight copy, lane l moving bytes
// 1024 k + 16 l of the page (the whole offset in voffset, so the range check
// of a resource sized to the live tokens covers it).
__device__ __forceinline__ void f8_copy(MLA_LDS char* buf, __amdgpu_buffer_rsrc_t rs, int k,
                                        int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MLA_LDS void*)(buf + 1024 * k), 16,
                                           1024 * k + 16 * lane, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f8_resource(const char* page, int live) {
  const int n = live < kPage ? live : kPage;
  return __builtin_amdgcn_make_buffer_rsrc((void*)page, (short)0, n * kF8TokenBytes, kBufferFlags);
}

// kFused: no tile_metadata, every workgroup schedules itself.  kFp8: the
// cache holds FP8 records; each page is copied as is into one of two FP8
// buffers and converted into the bf16 tile the products read (the
// dequantized values are exact bf16 values), so everything after the
// conversion is the bf16 kernel.
template <bool kFused, bool kFp8>
__global__ void __launch_bounds__(kThreads, 1)
    decode_kernel_t16(const DecodeParams prm, const uint16_t* __restrict__ q_ptr,
                      const uint16_t* __restrict__ kv_ptr, const int32_t* __restrict__ block_table,
                      const int32_t* __restrict__ seqlens, const int32_t* __restrict__ meta,
                      int32_t* __restrict__ splits, uint16_t* __restrict__ out_ptr,
                      float* __restrict__ lse_ptr, uint16_t* __restrict__ o_acc,
                      float* __restrict__ lse_acc) {
  using namespace t16;
  __shared__ __attribute__((aligned(1024))) char tile0_[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char tile1_[kFp8 ? 2 * kF8PageBytes : kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][64];  // [32-token k-step][lane]
  __shared__ float mx_buf[kWaves][16];                          // [wave][row]: tile max
  __shared__ float stat_l[kWaves][16];                          // [wave][row]: weight sums
  __shared__ std::conditional_t<kFused, InLaunchShared<kThreads>, char> sched_sh;
  MLA_LDS char* tile0 = (MLA_LDS char*)tile0_;
  MLA_LDS char* tile1 = (MLA_LDS char*)tile1_;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);  // wave-uniform: SGPR offsets and M0
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // one partition per workgroup: partitions read disjoint pages (no L2
  // reuse between workgroups), so their placement over the XCDs is left to
  // the dispatcher's round robin
  const int part = blockIdx.x;
  if (part >= prm.num_parts) return;

  int eb, ej, split_idx;
  Item cur;
  int L0 = 0, phys0 = 0;  // in-launch schedule: the first item's length and page

  if constexpr (!kFused) {
    const int32_t* m = meta + part * kMetaInts;
    eb = uni(m[2]);
    ej = uni(m[3]);
    cur = Item{uni(m[0]), uni(m[1])};
    split_idx = uni(m[4]);
  } else {
    // the separate scheduler's cuts, computed by this workgroup
    const InLaunchStart st = schedule_in_launch<kThreads>(
        sched_sh, part, prm.num_parts, prm.batch, prm.sched_c0, prm.max_pages, seqlens,
        block_table, splits, part == 0);
    cur = st.cur;
    eb = st.eb;
    ej = st.ej;
    split_idx = st.split_idx;
    L0 = st.L0;
    phys0 = st.phys0;
  }
  if (!item_before(cur, eb, ej)) return;

  const int col_base = wave * (kDv / kWaves);
  const bool row_live = l16 < prm.R;

  // K fragment (A of the score product): token 16 wave + l16 of the page,
  // logical chunk 4 ks + g at physical (4 ks + g) ^ (token & 7)
  const int sw = l16 & 7;
  const int k_lane = (16 * wave + l16) * kRowBytes + 16 * (g ^ (sw & 3));
  const int k_even = k_lane + ((sw & 4) ? 64 : 0);
  const int k_odd = k_lane - ((sw & 4) ? 64 : 0);
  // V^T fragment (A of the value product) by transposed read
  const int vt = 4 * g + (l16 >> 2);
  const int vsw = swz(vt);
  const int ve = (l16 & 3) >> 1;
  int v_off[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4)
    v_off[c4] = vt * kRowBytes + 16 * ((2 * c4 + ve) ^ vsw) + 8 * (l16 & 1);

  bf16x8 qf[kKS];
  f32x4 o[kCT];  // O^T tiles: row l16, columns col_base + 16 ct + 4 g + r
  float m_used = -INFINITY, l_part = 0.f;  // running max (raw units); own tokens' sum
  int n_vis = 0;
  int L = 0;
  int seg_s_lo = 0, seg_nsplit = 0;

  const char* kvbase = (const char*)kv_ptr;
  PageLoader loader;
  loader.init(lane);

  // load_q: the query rows come by global loads (every segment but the
  // partition's first, whose rows are staged in LDS; see below)
  auto begin_segment = [&](int b, int Lb, bool load_q) __attribute__((always_inline)) {
    L = Lb;
    if constexpr (kFused) {
      seg_s_lo = uni(split_of<kThreads>(sched_sh, b, prm.batch));
      seg_nsplit = uni(split_of<kThreads>(sched_sh, b + 1, prm.batch)) - seg_s_lo;
    } else {
      seg_s_lo = uni(splits[b]);
      seg_nsplit = uni(splits[b + 1]) - seg_s_lo;
    }
    // rows past R read row 0 and are never stored; they see no tokens
    const uint16_t* qrow = q_ptr + ((size_t)b * prm.R + (row_live ? l16 : 0)) * kD + 8 * g;
    if (load_q) static_for<0, kKS>([&](auto kc) __attribute__((always_inline)) {
      qf[decltype(kc)::value] = *(const bf16x8*)(qrow + 32 * decltype(kc)::value);
    });
    const int i = (row_live ? l16 : 0) / prm.h_q;
    int n = prm.causal ? (L - prm.s_q + 1 + i) : L;
    n = n < 0 ? 0 : (n > L ? L : n);
    n_vis = row_live ? n : 0;
    m_used = -INFINITY;
    l_part = 0.f;
    static_for<0, kCT>([&](auto c) __attribute__((always_inline)) {
      o[decltype(c)::value] = f32x4{0.f, 0.f, 0.f, 0.f};
    });
  };

  // all copies of one page into `tile` (bf16) or an FP8 buffer
  auto issue_page = [&](MLA_LDS char* tile, int phys, int live) __attribute__((always_inline)) {
    if constexpr (kFp8) {
      const __amdgpu_buffer_rsrc_t rs = f8_resource(kvbase + (size_t)phys * kF8PageBytes, live);
      for (int k = wave; k < kF8Copies; k += kWaves) f8_copy(tile, rs, k, lane);
    } else {
      loader.issue(tile, kvbase + (size_t)phys * kTileBytes, live, wave);
    }
  };
  auto load_item = [&](MLA_LDS char* tile, Item it) __attribute__((always_inline)) -> bool {
    const int L_it = uni(seqlens[it.b]);
    if (it.j * kPage >= L_it) return false;
    const int phys = uni(block_table[(size_t)it.b * prm.max_pages + it.j]);
    issue_page(tile, phys, L_it - it.j * kPage);
    return true;
  };

  auto next_copy = [&](MLA_LDS char* tile, Item it, bool has) __attribute__((always_inline)) {
    PendingCopy cp;
    cp.tile = tile;
    cp.valid = false;
    cp.rsrc = PageLoader::resource(kvbase, 0);
    if (has) {
      const int L_it = uni(seqlens[it.b]);
      if (it.j * kPage < L_it) {
        const int phys = uni(block_table[(size_t)it.b * prm.max_pages + it.j]);
        if constexpr (kFp8)
          cp.rsrc = f8_resource(kvbase + (size_t)phys * kF8PageBytes, L_it - it.j * kPage);
        else
          cp.rsrc = PageLoader::resource(kvbase + (size_t)phys * kTileBytes, L_it - it.j * kPage);
        cp.valid = true;
      }
    }
    return cp;
  };

  // next item after `it` of the current sequence (whose length is L)
  auto advance = [&](Item it) __attribute__((always_inline)) {
    Item nx = it;
    const int n_slots = (L + kPage - 1) / kPage;
    if (it.j + 1 < (n_slots > 0 ? n_slots : 1)) {
      nx.j = uni(it.j + 1);
    } else {
      nx.b = uni(it.b + 1);
      nx.j = 0;
    }
    return nx;
  };

  // V^T fragment ct (16 columns x 32 tokens 32 kk ..) by transposed reads
  auto load_v = [&](MLA_LDS char* tile, int kk, bf16x8& vf, int ct) __attribute__((always_inline)) {
    const int cta = col_base / 16 + ct;
    const int a = v_off[cta & 3] + 128 * (cta >> 2) + kk * 32 * kRowBytes;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a + 16 * kRowBytes));
    vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One page: scores of this wave's token tile, max exchange, softmax,
  // weights to LDS, value product of this wave's 128 columns.
  auto compute_page = [&](MLA_LDS char* tile, int j, const PendingCopy& cp)
                          __attribute__((always_inline)) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    auto load_k = [&](int ks) __attribute__((always_inline)) {
      return *(MLA_LDS bf16x8*)(tile + ((ks & 1) ? k_odd : k_even) + 64 * ks);
    };
    constexpr int DK = 6;  // K fragments in flight ahead of their product
    bf16x8 kr[DK + 1];
    static_for<0, DK>([&](auto ic) __attribute__((always_inline)) {
      kr[decltype(ic)::value] = load_k(decltype(ic)::value);
    });
    static_for<0, kKS>([&](auto ksc) __attribute__((always_inline)) {
      constexpr int ks = decltype(ksc)::value;
      if constexpr (ks + DK < kKS) kr[(ks + DK) % (DK + 1)] = load_k(ks + DK);
      // the next page's copy instructions, one per k-step (18 per wave for
      // a bf16 page; 11 or 10 of the 41 for an FP8 page)
      static_assert(kKS == kLoadsPerWave, "one copy per k-step");
      if constexpr (kFp8) {
        if constexpr (kWaves * ks < kF8Copies + kWaves) {
          if (cp.valid && wave + kWaves * ks < kF8Copies)
            f8_copy(cp.tile, cp.rsrc, wave + kWaves * ks, lane);
        }
      } else {
        if (cp.valid) loader.issue_one(cp.tile, cp.rsrc, wave, ks);
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (DK + 1)], qf[ks], s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // ---- tile max (raw score units; the scale is positive), shared
    const int tok0 = j * kPage + 16 * wave + 4 * g;
    float x[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (tok0 + r < n_vis) ? s[r] : -INFINITY;
      mt = fmaxf(mt, x[r]);
    }
    mt = wave_max_x4(mt);
    if (g == 0) mx_buf[wave][l16] = mt;
    // the first V^T fragments do not depend on the weights
    constexpr int DV = 4;
    bf16x8 vr[DV + 1];
    static_for<0, DV>([&](auto ic) __attribute__((always_inline)) {
      constexpr int u = decltype(ic)::value;  // fragment u: column tile u / 2, k-step u % 2
      load_v(tile, u % 2, vr[u], u / 2);
    });
    lds_barrier();
    const float mx = fmaxf(fmaxf(mx_buf[0][l16], mx_buf[1][l16]),
                           fmaxf(mx_buf[2][l16], mx_buf[3][l16]));
    // ---- online softmax (log2 domain): every wave sees the same mx and
    //      m_used, so every wave takes the same decision
    const bool upd = __builtin_amdgcn_ballot_w64((mx - m_used) * prm.scale_log2 >
                                                 kRescaleThreshold) != 0;
    const float mn = upd ? fmaxf(m_used, mx) : m_used;
    const float alpha = (upd && mn != -INFINITY)
                            ? __builtin_amdgcn_exp2f((m_used - mn) * prm.scale_log2)
                            : 1.f;
    m_used = mn;
    l_part *= alpha;
    const float nref = (mn == -INFINITY) ? 0.f : -mn * prm.scale_log2;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], prm.scale_log2, nref));
      l_part += p[r];
    }
    // k-step kk = wave / 2 of the value product; k-slot 8g + 4 (wave & 1) + r
    // <-> token 32 kk + 16 (wave & 1) + 4g + r: this wave's half of the slot
    const bf16x2 a0 = to_bf16x2(p[0], p[1]);
    const bf16x2 a1 = to_bf16x2(p[2], p[3]);
    *(MLA_LDS bf16x4*)((MLA_LDS char*)&pbuf[wave >> 1][lane] + 8 * (wave & 1)) =
        bf16x4{a0[0], a0[1], a1[0], a1[1]};
    if (upd) {
      static_for<0, kCT>([&](auto c) __attribute__((always_inline)) {
        o[decltype(c)::value] *= alpha;
      });
    }
    lds_barrier();
    // ---- value product: all 16 rows, this wave's 128 columns, 64 tokens
    const bf16x8 pb0 = pbuf[0][lane];
    const bf16x8 pb1 = pbuf[1][lane];
    static_for<0, 2 * kCT>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;  // column tile u / 2, k-step u % 2
      if constexpr (u + DV < 2 * kCT) load_v(tile, (u + DV) % 2, vr[(u + DV) % (DV + 1)], (u + DV) / 2);
      o[u / 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[u % (DV + 1)], (u % 2) ? pb1 : pb0,
                                                         o[u / 2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto finish_segment = [&](int b) __attribute__((always_inline)) {
    const bool direct = seg_nsplit <= 1;
    const int slot = seg_s_lo + split_idx;
    const float lw = wave_sum_x4(l_part);
    if (g == 0) stat_l[wave][l16] = lw;
    lds_barrier();
    const float lt = (stat_l[0][l16] + stat_l[1][l16]) + (stat_l[2][l16] + stat_l[3][l16]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row_live) {
      if (wave == 0 && g == 0) {
        const float lse2 = lt > 0.f ? m_used * prm.scale_log2 + __builtin_amdgcn_logf(lt) : -INFINITY;
        if (direct)
          lse_ptr[(size_t)b * prm.R + l16] = lse2 * kLn2;
        else
          lse_acc[(size_t)slot * prm.R + l16] = lse2;
      }
      // 16 bytes per lane: lanes g and g ^ 1 (lane ^ 16, the same row) swap
      // halves so that the even one holds 8 columns of tile c and the odd
      // one 8 columns of tile c + 1
      uint16_t* orow = direct ? out_ptr + ((size_t)b * prm.R + l16) * kDv + col_base
                              : o_acc + ((size_t)slot * prm.R + l16) * kDv + col_base;
      const bool even = (g & 1) == 0;
      static_for<0, kCT / 2>([&](auto pc) __attribute__((always_inline)) {
        constexpr int c = 2 * decltype(pc)::value;
        const f32x4 va = o[c] * inv;
        const f32x4 vb = o[c + 1] * inv;
        const int a0 = __builtin_bit_cast(int, to_bf16x2(va[0], va[1]));
        const int a1 = __builtin_bit_cast(int, to_bf16x2(va[2], va[3]));
        const int b0 = __builtin_bit_cast(int, to_bf16x2(vb[0], vb[1]));
        const int b1 = __builtin_bit_cast(int, to_bf16x2(vb[2], vb[3]));
        const int r0 = __shfl_xor(even ? b0 : a0, 16);
        const int r1 = __shfl_xor(even ? b1 : a1, 16);
        const i32x4 w = even ? i32x4{a0, a1, r0, r1} : i32x4{r0, r1, b0, b1};
        *(i32x4*)(orow + (even ? 16 * c + 4 * g : 16 * (c + 1) + 4 * (g - 1))) = w;
      });
    }
    split_idx = 0;  // later sequences of this partition start at their page 0
  };

  // FP8 page (64 records of 656 bytes) -> the bf16 tile: item (t, c) is
  // 16-byte chunk c of token t, 8 latent values converted with their
  // block's scale (exact: the scale is a power of two) or 8 rotary values
  // copied; stored at the tile's swizzled chunk c ^ (t & 7).  Tokens past
  // the live ones arrived as zeros and convert to zeros.
  auto convert_page = [&](MLA_LDS char* f8) __attribute__((always_inline)) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
#pragma unroll 6
    for (int u = 0; u < kPage * kChunksPerRow / kThreads; ++u) {  // 18
      const int i = threadIdx.x + kThreads * u;
      const int t = i / kChunksPerRow;
      const int c = i - kChunksPerRow * t;
      MLA_LDS char* rec = f8 + t * kF8TokenBytes;
      i32x4 v;
      if (c < kDv / 8) {
        const i32x2 w = *(MLA_LDS i32x2*)(rec + 8 * c);
        const float sc = *(MLA_LDS float*)(rec + kDv + 4 * (c >> 4));
        const bf2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], sc, false);
        const bf2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], sc, true);
        const bf2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], sc, false);
        const bf2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], sc, true);
        v = i32x4{__builtin_bit_cast(int, a0), __builtin_bit_cast(int, a1),
                  __builtin_bit_cast(int, a2), __builtin_bit_cast(int, a3)};
      } else {
        v = *(MLA_LDS i32x4*)(rec + kDv + 16 + 16 * (c - kDv / 8));
      }
      *(MLA_LDS i32x4*)(tile0 + t * kRowBytes + 16 * (c ^ swz(t))) = v;
    }
  };

  // One step: compute `cur` from tile A while the next page streams into B.
  // kFirst: the partition's first step, whose query rows wait in B (staged
  // there with the first page's copies): read into registers, then one more
  // barrier before the next page's copies overwrite B
  auto step = [&](MLA_LDS char* tA, MLA_LDS char* tB, auto first_c) __attribute__((always_inline))
      -> bool {
    constexpr bool kFirst = decltype(first_c)::value;
    const Item nx = advance(cur);
    const bool has_next = item_before(nx, eb, ej);
    // descriptor of the next copy first: its scalar loads (block table and
    // lengths, never written here) overlap the wait below
    PendingCopy cp = next_copy(tB, nx, has_next);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's part of tile A landed
    __syncthreads();                       // ... and every wave's; B is free
    if constexpr (kFirst) {
      // row l16 of the staged query, in the page layout: the K fragment's
      // addressing with token l16
      const int q_lane = l16 * kRowBytes + 16 * (g ^ (sw & 3));
      const int q_even = q_lane + ((sw & 4) ? 64 : 0);
      const int q_odd = q_lane - ((sw & 4) ? 64 : 0);
      static_for<0, kKS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int ks = decltype(kc)::value;
        qf[ks] = *(MLA_LDS bf16x8*)(tB + ((ks & 1) ? q_odd : q_even) + 64 * ks);
      });
      lds_barrier();
    }
    if (cur.j * kPage < L) {
      if constexpr (kFp8) {
        convert_page(tA);  // A (FP8) -> the bf16 tile, free since the barrier
        __syncthreads();
        compute_page(tile0, cur.j, cp);
      } else {
        compute_page(tA, cur.j, cp);
      }
    } else if (cp.valid) {
      if constexpr (kFp8) {
        for (int k = wave; k < kF8Copies; k += kWaves) f8_copy(cp.tile, cp.rsrc, k, lane);
      } else {
        for (int i = 0; i < kLoadsPerWave; ++i) loader.issue_one(cp.tile, cp.rsrc, wave, i);
      }
    }
    if (!has_next || nx.b != cur.b) {
      finish_segment(cur.b);
      if (has_next) begin_segment(nx.b, uni(seqlens[nx.b]), true);
    }
    cur = nx;
    return has_next;
  };

  // page buffers: the two bf16 tiles, or two FP8 buffers (the bf16 tile
  // then only receives conversions)
  MLA_LDS char* bufA = kFp8 ? tile1 : tile0;
  MLA_LDS char* bufB = kFp8 ? tile1 + kF8PageBytes : tile1;
  // The first segment's query rows (R <= 16, rows past R arrive as zeros
  // and see no tokens) are staged in B by two waves' 9 copies each, in the
  // page layout, instead of 18 global loads in every wave: a quarter of the
  // bytes through the CU's address path ahead of the first page.
  {
    const __amdgpu_buffer_rsrc_t qrs =
        PageLoader::resource((const char*)(q_ptr + (size_t)cur.b * prm.R * kD), prm.R);
    if (wave < 2) {
#pragma unroll
      for (int i = 0; i < 9; ++i) loader.issue_one(bufB, qrs, wave, i);
    }
  }
  if constexpr (kFused) {
    // length and page of the first item were read with the schedule
    begin_segment(cur.b, L0, false);
    if (cur.j * kPage < L0) issue_page(bufA, phys0, L0 - cur.j * kPage);
  } else {
    begin_segment(cur.b, uni(seqlens[cur.b]), false);
    load_item(bufA, cur);
  }
  if (step(bufA, bufB, std::true_type{})) {
    while (true) {
      if (!step(bufB, bufA, std::false_type{})) break;
      if (!step(bufA, bufB, std::false_type{})) break;
    }
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_decode_t16(const mla::DecodeParams* prm, hipStream_t stream) {
  using namespace mla;
  const int groups = (prm->num_parts + 7) / 8;
  if (prm->meta != nullptr)
    hipLaunchKernelGGL((decode_kernel_t16<false, false>), dim3(groups * 8), dim3(kThreads), 0, stream, *prm,
                       prm->q, prm->kv, prm->block_table, prm->seqlens, prm->meta,
                       prm->splits, prm->out, prm->lse, prm->o_acc, prm->lse_acc);
  else  // schedule inside the launch (batch <= kFusedMaxBatch, checked by the caller)
    hipLaunchKernelGGL((decode_kernel_t16<true, false>), dim3(groups * 8), dim3(kThreads), 0, stream, *prm,
                       prm->q, prm->kv, prm->block_table, prm->seqlens, prm->meta,
                       prm->splits, prm->out, prm->lse, prm->o_acc, prm->lse_acc);
  return hipGetLastError();
}

// FP8 latent cache (<= 16 rows per sequence; tile_metadata required: the two
// FP8 buffers and the bf16 tile leave no LDS for the in-launch schedule).
extern "C" hipError_t mla_launch_decode_t16_fp8(const mla::DecodeParams* prm, hipStream_t stream) {
  using namespace mla;
  if (prm->meta == nullptr) return hipErrorInvalidValue;
  const int groups = (prm->num_parts + 7) / 8;
  hipLaunchKernelGGL((decode_kernel_t16<false, true>), dim3(groups * 8), dim3(kThreads), 0, stream,
                     *prm, prm->q, prm->kv, prm->block_table, prm->seqlens, prm->meta,
                     prm->splits, prm->out, prm->lse, prm->o_acc, prm->lse_acc);
  return hipGetLastError();
}
