// Paged MLA decode, 64 query rows per workgroup of 8 waves (two per SIMD).
//
// What is computed, and the layouts shared with the other decode kernels,
// are described in mla_decode.hip (FlashMLA release note: MLA principles and
// the paged bf16 cache; DeepSeek-V3 summary: one latent shared by all heads).
//
// With one wave per SIMD a wave's own softmax, LDS waits and barriers leave
// the matrix core idle: a wave hides only about two VALU instructions behind
// each of its MFMAs.  Here every SIMD runs two waves, so one wave's softmax
// and LDS latency overlap the other's matrix instructions.  The price is a
// register budget of 256 per wave, which sets the split of the work:
//
//   score product  wave w = (row tile rt = w & 3, token tile th = w >> 2):
//                  S^T for the 16 tokens 16 th .. of each 32-token half and
//                  the 16 query rows 16 rt .. (18 MFMA 16x16x32 per half);
//   softmax        the two waves holding the same rows (w, w ^ 4) exchange
//                  their 16-token row maxima through LDS, so both take the
//                  same running max and the same rescale decision; each sums
//                  its own tokens' weights;
//   weights        each wave writes its 4 bf16 weights per lane into its
//                  8-byte half of the value product's B-operand slot;
//   value product  wave w owns output columns 64 w .. 64 w + 63 for all 64
//                  rows (16 MFMA 16x16x32 per half, 64 accumulator registers).
//
// Each wave copies one 8-token block of every page (9 wave-wide 1 KiB
// buffer loads into LDS, resource bounded by the live tokens).  A CU moves
// only about 50 B/clk into LDS, so a page costs about 1,500 cycles of copy
// time, and a wave whose copy instruction finds the queue full stalls; the
// next page's nine copies are therefore spread over the first half of the
// current page, one every four matrix instructions, which leaves the second
// half for them to land.  The top of a page waits for this wave's copies,
// then a barrier.

#include "mla_decode_common.h"

namespace mla {

namespace s8 {
constexpr int kWaves8 = 8;
constexpr int kThreads8 = 64 * kWaves8;
constexpr int kRows = 64;
constexpr int kRT = 4;               // 16-row tiles of the workgroup
constexpr int kCT = 4;               // 16-column tiles per wave (64 columns)
constexpr int kKS = kD / 32;         // 18 k-steps of the score product
constexpr int kCopies = 9;           // per wave and page: one 8-token block
}  // namespace s8

__global__ void __launch_bounds__(s8::kThreads8, 1)
    decode_kernel_split8(const DecodeParams prm, const uint16_t* __restrict__ q_ptr,
                         const uint16_t* __restrict__ kv_ptr,
                         const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ seqlens, const int32_t* __restrict__ meta,
                         const int32_t* __restrict__ splits, uint16_t* __restrict__ out_ptr,
                         float* __restrict__ lse_ptr, float* __restrict__ o_acc,
                         float* __restrict__ lse_acc) {
  using namespace s8;
  __shared__ __attribute__((aligned(1024))) char tile0_[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char tile1_[kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][kRT][64];  // [half][row tile][lane]
  __shared__ float alpha_buf[2][kRows];   // [half][row]: rescale factor of the row
  __shared__ float mx_buf[2][kWaves8][16];  // [half][wave][row in tile]: 16-token row max
  __shared__ float stat_l[2][kRows];      // [token tile][row]: softmax sums at segment end
  MLA_LDS char* tile0 = (MLA_LDS char*)tile0_;
  MLA_LDS char* tile1 = (MLA_LDS char*)tile1_;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int rt = wave & 3;   // row tile this wave scores
  const int th = wave >> 2;  // token tile (of each half) this wave scores

  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int rr = bid >> 3;
  const int rg = rr % prm.row_groups;
  const int part = (rr / prm.row_groups) * 8 + xcd;
  if (part >= prm.num_parts) return;

  const int32_t* m = meta + part * kMetaInts;
  const int eb = uni(m[2]), ej = uni(m[3]);
  Item cur = {uni(m[0]), uni(m[1])};
  if (!item_before(cur, eb, ej)) return;
  int split_idx = uni(m[4]);

  const int row0 = rg * kRows;
  const int qk_row = row0 + 16 * rt + l16;  // the row this lane scores
  const int col_base = wave * (kDv / kWaves8);

  // K fragment offsets (token 16 th + l16 of a half, logical chunk 4 ks + g)
  const int sw = l16 & 7;
  const int k_lane = (16 * th + l16) * kRowBytes + 16 * (g ^ (sw & 3));
  const int k_even = k_lane + ((sw & 4) ? 64 : 0);
  const int k_odd = k_lane - ((sw & 4) ? 64 : 0);
  // V^T fragment offsets for the transposed read
  const int vt = 4 * g + (l16 >> 2);
  const int vsw = swz(vt);
  const int ve = (l16 & 3) >> 1;
  int v_off[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4)
    v_off[c4] = vt * kRowBytes + 16 * ((2 * c4 + ve) ^ vsw) + 8 * (l16 & 1);

  bf16x8 qf[kKS];       // this lane's scoring row, 8 features per k-step
  f32x4 o[kRT][kCT];    // O^T tiles: row 16 rt' + l16, columns col_base + 16 ct + 4 g + r
  float m_used = -INFINITY, l_part = 0.f;  // running max (raw units); own tokens' sum
  int n_vis = 0;
  int L = 0;
  int seg_s_lo = 0, seg_nsplit = 0;

  const char* kvbase = (const char*)kv_ptr;
  // copy k (0..8) of this wave: LDS chunk 64 k + l of block `wave`
  int coff[kCopies];
#pragma unroll
  for (int k = 0; k < kCopies; ++k) {
    const int pc = 64 * k + lane;
    const int t = pc / kChunksPerRow;
    const int p = pc - t * kChunksPerRow;
    coff[k] = t * kRowBytes + 16 * (p ^ swz(t));
  }
  const int blk = wave * 8 * kRowBytes;  // this wave's 8-token block, 9216 B
  auto issue_copy = [&](MLA_LDS char* tile, __amdgpu_buffer_rsrc_t rs, int k)
                        __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MLA_LDS void*)(tile + blk + 1024 * k), 16,
                                             coff[k], blk, 0, 0);
  };

  auto begin_segment = [&](int b) __attribute__((always_inline)) {
    L = uni(seqlens[b]);
    seg_s_lo = uni(splits[b]);
    seg_nsplit = uni(splits[b + 1]) - seg_s_lo;
    const bool live = qk_row < prm.R;
    // rows past R read row 0 and are never stored; they see no tokens
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
    static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
      static_for<0, kCT>([&](auto cc) __attribute__((always_inline)) {
        o[decltype(rc)::value][decltype(cc)::value] = f32x4{0.f, 0.f, 0.f, 0.f};
      });
    });
  };

  auto load_item = [&](MLA_LDS char* tile, Item it) __attribute__((always_inline)) -> bool {
    const int L_it = uni(seqlens[it.b]);
    if (it.j * kPage >= L_it) return false;
    const int phys = uni(block_table[(size_t)it.b * prm.max_pages + it.j]);
    const __amdgpu_buffer_rsrc_t rs =
        PageLoader::resource(kvbase + (size_t)phys * kTileBytes, L_it - it.j * kPage);
#pragma unroll
    for (int k = 0; k < kCopies; ++k) issue_copy(tile, rs, k);
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

  // V^T fragment ct (16 columns x 32 tokens of half h) by transposed reads
  auto load_v = [&](MLA_LDS char* tile, int h, bf16x8& vf, int ct) __attribute__((always_inline)) {
    const int cta = col_base / 16 + ct;
    const int a = v_off[cta & 3] + 128 * (cta >> 2) + h * 32 * kRowBytes;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a + 16 * kRowBytes));
    vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One 32-token half of a page: scores of this wave's tile, max exchange,
  // softmax, weights to LDS, value product of this wave's 64 columns.
  auto compute_half = [&](MLA_LDS char* tile, int j, auto hc, const PendingCopy& cp)
                          __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
    // ---- scores: tokens 32 h + 16 th + (0..15), rows 16 rt + (0..15)
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    auto load_k = [&](int ks) __attribute__((always_inline)) {
      return *(MLA_LDS bf16x8*)(tile + ((ks & 1) ? k_odd : k_even) + 64 * ks +
                                h * 32 * kRowBytes);
    };
    constexpr int DK = 6;
    bf16x8 kr[DK + 1];
    static_for<0, DK>([&](auto ic) __attribute__((always_inline)) {
      kr[decltype(ic)::value] = load_k(decltype(ic)::value);
    });
    static_for<0, kKS>([&](auto ksc) __attribute__((always_inline)) {
      constexpr int ks = decltype(ksc)::value;
      if constexpr (ks + DK < kKS) kr[(ks + DK) % (DK + 1)] = load_k(ks + DK);
      // the next page's nine copies go out during the first half page:
      // k-steps 0, 4, 8, 12, 16 of its score product and the first four
      // column tiles of its value product
      if constexpr (h == 0 && ks % 4 == 0)
        if (cp.valid) issue_copy(cp.tile, cp.rsrc, ks / 4);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (DK + 1)], qf[ks], s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // ---- 16-token row max of this wave's tile (raw score units), shared
    //      with the wave holding the other token tile of the same rows
    const int tok0 = j * kPage + 32 * h + 16 * th + 4 * g;
    float x[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (tok0 + r < n_vis) ? s[r] : -INFINITY;
      mt = fmaxf(mt, x[r]);
    }
    mt = wave_max_x4(mt);
    if (g == 0) mx_buf[h][wave][l16] = mt;
    // the first V^T fragments do not depend on the weights
    constexpr int DV = 3;
    bf16x8 vr[DV + 1];
    static_for<0, DV>([&](auto ic) __attribute__((always_inline)) {
      load_v(tile, h, vr[decltype(ic)::value], decltype(ic)::value);
    });
    lds_barrier();
    const float mx = fmaxf(mt, mx_buf[h][wave ^ 4][l16]);
    // ---- online softmax (log2 domain); both waves of the pair see the same
    //      mx and m_used, so they take the same decision
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
    // k-slot 8g + 4 th + r <-> token 32h + 16 th + 4g + r: this wave's half of
    // the 16-byte B-operand slot of row tile rt
    const bf16x2 a0 = to_bf16x2(p[0], p[1]);
    const bf16x2 a1 = to_bf16x2(p[2], p[3]);
    *(MLA_LDS bf16x4*)((MLA_LDS char*)&pbuf[h][rt][lane] + 8 * th) = bf16x4{a0[0], a0[1], a1[0], a1[1]};
    if (th == 0 && g == 0) alpha_buf[h][16 * rt + l16] = alpha;
    lds_barrier();
    // ---- value product: all 64 rows, this wave's 64 columns
    bf16x8 pb[kRT];
    float al[kRT];
    bool resc = false;
#pragma unroll
    for (int r2 = 0; r2 < kRT; ++r2) {
      pb[r2] = pbuf[h][r2][lane];
      al[r2] = alpha_buf[h][16 * r2 + l16];
      resc |= al[r2] != 1.f;
    }
    if (__builtin_amdgcn_ballot_w64(resc) != 0) {
      static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r2 = decltype(rc)::value;
        static_for<0, kCT>([&](auto cc) __attribute__((always_inline)) {
          o[r2][decltype(cc)::value] *= al[r2];
        });
      });
    }
    static_for<0, kCT>([&](auto ctc) __attribute__((always_inline)) {
      constexpr int ct = decltype(ctc)::value;
      if constexpr (ct + DV < kCT) load_v(tile, h, vr[(ct + DV) % (DV + 1)], ct + DV);
      if constexpr (h == 0 && ct < 4)
        if (cp.valid) issue_copy(cp.tile, cp.rsrc, 5 + ct);
      static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r2 = decltype(rc)::value;
        o[r2][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[ct % (DV + 1)], pb[r2], o[r2][ct],
                                                            0, 0, 0);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto finish_segment = [&](int b) __attribute__((always_inline)) {
    const bool direct = seg_nsplit <= 1;
    const int slot = seg_s_lo + split_idx;
    // each scoring wave publishes its tokens' sum; the pair's sums add up
    const float lw = wave_sum_x4(l_part);
    if (g == 0) stat_l[th][16 * rt + l16] = lw;
    lds_barrier();
    if (th == 0 && g == 0 && qk_row < prm.R) {
      const float lt = lw + stat_l[1][16 * rt + l16];
      const float lse2 = lt > 0.f ? m_used * prm.scale_log2 + __builtin_amdgcn_logf(lt) : -INFINITY;
      if (direct)
        lse_ptr[(size_t)b * prm.R + qk_row] = lse2 * kLn2;
      else
        lse_acc[(size_t)slot * prm.R + qk_row] = lse2;
    }
    static_for<0, kRT>([&](auto rc) __attribute__((always_inline)) {
      constexpr int r2 = decltype(rc)::value;
      const int row = row0 + 16 * r2 + l16;
      const float lr = stat_l[0][16 * r2 + l16] + stat_l[1][16 * r2 + l16];
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      if (row < prm.R) {
        if (direct) {
          uint16_t* orow = out_ptr + ((size_t)b * prm.R + row) * kDv + col_base + 4 * g;
          static_for<0, kCT>([&](auto cc) __attribute__((always_inline)) {
            constexpr int ct = decltype(cc)::value;
            const f32x4 v = o[r2][ct] * inv;
            const bf16x2 a = to_bf16x2(v[0], v[1]);
            const bf16x2 c = to_bf16x2(v[2], v[3]);
            *(bf16x4*)(orow + 16 * ct) = bf16x4{a[0], a[1], c[0], c[1]};
          });
        } else {
          float* orow = o_acc + ((size_t)slot * prm.R + row) * kDv + col_base + 4 * g;
          static_for<0, kCT>([&](auto cc) __attribute__((always_inline)) {
            constexpr int ct = decltype(cc)::value;
            *(f32x4*)(orow + 16 * ct) = o[r2][ct] * inv;
          });
        }
      }
    });
    split_idx = 0;  // later sequences of this partition start at their page 0
    // stat_l is rewritten at the next segment end only after that
    // segment's page barriers
  };

  // One step: compute `cur` from tile A while the next page streams into B.
  auto step = [&](MLA_LDS char* tA, MLA_LDS char* tB) __attribute__((always_inline)) -> bool {
    const Item nx = advance(cur);
    const bool has_next = item_before(nx, eb, ej);
    PendingCopy cp = next_copy(tB, nx, has_next);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's block of tile A landed
    __syncthreads();                       // ... and every wave's; B is free
    const bool has_tokens = cur.j * kPage < L;
    if (has_tokens) {
      compute_half(tA, cur.j, std::integral_constant<int, 0>{}, cp);
      compute_half(tA, cur.j, std::integral_constant<int, 1>{}, cp);
    } else if (cp.valid) {
      for (int k = 0; k < kCopies; ++k) issue_copy(cp.tile, cp.rsrc, k);
    }
    if (!has_next || nx.b != cur.b) {
      finish_segment(cur.b);
      if (has_next) begin_segment(nx.b);
    }
    cur = nx;
    return has_next;
  };

  begin_segment(cur.b);
  load_item(tile0, cur);
  while (true) {
    if (!step(tile0, tile1)) break;
    if (!step(tile1, tile0)) break;
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_decode_split8(const mla::DecodeParams* prm, hipStream_t stream) {
  using namespace mla;
  const int groups = (prm->num_parts + 7) / 8;
  const dim3 grid(groups * 8 * prm->row_groups);
  hipLaunchKernelGGL(decode_kernel_split8, grid, dim3(s8::kThreads8), 0, stream, *prm, prm->q,
                     prm->kv, prm->block_table, prm->seqlens, prm->meta, prm->splits, prm->out,
                     prm->lse, prm->o_acc, prm->lse_acc);
  return hipGetLastError();
}
