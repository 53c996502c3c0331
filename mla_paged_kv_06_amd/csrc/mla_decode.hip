// Paged MLA decode for gfx950 (CDNA4): page gather -> LDS, S^T = K Q^T and
// O^T += V^T P^T on bf16 MFMA, online softmax in registers.
//
// What is computed (FlashMLA release note, paragraphs on MLA core principles
// and on the released paged bf16 cache; DeepSeek-V3 hardware paper summary,
// paragraph on memory efficiency): every query head attends over one shared
// 576-value latent per token, the first 512 values of which are the value.
// Because all heads read the same latent, the score and value products of a
// page are dense contractions with one row per (query token, head) -- the
// work that goes on the matrix cores.  The exact-softmax tiling with a
// running max and sum follows the FlashAttention line the release note's
// acknowledgements name; the layout below is our own for CDNA4.
//
// Workgroup = 4 waves (256 threads), one per SIMD; one workgroup per CU
// (two 72 KiB page buffers fill most of the 160 KiB LDS).
//
// Per page (64 tokens) and wave:
//   * the page is copied HBM -> LDS by global_load_lds (16 B per lane, 72
//     wave-wide loads split over the 4 waves), double-buffered: page k+1 is
//     in flight while page k is computed;
//   * S^T[token][row] = sum_d K[token][d] Q[row][d]: MFMA 16x16x32 with the
//     K tile (LDS, 16-byte reads) as A and the query rows (registers, loaded
//     once per sequence) as B.  The accumulator gives each lane one query row
//     (lane % 16) and 16 tokens, so the row max / sum needs only a 4-lane
//     reduction and the weights are already laid out as the B operand of the
//     next product;
//   * O^T[col][row] += sum_t V[t][col] P[row][t]: MFMA 16x16x32 with V^T read
//     by ds_read_b64_tr_b16 straight from the same LDS tile (the value is the
//     first 512 values of the latent) and the bf16 weights as B.  Each lane
//     again holds one query row, so the rescale of O is a per-lane scalar.
//
// Variants (query rows per workgroup; waves as row groups x column groups):
//   16 rows: 1 x 4, each wave all 16 rows and 128 output columns;
//   32 rows: 1 x 4, each wave all 32 rows (two 16-row tiles) and 128 columns;
//   64 rows: 2 x 2, each wave 32 rows and 256 columns.
// Waves of one row group repeat its score product (cheap next to the LDS
// traffic it saves): every K fragment read serves 32 rows, and each wave
// reads only its columns of V^T, whose transposed reads are the slowest LDS
// access on gfx950 (about 85 B/clk per CU against 200 B/clk for ds_read_b128).

#include "mla_decode_common.h"
#include "mla_sched_inlaunch.h"

namespace mla {


template <int RT, int RGW, int CGW>
struct Variant {
  static constexpr int kRT = RT;                 // 16-row tiles per wave
  static constexpr int kRows = 16 * RT * RGW;    // rows per workgroup
  static constexpr int kColsPerWave = kDv / CGW;
  static constexpr int kCT = kColsPerWave / 16;  // 16-column output tiles per wave
  static constexpr int kKS = kD / 32;            // 18 k-steps of the score product
};

// kFused: no tile_metadata; every workgroup computes the schedule itself.
template <int RT, int RGW, int CGW, bool kFused>
__global__ void __launch_bounds__(kThreads, 1)
    decode_kernel(const DecodeParams prm, const uint16_t* __restrict__ q_ptr,
                  const uint16_t* __restrict__ kv_ptr, const int32_t* __restrict__ block_table,
                  const int32_t* __restrict__ seqlens, const int32_t* __restrict__ meta,
                  int32_t* __restrict__ splits, uint16_t* __restrict__ out_ptr,
                  float* __restrict__ lse_ptr, uint16_t* __restrict__ o_acc,
                  float* __restrict__ lse_acc) {
  using V = Variant<RT, RGW, CGW>;
  constexpr int CT = V::kCT;
  constexpr int KS = V::kKS;

  __shared__ __attribute__((aligned(1024))) char tile0_[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char tile1_[kTileBytes];
  __shared__ std::conditional_t<kFused, InLaunchShared<kThreads>, char> sched_sh;
  MLA_LDS char* tile0 = (MLA_LDS char*)tile0_;
  MLA_LDS char* tile1 = (MLA_LDS char*)tile1_;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);  // wave-uniform: SGPR offsets and M0
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wr = wave % RGW;  // row sub-group of this wave
  const int wc = wave / RGW;  // column group of this wave

  // XCD-aware mapping: workgroups of the same partition (its row groups)
  // share blockIdx % 8 and so land on the same XCD and read its pages
  // through the same L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int rr = bid >> 3;
  const int rg = rr % prm.row_groups;
  const int part = (rr / prm.row_groups) * 8 + xcd;
  if (part >= prm.num_parts) return;

  int eb, ej, split_idx;
  Item cur;
  int L0 = 0, phys0 = 0;  // in-launch schedule: the first item's length and page
  if constexpr (kFused) {
    // the separate scheduler's cuts, computed by this workgroup
    const InLaunchStart st =
        schedule_in_launch<kThreads>(sched_sh, part, prm.num_parts, prm.batch, prm.sched_c0,
                                     prm.max_pages, seqlens, block_table, splits,
                                     part == 0 && rg == 0);
    cur = st.cur;
    eb = st.eb;
    ej = st.ej;
    split_idx = st.split_idx;
    L0 = st.L0;
    phys0 = st.phys0;
  } else {
    const int32_t* m = meta + part * kMetaInts;
    eb = uni(m[2]);
    ej = uni(m[3]);
    cur = Item{uni(m[0]), uni(m[1])};
    split_idx = uni(m[4]);
  }
  if (!item_before(cur, eb, ej)) return;

  const int row_base = rg * V::kRows + wr * 16 * RT;  // first row of this wave
  const int col_base = wc * V::kColsPerWave;

  // lane-constant LDS offsets
  // K fragment (A of the score product): token 16*tt + l16, logical chunk
  // 4*ks + g -> physical ((4 ks + g) ^ (l16 & 7)).  The XOR splits into a
  // per-lane part and a part depending only on ks parity.
  const int sw = l16 & 7;
  const int k_lane = l16 * kRowBytes + 16 * (g ^ (sw & 3));
  const int k_even = k_lane + ((sw & 4) ? 64 : 0);   // ks even: bit 2 of chunk 0 -> sw bit
  const int k_odd = k_lane - ((sw & 4) ? 64 : 0);    // ks odd:  bit 2 of chunk 1 -> flipped
  // V^T fragment (A of the value product) by transposed read: token
  // 32*qq + 16*h + 4*g + (l16 >> 2), columns 16*ct + 4*(l16 & 3) .. +3,
  // i.e. chunk 2*ct + ((l16 & 3) >> 1), byte 8*(l16 & 1) inside it.
  const int vt = 4 * g + (l16 >> 2);  // token within a 16-token block
  const int vsw = swz(vt);
  const int ve = (l16 & 3) >> 1;
  int v_off[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    const int chunk = (2 * c4 + ve) ^ vsw;  // low 3 bits of 2*ct + ve, ct % 4 = c4
    v_off[c4] = vt * kRowBytes + 16 * chunk + 8 * (l16 & 1);
  }

  bf16x8 qf[RT][KS];
  f32x4 o[RT][CT];
  float m_used[RT], l_part[RT];
  int n_vis[RT];
  int L = 0;
  // split bookkeeping of the current sequence, fetched when it begins so that
  // the epilogue does not wait for a load
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
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = row_base + 16 * rt + l16;
      const bool live = row < prm.R;
      // rows past R read row 0 and are never stored; they see no tokens, so
      // their weights are exactly 0
      const uint16_t* qrow = q_ptr + ((size_t)b * prm.R + (live ? row : 0)) * kD + 8 * g;
      if (load_q) static_for<0, KS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int ks = decltype(kc)::value;
        qf[rt][ks] = *(const bf16x8*)(qrow + 32 * ks);
      });
      const int i = (live ? row : 0) / prm.h_q;
      int n = prm.causal ? (L - prm.s_q + 1 + i) : L;
      n = n < 0 ? 0 : (n > L ? L : n);
      n_vis[rt] = live ? n : 0;
      m_used[rt] = -INFINITY;
      l_part[rt] = 0.f;
      static_for<0, CT>([&](auto c) __attribute__((always_inline)) { o[rt][decltype(c)::value] = f32x4{0.f, 0.f, 0.f, 0.f}; });
    }
  };

  // Start the copy of item `it`'s page; false if it has no tokens.
  auto load_item = [&](MLA_LDS char* tile, Item it) __attribute__((always_inline)) -> bool {
    const int L_it = uni(seqlens[it.b]);
    if (it.j * kPage >= L_it) return false;
    const int phys = uni(block_table[(size_t)it.b * prm.max_pages + it.j]);
    loader.issue(tile, kvbase + (size_t)phys * kTileBytes, L_it - it.j * kPage, wave);
    return true;
  };

  // The copy of the next item's page, to be issued during the score product.
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

  // One 32-token half of a page: scores, online softmax, value product.
  auto compute_half = [&](MLA_LDS char* tile, int j, auto hc, const PendingCopy& cp)
                          __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
    // ---- scores S^T = K Q^T for tokens 32h .. 32h+31 (token tiles 2h, 2h+1)
    f32x4 s[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) s[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_k = [&](bf16x8* kf, int ks) __attribute__((always_inline)) {
      const int base = ((ks & 1) ? k_odd : k_even) + 64 * ks + h * 32 * kRowBytes;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        kf[tt] = *(MLA_LDS bf16x8*)(tile + base + tt * 16 * kRowBytes);
    };
    auto mma_k = [&](const bf16x8* kf, int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          s[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tt], qf[rt][ks], s[rt][tt], 0, 0, 0);
    };
    auto load_v = [&](bf16x8& vf, int ct) __attribute__((always_inline)) {
      const int cta = col_base / 16 + ct;  // absolute 16-column tile
      const int a = v_off[cta & 3] + 128 * (cta >> 2) + h * 32 * kRowBytes;
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a + 16 * kRowBytes));
      vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // K fragments run DK k-steps ahead of the products that use them: with
    // one wave per SIMD nothing else hides the LDS latency.
    constexpr int DK = RT == 1 ? 6 : 2;
    bf16x8 kr[DK + 1][2];
    static_for<0, DK>([&](auto ic) __attribute__((always_inline)) {
      load_k(kr[decltype(ic)::value], decltype(ic)::value);
    });
    static_for<0, KS>([&](auto ksc) __attribute__((always_inline)) {
      constexpr int ks = decltype(ksc)::value;
      if constexpr (ks + DK < KS) load_k(kr[(ks + DK) % (DK + 1)], ks + DK);
      // the next page's 18 copy instructions go out at every other k-step of
      // both halves: issued in one burst they outrun the CU's address unit
      // (16 cycles per 1 KiB instruction, four waves sharing it) and stall
      // the wave, and the matrix pipe with it
      if constexpr (ks % 2 == 0) {
        static_assert(KS == kLoadsPerWave, "nine copies per half, at the even k-steps");
        if (cp.valid) loader.issue_one(cp.tile, cp.rsrc, wave, 9 * h + ks / 2);
      }
      mma_k(kr[ks % (DK + 1)], ks);
      __builtin_amdgcn_sched_barrier(0);
    });
    // the first V^T fragments are independent of the weights: start them now
    constexpr int DV = RT == 1 ? 4 : 3;
    bf16x8 vr[DV + 1];
    static_for<0, DV>([&](auto ic) __attribute__((always_inline)) {
      load_v(vr[decltype(ic)::value], decltype(ic)::value);
    });
    // ---- online softmax (log2 domain); lane holds row l16, tokens
    //      32h + 16tt + 4g + r
    const int tok0 = j * kPage + 32 * h + 4 * g;
    float rowmax[RT];
    bool need = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = tok0 + 16 * tt + r;
          float x = s[rt][tt][r] * prm.scale_log2;
          x = (tok < n_vis[rt]) ? x : -INFINITY;
          s[rt][tt][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = wave_max_x4(mx);
      rowmax[rt] = mx;
      need |= mx > m_used[rt] + kRescaleThreshold;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mn = fmaxf(m_used[rt], rowmax[rt]);
        const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_used[rt] - mn);
        m_used[rt] = mn;
        l_part[rt] *= alpha;
        static_for<0, CT>([&](auto c) __attribute__((always_inline)) { o[rt][decltype(c)::value] *= alpha; });
      }
    }
    // weights as the B operand of the value product: k-slot 8g + i is token
    // 32h + 4g + i (i < 4) or 32h + 16 + 4g + (i - 4)
    bf16x8 pf[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mref = (m_used[rt] == -INFINITY) ? 0.f : m_used[rt];
      float p[2][4];
      float acc = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[tt][r] = __builtin_amdgcn_exp2f(s[rt][tt][r] - mref);
          acc += p[tt][r];
        }
      l_part[rt] += acc;
      bf16x2 a0 = to_bf16x2(p[0][0], p[0][1]);
      bf16x2 a1 = to_bf16x2(p[0][2], p[0][3]);
      bf16x2 a2 = to_bf16x2(p[1][0], p[1][1]);
      bf16x2 a3 = to_bf16x2(p[1][2], p[1][3]);
      pf[rt] = bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
    }
    // ---- O^T += V^T P^T over the same 32 tokens
    auto mma_v = [&](const bf16x8& vf, int ct) __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rt], o[rt][ct], 0, 0, 0);
    };
    static_for<0, CT>([&](auto ctc) __attribute__((always_inline)) {
      constexpr int ct = decltype(ctc)::value;
      if constexpr (ct + DV < CT) load_v(vr[(ct + DV) % (DV + 1)], ct + DV);
      mma_v(vr[ct % (DV + 1)], ct);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto compute_page = [&](MLA_LDS char* tile, int j, const PendingCopy& cp)
                          __attribute__((always_inline)) {
    compute_half(tile, j, std::integral_constant<int, 0>{}, cp);
    compute_half(tile, j, std::integral_constant<int, 1>{}, cp);
  };

  // one row of this wave's columns, 16 bytes per lane: lanes g and g ^ 1
  // (lane ^ 16, the same row) swap halves so that the even one holds 8
  // columns of tile c and the odd one 8 columns of tile c + 1
  auto store_row = [&](uint16_t* orow, int rt, float inv) __attribute__((always_inline)) {
    const bool even = (g & 1) == 0;
    static_for<0, CT / 2>([&](auto pc) __attribute__((always_inline)) {
      constexpr int c = 2 * decltype(pc)::value;
      const f32x4 va = o[rt][c] * inv;
      const f32x4 vb = o[rt][c + 1] * inv;
      const int a0 = __builtin_bit_cast(int, to_bf16x2(va[0], va[1]));
      const int a1 = __builtin_bit_cast(int, to_bf16x2(va[2], va[3]));
      const int b0 = __builtin_bit_cast(int, to_bf16x2(vb[0], vb[1]));
      const int b1 = __builtin_bit_cast(int, to_bf16x2(vb[2], vb[3]));
      const int x0 = __shfl_xor(even ? b0 : a0, 16);
      const int x1 = __shfl_xor(even ? b1 : a1, 16);
      const i32x4 w = even ? i32x4{a0, a1, x0, x1} : i32x4{x0, x1, b0, b1};
      *(i32x4*)(orow + (even ? 16 * c + 4 * g : 16 * (c + 1) + 4 * (g - 1))) = w;
    });
  };

  auto finish_segment = [&](int b) __attribute__((always_inline)) {
    const int s_lo = seg_s_lo;
    const int nsplit = seg_nsplit;
    const bool direct = nsplit <= 1;
    const int slot = s_lo + split_idx;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = row_base + 16 * rt + l16;
      const float lt = wave_sum_x4(l_part[rt]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse2 = lt > 0.f ? m_used[rt] + __builtin_amdgcn_logf(lt) : -INFINITY;
      if (row < prm.R) {
        if (direct) {
          store_row(out_ptr + ((size_t)b * prm.R + row) * kDv + col_base, rt, inv);
          if (g == 0 && wc == 0) lse_ptr[(size_t)b * prm.R + row] = lse2 * kLn2;
        } else {
          // the normalized partial, rounded to bf16 like the output
          store_row(o_acc + ((size_t)slot * prm.R + row) * kDv + col_base, rt, inv);
          if (g == 0 && wc == 0) lse_acc[(size_t)slot * prm.R + row] = lse2;
        }
      }
    }
    split_idx = 0;  // later sequences of this partition start at their page 0
  };

  // One step: compute `cur` from tile A while the next item streams into B.
  // The query fragments of a sequence are loaded at the end of the step
  // before its first page, so the wait at the top of the step (needed for
  // the page anyway) also covers them and no load into registers is ever
  // pending next to a page copy.
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
      // row 16 rt + l16 of the staged query, in the page layout: the K
      // fragment's addressing with token 16 rt + l16 (same swizzle)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        static_for<0, KS>([&](auto kc) __attribute__((always_inline)) {
          constexpr int ks = decltype(kc)::value;
          qf[rt][ks] = *(MLA_LDS bf16x8*)(tB + 16 * rt * kRowBytes +
                                          ((ks & 1) ? k_odd : k_even) + 64 * ks);
        });
      }
      lds_barrier();
    }
    const bool has_tokens = cur.j * kPage < L;
    if (has_tokens) {
      compute_page(tA, cur.j, cp);
    } else if (cp.valid) {
      for (int i = 0; i < kLoadsPerWave; ++i) loader.issue_one(cp.tile, cp.rsrc, wave, i);
    }
    if (!has_next || nx.b != cur.b) {
      finish_segment(cur.b);
      if (has_next) begin_segment(nx.b, uni(seqlens[nx.b]), true);
    }
    cur = nx;
    return has_next;
  };

  // The first segment's query rows (R <= 32; rows past R arrive as zeros
  // and see no tokens) are staged in tile 1, each wave copying one 8-row
  // block, instead of all 32 rows loaded by every wave.
  {
    static_assert(RT * 16 <= 4 * 8, "four 8-row blocks");
    const __amdgpu_buffer_rsrc_t qrs =
        PageLoader::resource((const char*)(q_ptr + (size_t)cur.b * prm.R * kD), prm.R);
#pragma unroll
    for (int i = 0; i < 9; ++i) loader.issue_one(tile1, qrs, wave, i);
  }
  if constexpr (kFused) {
    // length and page of the first item were read with the schedule
    begin_segment(cur.b, L0, false);
    if (cur.j * kPage < L0)
      loader.issue(tile0, kvbase + (size_t)phys0 * kTileBytes, L0 - cur.j * kPage, wave);
  } else {
    begin_segment(cur.b, uni(seqlens[cur.b]), false);
    load_item(tile0, cur);
  }
  if (step(tile0, tile1, std::true_type{})) {
    while (true) {
      if (!step(tile1, tile0, std::false_type{})) break;
      if (!step(tile0, tile1, std::false_type{})) break;
    }
  }
}

}  // namespace mla

// ---------------------------------------------------------------------------
// launchers (called by the C ABI after argument checks)
extern "C" hipError_t mla_launch_decode(const mla::DecodeParams* prm, int rows_variant,
                                        hipStream_t stream) {
  using namespace mla;
  const int groups = (prm->num_parts + 7) / 8;
  const dim3 grid(groups * 8 * prm->row_groups);
  const dim3 block(kThreads);
#define MLA_DECODE_ARGS                                                                  \
  *prm, prm->q, prm->kv, prm->block_table, prm->seqlens, prm->meta, prm->splits, prm->out, \
      prm->lse, prm->o_acc, prm->lse_acc
  // (16 rows run in mla_decode_t16.hip)
  if (rows_variant != 32) return hipErrorInvalidValue;
  if (prm->meta)
    hipLaunchKernelGGL((decode_kernel<2, 1, 4, false>), grid, block, 0, stream, MLA_DECODE_ARGS);
  else  // schedule inside the launch (batch <= kFusedMaxBatch, checked by the caller)
    hipLaunchKernelGGL((decode_kernel<2, 1, 4, true>), grid, block, 0, stream, MLA_DECODE_ARGS);
#undef MLA_DECODE_ARGS
  return hipGetLastError();
}
