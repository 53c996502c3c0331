// Paged MLA decode, 64 query rows per workgroup, with the work of each
// 32-token half page split differently in its two products:
//
//   score product  S^T = K Q^T   -- wave w owns query rows 16w .. 16w+15 and
//                                   scores them against all 32 tokens;
//   value product  O^T += V^T P^T -- wave w owns output columns 128w .. +127
//                                   for all 64 rows.
//
// Between them each wave leaves its bf16 weights in LDS, already in the
// layout of the value product's B operand (one 16-byte read per 16 rows),
// together with the factor each of its rows was rescaled by.  Nothing is
// computed twice: the score product of a row happens once, every K fragment
// read serves 16 rows, and every (slow) transposed V^T read serves 64 rows.
//
// What is computed, and the choices shared with the other decode kernel,
// are described in mla_decode.hip (FlashMLA release note: MLA principles and
// the paged bf16 cache; DeepSeek-V3 summary: one latent shared by all heads).

#include "mla_decode_common.h"

namespace mla {

constexpr int kSplitRows = 64;   // query rows per workgroup
constexpr int kPvRT = 4;         // 16-row tiles in the value product (all 64 rows)
constexpr int kPvCT = 8;         // 16-column tiles per wave (128 columns)
constexpr int kKS = kD / 32;     // 18 k-steps of the score product

__global__ void __launch_bounds__(kThreads, 1)
    decode_kernel_split(const DecodeParams prm, const uint16_t* q_ptr,
                        const uint16_t* __restrict__ kv_ptr, const int32_t* __restrict__ block_table,
                        const int32_t* __restrict__ seqlens, const int32_t* __restrict__ meta,
                        const int32_t* __restrict__ splits, uint16_t* __restrict__ out_ptr,
                        float* __restrict__ lse_ptr, float* __restrict__ o_acc,
                        float* __restrict__ lse_acc) {
  __shared__ __attribute__((aligned(1024))) char tile0_[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char tile1_[kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][kWaves][64];  // [half][scoring wave][lane]
  __shared__ float alpha_buf[2][kSplitRows];  // [half][row]: factor the row was rescaled by
  __shared__ float stat_l[kSplitRows];  // per-row softmax sum at segment end
  MLA_LDS char* tile0 = (MLA_LDS char*)tile0_;
  MLA_LDS char* tile1 = (MLA_LDS char*)tile1_;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;

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

  const int row0 = rg * kSplitRows;        // first row of this workgroup
  const int qk_row = row0 + 16 * wave + l16;  // the row this lane scores
  const int col_base = wave * (kDv / kWaves);

  // K fragment offsets (token 16 tt + l16, logical chunk 4 ks + g)
  const int sw = l16 & 7;
  const int k_lane = l16 * kRowBytes + 16 * (g ^ (sw & 3));
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

  bf16x8 qf[kKS];           // this lane's scoring row, 8 features per k-step
  f32x4 o[kPvRT][kPvCT];    // O^T tiles: row 16 rt + l16, columns col_base + 16 ct + 4g + r
  float m_used = -INFINITY, l_part = 0.f;  // running max in raw score units
  int n_vis = 0;
  int wave_min_vis = 0;  // fewest visible tokens over this wave's rows
  int L = 0;
  // split bookkeeping of the current sequence, fetched when it begins so that
  // the epilogue does not wait for a load
  int seg_s_lo = 0, seg_nsplit = 0;

  const char* kvbase = (const char*)kv_ptr;
  // q_ptr is not restrict-qualified: the query loads must stay ordered
  // against the fenced waits for the (compiler-invisible) page copies
  AsmPageLoader loader;
  loader.init(lane);

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
    int v = n_vis;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d));
    wave_min_vis = v;
    m_used = -INFINITY;
    l_part = 0.f;
    static_for<0, kPvRT>([&](auto rc) __attribute__((always_inline)) {
      static_for<0, kPvCT>([&](auto cc) __attribute__((always_inline)) {
        o[decltype(rc)::value][decltype(cc)::value] = f32x4{0.f, 0.f, 0.f, 0.f};
      });
    });
  };

  auto load_item = [&](MLA_LDS char* tile, Item it) __attribute__((always_inline)) -> bool {
    const int L_it = uni(seqlens[it.b]);
    if (it.j * kPage >= L_it) return false;
    const int phys = uni(block_table[(size_t)it.b * prm.max_pages + it.j]);
    const i32x4 d = AsmPageLoader::desc(kvbase + (size_t)phys * kTileBytes, L_it - it.j * kPage);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) loader.issue_one(tile, d, wave, i);
    return true;
  };

  // The copy of the next item's page, to be issued during the score product.
  auto next_copy = [&](MLA_LDS char* tile, Item it, bool has) __attribute__((always_inline)) {
    AsmPendingCopy cp;
    cp.tile = tile;
    cp.valid = false;
    cp.desc = AsmPageLoader::desc(kvbase, 0);
    if (has) {
      const int L_it = uni(seqlens[it.b]);
      if (it.j * kPage < L_it) {
        const int phys = uni(block_table[(size_t)it.b * prm.max_pages + it.j]);
        cp.desc = AsmPageLoader::desc(kvbase + (size_t)phys * kTileBytes, L_it - it.j * kPage);
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

  // ---- the pieces of a page ------------------------------------------------
  // Score product of half h (tokens 32 h .. 32 h + 31) for this wave's 16
  // rows; at(u) adds work after matrix instruction u = 2 ks + tt (page
  // copies, a slice of the other half's softmax), so that it issues in the
  // shadow of the matrix core.
  auto qk_half = [&](MLA_LDS char* tile, auto hc, f32x4* s, auto&& at)
                     __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
    s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_k = [&](bf16x8* kf, int ks) __attribute__((always_inline)) {
      const int base = ((ks & 1) ? k_odd : k_even) + 64 * ks + h * 32 * kRowBytes;
      kf[0] = *(MLA_LDS bf16x8*)(tile + base);
      kf[1] = *(MLA_LDS bf16x8*)(tile + base + 16 * kRowBytes);
    };
    constexpr int DK = 6;
    bf16x8 kr[DK + 1][2];
    static_for<0, DK>([&](auto ic) __attribute__((always_inline)) {
      load_k(kr[decltype(ic)::value], decltype(ic)::value);
    });
    static_for<0, kKS>([&](auto ksc) __attribute__((always_inline)) {
      constexpr int ks = decltype(ksc)::value;
      if constexpr (ks + DK < kKS) load_k(kr[(ks + DK) % (DK + 1)], ks + DK);
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (DK + 1)][0], qf[ks], s[0], 0, 0, 0);
      at(std::integral_constant<int, 2 * ks>{});
      __builtin_amdgcn_sched_barrier(0);
      s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (DK + 1)][1], qf[ks], s[1], 0, 0, 0);
      at(std::integral_constant<int, 2 * ks + 1>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // V^T fragment ct (16 columns x 32 tokens of half h) by transposed reads
  auto load_v = [&](MLA_LDS char* tile, int h, bf16x8& vf, int ct) __attribute__((always_inline)) {
    const int cta = col_base / 16 + ct;
    const int a = v_off[cta & 3] + 128 * (cta >> 2) + h * 32 * kRowBytes;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a + 16 * kRowBytes));
    vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  constexpr int DV = 5;  // V^T fragments in flight ahead of their product

  // Value product of half h: all 64 rows, this wave's 128 columns.  vr holds
  // fragments 0 .. DV-1 on entry; at(u) adds work after matrix instruction
  // u = 4 ct + rt.
  auto pv_half = [&](MLA_LDS char* tile, auto hc, bf16x8* vr, auto&& at)
                     __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
    bf16x8 pb[kPvRT];
    float al[kPvRT];
    bool resc = false;
#pragma unroll
    for (int rt = 0; rt < kPvRT; ++rt) {
      pb[rt] = pbuf[h][rt][lane];
      al[rt] = alpha_buf[h][16 * rt + l16];
      resc |= al[rt] != 1.f;
    }
    if (__builtin_amdgcn_ballot_w64(resc) != 0) {
      static_for<0, kPvRT>([&](auto rc) __attribute__((always_inline)) {
        constexpr int rt = decltype(rc)::value;
        static_for<0, kPvCT>([&](auto cc) __attribute__((always_inline)) {
          o[rt][decltype(cc)::value] *= al[rt];
        });
      });
    }
    static_for<0, kPvCT>([&](auto ctc) __attribute__((always_inline)) {
      constexpr int ct = decltype(ctc)::value;
      if constexpr (ct + DV < kPvCT) load_v(tile, h, vr[(ct + DV) % (DV + 1)], ct + DV);
      static_for<0, kPvRT>([&](auto rc) __attribute__((always_inline)) {
        constexpr int rt = decltype(rc)::value;
        o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[ct % (DV + 1)], pb[rt], o[rt][ct], 0, 0, 0);
        at(std::integral_constant<int, kPvRT * ct + rt>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };

  // Online softmax of one half for this wave's rows (log2 domain), cut into
  // kSmStages slices of a few VALU instructions each, so that another phase
  // can place one slice after each of its matrix instructions (a wave hides
  // about two VALU instructions in the shadow of one 16x16x32 MFMA).  The
  // running max is kept in raw score units (the scale is positive), and the
  // scale is folded into one FMA ahead of each exponential:
  //   p = 2^(s * scale - m * scale).
  // Masking is skipped when every token of the half is visible to every row
  // of the wave (`full`, uniform).
  //   0-7 mask one score (partial halves only)   8-9 local max
  //   10-11 row max   12-13 lazy rescale decision   14-21 one exponential each
  //   22-23 sums      24-25 bf16 weights and factor to LDS
  // Branch-free: when any row of the wave exceeds its running max by the
  // threshold, every row moves its max up to the current one.
  struct SmState {
    float x[8];
    float m4, mx, mn, alpha, nref;
    float p[8];
    bool upd;
    bf16x2 a[4];
  };
  auto sm_stage = [&](auto stc, SmState& st, const f32x4* s, int tok0, bool full, auto hc)
                      __attribute__((always_inline)) {
    constexpr int u = decltype(stc)::value;
    constexpr int h = decltype(hc)::value;
    if constexpr (u < 8) {
      constexpr int tt = u / 4, r = u % 4;
      st.x[u] = (full || tok0 + 16 * tt + r < n_vis) ? s[tt][r] : -INFINITY;
    } else if constexpr (u == 8) {
      st.m4 = fmaxf(fmaxf(st.x[0], st.x[1]), fmaxf(st.x[2], st.x[3]));
    } else if constexpr (u == 9) {
      st.mx = fmaxf(st.m4, fmaxf(fmaxf(st.x[4], st.x[5]), fmaxf(st.x[6], st.x[7])));
    } else if constexpr (u == 10) {
      typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
      const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(st.mx),
                                                       __float_as_uint(st.mx), false, false);
      st.mx = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    } else if constexpr (u == 11) {
      typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
      const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.mx),
                                                       __float_as_uint(st.mx), false, false);
      st.mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    } else if constexpr (u == 12) {
      // m_used is in raw score units; the threshold is in log2 units
      st.upd = __builtin_amdgcn_ballot_w64((st.mx - m_used) * prm.scale_log2 > kRescaleThreshold) != 0;
      st.mn = st.upd ? fmaxf(m_used, st.mx) : m_used;
    } else if constexpr (u == 13) {
      st.alpha = (st.upd && st.mn != -INFINITY)
                     ? __builtin_amdgcn_exp2f((m_used - st.mn) * prm.scale_log2)
                     : 1.f;
      m_used = st.mn;
      l_part *= st.alpha;
      st.nref = (st.mn == -INFINITY) ? 0.f : -st.mn * prm.scale_log2;
    } else if constexpr (u < 22) {
      st.p[u - 14] = __builtin_amdgcn_exp2f(__builtin_fmaf(st.x[u - 14], prm.scale_log2, st.nref));
    } else if constexpr (u == 22) {
      l_part += (st.p[0] + st.p[1]) + (st.p[2] + st.p[3]);
    } else if constexpr (u == 23) {
      l_part += (st.p[4] + st.p[5]) + (st.p[6] + st.p[7]);
    } else if constexpr (u == 24) {
      // k-slot 8g + i <-> token 32h + 4g + i (i < 4) or 32h + 16 + 4g + (i - 4)
      st.a[0] = to_bf16x2(st.p[0], st.p[1]);
      st.a[1] = to_bf16x2(st.p[2], st.p[3]);
      st.a[2] = to_bf16x2(st.p[4], st.p[5]);
      st.a[3] = to_bf16x2(st.p[6], st.p[7]);
    } else if constexpr (u == 25) {
      pbuf[h][wave][lane] = bf16x8{st.a[0][0], st.a[0][1], st.a[1][0], st.a[1][1],
                                   st.a[2][0], st.a[2][1], st.a[3][0], st.a[3][1]};
      if (g == 0) alpha_buf[h][16 * wave + l16] = st.alpha;
    }
  };
  constexpr int kSmStages = 26;

  // One page (in `tile`), software-pipelined across its two halves so that
  // the softmax VALU work of each half runs under matrix instructions:
  //   scores h0 | scores h1 + softmax h0 | barrier | values h0 + softmax h1 |
  //   barrier | values h1
  // The next page's 18 copy instructions go out at the even k-steps of the
  // two score products (copies 0..8 fill its first half, 9..17 its second).
  auto compute_page = [&](MLA_LDS char* tile, int j, const AsmPendingCopy& cp)
                          __attribute__((always_inline)) {
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    const int tok0 = j * kPage + 4 * g;
    // halves every token of which every row of this wave sees (uniform)
    const int vis_min = uni(wave_min_vis);
    const bool full0 = j * kPage + 32 <= vis_min;
    const bool full1 = j * kPage + 64 <= vis_min;
    f32x4 s0[2], s1[2];
    // copies at every fourth matrix instruction (every other k-step)
    qk_half(tile, H0{}, s0, [&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u % 4 == 0)
        if (cp.valid) loader.issue_one(cp.tile, cp.desc, wave, u / 4);
    });
    // this page's second half (this wave's copies 9..17) has landed, for
    // every wave after the barrier; only the next page's first nine copies
    // may still be in flight
    if (cp.valid)
      fenced_wait<kWaitVm9>();
    else
      fenced_wait<kWaitVm0>();
    lds_barrier();
    SmState st0;
    qk_half(tile, H1{}, s1, [&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u % 4 == 0)
        if (cp.valid) loader.issue_one(cp.tile, cp.desc, wave, 9 + u / 4);
      if constexpr (u < kSmStages) sm_stage(uc, st0, s0, tok0, full0, H0{});
    });
    bf16x8 vr[DV + 1];
    static_for<0, DV>([&](auto ic) __attribute__((always_inline)) {
      load_v(tile, 0, vr[decltype(ic)::value], decltype(ic)::value);
    });
    lds_barrier();  // weights and factors of half 0 visible
    SmState st1;
    pv_half(tile, H0{}, vr, [&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < kSmStages) sm_stage(uc, st1, s1, tok0 + 32, full1, H1{});
    });
    static_for<0, DV>([&](auto ic) __attribute__((always_inline)) {
      load_v(tile, 1, vr[decltype(ic)::value], decltype(ic)::value);
    });
    lds_barrier();  // weights and factors of half 1 visible
    pv_half(tile, H1{}, vr, [&](auto) __attribute__((always_inline)) {});
  };

  auto finish_segment = [&](int b) __attribute__((always_inline)) {
    const int s_lo = seg_s_lo;
    const int nsplit = seg_nsplit;
    const bool direct = nsplit <= 1;
    const int slot = s_lo + split_idx;
    // the scoring wave of each row publishes its sum, and writes its lse
    const float lt = wave_sum_x4(l_part);
    if (g == 0) {
      stat_l[16 * wave + l16] = lt;
      if (qk_row < prm.R) {
        const float lse2 = lt > 0.f ? m_used * prm.scale_log2 + __builtin_amdgcn_logf(lt) : -INFINITY;
        if (direct)
          lse_ptr[(size_t)b * prm.R + qk_row] = lse2 * kLn2;
        else
          lse_acc[(size_t)slot * prm.R + qk_row] = lse2;
      }
    }
    lds_barrier();
    static_for<0, kPvRT>([&](auto rc) __attribute__((always_inline)) {
      constexpr int rt = decltype(rc)::value;
      const int row = row0 + 16 * rt + l16;
      const float lr = stat_l[16 * rt + l16];
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      if (row < prm.R) {
        if (direct) {
          uint16_t* orow = out_ptr + ((size_t)b * prm.R + row) * kDv + col_base + 4 * g;
          static_for<0, kPvCT>([&](auto cc) __attribute__((always_inline)) {
            constexpr int ct = decltype(cc)::value;
            const f32x4 v = o[rt][ct] * inv;
            const bf16x2 a = to_bf16x2(v[0], v[1]);
            const bf16x2 c = to_bf16x2(v[2], v[3]);
            *(bf16x4*)(orow + 16 * ct) = bf16x4{a[0], a[1], c[0], c[1]};
          });
        } else {
          float* orow = o_acc + ((size_t)slot * prm.R + row) * kDv + col_base + 4 * g;
          static_for<0, kPvCT>([&](auto cc) __attribute__((always_inline)) {
            constexpr int ct = decltype(cc)::value;
            *(f32x4*)(orow + 16 * ct) = o[rt][ct] * inv;
          });
        }
      }
    });
    split_idx = 0;
  };

  auto step = [&](MLA_LDS char* tA, MLA_LDS char* tB) __attribute__((always_inline)) -> bool {
    const Item nx = advance(cur);
    const bool has_next = item_before(nx, eb, ej);
    // descriptor of the next copy first: its scalar loads (block table and
    // lengths, never written here) overlap the wait below
    AsmPendingCopy cp = next_copy(tB, nx, has_next);
    // this wave's copies of the first half of tile A landed (the nine of its
    // second half may still fly) ... and every wave's after the barrier; B is
    // free
    fenced_wait<kWaitVm9>();
    __syncthreads();
    const bool has_tokens = cur.j * kPage < L;
    if (has_tokens) {
      compute_page(tA, cur.j, cp);
    } else if (cp.valid) {
      for (int i = 0; i < kLoadsPerWave; ++i) loader.issue_one(cp.tile, cp.desc, wave, i);
    }
    if (!has_next || nx.b != cur.b) {
      finish_segment(cur.b);
      if (has_next) {
        begin_segment(nx.b);
        // the stores and query loads above are newer than the next page's
        // copies: drain once per sequence so the count waits stay exact
        fenced_wait<kWaitVm0>();
      }
    }
    cur = nx;
    return has_next;
  };

  begin_segment(cur.b);
  load_item(tile0, cur);
  // queries and the first page (once per workgroup; afterwards the waits
  // count page halves)
  fenced_wait<kWaitVm0>();
  while (true) {
    if (!step(tile0, tile1)) break;
    if (!step(tile1, tile0)) break;
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_decode_split(const mla::DecodeParams* prm, hipStream_t stream) {
  using namespace mla;
  const int groups = (prm->num_parts + 7) / 8;
  const dim3 grid(groups * 8 * prm->row_groups);
  hipLaunchKernelGGL(decode_kernel_split, grid, dim3(kThreads), 0, stream, *prm, prm->q, prm->kv,
                     prm->block_table, prm->seqlens, prm->meta, prm->splits, prm->out, prm->lse,
                     prm->o_acc, prm->lse_acc);
  return hipGetLastError();
}
