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
    decode_kernel_split(const DecodeParams prm, const uint16_t* __restrict__ q_ptr,
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
  float m_used = -INFINITY, l_part = 0.f;
  int n_vis = 0;
  int L = 0;
  // split bookkeeping of the current sequence, fetched when it begins so that
  // the epilogue does not wait for a load
  int seg_s_lo = 0, seg_nsplit = 0;

  const char* kvbase = (const char*)kv_ptr;
  PageLoader loader;
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
    loader.issue(tile, kvbase + (size_t)phys * kTileBytes, wave);
    return true;
  };

  // The copy of the next item's page, to be issued during the score product.
  auto next_copy = [&](MLA_LDS char* tile, Item it, bool has) __attribute__((always_inline)) {
    PendingCopy cp;
    cp.tile = tile;
    cp.valid = false;
    cp.rsrc = PageLoader::resource(kvbase);
    if (has) {
      const int L_it = uni(seqlens[it.b]);
      if (it.j * kPage < L_it) {
        const int phys = uni(block_table[(size_t)it.b * prm.max_pages + it.j]);
        cp.rsrc = PageLoader::resource(kvbase + (size_t)phys * kTileBytes);
        cp.valid = true;
      }
    }
    return cp;
  };

  auto advance = [&](Item it) __attribute__((always_inline)) {
    Item nx = it;
    if (it.j + 1 < page_slots(seqlens, it.b)) {
      nx.j = uni(it.j + 1);
    } else {
      nx.b = uni(it.b + 1);
      nx.j = 0;
    }
    return nx;
  };

  // One 32-token half page (tokens 32h .. 32h+31 of page j in `tile`).
  auto compute_half = [&](MLA_LDS char* tile, int j, auto hc, const PendingCopy& cp)
                          __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
    // ---- scores for this wave's 16 rows
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
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
      if constexpr (h == 0) {
        static_assert(kKS == kLoadsPerWave, "one page-copy instruction per k-step");
        if (cp.valid) loader.issue_one(cp.tile, cp.rsrc, wave, ks);
      }
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (DK + 1)][0], qf[ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (DK + 1)][1], qf[ks], s[1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // ---- the first V^T fragments do not depend on the weights
    auto load_v = [&](bf16x8& vf, int ct) __attribute__((always_inline)) {
      const int cta = col_base / 16 + ct;
      const int a = v_off[cta & 3] + 128 * (cta >> 2) + h * 32 * kRowBytes;
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(tile + a + 16 * kRowBytes));
      vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int DV = 5;
    bf16x8 vr[DV + 1];
    static_for<0, DV>([&](auto ic) __attribute__((always_inline)) {
      load_v(vr[decltype(ic)::value], decltype(ic)::value);
    });
    // ---- online softmax of this wave's rows (log2 domain)
    const int tok0 = j * kPage + 32 * h + 4 * g;
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = s[tt][r] * prm.scale_log2;
        x[tt][r] = (tok0 + 16 * tt + r < n_vis) ? v : -INFINITY;
        mx = fmaxf(mx, x[tt][r]);
      }
    mx = wave_max_x4(mx);
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mx > m_used + kRescaleThreshold) != 0) {
      const float mn = fmaxf(m_used, mx);
      alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_used - mn);
      m_used = mn;
      l_part *= alpha;
    }
    const float mref = (m_used == -INFINITY) ? 0.f : m_used;
    float p[2][4];
    float acc = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[tt][r] = __builtin_amdgcn_exp2f(x[tt][r] - mref);
        acc += p[tt][r];
      }
    l_part += acc;
    // k-slot 8g + i <-> token 32h + 4g + i (i < 4) or 32h + 16 + 4g + (i - 4)
    const bf16x2 a0 = to_bf16x2(p[0][0], p[0][1]);
    const bf16x2 a1 = to_bf16x2(p[0][2], p[0][3]);
    const bf16x2 a2 = to_bf16x2(p[1][0], p[1][1]);
    const bf16x2 a3 = to_bf16x2(p[1][2], p[1][3]);
    pbuf[h][wave][lane] = bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
    if (g == 0) alpha_buf[h][16 * wave + l16] = alpha;
    lds_barrier();
    // ---- value product: all 64 rows, this wave's 128 columns
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
      if constexpr (ct + DV < kPvCT) load_v(vr[(ct + DV) % (DV + 1)], ct + DV);
      static_for<0, kPvRT>([&](auto rc) __attribute__((always_inline)) {
        constexpr int rt = decltype(rc)::value;
        o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[ct % (DV + 1)], pb[rt], o[rt][ct], 0, 0, 0);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto zero_tail = [&](MLA_LDS char* tile, int first_dead) __attribute__((always_inline)) {
    const int start = first_dead * kRowBytes;
    for (int off = start + threadIdx.x * 16; off < kTileBytes; off += kThreads * 16)
      *(MLA_LDS i32x4*)(tile + off) = i32x4{0, 0, 0, 0};
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
        const float lse2 = lt > 0.f ? m_used + __builtin_amdgcn_logf(lt) : -INFINITY;
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
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    PendingCopy cp = next_copy(tB, nx, has_next);
    const bool has_tokens = cur.j * kPage < L;
    if (has_tokens) {
      const int live = L - cur.j * kPage;
      if (live < kPage) {
        zero_tail(tA, live);
        lds_barrier();
      }
      compute_half(tA, cur.j, std::integral_constant<int, 0>{}, cp);
      compute_half(tA, cur.j, std::integral_constant<int, 1>{}, cp);
    } else if (cp.valid) {
      for (int i = 0; i < kLoadsPerWave; ++i) loader.issue_one(cp.tile, cp.rsrc, wave, i);
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

extern "C" hipError_t mla_launch_decode_split(const mla::DecodeParams* prm, hipStream_t stream) {
  using namespace mla;
  const int groups = (prm->num_parts + 7) / 8;
  const dim3 grid(groups * 8 * prm->row_groups);
  hipLaunchKernelGGL(decode_kernel_split, grid, dim3(kThreads), 0, stream, *prm, prm->q, prm->kv,
                     prm->block_table, prm->seqlens, prm->meta, prm->splits, prm->out, prm->lse,
                     prm->o_acc, prm->lse_acc);
  return hipGetLastError();
}
