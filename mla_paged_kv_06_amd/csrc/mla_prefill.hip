// MLA prefill: causal attention over whole prompts in per-head form.
//
// FlashMLA itself is a decode kernel (FlashMLA release note, introduction),
// and the DeepSeek-V3 summary (paragraph on inference speed) runs prefill
// and decode as separate stages.  For a prompt every token attends to every
// earlier one, so the latent is widened per head first (release note,
// paragraph on the MLA core principles): head h's key of token t is
// [k_nope[t, h] ; k_rope[t]] (128 + 64 values, the rotary part shared by the
// heads) and its value v[t, h] (128 values).  Query t of a prompt sees keys
// 0 .. t of its own prompt.  Several prompts are packed one after another
// (cu_seqlens).
//
// A workgroup of 8 waves owns 256 query rows of one prompt and one head;
// wave w holds rows 32 w .. 32 w + 31 as two 16-row tiles whose query
// fragments stay in registers.  Keys and values stream through LDS in
// 64-key blocks, double-buffered: every thread loads its share of the next
// block into registers before the current block's products and writes it to
// LDS after them, so one barrier per block suffices.
//   scores  S^T = K Q^T      MFMA 16x16x32 bf16, K from LDS (A), Q (B)
//   values  O^T += V^T P^T   MFMA 16x16x32 bf16, V^T from LDS (A), P (B)
// S^T puts one query row per lane (lane % 16), so each lane's weights are
// already the B operand of the value product once the value tile is stored
// transposed with its keys permuted to match the k-slots: k-slot 8 g + i of
// a 32-key step is key 4 g + i (i < 4) or 16 + 4 g + i - 4.  The transpose
// happens when the block is staged (each thread packs two keys of eight
// columns into eight 4-byte LDS writes), so every fragment read is a plain
// 16-byte LDS read.  LDS rows are laid out so that the 16 lanes of a
// fragment read hit distinct banks: key rows of 384 bytes with chunk c of
// key t at chunk (c & ~7) | ((c & 7) ^ ((t >> 1) & 7)), value columns of
// 64 keys padded to 144 bytes.
//
// Online softmax in the log2 domain with the decode's lazy rescale: the
// running max only moves when a score beats it by more than 8 (log2 units),
// one decision per wave; the max is kept in raw score units (the scale is
// positive).

#include "mla_decode_common.h"

namespace mla {

namespace pf {
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;         // 256 query rows per workgroup
constexpr int kBK = 64;                  // keys per block
constexpr int kNopeD = 128;
constexpr int kRopeD = 64;
constexpr int kQK = kNopeD + kRopeD;     // 192
constexpr int kVD = 128;
constexpr int kKS = kQK / 32;            // 6 k-steps of the score product
constexpr int kKRowB = kQK * 2;          // 384 B per key row in LDS
constexpr int kKRowChunks = kKRowB / 16; // 24
constexpr int kKTileB = kBK * kKRowB;    // 24576
constexpr int kKPer = kKTileB / 16 / kThreads;  // 3 16-byte key pieces per thread
constexpr int kVRowB = kBK * 2 + 16;     // 144: one value column of 64 keys, padded
constexpr int kVTileB = kVD * kVRowB;    // 18432
constexpr int kCT = kVD / 16;            // 8 column tiles of the value product
static_assert(kKPer * 16 * kThreads == kKTileB, "key staging");
static_assert(32 * 16 == kThreads, "value staging: 32 key pairs x 16 column groups");
}  // namespace pf

// physical 16-byte chunk of logical chunk c in key row t
__device__ __forceinline__ int pf_kchunk(int t, int c) { return (c & ~7) | ((c & 7) ^ ((t >> 1) & 7)); }

// position of key t (0..63) of a block in a value column (k-slot order)
__device__ __forceinline__ int pf_vpos(int t) {
  const int u = t & 31;
  const int in32 = u < 16 ? 8 * (u >> 2) + (u & 3) : 8 * ((u - 16) >> 2) + 4 + (u & 3);
  return (t & 32) + in32;
}

__global__ void __launch_bounds__(pf::kThreads, 1) prefill_attention_kernel(const PrefillParams p) {
  using namespace pf;
  using pf::kThreads;
  __shared__ __attribute__((aligned(16))) char k_lds[2][kKTileB];
  __shared__ __attribute__((aligned(16))) char v_lds[2][kVTileB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  // grid (head, prompt, q-block counted from the last): the heaviest
  // q-blocks of every prompt and head are dispatched first
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int seq0 = load_uniform(p.cu, s);
  const int n = load_uniform(p.cu, s + 1) - seq0;
  const int nqb = (n + kBQ - 1) / kBQ;
  if ((int)blockIdx.z >= nqb) return;
  const int q0 = (nqb - 1 - (int)blockIdx.z) * kBQ;
  const int kend = p.causal ? min(n, q0 + kBQ) : n;  // keys [0, kend) matter
  const int nblocks = (kend + kBK - 1) / kBK;
  const size_t H = p.H;
  const float sl2 = p.scale_log2;

  // ---- this wave's query rows (B operand: lane (l16, g) holds row l16 of
  //      the tile, values 32 ks + 8 g .. + 7)
  const int row_base = q0 + 32 * wave;
  bf16x8 qf[2][kKS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    int row = row_base + 16 * rt + l16;
    row = row < n ? row : n - 1;
    const uint16_t* qp = p.q + ((size_t)(seq0 + row) * H + h) * kQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[rt][ks] = *(const bf16x8*)(qp + 32 * ks);
  }

  // ---- staging of a key/value block: loads into registers, then LDS
  uint4 kreg[kKPer];
  uint4 vreg[2];
  const int vtp = tid & 31;  // key pair 2 vtp, 2 vtp + 1
  const int vcg = tid >> 5;  // columns 8 vcg .. 8 vcg + 7
  auto load_block = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * kBK;
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int i = tid + pf::kThreads * u;
      const int t = i / kKRowChunks;
      const int c = i - kKRowChunks * t;
      const int tok = k0 + t;
      uint4 val = {0u, 0u, 0u, 0u};
      if (tok < kend) {
        const uint16_t* src =
            c < 16 ? p.k_nope + ((size_t)(seq0 + tok) * H + h) * kNopeD + 8 * c
                   : p.k_rope + (size_t)(seq0 + tok) * p.rope_stride + 8 * (c - 16);
        val = *(const uint4*)src;
      }
      kreg[u] = val;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tok = k0 + 2 * vtp + e;
      uint4 val = {0u, 0u, 0u, 0u};
      if (tok < kend) val = *(const uint4*)(p.v + ((size_t)(seq0 + tok) * H + h) * kVD + 8 * vcg);
      vreg[e] = val;
    }
  };
  auto store_block = [&](int buf) __attribute__((always_inline)) {
    char* kb = k_lds[buf];
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int i = tid + pf::kThreads * u;
      const int t = i / kKRowChunks;
      const int c = i - kKRowChunks * t;
      *(uint4*)(kb + t * kKRowB + 16 * pf_kchunk(t, c)) = kreg[u];
    }
    // keys 2 vtp and 2 vtp + 1 sit next to each other in k-slot order
    char* vb = v_lds[buf] + 2 * pf_vpos(2 * vtp);
    const unsigned a[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
    const unsigned b[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned lo = (a[w] & 0xFFFFu) | (b[w] << 16);          // column 8 vcg + 2 w
      const unsigned hi = (a[w] >> 16) | (b[w] & 0xFFFF0000u);      // column 8 vcg + 2 w + 1
      *(unsigned*)(vb + (8 * vcg + 2 * w) * kVRowB) = lo;
      *(unsigned*)(vb + (8 * vcg + 2 * w + 1) * kVRowB) = hi;
    }
  };

  f32x4 o[2][kCT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) o[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};

  // the key-row part of every fragment address that does not change
  const int sw = (l16 >> 1) & 7;  // keys 16 tt + l16: same swizzle for every tt

  load_block(0);
  store_block(0);
  __syncthreads();
  for (int j = 0; j < nblocks; ++j) {
    const int buf = j & 1;
    if (j + 1 < nblocks) load_block(j + 1);
    const int k0 = j * kBK;
    // wave-uniform: rows past the prompt, or keys all after the last row
    const bool active = row_base < n && (!p.causal || k0 <= row_base + 31);
    if (active) {
      // ---- S^T = K Q^T over 4 key tiles of 16
      const char* kb = k_lds[buf] + l16 * kKRowB;
      f32x4 sacc[2][4];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sacc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          const int c = 4 * ks + g;
          const bf16x8 kf =
              *(const bf16x8*)(kb + tt * 16 * kKRowB + 16 * ((c & ~7) | ((c & 7) ^ sw)));
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            sacc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rt][ks], sacc[rt][tt],
                                                                  0, 0, 0);
        }
      }
      // ---- masks and row maxima (lane holds keys 16 tt + 4 g + r); a block
      //      every key of which every row of the wave sees needs no mask
      float x[2][16];
      float mt[2];
      const bool whole = k0 + kBK <= kend && (!p.causal || k0 + kBK - 1 <= row_base);
      if (whole) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[rt][4 * tt + r] = sacc[rt][tt][r];
          float m0 = fmaxf(fmaxf(x[rt][0], x[rt][1]), fmaxf(x[rt][2], x[rt][3]));
          float m1 = fmaxf(fmaxf(x[rt][4], x[rt][5]), fmaxf(x[rt][6], x[rt][7]));
          float m2 = fmaxf(fmaxf(x[rt][8], x[rt][9]), fmaxf(x[rt][10], x[rt][11]));
          float m3 = fmaxf(fmaxf(x[rt][12], x[rt][13]), fmaxf(x[rt][14], x[rt][15]));
          mt[rt] = wave_max_x4(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)));
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int row = row_base + 16 * rt + l16;
          mt[rt] = -INFINITY;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = k0 + 16 * tt + 4 * g + r;
              const bool ok = key < kend && (!p.causal || key <= row);
              x[rt][4 * tt + r] = ok ? sacc[rt][tt][r] : -INFINITY;
              mt[rt] = fmaxf(mt[rt], x[rt][4 * tt + r]);
            }
          }
          mt[rt] = wave_max_x4(mt[rt]);
        }
      }
      // ---- online softmax, one rescale decision for the wave
      const bool grow = (mt[0] - m_used[0]) * sl2 > kRescaleThreshold ||
                        (mt[1] - m_used[1]) * sl2 > kRescaleThreshold;
      const bool upd = __builtin_amdgcn_ballot_w64(grow) != 0;
      float alpha[2], nref[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float mn = upd ? fmaxf(m_used[rt], mt[rt]) : m_used[rt];
        alpha[rt] = (upd && mn != -INFINITY) ? __builtin_amdgcn_exp2f((m_used[rt] - mn) * sl2) : 1.f;
        m_used[rt] = mn;
        l_part[rt] *= alpha[rt];
        nref[rt] = mn == -INFINITY ? 0.f : -mn * sl2;
      }
      bf16x8 pb[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[rt][i], sl2, nref[rt]));
          l_part[rt] += pv[i];
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x2 a0 = to_bf16x2(pv[8 * kk + 0], pv[8 * kk + 1]);
          const bf16x2 a1 = to_bf16x2(pv[8 * kk + 2], pv[8 * kk + 3]);
          const bf16x2 a2 = to_bf16x2(pv[8 * kk + 4], pv[8 * kk + 5]);
          const bf16x2 a3 = to_bf16x2(pv[8 * kk + 6], pv[8 * kk + 7]);
          pb[rt][kk] = bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
        }
      }
      if (upd) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) o[rt][ct] *= alpha[rt];
      }
      // ---- O^T += V^T P^T over 8 column tiles and 2 k-steps of 32 keys
      const char* vb = v_lds[buf] + l16 * kVRowB + 16 * g;
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 vf = *(const bf16x8*)(vb + ct * 16 * kVRowB + 64 * kk);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[rt][kk], o[rt][ct], 0, 0, 0);
        }
      }
    }
    if (j + 1 < nblocks) store_block((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane (l16, g) holds columns 16 ct + 4 g .. + 3 of its
  //      row; a swap between 16-lane groups over tiles 2 c and 2 c + 1
  //      leaves lane group g with 8 consecutive columns 16 (2 c + (g & 1)) +
  //      8 (g >> 1) .. + 7, so each store writes 64 contiguous bytes of a row
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = row_base + 16 * rt + l16;
    const float lt = wave_sum_x4(l_part[rt]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* op = p.o + ((size_t)(seq0 + (row < n ? row : 0)) * H + h) * kVD;
#pragma unroll
    for (int c = 0; c < kCT / 2; ++c) {
      const f32x4 x0 = o[rt][2 * c] * inv, x1 = o[rt][2 * c + 1] * inv;
      const bf16x2 a0 = to_bf16x2(x0[0], x0[1]), b0 = to_bf16x2(x0[2], x0[3]);
      const bf16x2 a1 = to_bf16x2(x1[0], x1[1]), b1 = to_bf16x2(x1[2], x1[3]);
      const u32x2 s0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a0),
                                                        __builtin_bit_cast(unsigned, a1), false,
                                                        false);
      const u32x2 s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, b0),
                                                        __builtin_bit_cast(unsigned, b1), false,
                                                        false);
      if (row < n)
        *(i32x4*)(op + 16 * (2 * c + (g & 1)) + 8 * (g >> 1)) =
            i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
    }
    if (row < n && g == 0)
      p.lse[(size_t)(seq0 + row) * H + h] =
          lt > 0.f ? (m_used[rt] * sl2 + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_prefill_attention(const mla::PrefillParams* prm, int batch,
                                                   int max_seqlen, hipStream_t stream) {
  const int qblocks = (max_seqlen + mla::pf::kBQ - 1) / mla::pf::kBQ;
  if (qblocks <= 0) return hipSuccess;
  const dim3 grid(prm->H, batch, qblocks);
  hipLaunchKernelGGL(mla::prefill_attention_kernel, grid, dim3(mla::pf::kThreads), 0, stream,
                     *prm);
  return hipGetLastError();
}
