// Absorption products on either side of the latent decode.
//
// Keys and values are kept as one compressed latent per token and widened
// per head only at compute time (FlashMLA release note, paragraph on the MLA
// core principles; DeepSeek-V3 summary, paragraph on memory efficiency: the
// up-projections fold every head's K and V into the one latent).  With head h
// keys k = [W_UK,h c ; r] and values v = W_UV,h c, the score of query
// [q_c ; q_r] is (W_UK,h^T q_c) . c + q_r . r, so the decode runs on the
// absorbed query q~ = [W_UK,h^T q_c ; q_r] (576 values) against the cached
// [c ; r], and the head's output is W_UV,h applied to the 512-value latent
// output.  The per-head query part is 128 values (the 192 = 128 + 64 query
// width behind the 1/sqrt(192) scale) and so is the value head.
//
// Both products are C[m][n] = sum_k A[m][k] W[n][k] per head, with the
// contraction index contiguous in W:
//   query:  A = q_c rows (K = 128), W = W_UK,h^T stored [512][128], C = q~[0:512]
//   output: A = latent output rows (K = 512), W = W_UV,h stored [128][512], C = o
// m runs over the batch * s_q query tokens.  They are bound by reading the
// weights and activations once (2 flops per weight byte per row, far below
// the matrix-core ridge at decode batch sizes).
//
// A workgroup of 4 waves owns one head, 4 * 16 * NT output columns and up
// to kRowChunk rows; each wave keeps its 16 NT columns of W (all of K) in
// registers and walks the rows in 16-row tiles: MFMA 16x16x32 with W as the
// A operand and the activation rows as B gives D^T[n][m], so each lane
// stores 4 consecutive output columns of one row.  Every weight is read once
// per kRowChunk rows (once at decode batch sizes).

#include "mla_device.h"

namespace mla {

constexpr int kNope = 128;       // per-head query part and value head width
constexpr int kRope = kD - kDv;  // 64
constexpr int kRowChunk = 256;   // rows per workgroup (blockIdx.x)

// A workgroup walks its rows in 16-row tiles with the next D tiles' rows
// already in flight (a ring of D + 1 register buffers), so the loads of later
// tiles overlap the matrix instructions of the current one.
template <int K, int NT, int D>
__global__ void __launch_bounds__(256) absorb_kernel(const uint16_t* __restrict__ act,
                                                     int act_stride,
                                                     const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ out, int out_stride,
                                                     int M, int H, int N,
                                                     const uint16_t* __restrict__ rope,
                                                     int rope_stride) {
  constexpr int KS = K / 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int h = blockIdx.z;
  const int n0 = (blockIdx.y * 4 + wave) * 16 * NT;
  const int m_begin = blockIdx.x * kRowChunk;
  const int m_end = min(M, m_begin + kRowChunk);
  const int n_tiles = (m_end - m_begin + 15) / 16;

  // this wave's W columns: row n0 + 16 nt + l16 of head h, k = 32 ks + 8 g ..
  bf16x8 wf[NT][KS];
  const uint16_t* wh = w + (size_t)h * N * K;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      wf[nt][ks] = *(const bf16x8*)(wh + (size_t)(n0 + 16 * nt + l16) * K + 32 * ks + 8 * g);

  // rows of tile t: row m_begin + 16 t + l16 of head h (rows past the end
  // load the first row and are never stored)
  auto load_tile = [&](int t, bf16x8 (&af)[KS]) __attribute__((always_inline)) {
    int m = m_begin + 16 * t + l16;
    m = m < m_end ? m : m_begin;
    const uint16_t* a = act + ((size_t)m * H + h) * act_stride + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) af[ks] = *(const bf16x8*)(a + 32 * ks);
  };
  auto compute_tile = [&](int t, const bf16x8 (&af)[KS], bool full) __attribute__((always_inline)) {
    const int m = m_begin + 16 * t + l16;
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nt][ks], af[ks], acc[nt], 0, 0, 0);
    // lane (g, l16) holds columns n0 + 16 nt + 4 g + r of row m
    if (full || m < m_end) {
      uint16_t* o = out + ((size_t)m * H + h) * out_stride + n0 + 4 * g;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x2 a = to_bf16x2(acc[nt][0], acc[nt][1]);
        const bf16x2 b = to_bf16x2(acc[nt][2], acc[nt][3]);
        *(bf16x4*)(o + 16 * nt) = bf16x4{a[0], a[1], b[0], b[1]};
      }
    }
  };

  // Main loop over whole tiles with no branch inside: every step issues the
  // loads of the tile D ahead (clamped rows past the end) and stores a whole
  // tile, so the compiler can count the loads in flight and wait only for
  // the tile it computes.  The last whole tiles and a ragged one follow.
  const int n_full = (m_end - m_begin) / 16;
  bf16x8 ring[D + 1][KS];
  static_for<0, D>([&](auto ic) __attribute__((always_inline)) {
    load_tile(decltype(ic)::value, ring[decltype(ic)::value]);
  });
  int t0 = 0;
  for (; t0 + D + 1 <= n_full; t0 += D + 1) {
    static_for<0, D + 1>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      load_tile(t0 + u + D, ring[(u + D) % (D + 1)]);
      compute_tile(t0 + u, ring[u], true);
    });
  }
  // tiles t0 .. n_tiles - 1 (at most D + 1): tiles t0 .. t0 + D - 1 are in
  // ring buffers 0 .. D - 1 already; tile t0 + D (a ragged last tile after D
  // whole ones) still has to be loaded
  load_tile(t0 + D, ring[D]);
  static_for<0, D + 1>([&](auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    if (t0 + u < n_tiles) compute_tile(t0 + u, ring[u], false);
  });

  // the rotary part of the absorbed query passes through unchanged
  if (rope != nullptr && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < (m_end - m_begin) * (kRope / 4); i += 256) {
      const int m = m_begin + i / (kRope / 4);
      const int c = 4 * (i % (kRope / 4));
      *(uint2*)(out + ((size_t)m * H + h) * out_stride + kDv + c) =
          *(const uint2*)(rope + ((size_t)m * H + h) * rope_stride + c);
    }
  }
}

// tiles in flight ahead of the one computed (registers: W 64 + rows
// 4 KS (D + 1))
constexpr int kQueryDepth = 5;   // K = 128: 16 per tile
constexpr int kOutputDepth = 2;  // K = 512: 64 per tile

}  // namespace mla

// q_out[m, h, 0:512] = W_UK,h^T q_c[m, h];  q_out[m, h, 512:576] = q_r[m, h]
extern "C" hipError_t mla_launch_absorb_query(const uint16_t* q_c, const uint16_t* q_r,
                                              const uint16_t* w_uk_t, int M, int H,
                                              uint16_t* q_out, hipStream_t stream) {
  using namespace mla;
  // 4 waves x 64 columns = 256 columns per workgroup
  const dim3 grid((M + kRowChunk - 1) / kRowChunk, kDv / 256, H);
  hipLaunchKernelGGL((absorb_kernel<kNope, 4, kQueryDepth>), grid, dim3(256), 0, stream, q_c, kNope, w_uk_t,
                     q_out, kD, M, H, kDv, q_r, kRope);
  return hipGetLastError();
}

// o[m, h, :] = W_UV,h out[m, h, :]
extern "C" hipError_t mla_launch_absorb_output(const uint16_t* lat_out, const uint16_t* w_uv,
                                               int M, int H, uint16_t* o, hipStream_t stream) {
  using namespace mla;
  // 4 waves x 16 columns = 64 columns per workgroup
  const dim3 grid((M + kRowChunk - 1) / kRowChunk, kNope / 64, H);
  hipLaunchKernelGGL((absorb_kernel<kDv, 1, kOutputDepth>), grid, dim3(256), 0, stream, lat_out, kDv, w_uv, o,
                     kNope, M, H, kNope, (const uint16_t*)nullptr, 0);
  return hipGetLastError();
}
