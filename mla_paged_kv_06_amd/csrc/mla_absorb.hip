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
// A workgroup of 4 waves owns one head, NCOL output columns and up to
// kRowChunk rows.  Its NCOL x K slice of W (64 KiB) is staged in LDS once;
// the waves split the rows, wave w taking 16-row tiles w, w + 4, ..., each
// streaming its own activation rows with the next D tiles in flight (a ring
// of D + 1 register buffers), so the four waves keep distinct bytes in
// flight.  MFMA 16x16x32 with W as the A operand (read from LDS) and the
// activation rows as B gives D^T[n][m], so each lane stores 4 consecutive
// output columns of one row.  Every weight is read from HBM once per
// kRowChunk rows (once at decode batch sizes).

#include "mla_device.h"

namespace mla {

constexpr int kNope = 128;       // per-head query part and value head width
constexpr int kRope = kD - kDv;  // 64
constexpr int kRowChunk = 256;   // rows per workgroup (blockIdx.x)

template <int K, int NCOL, int D>
__global__ void __launch_bounds__(256, 2) absorb_kernel(const uint16_t* __restrict__ act,
                                                     int act_stride,
                                                     const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ out, int out_stride,
                                                     int M, int H, int N,
                                                     const uint16_t* __restrict__ rope,
                                                     int rope_stride) {
  constexpr int KS = K / 32;       // k-steps per tile
  constexpr int CT = NCOL / 16;    // 16-column output tiles
  constexpr int kRowB = 2 * K + 16;  // LDS row of W: padded so that the 16 rows
                                     // one fragment read touches hit distinct banks
  __shared__ __attribute__((aligned(16))) char w_lds[NCOL * kRowB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int h = blockIdx.z;
  const int n0 = blockIdx.y * NCOL;
  const int m_begin = blockIdx.x * kRowChunk;
  const int m_end = min(M, m_begin + kRowChunk);
  const int n_tiles = (m_end - m_begin + 15) / 16;

  // rows of tile t: row m_begin + 16 t + l16 of head h (rows past the end
  // load the first row and are never stored)
  auto load_tile = [&](int t, bf16x8 (&af)[KS]) __attribute__((always_inline)) {
    int m = m_begin + 16 * t + l16;
    m = m < m_end ? m : m_begin;
    const uint16_t* a = act + ((size_t)m * H + h) * act_stride + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) af[ks] = *(const bf16x8*)(a + 32 * ks);
  };

  // this wave's tiles: wave, wave + 4, ...; the first D go out before W is staged
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;
  bf16x8 ring[D + 1][KS];
  static_for<0, D>([&](auto ic) __attribute__((always_inline)) {
    load_tile(wave + 4 * decltype(ic)::value, ring[decltype(ic)::value]);
  });

  // W slice into LDS: NCOL rows of K values (row n0 + r of head h), 16-byte pieces
  {
    constexpr int kPieces = NCOL * K / 8;
    constexpr int kPer = kPieces / 256;
    const uint16_t* wh = w + ((size_t)h * N + n0) * K;
    uint4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) v[u] = *(const uint4*)(wh + 8 * (u * 256 + tid));
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * 256 + tid;
      const int r = i / (K / 8), c = i % (K / 8);
      *(uint4*)(w_lds + r * kRowB + 16 * c) = v[u];
    }
  }
  __syncthreads();

  // A fragment of column tile ct, k-step ks: row 16 ct + l16, k = 32 ks + 8 g
  const char* wl = w_lds + l16 * kRowB + 16 * g;
  auto compute_tile = [&](int t, const bf16x8 (&af)[KS], bool full) __attribute__((always_inline)) {
    const int m = m_begin + 16 * t + l16;
    // W fragments are read from LDS for every tile: left to itself the
    // compiler keeps the whole 64 KiB slice in registers (one wave per SIMD)
    int wo = 0;
    asm volatile("" : "+v"(wo));
    uint16_t* o = out + ((size_t)m * H + h) * out_stride + n0 + 4 * g;
    const bool live = full || m < m_end;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 wf = *(const bf16x8*)(wl + wo + 16 * ct * kRowB + 64 * ks);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, af[ks], acc, 0, 0, 0);
      }
      // lane (g, l16) holds columns n0 + 16 ct + 4 g + r of row m
      if (live) {
        const bf16x2 a = to_bf16x2(acc[0], acc[1]);
        const bf16x2 b = to_bf16x2(acc[2], acc[3]);
        *(bf16x4*)(o + 16 * ct) = bf16x4{a[0], a[1], b[0], b[1]};
      }
    }
  };

  // Main loop over this wave's whole tiles with no branch inside: every step
  // issues the loads of the tile D ahead (clamped rows past the end) and
  // stores a whole tile, so the compiler can count the loads in flight and
  // wait only for the tile it computes.  The last ones follow, with the
  // ragged tile (if any, the batch's last) stored row by row.
  const int n_full = (m_end - m_begin) / 16;
  const int my_full = n_full > wave ? (n_full - wave + 3) / 4 : 0;
  int i0 = 0;
  for (; i0 + D + 1 <= my_full; i0 += D + 1) {
    static_for<0, D + 1>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      load_tile(wave + 4 * (i0 + u + D), ring[(u + D) % (D + 1)]);
      compute_tile(wave + 4 * (i0 + u), ring[u], true);
    });
  }
  // this wave's tiles i0 .. my_tiles - 1 (at most D + 1): i0 .. i0 + D - 1
  // are in ring buffers 0 .. D - 1; i0 + D still has to be loaded
  load_tile(wave + 4 * (i0 + D), ring[D]);
  static_for<0, D + 1>([&](auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    if (i0 + u < my_tiles) compute_tile(wave + 4 * (i0 + u), ring[u], false);
  });

  // the rotary part of the absorbed query passes through unchanged: 16-byte
  // pieces (8 per row), shared by the head's column workgroups, all of a
  // thread's loads in flight before its stores
  if (rope != nullptr) {
    constexpr int kPieces = kRope / 8;
    constexpr int kU = 8;
    const int total = (m_end - m_begin) * kPieces;
    const int stride = 256 * gridDim.y;
    for (int base = blockIdx.y * 256 + threadIdx.x; base < total; base += kU * stride) {
      uint4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * stride;
        const int m = m_begin + (i < total ? i : 0) / kPieces;
        const int c = 8 * ((i < total ? i : 0) % kPieces);
        v[u] = *(const uint4*)(rope + ((size_t)m * H + h) * rope_stride + c);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * stride;
        if (i < total) {
          const int m = m_begin + i / kPieces;
          const int c = 8 * (i % kPieces);
          *(uint4*)(out + ((size_t)m * H + h) * out_stride + kDv + c) = v[u];
        }
      }
    }
  }
}

// tiles in flight ahead of the one computed, per wave (registers: rows
// 4 KS (D + 1)); a workgroup's 16 tiles are 4 per wave.  Two workgroups fit
// a CU (registers and 2 x 68 KiB of LDS).
constexpr int kQueryDepth = 3;   // K = 128: 16 registers per tile
constexpr int kOutputDepth = 2;  // K = 512: 64 per tile

}  // namespace mla

// q_out[m, h, 0:512] = W_UK,h^T q_c[m, h];  q_out[m, h, 512:576] = q_r[m, h]
extern "C" hipError_t mla_launch_absorb_query(const uint16_t* q_c, const uint16_t* q_r,
                                              const uint16_t* w_uk_t, int M, int H,
                                              uint16_t* q_out, hipStream_t stream) {
  using namespace mla;
  // 256 columns (a 64 KiB slice of W) per workgroup
  const dim3 grid((M + kRowChunk - 1) / kRowChunk, kDv / 256, H);
  hipLaunchKernelGGL((absorb_kernel<kNope, 256, kQueryDepth>), grid, dim3(256), 0, stream, q_c,
                     kNope, w_uk_t, q_out, kD, M, H, kDv, q_r, kRope);
  return hipGetLastError();
}

// o[m, h, :] = W_UV,h out[m, h, :]
extern "C" hipError_t mla_launch_absorb_output(const uint16_t* lat_out, const uint16_t* w_uv,
                                               int M, int H, uint16_t* o, hipStream_t stream) {
  using namespace mla;
  // 64 columns (a 64 KiB slice of W) per workgroup
  const dim3 grid((M + kRowChunk - 1) / kRowChunk, kNope / 64, H);
  hipLaunchKernelGGL((absorb_kernel<kDv, 64, kOutputDepth>), grid, dim3(256), 0, stream, lat_out,
                     kDv, w_uv, o, kNope, M, H, kNope, (const uint16_t*)nullptr, 0);
  return hipGetLastError();
}
