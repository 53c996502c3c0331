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

// the LDS-DMA copies write M0 in inline assembly (no compiled code of the
// expansion kernel uses M0)
#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

constexpr int kNope = 128;       // per-head query part and value head width
constexpr int kRope = kD - kDv;  // 64
constexpr int kRowChunk = 256;   // rows per workgroup (blockIdx.x)

template <int K, int NCOL, int D>
__global__ void __launch_bounds__(256, 2) absorb_kernel(const uint16_t* __restrict__ act,
                                                     int act_row, int act_head,
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
    const uint16_t* a = act + (size_t)m * act_row + (size_t)h * act_head + 8 * g;
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
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
#pragma unroll
    for (int cp = 0; cp < CT / 2; ++cp) {
      f32x4 acc[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 wf = *(const bf16x8*)(wl + wo + 16 * (2 * cp + e) * kRowB + 64 * ks);
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, af[ks], acc[e], 0, 0, 0);
        }
      }
      // lane (g, l16) holds columns n0 + 16 ct + 4 g + r of row m for the
      // tiles ct = 2 cp, 2 cp + 1; a swap between 16-lane groups leaves lane
      // group g with 8 consecutive columns 16 (2 cp + (g & 1)) + 8 (g >> 1)
      // .. + 7, so each store writes 64 contiguous bytes of a row
      const bf16x2 a0 = to_bf16x2(acc[0][0], acc[0][1]), b0 = to_bf16x2(acc[0][2], acc[0][3]);
      const bf16x2 a1 = to_bf16x2(acc[1][0], acc[1][1]), b1 = to_bf16x2(acc[1][2], acc[1][3]);
      const u32x2 s0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a0),
                                                        __builtin_bit_cast(unsigned, a1), false,
                                                        false);
      const u32x2 s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, b0),
                                                        __builtin_bit_cast(unsigned, b1), false,
                                                        false);
      if (live) {
        const int col = 16 * (2 * cp + (g & 1)) + 8 * (g >> 1);
        *(i32x4*)(o - 4 * g + col) = i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
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

// Prefill expansion as one matrix product per weight:
//   C[t][n] = sum_k latent[t][k] W[n][k],  n = 128 h + d,  k < 512,
// k_nope (W_UK) and v (W_UV) both [T][H][128] = [T][N].  One workgroup of 8
// waves per compute unit walks 256 x 256 tiles of C (wave w: rows 64 (w & 3)
// .., columns 128 (w >> 2) ..; 4 x 8 MFMA 16x16x32 tiles, 128 accumulators).
// The contraction runs in 8 stages of 64 values (two MFMA k-steps); each
// stage's 256 x 64 slices of the latents and of W (32 KiB each) are copied
// HBM -> LDS by LDS-DMA (buffer_load ... lds, eight 1 KiB copies per wave)
// into the other of two buffers while the current stage computes, and the
// last stage of a tile copies the first of the workgroup's next tile, so
// neither a tile's first copies nor its stores leave the matrix cores idle
// between tiles.  LDS
// rows are 128 bytes; the 16-byte chunk c of row r sits at c ^ (r & 7), so
// the rows one fragment read touches fall on distinct banks.  Buffer
// resources bounded at the last row (T, N) make rows past the ends read as
// zero.
namespace ex {
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kStages = kDv / kBK;  // 8
constexpr int kRing = 2;
constexpr int kSliceB = kBM * kBK * 2;  // 32 KiB
constexpr int kThreads = 512;
}  // namespace ex

__device__ __forceinline__ void ex_copy16(MLA_LDS char* lds, int voff, i32x4 rsrc, int soff) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)(size_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ i32x4 ex_rsrc(const void* base, int bytes) {
  const unsigned long long a = (unsigned long long)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF)),
               __builtin_amdgcn_readfirstlane(bytes), kBufferFlags};
}

template <int kImm>
__device__ __forceinline__ void ex_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(ex::kThreads, 1)
    expand_gemm_kernel(const uint16_t* __restrict__ latent, int latent_stride, int T,
                       const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, int N,
                       uint16_t* __restrict__ out0, uint16_t* __restrict__ out1, int n_tiles,
                       int tiles_m, int tiles_n) {
  using namespace ex;
  __shared__ __attribute__((aligned(1024))) char ring_[kRing * 2 * kSliceB];
  MLA_LDS char* ring = (MLA_LDS char*)ring_;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  // this wave's copies of a stage: 1 KiB pieces 4 w .. 4 w + 3 of the A and
  // of the B slice (piece i, lane l: row 8 i + l / 8, physical chunk l & 7)
  int va[4], vb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 8 * (4 * wave + u) + (lane >> 3);
    const int lc = (lane & 7) ^ (row & 7);
    va[u] = row * latent_stride * 2 + 16 * lc;
    vb[u] = row * kDv * 2 + 16 * lc;
  }
  // tiles of this workgroup: blockIdx.x, + gridDim.x, ...  (tile id: m
  // fastest, then n, then the weight); with a grid that is a multiple of
  // tiles_m every tile of a workgroup shares its latent rows
  struct Tile {
    int m0, n0, z;
  };
  auto tile_of = [&](int id) __attribute__((always_inline)) {
    Tile t;
    t.m0 = (id % tiles_m) * kBM;
    t.n0 = ((id / tiles_m) % tiles_n) * kBN;
    t.z = id / (tiles_m * tiles_n);
    return t;
  };
  auto issue = [&](const Tile& t, int st, int slot) __attribute__((always_inline)) {
    const uint16_t* w = t.z ? w1 : w0;
    const int rows_a = min(kBM, T - t.m0), rows_b = min(kBN, N - t.n0);
    const i32x4 ra = ex_rsrc(latent + (size_t)t.m0 * latent_stride, rows_a * latent_stride * 2);
    const i32x4 rb = ex_rsrc(w + (size_t)t.n0 * kDv, rows_b * kDv * 2);
    MLA_LDS char* buf = ring + slot * 2 * kSliceB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ex_copy16(buf + 1024 * (4 * wave + u), va[u], ra, st * kBK * 2);
      ex_copy16(buf + kSliceB + 1024 * (4 * wave + u), vb[u], rb, st * kBK * 2);
    }
  };
  // fragment rows: A row 64 (w & 3) + 16 mt + l16, B row 128 (w >> 2) + 16 nt + l16;
  // k-step ks of a stage reads logical chunk 4 ks + g of its row
  const int fa0 = (64 * (wave & 3) + l16) * 128 + 16 * (g ^ (l16 & 7));
  const int fa1 = (64 * (wave & 3) + l16) * 128 + 16 * ((4 + g) ^ (l16 & 7));
  const int fb0 = kSliceB + (128 * (wave >> 2) + l16) * 128 + 16 * (g ^ (l16 & 7));
  const int fb1 = kSliceB + (128 * (wave >> 2) + l16) * 128 + 16 * ((4 + g) ^ (l16 & 7));

  int id = blockIdx.x;
  if (id >= n_tiles) return;
  Tile cur = tile_of(id);
  issue(cur, 0, 0);
  int gstage = 0;  // stages computed by this workgroup so far (ring position)
  for (;;) {
    const int next_id = id + (int)gridDim.x;
    const bool has_next = next_id < n_tiles;
    const Tile nxt = tile_of(has_next ? next_id : id);
    f32x4 acc[8][4];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < kStages; ++st, ++gstage) {
      ex_wait<0x0F70>();             // this wave's copies of this stage landed
      __builtin_amdgcn_s_barrier();  // every wave's copies landed; the last stage read
      asm volatile("" ::: "memory");
      // the next stage: of this tile, or the first of the next one
      if (st + 1 < kStages)
        issue(cur, st + 1, (gstage + 1) & (kRing - 1));
      else if (has_next)
        issue(nxt, 0, (gstage + 1) & (kRing - 1));
      const MLA_LDS char* buf = ring + (gstage & (kRing - 1)) * 2 * kSliceB;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 af[4], bf[8];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = *(const MLA_LDS bf16x8*)(buf + (ks ? fa1 : fa0) + 2048 * mt);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          bf[nt] = *(const MLA_LDS bf16x8*)(buf + (ks ? fb1 : fb0) + 2048 * nt);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[nt][mt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[nt], af[mt], acc[nt][mt], 0, 0, 0);
      }
    }
    // lane (g, l16) holds columns 4 g .. 4 g + 3 of each 16-column tile, row
    // l16; a swap between 16-lane groups over tiles 2 p and 2 p + 1 leaves
    // lane group g with 8 consecutive columns 16 (2 p + (g & 1)) + 8 (g >> 1)
    // .. + 7, so each store writes 64 contiguous bytes of a row
    const int ncol = cur.n0 + 128 * (wave >> 2);
    uint16_t* out = cur.z ? out1 : out0;
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = cur.m0 + 64 * (wave & 3) + 16 * mt + l16;
      uint16_t* o = out + (size_t)m * N + ncol;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f32x4 x0 = acc[2 * p][mt], x1 = acc[2 * p + 1][mt];
        const bf16x2 a0 = to_bf16x2(x0[0], x0[1]), b0 = to_bf16x2(x0[2], x0[3]);
        const bf16x2 a1 = to_bf16x2(x1[0], x1[1]), b1 = to_bf16x2(x1[2], x1[3]);
        const u32x2 s0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a0),
                                                          __builtin_bit_cast(unsigned, a1), false,
                                                          false);
        const u32x2 s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, b0),
                                                          __builtin_bit_cast(unsigned, b1), false,
                                                          false);
        if (m < T && ncol < N)
          *(i32x4*)(o + 16 * (2 * p + (g & 1)) + 8 * (g >> 1)) =
              i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
      }
    }
    if (!has_next) break;
    id = next_id;
    cur = nxt;
  }
  ex_wait<0x0F70>();  // nothing may still fly when the wave ends
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
  // 256 columns (a 64 KiB slice of W) per workgroup; with fewer workgroups
  // than compute units that way (decode-size batches), 128 columns, so that
  // twice as many CUs stream the weights
  const int chunks = (M + kRowChunk - 1) / kRowChunk;
  if ((long long)chunks * (kDv / 256) * H < 256) {
    const dim3 grid(chunks, kDv / 128, H);
    hipLaunchKernelGGL((absorb_kernel<kNope, 128, kQueryDepth>), grid, dim3(256), 0, stream,
                       q_c, H * kNope, kNope, w_uk_t, q_out, kD, M, H, kDv, q_r, kRope);
  } else {
    const dim3 grid(chunks, kDv / 256, H);
    hipLaunchKernelGGL((absorb_kernel<kNope, 256, kQueryDepth>), grid, dim3(256), 0, stream,
                       q_c, H * kNope, kNope, w_uk_t, q_out, kD, M, H, kDv, q_r, kRope);
  }
  return hipGetLastError();
}

// o[m, h, :] = W_UV,h out[m, h, :]
extern "C" hipError_t mla_launch_absorb_output(const uint16_t* lat_out, const uint16_t* w_uv,
                                               int M, int H, uint16_t* o, hipStream_t stream) {
  using namespace mla;
  // 64 columns (a 64 KiB slice of W) per workgroup, 32 for decode-size
  // batches (as for the query product)
  const int chunks = (M + kRowChunk - 1) / kRowChunk;
  if ((long long)chunks * (kNope / 64) * H < 256) {
    const dim3 grid(chunks, kNope / 32, H);
    hipLaunchKernelGGL((absorb_kernel<kDv, 32, kOutputDepth>), grid, dim3(256), 0, stream,
                       lat_out, H * kDv, kDv, w_uv, o, kNope, M, H, kNope,
                       (const uint16_t*)nullptr, 0);
  } else {
    const dim3 grid(chunks, kNope / 64, H);
    hipLaunchKernelGGL((absorb_kernel<kDv, 64, kOutputDepth>), grid, dim3(256), 0, stream,
                       lat_out, H * kDv, kDv, w_uv, o, kNope, M, H, kNope,
                       (const uint16_t*)nullptr, 0);
  }
  return hipGetLastError();
}

// Prefill: every head's key (latent part) and value widened from the shared
// latent of each token, k_nope[t, h, :] = W_UK,h c_t and v[t, h, :] = W_UV,h c_t
// (the same product with the activation row shared by the heads: head
// stride 0).  c_t is the first 512 values of row t of `latent` (row stride
// latent_stride values).
extern "C" hipError_t mla_launch_prefill_expand(const uint16_t* latent, int latent_stride, int T,
                                                const uint16_t* w_uk, const uint16_t* w_uv, int H,
                                                uint16_t* k_nope, uint16_t* v, hipStream_t stream) {
  using namespace mla;
  const int N = H * kNope;
  const int tiles_m = (T + ex::kBM - 1) / ex::kBM, tiles_n = (N + ex::kBN - 1) / ex::kBN;
  const int n_tiles = tiles_m * tiles_n * 2;
  // persistent workgroups, one per compute unit, a multiple of tiles_m so
  // that each keeps its latent rows
  int grid = 256 / tiles_m * tiles_m;
  if (grid < tiles_m) grid = tiles_m;
  if (grid > n_tiles) grid = n_tiles;
  hipLaunchKernelGGL(expand_gemm_kernel, dim3(grid), dim3(ex::kThreads), 0, stream, latent,
                     latent_stride, T, w_uk, w_uv, N, k_nope, v, n_tiles, tiles_m, tiles_n);
  return hipGetLastError();
}
