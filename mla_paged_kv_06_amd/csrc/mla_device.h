// Device-side types, constants and small helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mla {

// Problem geometry: one 576-value bf16 latent per token (512 latent + 64
// rotary), 64 tokens per page, 512-value output (FlashMLA release note,
// paragraph on the released paged BF16 cache with block size 64).
constexpr int kD = 576;
constexpr int kDv = 512;
constexpr int kPage = 64;
constexpr int kRowBytes = kD * 2;                  // 1152 B per token
constexpr int kTileBytes = kPage * kRowBytes;      // 73728 B per page
constexpr int kChunksPerRow = kRowBytes / 16;      // 72 x 16 B
constexpr int kTileChunks = kPage * kChunksPerRow; // 4608
constexpr int kLoadsPerTile = kTileChunks / 64;    // 72 wave-wide 1 KiB loads
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerWave = kLoadsPerTile / kWaves;  // 18
constexpr int kRowGroup = 64;  // most query rows one workgroup holds
constexpr int kMetaInts = 8;
constexpr int kMaxParts = 4096;

// Word 3 of a raw buffer resource on CDNA3/4 (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max used for exponentiation is only raised when a new score
// exceeds it by this much (log2 units), so the accumulator is rarely rescaled;
// weights stay below 2^8, well inside fp32/bf16 range.
constexpr float kRescaleThreshold = 8.0f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

#define MLA_LDS __attribute__((address_space(3)))

// LDS layout of a page: token t's 72 16-byte chunks in row t (1152 B apart);
// logical chunk c sits at physical chunk c ^ swz(t), which spreads the 16
// tokens one MFMA fragment reads over distinct banks.  The XOR only touches
// the low 3 bits, so a chunk stays inside its 128-byte group and row.
__device__ __forceinline__ int swz(int t) { return t & 7; }

// s_waitcnt immediates for gfx9: vmcnt in [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8].
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0), others unconstrained
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0), others unconstrained
// vmcnt(9): all but the newest 9 vector-memory ops (one wave's half-page copy)
constexpr int kWaitVm9 = 0x0F70 | 9;
// vmcnt(18): all but the newest 18 vector-memory ops (one wave's page copy)
constexpr int kWaitVmPrefetch = 0x0F70 | (kLoadsPerWave & 15) | ((kLoadsPerWave >> 4) << 14);

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E) step S, so
// indices into register arrays are constants and never force scratch.
template <int B, int E, int S = 1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + S, E, S>(f);
  }
}

// Reductions over the four lanes l, l^16, l^32, l^48 that hold one query
// row.  v_permlane16_swap / v_permlane32_swap give each lane its own value and
// its xor-16 (xor-32) partner's, in either order; combining the two with a
// commutative op leaves bitwise-identical results in all four lanes.  Plain
// VALU: no trip through the LDS pipeline as a ds_bpermute shuffle would take.
__device__ __forceinline__ float wave_max_x4(float v) {
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_x4(float v) {
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, nearest-even
}

// Arguments of the decode kernel (filled by the C ABI after its checks).
struct DecodeParams {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* meta;
  int32_t* splits;  // written by kernels that schedule in-launch
  uint16_t* out;
  float* lse;
  uint16_t* o_acc;  // [slots][R][512] bf16: normalized split partials
  float* lse_acc;  // [slots][R]   (log2 domain)
  int batch, s_q, h_q, R, max_pages, num_parts, row_groups;
  int causal;
  float scale_log2;  // softmax_scale * log2(e)
  int sched_c0;      // fixed cost of the schedule rule (kernels that schedule in-launch)
};

// Arguments of the prefill attention kernel (filled by the C ABI after its checks).
struct PrefillParams {
  const uint16_t* q;       // [T][H][192]
  const uint16_t* k_nope;  // [T][H][128]
  const uint16_t* k_rope;  // row t at k_rope + t * rope_stride, 64 values
  const uint16_t* v;       // [T][H][128]
  const int32_t* cu;       // [batch + 1]
  uint16_t* o;             // [T][H][128]
  float* lse;              // [T][H]
  int rope_stride;
  int H;
  float scale_log2;
  int causal;
};

}  // namespace mla
