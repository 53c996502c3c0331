// Quantization of the latent cache to FP8 records.
//
// FP8 is the pages' format for matrix products, training and communication
// (DeepSeek-V3 hardware paper summary, section on FP8 mixed precision); using
// it for the attention cache is an extension of this library.  Each 576-value
// bf16 cache entry becomes a 656-byte record:
//   [0, 512)    the latent values as OCP E4M3 codes,
//   [512, 528)  four float32 scales 2^e, one per 128 latent values,
//   [528, 656)  the 64 rotary values, bf16, unchanged.
// A block's e is the smallest integer with max|x| <= 448 * 2^e (0 for an
// all-zero block); a value is stored as the E4M3 code nearest x * 2^-e,
// ties to the even code, with the sign of x.  Since the scale is a power of
// two, code * scale is exactly a bf16 value again.
//
// One wave per token: lane l holds latent values 8 l .. 8 l + 7 (block
// l / 16); the block maximum is a 16-lane reduction.

#include "mla_device.h"

namespace mla {

constexpr int kF8Bytes = 656;

// Smallest e with a <= 448 * 2^e: a = f * 2^k with f in [0.5, 1), and
// 448 * 2^(k - 9) = 1.75 * 2^(k - 1).
__device__ __forceinline__ int f8_block_exponent(float a) {
  if (a == 0.f) return 0;
  int k;
  const float f = frexpf(a, &k);
  return (k - 1) - 8 + (2.f * f > 1.75f ? 1 : 0);
}

// Magnitude code of E4M3 nearest to a in [0, 448]: with k = max(floor(log2 a),
// -6) the codes of binade k are (k + 6) * 8 + n for n = a / 2^(k - 3) in
// [8, 16] (n = 16 is the next binade's first code), and the subnormals below
// 2^-6 are n = a / 2^-9 in [0, 8]; rint rounds half to even, and the code's
// parity is n's, so ties go to the even code.
__device__ __forceinline__ unsigned f8_code(float y, unsigned sign) {
  const float a = fminf(fabsf(y), 448.f);
  int k = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
  k = k < -6 ? -6 : k;
  const int n = (int)__builtin_rintf(ldexpf(a, 3 - k));
  int mag = (k + 6) * 8 + n;
  mag = mag > 126 ? 126 : mag;
  return sign | (unsigned)mag;
}

__global__ void __launch_bounds__(256) kv_quantize_fp8_kernel(const uint16_t* __restrict__ kv,
                                                              int n_tokens,
                                                              uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= n_tokens) return;  // whole waves
  const uint16_t* x = kv + (size_t)tok * kD;
  uint8_t* rec = out + (size_t)tok * kF8Bytes;
  const i32x4 raw = *(const i32x4*)(x + 8 * lane);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float((unsigned)raw[i] << 16);
    f[2 * i + 1] = __uint_as_float((unsigned)raw[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const int e = f8_block_exponent(amax);
  unsigned lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned sign = (__float_as_uint(f[i]) >> 24) & 0x80u;
    const unsigned c = f8_code(ldexpf(f[i], -e), sign);
    if (i < 4)
      lo |= c << (8 * i);
    else
      hi |= c << (8 * (i - 4));
  }
  *(i32x2*)(rec + 8 * lane) = i32x2{(int)lo, (int)hi};
  if ((lane & 15) == 0) *(float*)(rec + kDv + 4 * (lane >> 4)) = ldexpf(1.f, e);
  if (lane < 8) *(i32x4*)(rec + kDv + 16 + 16 * lane) = *(const i32x4*)(x + kDv + 8 * lane);
}

}  // namespace mla

extern "C" hipError_t mla_launch_kv_quantize_fp8(const uint16_t* kv, int n_tokens, uint8_t* out,
                                                 hipStream_t stream) {
  hipLaunchKernelGGL(mla::kv_quantize_fp8_kernel, dim3((n_tokens + 3) / 4), dim3(256), 0, stream, kv,
                     n_tokens, out);
  return hipGetLastError();
}
