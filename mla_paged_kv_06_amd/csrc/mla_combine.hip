// LSE combine of split partials.  Splitting one sequence's keys over several
// compute units and merging the partial results is this library's design for
// balancing variable-length sequences (the FlashMLA release note says only
// that its kernel is tuned for variable-length sequences; the get-metadata /
// decode / combine call split follows the problem statement).  The merge is
// exact: with s_k the scores of split k, lse = ln sum_k exp(lse_k) and
// out = sum_k exp(lse_k - lse) o_k reproduce the unsplit softmax.

#include "mla_device.h"

namespace mla {

// Combine: merge split partials by log-sum-exp.  One wave per query row
// (4 rows per workgroup), 8 output columns per lane.  The partial rows of the
// first kCombineUnroll splits are requested before anything else, so their
// loads overlap those of the split lse values; lane t computes the weights
// of splits t and t + 64, broadcast from it where they are summed (weights
// of splits past 128 are computed again from memory).
constexpr int kCombineRows = 4;
constexpr int kCombineUnroll = 8;  // partial rows in flight per lane

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// 8 bf16 partial values (16 bytes) -> two float32 quadruples, exactly
__device__ __forceinline__ void widen8(i32x4 r, f32x4& lo, f32x4& hi) {
  lo = f32x4{__uint_as_float((unsigned)r[0] << 16), __uint_as_float((unsigned)r[0] & 0xFFFF0000u),
             __uint_as_float((unsigned)r[1] << 16), __uint_as_float((unsigned)r[1] & 0xFFFF0000u)};
  hi = f32x4{__uint_as_float((unsigned)r[2] << 16), __uint_as_float((unsigned)r[2] & 0xFFFF0000u),
             __uint_as_float((unsigned)r[3] << 16), __uint_as_float((unsigned)r[3] & 0xFFFF0000u)};
}

__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ o_acc,
                                                      const float* __restrict__ lse_acc,
                                                      const int32_t* __restrict__ splits, int R,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  constexpr int U = kCombineUnroll;
  const int b = blockIdx.y;
  const int wv = threadIdx.x >> 6;
  const int row = blockIdx.x * kCombineRows + wv;
  const int t = threadIdx.x & 63;
  const int s0 = __builtin_amdgcn_readfirstlane(splits[b]);
  const int ns = __builtin_amdgcn_readfirstlane(splits[b + 1]) - s0;
  if (ns <= 1 || row >= R) return;  // uniform per wave; no block barrier below
  const float* lrow = lse_acc + (size_t)s0 * R + row;
  const uint16_t* orow_acc = o_acc + ((size_t)s0 * R + row) * kDv + 8 * t;
  i32x4 v[U];  // raw bf16 partial values, widened where they are summed
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < ns) {
      const uint16_t* src = orow_acc + (size_t)u * R * kDv;
      v[u] = *(const i32x4*)src;
    } else {
      v[u] = i32x4{0, 0, 0, 0};
    }
  }
  // split weights: lanes over splits, a wave max and sum
  const float l0 = t < ns ? lrow[(size_t)t * R] : -INFINITY;
  float l1 = -INFINITY;
  if (ns > 64 && t + 64 < ns) l1 = lrow[(size_t)(t + 64) * R];  // ns is wave-uniform
  float mx = fmaxf(l0, l1);
  for (int s = t + 128; s < ns; s += 64) mx = fmaxf(mx, lrow[(size_t)s * R]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
  uint16_t* orow = out + ((size_t)b * R + row) * kDv + 8 * t;
  if (mx == -INFINITY) {
    *(i32x4*)orow = i32x4{0, 0, 0, 0};
    if (t == 0) lse[(size_t)b * R + row] = -INFINITY;
    return;
  }
  const float e0 = __builtin_amdgcn_exp2f(l0 - mx);  // -inf -> 0
  const float e1 = __builtin_amdgcn_exp2f(l1 - mx);
  float z = e0 + e1;
  for (int s = t + 128; s < ns; s += 64) z += __builtin_amdgcn_exp2f(lrow[(size_t)s * R] - mx);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) z += __shfl_xor(z, d);
  const float inv = 1.f / z;
  const float w0 = e0 * inv, w1 = e1 * inv;  // weights of splits t and t + 64
  auto weight = [&](int si) __attribute__((always_inline)) {
    return si < 64    ? lane_value(w0, si)
           : si < 128 ? lane_value(w1, si - 64)
                      : __builtin_amdgcn_exp2f(lrow[(size_t)si * R] - mx) * inv;
  };
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < ns) {
      const float w = weight(u);
      f32x4 lo, hi;
      widen8(v[u], lo, hi);
      a0 += w * lo;
      a1 += w * hi;
    }
  }
  for (int s = U; s < ns; s += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < ns) {
        const uint16_t* src = orow_acc + (size_t)(s + u) * R * kDv;
        v[u] = *(const i32x4*)src;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < ns) {
        const float w = weight(s + u);
        f32x4 lo, hi;
        widen8(v[u], lo, hi);
        a0 += w * lo;
        a1 += w * hi;
      }
    }
  }
  bf16x2 r0 = to_bf16x2(a0[0], a0[1]);
  bf16x2 r1 = to_bf16x2(a0[2], a0[3]);
  bf16x2 r2 = to_bf16x2(a1[0], a1[1]);
  bf16x2 r3 = to_bf16x2(a1[2], a1[3]);
  *(bf16x8*)orow = bf16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  if (t == 0) lse[(size_t)b * R + row] = (mx + __builtin_amdgcn_logf(z)) * kLn2;
}

// Combine for sequences split many ways (few long sequences spread over the
// whole GPU): one workgroup per query row, the four waves taking every fourth
// split, so that all partial rows of a row are in flight in one round.  Each
// wave accumulates its weighted partials (8 columns per lane); the four sums
// meet in LDS and each wave finishes 128 columns.
constexpr int kWideUnroll = 8;  // partial rows in flight per wave

__global__ void __launch_bounds__(256) combine_wide_kernel(const uint16_t* __restrict__ o_acc,
                                                           const float* __restrict__ lse_acc,
                                                           const int32_t* __restrict__ splits,
                                                           int R, uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  __shared__ f32x4 s_acc[kWaves][2][64];
  const int b = blockIdx.y;
  const int row = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = threadIdx.x & 63;
  const int s0 = __builtin_amdgcn_readfirstlane(splits[b]);
  const int ns = __builtin_amdgcn_readfirstlane(splits[b + 1]) - s0;
  if (ns <= 1) return;  // uniform over the workgroup
  const float* lrow = lse_acc + (size_t)s0 * R + row;
  const uint16_t* base = o_acc + ((size_t)s0 * R + row) * kDv + 8 * t;
  // this wave's first kWideUnroll partial rows (splits wv, wv + 4, ...) are
  // requested first: their loads overlap those of the lse values.  Indexes
  // past the last split read the last one again and are never summed (a
  // load under a branch made the compiler wait for it on the spot).
  i32x4 v[kWideUnroll];  // raw bf16 partial values, widened where they are summed
#pragma unroll
  for (int u = 0; u < kWideUnroll; ++u) {
    const int si = min(wv + kWaves * u, ns - 1);
    v[u] = *(const i32x4*)(base + (size_t)si * R * kDv);
  }
  // max and sum of the split weights (lanes over splits; every wave computes
  // the same values)
  const float l0 = t < ns ? lrow[(size_t)t * R] : -INFINITY;
  float l1 = -INFINITY;
  if (ns > 64 && t + 64 < ns) l1 = lrow[(size_t)(t + 64) * R];  // ns is wave-uniform
  float mx = fmaxf(l0, l1);
  for (int s = t + 128; s < ns; s += 64) mx = fmaxf(mx, lrow[(size_t)s * R]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
  uint16_t* orow = out + ((size_t)b * R + row) * kDv;
  if (mx == -INFINITY) {  // no split saw a token: uniform over the workgroup
    if (wv == 0) {
      *(i32x4*)(orow + 8 * t) = i32x4{0, 0, 0, 0};
      if (t == 0) lse[(size_t)b * R + row] = -INFINITY;
    }
    return;
  }
  const float e0 = __builtin_amdgcn_exp2f(l0 - mx);  // -inf -> 0
  const float e1 = __builtin_amdgcn_exp2f(l1 - mx);
  float z = e0 + e1;
  for (int s = t + 128; s < ns; s += 64) z += __builtin_amdgcn_exp2f(lrow[(size_t)s * R] - mx);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) z += __shfl_xor(z, d);
  const float inv = 1.f / z;
  const float w0 = e0 * inv, w1 = e1 * inv;  // weights of splits t and t + 64
  auto weight = [&](int si) __attribute__((always_inline)) {
    return si < 64    ? lane_value(w0, si)
           : si < 128 ? lane_value(w1, si - 64)
                      : __builtin_amdgcn_exp2f(lrow[(size_t)si * R] - mx) * inv;
  };
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  for (int s = wv; s < ns; s += kWaves * kWideUnroll) {
    if (s != wv) {
#pragma unroll
      for (int u = 0; u < kWideUnroll; ++u) {
        const int si = s + kWaves * u;
        if (si < ns) {
          const uint16_t* src = base + (size_t)si * R * kDv;
          v[u] = *(const i32x4*)src;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kWideUnroll; ++u) {
      const int si = s + kWaves * u;
      if (si < ns) {
        const float w = weight(si);
        f32x4 lo, hi;
        widen8(v[u], lo, hi);
        a0 += w * lo;
        a1 += w * hi;
      }
    }
  }
  s_acc[wv][0][t] = a0;
  s_acc[wv][1][t] = a1;
  __syncthreads();
  // wave wv finishes columns 128 wv .. 128 wv + 127: lane t < 32 takes the
  // four columns held by source lane 16 wv + t / 2, half t & 1
  if (t < 32) {
    const int src = 16 * wv + (t >> 1);
    const int h = t & 1;
    f32x4 acc = s_acc[0][h][src];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) acc += s_acc[k][h][src];
    const bf16x2 x = to_bf16x2(acc[0], acc[1]);
    const bf16x2 y = to_bf16x2(acc[2], acc[3]);
    *(bf16x4*)(orow + 8 * src + 4 * h) = bf16x4{x[0], x[1], y[0], y[1]};
  }
  if (wv == 0 && t == 0) lse[(size_t)b * R + row] = (mx + __builtin_amdgcn_logf(z)) * kLn2;
}

}  // namespace mla

// wide: the caller's estimate that sequences are split many ways (partitions
// well above the batch); the result is the same either way.
extern "C" hipError_t mla_launch_combine(const uint16_t* o_acc, const float* lse_acc,
                                         const int32_t* splits, int batch, int R, uint16_t* out,
                                         float* lse, int wide, hipStream_t stream) {
  if (wide) {
    hipLaunchKernelGGL(mla::combine_wide_kernel, dim3(R, batch), dim3(256), 0, stream, o_acc,
                       lse_acc, splits, R, out, lse);
  } else {
    const dim3 grid((R + mla::kCombineRows - 1) / mla::kCombineRows, batch);
    hipLaunchKernelGGL(mla::combine_kernel, grid, dim3(256), 0, stream, o_acc, lse_acc, splits, R,
                       out, lse);
  }
  return hipGetLastError();
}
