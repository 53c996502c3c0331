// Split-KV tile scheduler: balances variable-length sequences over the GPU.
//
// The pages name variable-length sequences as what the decode kernel is tuned
// for (FlashMLA release note, introduction and the paragraph on dynamic
// sequence processing) and block-based paging (Tom's Hardware FR article,
// paragraph on the techniques).  How the work is cut is our own design:
//
//   * sequence b has n_b = max(1, ceil(L_b / 64)) page slots (an empty
//     sequence keeps one slot so that some partition writes its output) and
//     costs c_b = c0 + n_b units, c0 being a fixed per-sequence overhead
//     (query load, epilogue) in page units;
//   * the units of all sequences are laid end to end (U_b = sum of c over
//     sequences before b, T = total) and cut into num_parts equal shares of
//     q = ceil(T / num_parts) units: partition p starts at unit p*q;
//   * a cut inside sequence b's overhead units starts at its page 0, a cut
//     inside its page units at page (p*q - U_b - c0);
//   * partition p owns the half-open (sequence, page) range between its start
//     and partition p+1's start.
// Every count below follows from that rule by integer arithmetic, so the
// schedule is deterministic and depends only on the lengths and num_parts.

#include "mla_device.h"

namespace mla {

__device__ __forceinline__ long long floor_div(long long a, long long b) {
  // b > 0, a >= 0 here
  return a / b;
}

__device__ long long block_scan_exclusive(long long v, long long* total, long long* s_wave) {
  // inclusive scan inside the wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  long long x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    long long y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    long long w = (lane < nwaves) ? s_wave[lane] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      long long y = __shfl_up(w, d);
      if (lane >= d) w += y;
    }
    if (lane < nwaves) s_wave[lane] = w;  // inclusive over waves
  }
  __syncthreads();
  long long before = (wave > 0) ? s_wave[wave - 1] : 0;
  *total = s_wave[nwaves - 1];
  __syncthreads();
  return before + x - v;
}

__global__ void __launch_bounds__(1024) sched_kernel(const int32_t* __restrict__ seqlens,
                                                     int batch, int num_parts, int c0,
                                                     int32_t* __restrict__ meta,
                                                     int32_t* __restrict__ splits) {
  __shared__ long long s_wave[16];
  __shared__ int s_beg_b[kMaxParts + 1];
  __shared__ int s_beg_j[kMaxParts + 1];
  __shared__ int s_first[kMaxParts + 1];
  const int tid = threadIdx.x;
  const int nt = blockDim.x;

  // pass 1: total units T
  long long T = 0;
  for (int base = 0; base < batch; base += nt) {
    int b = base + tid;
    long long c = 0;
    if (b < batch) {
      long long L = seqlens[b];
      long long n = (L + kPage - 1) / kPage;
      c = c0 + (n > 0 ? n : 1);
    }
    long long tot;
    block_scan_exclusive(c, &tot, s_wave);
    T += tot;
  }
  const long long q = (T + num_parts - 1) / num_parts;  // units per partition

  for (int p = tid; p <= num_parts; p += nt) {
    s_beg_b[p] = batch;
    s_beg_j[p] = 0;
    s_first[p] = 0;
  }
  __syncthreads();

  // pass 2: per-sequence split counts and the partition starts inside it
  long long carry_u = 0, carry_s = 0;
  for (int base = 0; base < batch; base += nt) {
    int b = base + tid;
    long long n = 0, c = 0;
    if (b < batch) {
      long long L = seqlens[b];
      n = (L + kPage - 1) / kPage;
      if (n < 1) n = 1;
      c = c0 + n;
    }
    long long tot_u;
    long long U = carry_u + block_scan_exclusive(c, &tot_u, s_wave);
    long long ns = 0;
    if (b < batch) {
      const long long A = U + c0;  // first page unit of b
      // cuts strictly inside b's page units: multiples of q in (A, A + n)
      ns = 1 + floor_div(A + n - 1, q) - floor_div(A, q);
      // partitions starting inside [U, U + c)
      long long p_lo = (U + q - 1) / q;
      long long p_hi = floor_div(U + c - 1, q);
      for (long long p = p_lo; p <= p_hi && p < num_parts; ++p) {
        long long u = p * q;
        s_beg_b[p] = b;
        s_beg_j[p] = (int)(u > A ? u - A : 0);
        s_first[p] = (int)(u > A ? p - floor_div(A, q) : 0);
      }
    }
    long long tot_s;
    long long S = carry_s + block_scan_exclusive(ns, &tot_s, s_wave);
    if (b < batch) splits[b] = (int)S;
    carry_u += tot_u;
    carry_s += tot_s;
  }
  if (tid == 0) splits[batch] = (int)carry_s;
  __syncthreads();

  // pass 3: ranges
  for (int p = tid; p < num_parts; p += nt) {
    int32_t* m = meta + (size_t)p * kMetaInts;
    m[0] = s_beg_b[p];
    m[1] = s_beg_j[p];
    m[2] = s_beg_b[p + 1];
    m[3] = s_beg_j[p + 1];
    m[4] = s_first[p];
    m[5] = (int)q;
    m[6] = c0;
    m[7] = (int)(T < 0x7fffffffLL ? T : 0x7fffffffLL);
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_sched(const int32_t* seqlens, int batch, int num_parts, int c0,
                                       int32_t* meta, int32_t* splits, hipStream_t stream) {
  hipLaunchKernelGGL(mla::sched_kernel, dim3(1), dim3(1024), 0, stream, seqlens, batch, num_parts,
                     c0, meta, splits);
  return hipGetLastError();
}
