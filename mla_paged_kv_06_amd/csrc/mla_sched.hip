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

template <int NT>
__device__ long long block_scan_exclusive(long long v, long long* total, long long* s_wave) {
  constexpr int kNW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  long long x = v;  // inclusive scan inside the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    long long y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  long long before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const long long sw = s_wave[w];
    before += (w < wave) ? sw : 0;
    tot += sw;
  }
  *total = tot;
  __syncthreads();  // s_wave is reused by the next scan
  return before + x - v;
}

// Partition starts that fall inside sequence b's units [U, U + c), and its
// split count.  I is int (totals below 2^31, the normal case: 32-bit
// divisions are a short VALU sequence) or long long.
template <typename I>
__device__ __forceinline__ int sequence_cuts(int b, I U, I n, int c0, I q, int num_parts,
                                             int* s_beg_b, int* s_beg_j, int* s_first) {
  const I c = c0 + n;
  const I A = U + c0;  // first page unit of b
  const I a_div = A / q;
  const I p_lo = (U + q - 1) / q;
  I p_hi = (U + c - 1) / q;
  if (p_hi > (I)(num_parts - 1)) p_hi = num_parts - 1;
  for (I p = p_lo; p <= p_hi; ++p) {
    const I u = p * q;
    s_beg_b[p] = b;
    s_beg_j[p] = (int)(u > A ? u - A : 0);
    s_first[p] = (int)(u > A ? p - a_div : 0);
  }
  // cuts strictly inside b's page units: multiples of q in (A, A + n)
  return (int)(1 + (A + n - 1) / q - a_div);
}

template <int NT>
__global__ void __launch_bounds__(NT) sched_kernel(const int32_t* __restrict__ seqlens,
                                                   int batch, int num_parts, int c0,
                                                   int32_t* __restrict__ meta,
                                                   int32_t* __restrict__ splits) {
  __shared__ long long s_wave[NT / 64];
  __shared__ int s_beg_b[kMaxParts + 1];
  __shared__ int s_beg_j[kMaxParts + 1];
  __shared__ int s_first[kMaxParts + 1];
  const int tid = threadIdx.x;

  for (int p = tid; p <= num_parts; p += NT) {
    s_beg_b[p] = batch;
    s_beg_j[p] = 0;
    s_first[p] = 0;
  }
  long long T = 0, q = 1;
  if (batch <= NT) {
    // one pass: every sequence in a register
    long long n = 0;
    if (tid < batch) {
      const long long L = seqlens[tid];
      n = (L + kPage - 1) / kPage;
      if (n < 1) n = 1;
    }
    const long long c = tid < batch ? c0 + n : 0;
    const long long U = block_scan_exclusive<NT>(c, &T, s_wave);  // barrier: init done
    q = (T + num_parts - 1) / num_parts;
    int ns = 0;
    if (tid < batch) {
      if (T < 0x7fffffffLL)
        ns = sequence_cuts<int>(tid, (int)U, (int)n, c0, (int)q, num_parts, s_beg_b, s_beg_j,
                                s_first);
      else
        ns = sequence_cuts<long long>(tid, U, n, c0, q, num_parts, s_beg_b, s_beg_j, s_first);
    }
    long long tot_s;
    const long long S = block_scan_exclusive<NT>(ns, &tot_s, s_wave);
    if (tid < batch) splits[tid] = (int)S;
    if (tid == 0) splits[batch] = (int)tot_s;
  } else {
    // pass 1: total units; pass 2: cuts chunk by chunk
    for (int base = 0; base < batch; base += NT) {
      const int b = base + tid;
      long long c = 0;
      if (b < batch) {
        const long long L = seqlens[b];
        const long long n = (L + kPage - 1) / kPage;
        c = c0 + (n > 0 ? n : 1);
      }
      long long tot;
      block_scan_exclusive<NT>(c, &tot, s_wave);
      T += tot;
    }
    q = (T + num_parts - 1) / num_parts;
    long long carry_u = 0, carry_s = 0;
    for (int base = 0; base < batch; base += NT) {
      const int b = base + tid;
      long long n = 0, c = 0;
      if (b < batch) {
        const long long L = seqlens[b];
        n = (L + kPage - 1) / kPage;
        if (n < 1) n = 1;
        c = c0 + n;
      }
      long long tot_u;
      const long long U = carry_u + block_scan_exclusive<NT>(c, &tot_u, s_wave);
      int ns = 0;
      if (b < batch) {
        if (T < 0x7fffffffLL)
          ns = sequence_cuts<int>(b, (int)U, (int)n, c0, (int)q, num_parts, s_beg_b, s_beg_j,
                                  s_first);
        else
          ns = sequence_cuts<long long>(b, U, n, c0, q, num_parts, s_beg_b, s_beg_j, s_first);
      }
      long long tot_s;
      const long long S = carry_s + block_scan_exclusive<NT>(ns, &tot_s, s_wave);
      if (b < batch) splits[b] = (int)S;
      carry_u += tot_u;
      carry_s += tot_s;
    }
    if (tid == 0) splits[batch] = (int)carry_s;
  }
  __syncthreads();

  // ranges
  for (int p = tid; p < num_parts; p += NT) {
    int32_t* m = meta + (size_t)p * kMetaInts;
    i32x4 lo = {s_beg_b[p], s_beg_j[p], s_beg_b[p + 1], s_beg_j[p + 1]};
    i32x4 hi = {s_first[p], (int)q, c0, (int)(T < 0x7fffffffLL ? T : 0x7fffffffLL)};
    *(i32x4*)m = lo;
    *(i32x4*)(m + 4) = hi;
  }
}

// Inclusive prefix sum over the block, one value per thread; the block total
// lands in *total.  Two barriers.
template <int NT, typename I>
__device__ __forceinline__ I block_scan_inclusive(I v, I* total, I* s_wave) {
  constexpr int kNW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  I x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const I y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  I before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    const I sw = s_wave[w];
    before += (w < wave) ? sw : 0;
    tot += sw;
  }
  *total = tot;
  __syncthreads();  // s_wave is reused by the next scan
  return before + x;
}

// Body of sched_small_kernel in index type I (int when every total is below
// 2^31, long long otherwise): the same rule as sched_kernel, with no serial
// loop -- each partition p finds the sequence holding its start unit p*q by
// binary search over the unit prefix sums.
template <int NT, typename I>
__device__ __forceinline__ void sched_small_body(int n, int batch, int num_parts, int c0,
                                                 int32_t* __restrict__ meta,
                                                 int32_t* __restrict__ splits, I* s_U,
                                                 I* s_wave, i32x2* s_start) {
  const int tid = threadIdx.x;
  const I c = tid < batch ? (I)(c0 + n) : (I)0;
  I T;
  const I U = block_scan_inclusive<NT, I>(c, &T, s_wave) - c;
  if (tid < batch) s_U[tid] = U;
  const I q = (T + num_parts - 1) / num_parts;
  // splits of sequence b: its start partition plus the cuts strictly inside
  // its page units (multiples of q in (A, A + n))
  I ns = 0;
  if (tid < batch) {
    const I A = U + c0;
    ns = 1 + (A + n - 1) / q - A / q;
  }
  I S_tot;
  const I S = block_scan_inclusive<NT, I>(ns, &S_tot, s_wave) - ns;  // barriers: s_U complete
  if (tid < batch) splits[tid] = (int32_t)S;
  if (tid == 0) splits[batch] = (int32_t)S_tot;
  // start (sequence, page, split index) of partition p
  auto start_of = [&](int p, int* b_out, int* j_out, int* f_out) {
    const I u = (I)p * q;
    if (u >= T) {
      *b_out = batch;
      *j_out = 0;
      *f_out = 0;
      return;
    }
    int lo = 0, hi = batch - 1;  // largest b with U[b] <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_U[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const I A = s_U[lo] + c0;
    *b_out = lo;
    *j_out = (int)(u > A ? u - A : 0);
    *f_out = (int)(u > A ? p - A / q : 0);
  };
  const int T32 = (int)(T < (I)0x7fffffff ? T : (I)0x7fffffff);
  // one search per partition: thread t finds the start of partition
  // base + t; the end of partition p is the start of p + 1, taken from the
  // neighbouring thread through LDS (the last thread searches it itself)
  for (int base = 0; base < num_parts; base += NT) {
    const int p = base + tid;
    int b0 = batch, j0 = 0, f0 = 0;
    if (p <= num_parts) start_of(p, &b0, &j0, &f0);
    s_start[tid] = i32x2{b0, j0};
    int b1 = batch, j1 = 0, f1 = 0;
    if (tid == NT - 1 && p + 1 <= num_parts) start_of(p + 1, &b1, &j1, &f1);
    __syncthreads();
    if (tid < NT - 1) {
      b1 = s_start[tid + 1][0];
      j1 = s_start[tid + 1][1];
    }
    if (p < num_parts) {
      int32_t* m = meta + (size_t)p * kMetaInts;
      *(i32x4*)m = i32x4{b0, j0, b1, j1};
      *(i32x4*)(m + 4) = i32x4{f0, (int)q, c0, T32};
    }
    __syncthreads();  // s_start is reused by the next round
  }
}

template <int NT>
__global__ void __launch_bounds__(NT) sched_small_kernel(const int32_t* __restrict__ seqlens,
                                                         int batch, int num_parts, int c0,
                                                         int32_t* __restrict__ meta,
                                                         int32_t* __restrict__ splits) {
  __shared__ long long s_U[NT];
  __shared__ long long s_wave[NT / 64];
  __shared__ i32x2 s_start[NT];
  const int tid = threadIdx.x;
  int n = 0;
  if (tid < batch) {
    const int L = seqlens[tid];
    n = (L + kPage - 1) / kPage;
    if (n < 1) n = 1;
  }
  // fewer than 2^20 units per sequence and at most 1024 sequences keep every
  // total below 2^30: 32-bit arithmetic is exact
  if (!__syncthreads_or(n >= (1 << 20) - 8))
    sched_small_body<NT, int>(n, batch, num_parts, c0, meta, splits, (int*)s_U, (int*)s_wave,
                              s_start);
  else
    sched_small_body<NT, long long>(n, batch, num_parts, c0, meta, splits, s_U, s_wave, s_start);
}

}  // namespace mla

extern "C" hipError_t mla_launch_sched(const int32_t* seqlens, int batch, int num_parts, int c0,
                                       int32_t* meta, int32_t* splits, hipStream_t stream) {
  // at least 256 threads: one partition per thread in the common case
  if (batch <= 256)
    hipLaunchKernelGGL(mla::sched_small_kernel<256>, dim3(1), dim3(256), 0, stream, seqlens,
                       batch, num_parts, c0, meta, splits);
  else if (batch <= 1024)
    hipLaunchKernelGGL(mla::sched_small_kernel<1024>, dim3(1), dim3(1024), 0, stream, seqlens,
                       batch, num_parts, c0, meta, splits);
  else
    hipLaunchKernelGGL(mla::sched_kernel<1024>, dim3(1), dim3(1024), 0, stream, seqlens, batch,
                       num_parts, c0, meta, splits);
  return hipGetLastError();
}
