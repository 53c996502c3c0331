// Paged KV append with page allocation: the step before every decode step.
//
// The cache is paged, 64 tokens per block (FlashMLA release note, paragraph
// on the released paged bf16 cache), and blocks are handed out on demand as
// sequences grow (Tom's Hardware FR article, paragraph on the techniques:
// block-based paging with dynamic allocation).  Each sequence's new tokens
// -- their 576-value cache entries [latent ; rotary key] -- are written into
// its pages; a sequence that crosses into a page it does not hold yet takes
// a fresh one from a stack of free pages.
//
// The allocation is deterministic: sequence b needs
//   k_b = ceil((L_b + n) / 64) - ceil(L_b / 64)
// new pages; with K_b = k_0 + .. + k_{b-1} and F free pages on the stack,
// its i-th new page is free_pages[F - 1 - (K_b + i)] (the stack is popped
// from the top in batch order), and the stack ends with F - K entries.  If
// the stack holds fewer than K pages, or a sequence would need more than
// max_pages, nothing is written and the status word is set to 1.
//
// Two launches: one workgroup scans the needs and writes the new block-table
// entries and the stack size (and the status); then one workgroup per
// sequence copies its tokens in 16-byte pieces and advances its length.

#include "mla_device.h"

namespace mla {

constexpr int kAllocThreads = 1024;

__global__ void __launch_bounds__(kAllocThreads) kv_alloc_kernel(
    const int32_t* __restrict__ seqlens, int batch, int n_new, int32_t* __restrict__ block_table,
    int max_pages, const int32_t* __restrict__ free_pages, int32_t* __restrict__ free_count,
    int32_t* __restrict__ status) {
  __shared__ long long s_wave[kAllocThreads / 64];
  __shared__ long long s_carry;
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    s_carry = 0;
    s_bad = 0;
  }
  __syncthreads();
  const long long F = free_count[0];
  // pass 1: total need and the max_pages check; pass 2 (only if it all fits):
  // block-table entries.  Both walk the batch in chunks of the block size.
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (s_bad || s_carry > F) break;
      __syncthreads();
      if (tid == 0) s_carry = 0;
      __syncthreads();
    }
    for (int base = 0; base < batch; base += kAllocThreads) {
      const int b = base + tid;
      long long k = 0, old_pages = 0;
      if (b < batch) {
        const long long L = seqlens[b];
        old_pages = (L + kPage - 1) / kPage;
        const long long new_pages = (L + n_new + kPage - 1) / kPage;
        k = new_pages - old_pages;
        if (new_pages > max_pages) atomicOr(&s_bad, 1);
      }
      // block-wide exclusive scan of k
      long long x = k;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const long long y = __shfl_up(x, d);
        if (lane >= d) x += y;
      }
      if (lane == 63) s_wave[wave] = x;
      __syncthreads();
      long long before = s_carry, tot = 0;
      for (int w = 0; w < kAllocThreads / 64; ++w) {
        before += (w < wave) ? s_wave[w] : 0;
        tot += s_wave[w];
      }
      const long long K_b = before + x - k;
      if (pass == 1 && b < batch) {
        for (long long i = 0; i < k; ++i)
          block_table[(size_t)b * max_pages + old_pages + i] = free_pages[F - 1 - (K_b + i)];
      }
      __syncthreads();
      if (tid == 0) s_carry += tot;
      __syncthreads();
    }
  }
  __syncthreads();
  if (tid == 0) {
    const bool ok = !s_bad && s_carry <= F;
    status[0] = ok ? 0 : 1;
    if (ok) free_count[0] = (int32_t)(F - s_carry);
  }
}

// One workgroup per sequence: token i goes to page (L + i) / 64, slot
// (L + i) % 64, 72 16-byte pieces per token.
__global__ void __launch_bounds__(256) kv_append_kernel(
    uint16_t* __restrict__ kv, const int32_t* __restrict__ block_table, int max_pages,
    int32_t* __restrict__ seqlens, const uint16_t* __restrict__ new_kv, int n_new,
    const int32_t* __restrict__ status) {
  if (status[0] != 0) return;
  const int b = blockIdx.x;
  const int L = seqlens[b];
  const int32_t* bt = block_table + (size_t)b * max_pages;
  const int pieces = n_new * kChunksPerRow;
  for (int p = threadIdx.x; p < pieces; p += 256) {
    const int i = p / kChunksPerRow;
    const int c = p - i * kChunksPerRow;
    const int t = L + i;
    const size_t page = (size_t)bt[t / kPage];
    const uint4 v = *(const uint4*)(new_kv + ((size_t)b * n_new + i) * kD + 8 * c);
    *(uint4*)(kv + (page * kPage + (t % kPage)) * kD + 8 * c) = v;
  }
  __syncthreads();  // every thread has read L
  if (threadIdx.x == 0) seqlens[b] = L + n_new;
}

}  // namespace mla

extern "C" hipError_t mla_launch_kv_append(uint16_t* kv, int32_t* block_table, int max_pages,
                                           int32_t* seqlens, int batch, const uint16_t* new_kv,
                                           int n_new, const int32_t* free_pages,
                                           int32_t* free_count, int32_t* status,
                                           hipStream_t stream) {
  using namespace mla;
  hipLaunchKernelGGL(kv_alloc_kernel, dim3(1), dim3(kAllocThreads), 0, stream, seqlens, batch,
                     n_new, block_table, max_pages, free_pages, free_count, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_append_kernel, dim3(batch), dim3(256), 0, stream, kv, block_table,
                     max_pages, seqlens, new_kv, n_new, status);
  return hipGetLastError();
}
