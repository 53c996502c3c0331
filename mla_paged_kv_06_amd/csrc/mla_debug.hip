// Device-content checks run before a decode when debug checks are on.
//
// The decode trusts two things it cannot check on the host without waiting
// for the device: every cache length lies in [0, max_pages * 64], and every
// block-table entry of a page that holds tokens names a page of the pool.
// This pass reads exactly the entries the decode would read (never past a
// row of the table, even for a length that is out of range) and reduces
// what it finds into one device word, which the host reads back.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kCheckThreads = 1024;

// bit 0: some length outside [0, max_pages * 64]; bit 1: some used entry
// outside [0, num_pages)
constexpr int kBadLength = 1;
constexpr int kBadEntry = 2;

// Error word of the pass, one per device (each GPU holds its own copy).
__device__ int g_check_word;

__global__ void __launch_bounds__(kCheckThreads)
    check_contents_kernel(const int32_t* __restrict__ seqlens,
                          const int32_t* __restrict__ block_table, int batch, int max_pages,
                          int num_pages, int* __restrict__ word) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int mine = 0;
  const long long cap = (long long)max_pages * 64;
  for (int b = threadIdx.x; b < batch; b += kCheckThreads) {
    const int L = seqlens[b];
    if (L < 0 || (long long)L > cap) mine |= kBadLength;
    long long pages = L > 0 ? ((long long)L + 63) / 64 : 0;
    if (pages > max_pages) pages = max_pages;  // read only inside the row
    const int32_t* row = block_table + (size_t)b * max_pages;
    for (long long j = 0; j < pages; ++j) {
      const int p = row[j];
      if (p < 0 || p >= num_pages) {
        mine |= kBadEntry;
        break;
      }
    }
  }
  if (mine) atomicOr(&flags, mine);
  __syncthreads();
  if (threadIdx.x == 0) *word = flags;  // written whole: no clearing needed
}

}  // namespace mla

// Address of this device's error word (looked up once per device by the caller).
extern "C" hipError_t mla_check_word_address(int** addr) {
  return hipGetSymbolAddress((void**)addr, HIP_SYMBOL(mla::g_check_word));
}

extern "C" hipError_t mla_launch_check_contents(const int32_t* seqlens, const int32_t* block_table,
                                                int batch, int max_pages, int num_pages, int* word,
                                                hipStream_t stream) {
  hipLaunchKernelGGL(mla::check_contents_kernel, dim3(1), dim3(mla::kCheckThreads), 0, stream,
                     seqlens, block_table, batch, max_pages, num_pages, word);
  return hipGetLastError();
}
