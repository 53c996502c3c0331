// Pieces shared by the decode kernels: work items, uniform values, LDS-only
// barrier, and the HBM -> LDS page copy.
#pragma once

#include "mla_device.h"

namespace mla {

struct Item {
  int b, j;
};

__device__ __forceinline__ bool item_before(Item a, int eb, int ej) {
  return a.b < eb || (a.b == eb && a.j < ej);
}

// Wave-uniform value (kept in an SGPR, so loads indexed by it are scalar).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wave-uniform read of memory that no kernel of the launch writes (lengths,
// block table).  Through the constant address space it is always a scalar
// load, counted by lgkmcnt.  A plain load becomes a vector load wherever the
// compiler cannot prove the memory unwritten (a kernel that also stores the
// split counts), and a vector load is counted by vmcnt with the page copies:
// waiting for it would wait for every copy in flight.
__device__ __forceinline__ int load_uniform(const int32_t* p, size_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Barrier for LDS traffic only: unlike __syncthreads it does not wait for
// outstanding global loads, so a page prefetch in flight keeps flying.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copy one 64-token page into an LDS tile.  The page is 8 blocks of 8 tokens
// (9216 B each = 9 wave-wide 1 KiB copies); wave w copies block w (first
// half page) with its copies 0..8 and block w + 4 (second half) with 9..17,
// so a wave's first nine copies complete the first half of the page.
// Inside a block, copy k, lane l fills LDS chunk 64 k + l of the block:
// token t' = (64 k + l) / 72, physical chunk p = (64 k + l) % 72, which
// holds logical chunk p ^ swz(t').  swz depends on t & 7 only, so the nine
// per-lane source offsets are the same for every block.
//
// The copy is buffer_load ... lds through a buffer resource covering exactly
// the page (reads past it return zero).  Its global_load_lds twin makes the
// compiler wait for every outstanding LDS operation before each LDS read
// while a copy is in flight, which serialises the fragment pipeline below.
struct PageLoader {
  int off[9];  // per-lane source byte offsets inside an 8-token block
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const int pc = 64 * k + lane;
      const int t = pc / kChunksPerRow;
      const int p = pc - t * kChunksPerRow;
      off[k] = t * kRowBytes + 16 * (p ^ swz(t));
    }
  }
  // Resource for a page of which `live` tokens (1..64) hold data: reads past
  // them return zero, so the tail of a sequence's last page arrives in LDS
  // already cleared (a zero weight times stale data could otherwise be NaN).
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t resource(const char* page, int live) {
    const int n = live < kPage ? live : kPage;
    return __builtin_amdgcn_make_buffer_rsrc((void*)page, (short)0, n * kRowBytes, kBufferFlags);
  }
  // Copy number i (0 .. 17) of this wave: block wave + 4 (i / 9), load i % 9.
  __device__ __forceinline__ void issue_one(MLA_LDS char* tile, __amdgpu_buffer_rsrc_t rsrc,
                                            int wave, int i) const {
    const int base = (wave + 4 * (i / 9)) * 8 * kRowBytes;  // == 9 KiB of LDS per block
    const int k = i % 9;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(tile + base + 1024 * k), 16,
                                             off[k], base, 0, 0);
  }
  __device__ __forceinline__ void issue(MLA_LDS char* tile, const char* page, int live,
                                        int wave) const {
    const __amdgpu_buffer_rsrc_t rsrc = resource(page, live);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) issue_one(tile, rsrc, wave, i);
  }
};

// A page copy whose 18 per-wave instructions are spread over the k-steps of
// a score product, so the wave never stalls on a long run of memory issues.
struct PendingCopy {
  MLA_LDS char* tile;
  __amdgpu_buffer_rsrc_t rsrc;
  bool valid;
};

}  // namespace mla
