// A whole decode step (schedule, decode, combine) that allocates nothing: the
// split-KV schedule, the split counts and the split partials live in one
// static device array of this library instead of caller-given buffers.
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it).  The same kernels as
// mla_get_metadata / mla_decode_paged / mla_combine run, through those entry
// points, on slices of the array.
//
// The array is per GPU: each device that loads this library holds its own
// copy until the process ends.  In host code its name is only a stand-in, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever handed to a kernel.
// Every call on one GPU uses the same array: calls that overlap on one GPU
// (two streams, two threads) race and must be ordered by the caller.  Nothing
// in it has to start at zero: the schedule writes every split count and
// every schedule entry the decode reads, and the combine reads only the
// partials the decode of the same call wrote.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>

#include "mla_paged.h"

namespace {

static_assert(MLA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<unsigned char*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on each device).
mla_status_t scratch_of_current_device(unsigned char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  unsigned char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return MLA_ERR_HIP;
    p = (unsigned char*)addr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MLA_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" {

mla_status_t mla_decode_step_noalloc(const void* q, const void* kv_cache,
                                     const int32_t* block_table, const int32_t* cache_seqlens,
                                     int32_t batch, int32_t s_q, int32_t h_q, int32_t num_pages,
                                     int32_t max_pages, float softmax_scale, int32_t causal,
                                     void* out, float* lse, hipStream_t stream) {
  if (batch <= 0 || s_q <= 0 || h_q <= 0) return MLA_ERR_INVALID_ARGUMENT;
  if (batch > MLA_MAX_BATCH || (long long)s_q * h_q > MLA_MAX_ROWS) return MLA_ERR_UNSUPPORTED;
  const int parts = mla_num_partitions(s_q, h_q, 0);
  if (parts <= 0) return MLA_ERR_HIP;
  const size_t ws = mla_workspace_bytes(batch, s_q, h_q, 0);
  if (ws == 0) return MLA_ERR_UNSUPPORTED;
  // scratch layout: split counts [batch + 1], schedule [parts][8], partials
  const size_t splits_bytes = align256((size_t)(batch + 1) * sizeof(int32_t));
  const size_t meta_bytes = align256(mla_metadata_ints(s_q, h_q, 0) * sizeof(int32_t));
  if (splits_bytes + meta_bytes + ws > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return MLA_ERR_SCRATCH_TOO_SMALL;
  unsigned char* base = nullptr;
  const mla_status_t st = scratch_of_current_device(&base);
  if (st != MLA_OK) return st;
  int32_t* splits = (int32_t*)base;
  int32_t* meta = (int32_t*)(base + splits_bytes);
  void* workspace = base + splits_bytes + meta_bytes;

  // the decode schedules itself where it can (at most MLA_MAX_FUSED_BATCH
  // sequences and a block table within its 32-bit unit range); otherwise the
  // separate schedule writes into the scratch first
  const bool fused = batch <= MLA_MAX_FUSED_BATCH &&
                     (long long)batch * ((long long)max_pages + 2) < (1LL << 30);
  if (!fused) {
    const mla_status_t s1 =
        mla_get_metadata(cache_seqlens, batch, s_q, h_q, 0, meta, splits, stream);
    if (s1 != MLA_OK) return s1;
  }
  const mla_status_t s2 = mla_decode_paged(q, kv_cache, block_table, cache_seqlens, batch, s_q,
                                           h_q, num_pages, max_pages, softmax_scale, causal,
                                           fused ? nullptr : meta, splits, 0, workspace, ws, out,
                                           lse, stream);
  if (s2 != MLA_OK) return s2;
  return mla_combine(workspace, ws, splits, batch, s_q, h_q, 0, out, lse, stream);
}

}  // extern "C"
