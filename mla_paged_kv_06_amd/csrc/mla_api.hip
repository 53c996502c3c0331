// C ABI of the paged MLA decode library: argument checks, launch shapes,
// status codes.  Declared in include/mla_paged.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "mla_paged.h"
#include "mla_device.h"

extern "C" hipError_t mla_check_word_address(int** addr);
extern "C" hipError_t mla_launch_check_contents(const int32_t* seqlens, const int32_t* block_table,
                                                int batch, int max_pages, int num_pages, int* word,
                                                hipStream_t stream);
extern "C" hipError_t mla_launch_probe_stream_read(const void* src, size_t bytes, unsigned* sink,
                                                   int blocks, hipStream_t stream);
extern "C" hipError_t mla_launch_probe_issue(int kind, int iters, int blocks, float* sink,
                                             unsigned long long* clk, hipStream_t stream);
extern "C" hipError_t mla_launch_probe_copy_ring(int kind, const void* src, int slots, int steps,
                                                 int blocks, int* sink, unsigned long long* clk,
                                                 hipStream_t stream);
extern "C" hipError_t mla_launch_probe_lds(int kind, int iters, int blocks, int* sink,
                                           unsigned long long* clk, hipStream_t stream);
extern "C" hipError_t mla_launch_probe_mfma(int iters, int blocks, float* sink,
                                            unsigned long long* clk, hipStream_t stream);
extern "C" hipError_t mla_launch_prefill_expand(const uint16_t* latent, int latent_stride, int T,
                                                const uint16_t* w_uk, const uint16_t* w_uv, int H,
                                                uint16_t* k_nope, uint16_t* v, hipStream_t stream);
extern "C" hipError_t mla_launch_prefill_attention(const mla::PrefillParams* prm, int batch,
                                                   int max_seqlen, hipStream_t stream);
extern "C" hipError_t mla_launch_sched(const int32_t* seqlens, int batch, int num_parts, int c0,
                                       int32_t* meta, int32_t* splits, hipStream_t stream);

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device, cached per device.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool rows_ok(int32_t s_q, int32_t h_q) {
  if (s_q <= 0 || h_q <= 0) return false;
  const long long R = (long long)s_q * h_q;
  return R <= MLA_MAX_ROWS;
}

// Debug checks of device contents: -1 = not decided yet (then MLA_DEBUG in
// the environment decides), 0 = off, 1 = on.
std::atomic<int> g_debug{-1};

bool debug_checks_on() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("MLA_DEBUG");
    v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expect = -1;
    g_debug.compare_exchange_strong(expect, v, std::memory_order_relaxed);
  }
  return v > 0;
}

// Address of the current device's check word, looked up once per device.
std::atomic<int*> g_check_word[kMaxDevices];

int* check_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  int* p = g_check_word[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (mla_check_word_address(&p) != hipSuccess) return nullptr;
  g_check_word[dev].store(p, std::memory_order_release);
  return p;
}

// Runs the content checks on `stream` and waits for them.  MLA_OK when the
// lengths and the used block-table entries are in range.
mla_status_t check_device_contents(const int32_t* seqlens, const int32_t* block_table,
                                   int batch, int max_pages, int num_pages, hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return MLA_ERR_HIP;
  if (cap != hipStreamCaptureStatusNone) return MLA_ERR_UNSUPPORTED;  // it must wait
  int* word = check_word();
  if (!word) return MLA_ERR_HIP;
  if (mla_launch_check_contents(seqlens, block_table, batch, max_pages, num_pages, word,
                                stream) != hipSuccess)
    return MLA_ERR_HIP;
  int flags = 0;
  if (hipMemcpyAsync(&flags, word, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return MLA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_HIP;
  return flags ? MLA_ERR_DEVICE_CONTENTS : MLA_OK;
}

int row_groups_of(int R) { return (R + mla::kRowGroup - 1) / mla::kRowGroup; }

// Query rows one workgroup holds: the smallest tuned size covering a row group.
int rows_variant_of(int R) {
  const int r = R < mla::kRowGroup ? R : mla::kRowGroup;
  if (r <= 16) return 16;
  if (r <= 32) return 32;
  return 64;
}

// Fixed cost of one (sequence, partition) segment in page units: the query
// load and the epilogue grow with the rows held.
int fixed_cost_of(int R) { return 1 + rows_variant_of(R) / 32; }

int parts_of(int32_t s_q, int32_t h_q, int32_t num_cus) {
  if (!rows_ok(s_q, h_q) || num_cus < 0) return 0;
  const int cus = num_cus > 0 ? num_cus : device_cus();
  if (cus <= 0) return 0;
  const int R = s_q * h_q;
  int parts = cus / row_groups_of(R);
  if (parts < 1) parts = 1;
  if (parts > MLA_MAX_PARTS) parts = MLA_MAX_PARTS;
  return parts;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// workspace: o_acc [slots][R][512] bf16, then lse_acc [slots][R] fp32.  With
// one partition no sequence is split (it owns every unit), so no slot is
// ever written; a token 256 bytes keep the pointer checks uniform.
size_t slots_of(int batch, int parts) { return parts > 1 ? (size_t)batch + parts : 0; }
size_t oacc_bytes(int batch, int R, int parts) {
  return align_up(slots_of(batch, parts) * R * MLA_V_DIM * sizeof(uint16_t), 256);
}
size_t ws_bytes(int batch, int R, int parts) {
  const size_t n = oacc_bytes(batch, R, parts) +
                   align_up(slots_of(batch, parts) * R * sizeof(float), 256);
  return n > 256 ? n : 256;
}

}  // namespace

extern "C" hipError_t mla_launch_decode(const mla::DecodeParams* prm, int rows_variant,
                                        hipStream_t stream);
extern "C" hipError_t mla_launch_decode_sv64(const mla::DecodeParams* prm, hipStream_t stream);
extern "C" hipError_t mla_launch_decode_t16(const mla::DecodeParams* prm, hipStream_t stream);
extern "C" hipError_t mla_launch_decode_t16_fp8(const mla::DecodeParams* prm, hipStream_t stream);
extern "C" hipError_t mla_launch_kv_quantize_fp8(const uint16_t* kv, int n_tokens, uint8_t* out,
                                                 hipStream_t stream);
extern "C" hipError_t mla_launch_combine(const uint16_t* o_acc, const float* lse_acc,
                                         const int32_t* splits, int batch, int R, uint16_t* out,
                                         float* lse, int wide, hipStream_t stream);

extern "C" hipError_t mla_launch_absorb_query(const uint16_t* q_c, const uint16_t* q_r,
                                              const uint16_t* w_uk_t, int M, int H,
                                              uint16_t* q_out, hipStream_t stream);
extern "C" hipError_t mla_launch_absorb_output(const uint16_t* lat_out, const uint16_t* w_uv,
                                               int M, int H, uint16_t* o, hipStream_t stream);

extern "C" hipError_t mla_launch_kv_append(uint16_t* kv, int32_t* block_table, int max_pages,
                                           int32_t* seqlens, int batch, const uint16_t* new_kv,
                                           int n_new, const int32_t* free_pages,
                                           int32_t* free_count, int32_t* status,
                                           hipStream_t stream);

extern "C" {

int32_t mla_set_debug_checks(int32_t on) {
  const int prev = debug_checks_on() ? 1 : 0;
  if (on >= 0) g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

int32_t mla_num_partitions(int32_t s_q, int32_t h_q, int32_t num_cus) {
  return parts_of(s_q, h_q, num_cus);
}

size_t mla_metadata_ints(int32_t s_q, int32_t h_q, int32_t num_cus) {
  return (size_t)parts_of(s_q, h_q, num_cus) * MLA_META_INTS;
}

size_t mla_workspace_bytes(int32_t batch, int32_t s_q, int32_t h_q, int32_t num_cus) {
  if (batch <= 0 || batch > MLA_MAX_BATCH) return 0;
  const int parts = parts_of(s_q, h_q, num_cus);
  if (parts <= 0) return 0;
  return ws_bytes(batch, s_q * h_q, parts);
}

mla_status_t mla_get_metadata(const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                              int32_t h_q, int32_t num_cus, int32_t* tile_metadata,
                              int32_t* num_splits, hipStream_t stream) {
  if (!cache_seqlens || !tile_metadata || !num_splits) return MLA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_cus < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (batch > MLA_MAX_BATCH || !rows_ok(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
  const int parts = parts_of(s_q, h_q, num_cus);
  if (parts <= 0) return MLA_ERR_HIP;
  const int c0 = fixed_cost_of(s_q * h_q);
  hipError_t e = mla_launch_sched(cache_seqlens, batch, parts, c0, tile_metadata, num_splits, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

static mla_status_t decode_impl(bool fp8, const void* q, const void* kv_cache, const int32_t* block_table,
                              const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                              int32_t h_q, int32_t num_pages, int32_t max_pages,
                              float softmax_scale, int32_t causal, const int32_t* tile_metadata,
                              int32_t* num_splits, int32_t num_cus, void* workspace,
                              size_t workspace_bytes, void* out, float* lse, hipStream_t stream) {
  if (!q || !kv_cache || !block_table || !cache_seqlens || !num_splits || !workspace || !out ||
      !lse)
    return MLA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_pages <= 0 || max_pages <= 0 || num_cus < 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
  if (batch > MLA_MAX_BATCH || !rows_ok(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
  if (((uintptr_t)q | (uintptr_t)kv_cache | (uintptr_t)out | (uintptr_t)workspace) & 15)
    return MLA_ERR_INVALID_ARGUMENT;
  const int parts = parts_of(s_q, h_q, num_cus);
  if (parts <= 0) return MLA_ERR_HIP;
  const int R = s_q * h_q;
  if (workspace_bytes < ws_bytes(batch, R, parts)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  // without tile_metadata the decode schedules itself: at most
  // MLA_MAX_FUSED_BATCH sequences, and a block table small enough that its
  // schedule units fit 32-bit arithmetic
  // the FP8 cache: workgroups of at most 16 rows, tile_metadata required
  if (fp8 && (rows_variant_of(R) != 16 || !tile_metadata)) return MLA_ERR_UNSUPPORTED;
  if (!tile_metadata && (batch > MLA_MAX_FUSED_BATCH ||
                         (long long)batch * ((long long)max_pages + 2) >= (1LL << 30)))
    return MLA_ERR_UNSUPPORTED;

  if (debug_checks_on()) {
    const mla_status_t st =
        check_device_contents(cache_seqlens, block_table, batch, max_pages, num_pages, stream);
    if (st != MLA_OK) return st;
  }

  mla::DecodeParams prm;
  prm.q = (const uint16_t*)q;
  prm.kv = (const uint16_t*)kv_cache;
  prm.block_table = block_table;
  prm.seqlens = cache_seqlens;
  prm.meta = tile_metadata;
  prm.splits = num_splits;
  prm.out = (uint16_t*)out;
  prm.lse = lse;
  prm.o_acc = (uint16_t*)workspace;
  prm.lse_acc = (float*)((char*)workspace + oacc_bytes(batch, R, parts));
  prm.batch = batch;
  prm.s_q = s_q;
  prm.h_q = h_q;
  prm.R = R;
  prm.max_pages = max_pages;
  prm.num_parts = parts;
  prm.row_groups = row_groups_of(R);
  prm.causal = causal ? 1 : 0;
  prm.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  prm.sched_c0 = fixed_cost_of(R);
  const int variant = rows_variant_of(R);
  hipError_t e = fp8             ? mla_launch_decode_t16_fp8(&prm, stream)
                 : variant == 64 ? mla_launch_decode_sv64(&prm, stream)
                 : variant == 16 ? mla_launch_decode_t16(&prm, stream)
                                 : mla_launch_decode(&prm, variant, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" {

mla_status_t mla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_table,
                              const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                              int32_t h_q, int32_t num_pages, int32_t max_pages,
                              float softmax_scale, int32_t causal, const int32_t* tile_metadata,
                              int32_t* num_splits, int32_t num_cus, void* workspace,
                              size_t workspace_bytes, void* out, float* lse, hipStream_t stream) {
  return decode_impl(false, q, kv_cache, block_table, cache_seqlens, batch, s_q, h_q, num_pages,
                     max_pages, softmax_scale, causal, tile_metadata, num_splits, num_cus,
                     workspace, workspace_bytes, out, lse, stream);
}

mla_status_t mla_decode_paged_fp8(const void* q, const void* kv_fp8, const int32_t* block_table,
                                  const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                                  int32_t h_q, int32_t num_pages, int32_t max_pages,
                                  float softmax_scale, int32_t causal,
                                  const int32_t* tile_metadata, int32_t* num_splits,
                                  int32_t num_cus, void* workspace, size_t workspace_bytes,
                                  void* out, float* lse, hipStream_t stream) {
  return decode_impl(true, q, kv_fp8, block_table, cache_seqlens, batch, s_q, h_q, num_pages,
                     max_pages, softmax_scale, causal, tile_metadata, num_splits, num_cus,
                     workspace, workspace_bytes, out, lse, stream);
}

mla_status_t mla_kv_quantize_fp8(const void* kv_cache, int32_t num_pages, void* kv_fp8,
                                 hipStream_t stream) {
  if (!kv_cache || !kv_fp8 || num_pages <= 0) return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)kv_cache | (uintptr_t)kv_fp8) & 15) return MLA_ERR_INVALID_ARGUMENT;
  if ((long long)num_pages * MLA_PAGE_SIZE > 0x7FFFFFFFLL) return MLA_ERR_UNSUPPORTED;
  hipError_t e = mla_launch_kv_quantize_fp8((const uint16_t*)kv_cache, num_pages * MLA_PAGE_SIZE,
                                            (uint8_t*)kv_fp8, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_combine(const void* workspace, size_t workspace_bytes, const int32_t* num_splits,
                         int32_t batch, int32_t s_q, int32_t h_q, int32_t num_cus, void* out,
                         float* lse, hipStream_t stream) {
  if (!workspace || !num_splits || !out || !lse) return MLA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_cus < 0) return MLA_ERR_INVALID_ARGUMENT;
  if (batch > MLA_MAX_BATCH || !rows_ok(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
  const int parts = parts_of(s_q, h_q, num_cus);
  if (parts <= 0) return MLA_ERR_HIP;
  const int R = s_q * h_q;
  if (workspace_bytes < ws_bytes(batch, R, parts)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (parts == 1) return MLA_OK;  // one partition: nothing was split
  const uint16_t* o_acc = (const uint16_t*)workspace;
  const float* lse_acc = (const float*)((const char*)workspace + oacc_bytes(batch, R, parts));
  // many partitions per sequence on average: spread each row's partials over
  // a whole workgroup
  const int wide = parts >= 8 * batch ? 1 : 0;
  hipError_t e = mla_launch_combine(o_acc, lse_acc, num_splits, batch, R, (uint16_t*)out, lse, wide,
                                    stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Shapes of the absorption products: the decode's limits.
static mla_status_t absorb_shape_ok(int32_t batch, int32_t s_q, int32_t h_q) {
  if (batch <= 0 || s_q <= 0 || h_q <= 0) return MLA_ERR_INVALID_ARGUMENT;
  if (batch > MLA_MAX_BATCH || !rows_ok(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status_t mla_absorb_query(const void* q_nope, const void* q_rope, const void* w_uk_t,
                              int32_t batch, int32_t s_q, int32_t h_q, void* q_out,
                              hipStream_t stream) {
  if (!q_nope || !q_rope || !w_uk_t || !q_out) return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)q_nope | (uintptr_t)q_rope | (uintptr_t)w_uk_t | (uintptr_t)q_out) & 15)
    return MLA_ERR_INVALID_ARGUMENT;
  const mla_status_t st = absorb_shape_ok(batch, s_q, h_q);
  if (st != MLA_OK) return st;
  hipError_t e = mla_launch_absorb_query((const uint16_t*)q_nope, (const uint16_t*)q_rope,
                                         (const uint16_t*)w_uk_t, batch * s_q, h_q,
                                         (uint16_t*)q_out, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_absorb_output(const void* out, const void* w_uv, int32_t batch, int32_t s_q,
                               int32_t h_q, void* o, hipStream_t stream) {
  if (!out || !w_uv || !o) return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)out | (uintptr_t)w_uv | (uintptr_t)o) & 15) return MLA_ERR_INVALID_ARGUMENT;
  const mla_status_t st = absorb_shape_ok(batch, s_q, h_q);
  if (st != MLA_OK) return st;
  hipError_t e = mla_launch_absorb_output((const uint16_t*)out, (const uint16_t*)w_uv,
                                          batch * s_q, h_q, (uint16_t*)o, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_kv_append(void* kv_cache, int32_t num_pages, int32_t* block_table,
                           int32_t max_pages, int32_t* cache_seqlens, int32_t batch,
                           const void* new_kv, int32_t n_new, const int32_t* free_pages,
                           int32_t* free_count, int32_t* status, hipStream_t stream) {
  if (!kv_cache || !block_table || !cache_seqlens || !free_pages || !free_count || !status ||
      (n_new > 0 && !new_kv))
    return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)kv_cache | (uintptr_t)new_kv) & 15) return MLA_ERR_INVALID_ARGUMENT;
  if (num_pages <= 0 || max_pages <= 0 || batch <= 0 || n_new < 0)
    return MLA_ERR_INVALID_ARGUMENT;
  if (batch > MLA_MAX_BATCH || n_new > MLA_MAX_APPEND) return MLA_ERR_UNSUPPORTED;
  hipError_t e = mla_launch_kv_append((uint16_t*)kv_cache, block_table, max_pages, cache_seqlens,
                                      batch, (const uint16_t*)new_kv, n_new, free_pages,
                                      free_count, status, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_prefill_expand_kv(const void* latent, int32_t latent_stride, int32_t tokens,
                                   const void* w_uk, const void* w_uv, int32_t h_q, void* k_nope,
                                   void* v, hipStream_t stream) {
  if (!latent || !w_uk || !w_uv || !k_nope || !v) return MLA_ERR_INVALID_ARGUMENT;
  if (tokens <= 0 || h_q <= 0 || latent_stride < MLA_V_DIM || (latent_stride & 7))
    return MLA_ERR_INVALID_ARGUMENT;
  // 256 latent rows stay addressable by 32-bit byte offsets
  if (latent_stride > (1 << 21)) return MLA_ERR_UNSUPPORTED;
  if (((uintptr_t)latent | (uintptr_t)w_uk | (uintptr_t)w_uv | (uintptr_t)k_nope |
       (uintptr_t)v) & 15)
    return MLA_ERR_INVALID_ARGUMENT;
  if (h_q > MLA_MAX_PREFILL_HEADS || (long long)tokens * h_q * MLA_NOPE_DIM >= (1LL << 31))
    return MLA_ERR_UNSUPPORTED;
  const hipError_t e = mla_launch_prefill_expand((const uint16_t*)latent, latent_stride, tokens,
                                                 (const uint16_t*)w_uk, (const uint16_t*)w_uv,
                                                 h_q, (uint16_t*)k_nope, (uint16_t*)v, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_prefill_attention(const void* q, const void* k_nope, const void* k_rope,
                                   int32_t rope_stride, const void* v,
                                   const int32_t* cu_seqlens, int32_t batch, int32_t h_q,
                                   int32_t max_seqlen, float softmax_scale, int32_t causal,
                                   void* o, float* lse, hipStream_t stream) {
  if (!q || !k_nope || !k_rope || !v || !cu_seqlens || !o || !lse)
    return MLA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || h_q <= 0 || max_seqlen < 0 || rope_stride < MLA_ROPE_DIM ||
      (rope_stride & 7))
    return MLA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)q | (uintptr_t)k_nope | (uintptr_t)k_rope | (uintptr_t)v | (uintptr_t)o) & 15)
    return MLA_ERR_INVALID_ARGUMENT;
  if (batch > MLA_MAX_BATCH || h_q > MLA_MAX_PREFILL_HEADS) return MLA_ERR_UNSUPPORTED;
  if (max_seqlen == 0) return MLA_OK;
  mla::PrefillParams prm;
  prm.q = (const uint16_t*)q;
  prm.k_nope = (const uint16_t*)k_nope;
  prm.k_rope = (const uint16_t*)k_rope;
  prm.v = (const uint16_t*)v;
  prm.cu = cu_seqlens;
  prm.o = (uint16_t*)o;
  prm.lse = lse;
  prm.rope_stride = rope_stride;
  prm.H = h_q;
  prm.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  prm.causal = causal ? 1 : 0;
  const hipError_t e = mla_launch_prefill_attention(&prm, batch, max_seqlen, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_probe_stream_read(const void* buf, size_t bytes, void* sink, int32_t blocks,
                                   hipStream_t stream) {
  if (!buf || !sink || blocks <= 0 || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15))
    return MLA_ERR_INVALID_ARGUMENT;
  return mla_launch_probe_stream_read(buf, bytes, (unsigned*)sink, blocks, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status_t mla_probe_mfma(int32_t iters, int32_t blocks, void* sink, void* clocks,
                            hipStream_t stream) {
  if (!sink || !clocks || iters <= 0 || blocks <= 0) return MLA_ERR_INVALID_ARGUMENT;
  return mla_launch_probe_mfma(iters, blocks, (float*)sink, (unsigned long long*)clocks, stream) ==
                 hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status_t mla_probe_lds(int32_t kind, int32_t iters, int32_t blocks, void* sink, void* clocks,
                           hipStream_t stream) {
  if (!sink || !clocks || iters <= 0 || blocks <= 0 || (kind != 0 && kind != 1))
    return MLA_ERR_INVALID_ARGUMENT;
  return mla_launch_probe_lds(kind, iters, blocks, (int*)sink, (unsigned long long*)clocks,
                              stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status_t mla_probe_issue(int32_t kind, int32_t iters, int32_t blocks, void* sink,
                             void* clocks, hipStream_t stream) {
  if (!sink || !clocks || iters <= 0 || blocks <= 0 || kind < 0 || kind > 4)
    return MLA_ERR_INVALID_ARGUMENT;
  return mla_launch_probe_issue(kind, iters, blocks, (float*)sink, (unsigned long long*)clocks,
                                stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status_t mla_probe_copy_ring(int32_t kind, const void* src, int32_t slots, int32_t steps,
                                 int32_t blocks, void* sink, void* clocks, hipStream_t stream) {
  if (!src || ((uintptr_t)src & 15) || !sink || !clocks || kind < 0 || kind > 2 || slots < 2 ||
      slots > (1 << 16) || steps < 3 || steps > (1 << 20) || blocks <= 0)
    return MLA_ERR_INVALID_ARGUMENT;
  return mla_launch_probe_copy_ring(kind, src, slots, steps, blocks, (int*)sink,
                                    (unsigned long long*)clocks, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

const char* mla_status_string(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_DEVICE_CONTENTS:
      return "cache length or block-table entry out of range (debug checks)";
    case MLA_ERR_SCRATCH_TOO_SMALL:
      return "shape needs more than the static scratch of the no-allocation decode";
  }
  return "unknown status";
}

}  // extern "C"
