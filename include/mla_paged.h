/*
 * mla_paged.h -- C ABI of the MI355X (gfx950) paged MLA decode library.
 *
 * Multi-head Latent Attention decode over a paged, variable-length bf16
 * latent cache.  Sources for what is computed (by page and paragraph):
 *   - FlashMLA release note (shoujike.com.cn): an MLA decode kernel tuned for
 *     variable-length sequences (introduction); the cache is paged, bf16, with
 *     64 tokens per block (paragraph on what was released); keys and values
 *     are held as one compressed latent per token and widened at compute time
 *     (paragraph on MLA core principles); exact softmax attention in the
 *     FlashAttention line (acknowledgements paragraph).
 *   - DeepSeek-V3 hardware paper summary (news.chathome.org), paragraph on
 *     memory efficiency: the latent is shared by every attention head.
 *   - Tom's Hardware FR article on FlashMLA, paragraph on the techniques:
 *     block-based paging allocated on demand for variable-length sequences.
 *
 * The operation.  For sequence b with L = cache_seqlens[b] cached tokens and
 * each query row (query token i < s_q, head h < h_q):
 *     n      = L                       (non-causal)
 *            = clamp(L - s_q + 1 + i, 0, L)   (causal: the s_q queries are
 *              the last s_q cache positions; query i sees positions
 *              0 .. L - s_q + i)
 *     k_t    = kv_cache[block_table[b][t / 64]][t % 64][0:576]     (t < n)
 *     s_t    = softmax_scale * dot(q[b][i][h][0:576], k_t)
 *     lse    = ln(sum_t exp(s_t))                    (natural log)
 *     out    = sum_t exp(s_t - lse) * k_t[0:512]     (the latent is the value)
 * An empty row (n = 0) gives out = 0 and lse = -inf.  out is rounded once to
 * bf16 (nearest-even); lse is float32.
 *
 * Dimensions are fixed: 576-value latent (512 latent + 64 rotary), 512-value
 * output, 64-token pages, one latent head shared by every query head.
 *
 * Layouts (all row-major, contiguous, device memory, 16-byte aligned):
 *   q             bf16  [batch][s_q][h_q][576]   query row r = i*h_q + h
 *   kv_cache      bf16  [num_pages][64][576]
 *   block_table   int32 [batch][max_pages]        entries < ceil(L/64) used
 *   cache_seqlens int32 [batch]
 *   out           bf16  [batch][s_q][h_q][512]
 *   lse           fp32  [batch][s_q][h_q]
 *
 * Call sequence for one decode step (every call is asynchronous on `stream`):
 *   mla_get_metadata(...)       once per step (depends only on cache_seqlens)
 *   mla_decode_paged(...)       per layer
 *   mla_combine(...)            per layer, after decode, same stream
 *
 * Ownership.  The caller allocates and frees every buffer; the library never
 * allocates, frees or synchronizes.  Pointers must stay valid until the work
 * queued on `stream` has finished.  The only library state is a per-device
 * cache of the compute-unit count.
 *
 * Errors.  Host-visible arguments are checked before anything is launched; a
 * failed check returns a status and launches nothing.  A failed launch
 * returns MLA_ERR_HIP.  Device-side contents are preconditions: every
 * cache_seqlens[b] in [0, max_pages*64], and every used block_table entry
 * (j < ceil(L_b/64)) in [0, num_pages).  They are not checked unless debug
 * checks are on (MLA_DEBUG=1 in the environment, or mla_set_debug_checks):
 * then each decode call first checks them on the device, waits for the
 * result, and returns MLA_ERR_DEVICE_CONTENTS without launching the decode
 * if any is violated.  No C++ exception crosses this ABI.
 */
#ifndef MLA_PAGED_H
#define MLA_PAGED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, bad scale */
  MLA_ERR_UNSUPPORTED = 2,      /* shape outside the supported limits below */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4,              /* a HIP runtime call or launch failed */
  MLA_ERR_DEVICE_CONTENTS = 5,  /* debug checks: a length or used block-table entry out of range */
  MLA_ERR_SCRATCH_TOO_SMALL = 6 /* mla_decode_step_noalloc: the shape needs more than its scratch */
} mla_status_t;

#define MLA_HEAD_DIM 576
#define MLA_V_DIM 512
#define MLA_PAGE_SIZE 64
#define MLA_META_INTS 8      /* ints per partition in tile_metadata */
#define MLA_MAX_BATCH 65536
#define MLA_MAX_ROWS 65536   /* s_q * h_q, e.g. a 512-token chunk at 128 heads */
#define MLA_MAX_PARTS 4096   /* partitions of the key range (see below) */
#define MLA_NOPE_DIM 128     /* per-head query part before absorption; value head width */
#define MLA_ROPE_DIM 64      /* rotary part of the query and of the cache entry */
#define MLA_MAX_APPEND 65536 /* new tokens per sequence in one mla_kv_append */
#define MLA_MAX_FUSED_BATCH 1024 /* sequences for a decode that schedules itself */
#define MLA_FP8_TOKEN_BYTES 656  /* one token of the FP8 latent cache (see mla_kv_quantize_fp8) */
#define MLA_MAX_PREFILL_HEADS 65535 /* heads of one mla_prefill_attention / mla_prefill_expand_kv */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20) /* static scratch of mla_decode_step_noalloc, per GPU */

/*
 * Debug checks of device contents before every mla_decode_paged /
 * mla_decode_paged_fp8 call (see "Errors" above).  on = 1 turns them on,
 * 0 off, a negative value leaves the setting as it is; returns the previous
 * setting (1 or 0).  The first call of the library takes the default from
 * the environment: on when MLA_DEBUG is set to anything but "0".  With the
 * checks on, a decode waits for its stream (one small check launch and a
 * 4-byte read back) and returns MLA_ERR_UNSUPPORTED on a stream under graph
 * capture.  The checks read only the lengths and the block-table entries
 * the decode would read; their error word is a 4-byte device variable per
 * GPU, shared by every call on it.
 */
int32_t mla_set_debug_checks(int32_t on);

/*
 * Number of key-range partitions used for `num_cus` compute units
 * (0 = the current device's count).  Query rows are processed in groups of up
 * to 64; the partitions times the row groups give about one workgroup per
 * compute unit.  Returns 0 for invalid arguments.
 */
int32_t mla_num_partitions(int32_t s_q, int32_t h_q, int32_t num_cus);

/* int32 entries of tile_metadata: mla_num_partitions(...) * MLA_META_INTS. */
size_t mla_metadata_ints(int32_t s_q, int32_t h_q, int32_t num_cus);

/*
 * Bytes of workspace mla_decode_paged / mla_combine need: bf16 normalized
 * partial outputs and float32 log-sum-exps for sequences whose keys are
 * split over several partitions, one slot per (sequence, split).  With a single partition
 * (s_q * h_q of 16384 rows or more on 256 CUs) nothing is split: 256 bytes,
 * never written, and mla_combine launches nothing.
 */
size_t mla_workspace_bytes(int32_t batch, int32_t s_q, int32_t h_q, int32_t num_cus);

/*
 * Split-KV schedule.  Reads cache_seqlens on the device and writes
 *   tile_metadata int32 [partitions][8]: per partition the half-open range of
 *       (sequence, page) work it owns, {b_begin, page_begin, b_end, page_end,
 *       first_split, units_per_partition, fixed_cost, total_units}, pages
 *       counted in 64-token units (an empty sequence counts as one page that
 *       holds nothing); first_split is the index, among the partitions that
 *       share sequence b_begin, of this one; the last three describe the cut
 *       (every sequence costs fixed_cost + its pages; partition p starts at
 *       unit p * units_per_partition);
 *   num_splits    int32 [batch + 1]: exclusive prefix over sequences of how
 *       many partitions share each one (num_splits[batch] = slots used).
 * Work is balanced by cutting the concatenation of every sequence's pages,
 * each sequence charged a fixed extra cost, into equal shares.  One
 * workgroup, asynchronous on `stream`.
 */
mla_status_t mla_get_metadata(const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                              int32_t h_q, int32_t num_cus, int32_t* tile_metadata,
                              int32_t* num_splits, hipStream_t stream);

/*
 * Decode.  Each workgroup walks its partition's pages, streams every 64-token
 * latent page from HBM into LDS once, and runs Q.K^T and P.V on bf16 matrix
 * cores with an online softmax.  Sequences owned by one partition are
 * written straight to out/lse; the others write bf16 partials into the
 * workspace for mla_combine.  tile_metadata and num_splits must come from
 * mla_get_metadata with the same cache_seqlens, batch, s_q, h_q and num_cus.
 * Alternatively, when batch <= MLA_MAX_FUSED_BATCH and
 * batch * (max_pages + 2) < 2^30, tile_metadata may be NULL: the decode then
 * computes the same schedule inside its launch (every workgroup for itself)
 * and writes num_splits (batch + 1 ints, device) for mla_combine; larger
 * batches or block tables with a NULL tile_metadata return
 * MLA_ERR_UNSUPPORTED.  With tile_metadata given, num_splits is only read.
 * softmax_scale must be finite and positive (the workloads use 1/sqrt(192),
 * the per-head query width before absorption; the pages state no scale);
 * anything else returns MLA_ERR_INVALID_ARGUMENT.
 */
mla_status_t mla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_table,
                              const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                              int32_t h_q, int32_t num_pages, int32_t max_pages,
                              float softmax_scale, int32_t causal, const int32_t* tile_metadata,
                              int32_t* num_splits, int32_t num_cus, void* workspace,
                              size_t workspace_bytes, void* out, float* lse, hipStream_t stream);

/*
 * Combine.  For every sequence split over several partitions, merges the
 * partials by log-sum-exp: lse = ln sum_s exp(lse_s), out = sum_s
 * exp(lse_s - lse) o_s, rounded to bf16.  Partials with lse_s = -inf carry no
 * weight; if every one is -inf the row is written as out = 0, lse = -inf.
 * Sequences owned by one partition are left untouched.
 */
mla_status_t mla_combine(const void* workspace, size_t workspace_bytes, const int32_t* num_splits,
                         int32_t batch, int32_t s_q, int32_t h_q, int32_t num_cus, void* out,
                         float* lse, hipStream_t stream);

/*
 * One whole decode step -- the split-KV schedule, mla_decode_paged and
 * mla_combine -- that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation).  Arguments, layouts and
 * results are those of mla_decode_paged followed by mla_combine (the
 * schedule inside the decode where mla_decode_paged accepts a NULL
 * tile_metadata, the separate mla_get_metadata otherwise), on the current
 * device's compute units.  The schedule, the split counts and the split
 * partials live in a static device array of MLA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that each GPU running this library holds until the process ends;
 * a shape that needs more (split counts + schedule + mla_workspace_bytes,
 * each rounded up to 256 bytes) returns MLA_ERR_SCRATCH_TOO_SMALL and
 * launches nothing.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other threads) race: the caller
 * orders them.  Asynchronous on `stream`; no hipMalloc or hipFree, no
 * synchronization (unless the debug checks are on).  Other errors as for
 * mla_decode_paged.
 */
mla_status_t mla_decode_step_noalloc(const void* q, const void* kv_cache,
                                     const int32_t* block_table, const int32_t* cache_seqlens,
                                     int32_t batch, int32_t s_q, int32_t h_q, int32_t num_pages,
                                     int32_t max_pages, float softmax_scale, int32_t causal,
                                     void* out, float* lse, hipStream_t stream);

/*
 * Query absorption, the step before mla_decode_paged.  Keys and values are
 * one compressed latent per token, widened per head only at compute time
 * (FlashMLA release note, paragraph on the MLA core principles; DeepSeek-V3
 * summary, paragraph on memory efficiency).  Head h's key for token t is
 * [W_UK,h c_t ; r_t] (c_t the 512-value latent, r_t the 64-value rotary key,
 * W_UK,h a 128 x 512 matrix), so its score with the query [q_nope ; q_rope]
 * equals the score of the absorbed query [W_UK,h^T q_nope ; q_rope] with the
 * cached [c_t ; r_t].  For every query token m = b * s_q + i and head h:
 *   q_out[m][h][0:512]   = W_UK,h^T q_nope[m][h]   (sum over 128 values)
 *   q_out[m][h][512:576] = q_rope[m][h]            (copied)
 *   q_nope  bf16 [batch][s_q][h_q][128]
 *   q_rope  bf16 [batch][s_q][h_q][64]
 *   w_uk_t  bf16 [h_q][512][128]: W_UK,h transposed, entry [h][c][d] = W_UK,h[d][c]
 *   q_out   bf16 [batch][s_q][h_q][576]: the q of mla_decode_paged
 * Products accumulate in fp32 and round once to bf16 (nearest even).  Device
 * pointers, 16-byte aligned, caller-owned; asynchronous on `stream`; the call
 * allocates nothing.  Errors: MLA_ERR_INVALID_ARGUMENT (null or misaligned
 * pointer, non-positive size), MLA_ERR_UNSUPPORTED (batch > MLA_MAX_BATCH or
 * s_q * h_q > MLA_MAX_ROWS), MLA_ERR_HIP.
 */
mla_status_t mla_absorb_query(const void* q_nope, const void* q_rope, const void* w_uk_t,
                              int32_t batch, int32_t s_q, int32_t h_q, void* q_out,
                              hipStream_t stream);

/*
 * Output absorption, the step after mla_decode_paged / mla_combine (same
 * passages): head h's value for token t is W_UV,h c_t, so its output is
 * W_UV,h applied to the latent output the decode returns.
 *   o[m][h][:] = W_UV,h out[m][h][:]                (128 values from 512)
 *   out   bf16 [batch][s_q][h_q][512]: the out of mla_decode_paged
 *   w_uv  bf16 [h_q][128][512]: W_UV,h as stored, entry [h][d][c]
 *   o     bf16 [batch][s_q][h_q][128]
 * Accumulation, pointers, errors: as mla_absorb_query.
 */
mla_status_t mla_absorb_output(const void* out, const void* w_uv, int32_t batch, int32_t s_q,
                               int32_t h_q, void* o, hipStream_t stream);

/*
 * Paged KV append with page allocation, the step before each decode step.
 * The cache is paged, 64 tokens per block (FlashMLA release note, paragraph
 * on the released paged BF16 cache), and blocks are handed out on demand as
 * sequences grow (Tom's Hardware FR article, paragraph on the techniques).
 * Sequence b's n_new new cache entries (each [512 latent ; 64 rotary]) go to
 * tokens L_b .. L_b + n_new - 1 of it: token t at page block_table[b][t/64],
 * slot t % 64.  A sequence that crosses into pages it does not hold yet
 * takes them from the free-page stack:
 *   k_b = ceil((L_b + n_new)/64) - ceil(L_b/64) new pages; with
 *   K_b = k_0 + .. + k_{b-1} and F = *free_count on entry, its i-th new page
 *   is free_pages[F - 1 - (K_b + i)] and goes to block_table[b][ceil(L_b/64) + i];
 *   on exit *free_count = F - (k_0 + .. + k_{batch-1}) and cache_seqlens[b] =
 *   L_b + n_new.
 * If the stack holds fewer pages than needed, or some ceil((L_b+n_new)/64)
 * exceeds max_pages, nothing at all is written except *status = 1;
 * otherwise *status = 0.
 *   kv_cache      bf16 [num_pages][64][576], written
 *   block_table   int32 [batch][max_pages]; the entries of held pages are read,
 *                 the new ones written
 *   cache_seqlens int32 [batch], read and advanced
 *   new_kv        bf16 [batch][n_new][576] (may be null when n_new = 0)
 *   free_pages    int32 [>= *free_count]: physical pages not in use (distinct,
 *                 < num_pages; not checked)
 *   free_count    int32 [1], status int32 [1]: device words
 * Device pointers, kv_cache and new_kv 16-byte aligned, caller-owned;
 * asynchronous on `stream` (two launches); allocates nothing.  Errors:
 * MLA_ERR_INVALID_ARGUMENT (null or misaligned pointer, non-positive size,
 * n_new < 0), MLA_ERR_UNSUPPORTED (batch > MLA_MAX_BATCH or n_new >
 * MLA_MAX_APPEND), MLA_ERR_HIP.  Shortage of pages is reported through
 * *status, on the device.
 */
mla_status_t mla_kv_append(void* kv_cache, int32_t num_pages, int32_t* block_table,
                           int32_t max_pages, int32_t* cache_seqlens, int32_t batch,
                           const void* new_kv, int32_t n_new, const int32_t* free_pages,
                           int32_t* free_count, int32_t* status, hipStream_t stream);

/*
 * FP8 latent cache (an extension: the DeepSeek-V3 hardware paper summary,
 * section on FP8 mixed precision, applies FP8 to matrix products, training
 * and communication, not to this cache).  Converts a bf16 cache
 * kv_cache [num_pages][64][576] (device) into kv_fp8 [num_pages][64][656]
 * bytes (device, caller-allocated), one record per token:
 *   bytes [0, 512)    the 512 latent values as OCP E4M3 codes,
 *   bytes [512, 528)  four float32 scales 2^e, one per 128 latent values,
 *   bytes [528, 656)  the 64 rotary values, bf16, unchanged.
 * A block's e is the smallest integer with max|x| <= 448 * 2^e (0 for an
 * all-zero block); each value becomes the E4M3 code nearest to x * 2^-e,
 * ties to the even code, with the sign of x.  code * 2^e is then exactly a
 * bf16 value, so the decode over the FP8 cache equals the bf16 decode over
 * the dequantized values.  Results for non-finite inputs are unspecified.
 * Both pointers 16-byte aligned.  Errors: MLA_ERR_INVALID_ARGUMENT (null or
 * misaligned pointer, num_pages <= 0), MLA_ERR_UNSUPPORTED (more than 2^31
 * tokens), MLA_ERR_HIP.
 */
mla_status_t mla_kv_quantize_fp8(const void* kv_cache, int32_t num_pages, void* kv_fp8,
                                 hipStream_t stream);

/*
 * Decode over the FP8 latent cache written by mla_kv_quantize_fp8
 * (kv_fp8 [num_pages][64][656] bytes); every other argument as for
 * mla_decode_paged, and the same combine follows.  Each page is copied as
 * is (41 KiB instead of 72 KiB) and converted in LDS into the bf16 tile the
 * matrix products read.  At most 16 query rows per sequence (s_q * h_q <=
 * 16) and tile_metadata required; other shapes return MLA_ERR_UNSUPPORTED.
 */
mla_status_t mla_decode_paged_fp8(const void* q, const void* kv_fp8, const int32_t* block_table,
                                  const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                                  int32_t h_q, int32_t num_pages, int32_t max_pages,
                                  float softmax_scale, int32_t causal,
                                  const int32_t* tile_metadata, int32_t* num_splits,
                                  int32_t num_cus, void* workspace, size_t workspace_bytes,
                                  void* out, float* lse, hipStream_t stream);

/*
 * MLA prefill, per-head form: the stage before decoding, run separately
 * from it (DeepSeek-V3 summary, paragraph on inference speed; FlashMLA
 * itself is a decode kernel, release note introduction).  For a whole
 * prompt the latent is widened per head first (release note, paragraph on
 * the MLA core principles): head h's key of token t is [W_UK,h c_t ; r_t]
 * and its value W_UV,h c_t, with c_t the 512-value latent and r_t the
 * 64-value rotary key shared by every head.
 *
 * mla_prefill_expand_kv widens the latents:
 *   latent  bf16 [tokens][latent_stride]: c_t = latent[t][0:512] (a cache
 *           entry [c ; r] has latent_stride 576); latent_stride >= 512, a
 *           multiple of 8, at most 2^21 (else MLA_ERR_UNSUPPORTED)
 *   w_uk, w_uv  bf16 [h_q][128][512]: W_UK,h and W_UV,h as stored
 *   k_nope  bf16 [tokens][h_q][128]: k_nope[t][h] = W_UK,h c_t
 *   v       bf16 [tokens][h_q][128]: v[t][h] = W_UV,h c_t
 * fp32 accumulation, one rounding to bf16 (nearest even).  One launch: both
 * products as [tokens][512] x [512][h_q * 128] matrix products.
 *
 * mla_prefill_attention: packed prompts, prompt s holding tokens
 * cu_seqlens[s] .. cu_seqlens[s+1] - 1 (cu_seqlens int32 [batch + 1],
 * device, non-decreasing from 0; max_seqlen >= the longest prompt, host).
 *   q       bf16 [tokens][h_q][192]: [q_nope (128) ; q_rope (64)] per head,
 *           rotary embedding already applied
 *   k_nope  bf16 [tokens][h_q][128], v bf16 [tokens][h_q][128]
 *   k_rope  bf16: row t at k_rope + t * rope_stride, 64 values (for the
 *           cache entries [c ; r]: k_rope = latent + 512, rope_stride 576);
 *           rope_stride >= 64, a multiple of 8
 *   o       bf16 [tokens][h_q][128]: sum_u exp(s_u - lse) v[u][h]
 *   lse     fp32 [tokens][h_q]: ln sum_u exp(s_u), natural log
 * with s_u = softmax_scale * dot(q[t][h], [k_nope[u][h] ; k_rope[u]]) over
 * the keys u of t's prompt at or before t (causal != 0) or all of them.
 * fp32 scores and accumulators, bf16 weights in the value product, out
 * rounded once to bf16.  softmax_scale finite and positive.  All pointers
 * device, 16-byte aligned, caller-owned; asynchronous on `stream`; nothing
 * allocated.  Errors: MLA_ERR_INVALID_ARGUMENT (null or misaligned pointer,
 * sizes or strides out of range, bad scale), MLA_ERR_UNSUPPORTED (batch >
 * MLA_MAX_BATCH, h_q > MLA_MAX_PREFILL_HEADS, or tokens * h_q * 128 >= 2^31
 * for the expansion), MLA_ERR_HIP.  cu_seqlens contents are a precondition.
 */
mla_status_t mla_prefill_expand_kv(const void* latent, int32_t latent_stride, int32_t tokens,
                                   const void* w_uk, const void* w_uv, int32_t h_q, void* k_nope,
                                   void* v, hipStream_t stream);
mla_status_t mla_prefill_attention(const void* q, const void* k_nope, const void* k_rope,
                                   int32_t rope_stride, const void* v,
                                   const int32_t* cu_seqlens, int32_t batch, int32_t h_q,
                                   int32_t max_seqlen, float softmax_scale, int32_t causal,
                                   void* o, float* lse, hipStream_t stream);

/*
 * Machine-limit probes (benchmark instruments, not part of the decode).
 * mla_probe_stream_read reads `bytes` (a multiple of 16, >= 16) of device
 * memory at `buf` (16-byte aligned) once with 16-byte loads from `blocks`
 * workgroups of 256 threads and writes one 4-byte word per workgroup to
 * `sink` (device, blocks * 4 bytes): its duration gives the streaming-read
 * rate this GPU reaches.  mla_probe_mfma runs `iters` x 4 independent bf16
 * 16x16x32 matrix instructions in each of 8 waves of `blocks` workgroups
 * (16384 flops each), no memory traffic; it writes blocks * 512 floats to
 * `sink` and, from workgroup 0, two 8-byte counts to `clocks` (device): the
 * shader-clock cycles and the 100 MHz real-time ticks its loop took, whose
 * ratio is the shader clock under matrix load.  Asynchronous on `stream`;
 * MLA_ERR_INVALID_ARGUMENT for null pointers or sizes out of range.
 */
mla_status_t mla_probe_stream_read(const void* buf, size_t bytes, void* sink, int32_t blocks,
                                   hipStream_t stream);
mla_status_t mla_probe_mfma(int32_t iters, int32_t blocks, void* sink, void* clocks,
                            hipStream_t stream);
/* mla_probe_lds: `iters` x 16 LDS reads per lane by 8 waves in each of
 * `blocks` workgroups (64 KiB of LDS each), kind 0 = 16-byte reads at the
 * decode's key-fragment addresses, kind 1 = transposed 8-byte reads
 * (ds_read_b64_tr_b16) at its value-fragment addresses; writes blocks * 512
 * ints to `sink` and workgroup 0's shader-clock cycles to `clocks` (one
 * 8-byte count), so bytes per clock per compute unit follow. */
mla_status_t mla_probe_lds(int32_t kind, int32_t iters, int32_t blocks, void* sink, void* clocks,
                           hipStream_t stream);
/* mla_probe_issue: whether matrix and vector work share a SIMD's time.  In
 * each of `blocks` workgroups of 8 waves (waves w and w + 4 on one SIMD),
 * kind 0: waves 0-3 run `iters` x 4 independent bf16 16x16x32 matrix
 * instructions, waves 4-7 nothing; kind 1: waves 4-7 run `iters` x 16
 * independent fp32 fused multiply-adds, waves 0-3 nothing; kind 2: waves 4-7
 * run `iters` x 4 independent exponentials; kind 3: kinds 0 and 1 at once;
 * kind 4: kinds 0 and 2 at once.  Writes blocks * 512 floats to `sink` and
 * workgroup 0's shader-clock cycles of waves 0 and 4 to `clocks` (two 8-byte
 * counts, device).  A launch of kind 3 that takes as long as kinds 0 and 1
 * back to back means the two kinds of work do not overlap. */
mla_status_t mla_probe_issue(int32_t kind, int32_t iters, int32_t blocks, void* sink,
                             void* clocks, hipStream_t stream);
/* mla_probe_copy_ring: the 64-row decode's page copies on their own.  Each
 * of `blocks` workgroups of 8 waves owns `slots` (2 .. 65536) consecutive
 * 36 KiB slots of `src` (device, 16-byte aligned, at least blocks x slots x
 * 36864 bytes, which the caller guarantees) and walks them cyclically for
 * `steps` (3 .. 2^20) steps: waves 4-7 copy each slot into a four-slot LDS
 * ring by LDS-DMA (nine 1 KiB copies per wave, two slots ahead, the decode's
 * chunk layout), wait for their copies of slot i, then one barrier opens
 * step i.  Waves 0-3: kind 0 only meet the barriers, kind 1 read the step's
 * slot as the decode's score waves read key fragments (576 bytes per lane),
 * kind 2 run 68 bf16 16x16x32 matrix instructions per step.  Writes blocks
 * x 512 ints to `sink` and, per workgroup g, two 8-byte counts to `clocks`
 * (device): the copying loop's shader-clock cycles (2 g) and the mean
 * cycles from the end of a slot's issue to the end of the wait for it
 * (2 g + 1).  With two slots per workgroup the data stays in L2; with
 * hundreds it streams from HBM. */
mla_status_t mla_probe_copy_ring(int32_t kind, const void* src, int32_t slots, int32_t steps,
                                 int32_t blocks, void* sink, void* clocks, hipStream_t stream);

/* Static, human-readable text of a status code. */
const char* mla_status_string(mla_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_H */
