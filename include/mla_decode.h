/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) paged MLA decode library.
 *
 * The operation (deepseek.csdn.net FlashMLA article, section 2.2, the MLA
 * output equation and the matrix-absorption paragraph after it): for every
 * sequence b, query token i and query head h,
 *
 *     O[b,i,h,:]  = sum_j softmax_j(sigma * q[b,i,h,:] . K_b[j,:]) * K_b[j, 0:dv]
 *     LSE[b,h,i]  = ln sum_j exp(sigma * q[b,i,h,:] . K_b[j,:])
 *
 * where K_b[j] is the cached latent row [c^KV (512); k^R (64)] of token j of
 * sequence b for latent head h / (h_q / h_kv), the sum runs over the tokens
 * the query sees (all L_b tokens, or with causal=1 tokens 0 .. L_b - s_q + i),
 * and sigma defaults to 1/sqrt(192).  Rows that see no token get O = 0 and
 * LSE = -inf.  The cache is paged in 64-token blocks addressed through
 * block_table (same article, section 4.2(1)).
 *
 * The two calls follow the usage on the dolphin-ai.jp FlashMLA page
 * ("FlashMLA の使用方法", steps 3 and 4):
 *     get_mla_metadata(cache_seqlens, s_q*h_q/h_kv, h_kv)
 *         -> tile_scheduler_metadata, num_splits
 *     flash_mla_with_kvcache(q, kvcache, block_table, cache_seqlens, dv,
 *                            tile_scheduler_metadata, num_splits, causal)
 *         -> o, lse
 *
 * Conventions for every entry point:
 *   - Pointers marked [dev] are device memory; the caller owns every buffer.
 *     The library allocates nothing and keeps only a per-device cache of the
 *     compute-unit count.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Launches are
 *     asynchronous and stream-ordered; nothing synchronises the host.  Inputs
 *     must stay alive until the stream has run the work.
 *   - Calls return MLA_OK or a negative status.  Arguments are checked on the
 *     host before anything is launched, so an invalid call launches nothing.
 *     The *contents* of block_table and cache_seqlens live on the device and
 *     are not checked by default.  The decode kernels never form an address
 *     outside the cache from them: a page id outside [0, num_pages) is read
 *     as a page of zeros, and blocks past max_pages_per_seq (a length above
 *     64 * max_pages_per_seq) as such a page too; the output for that
 *     sequence is then meaningless but finite.  mla_check_inputs() finds such
 *     entries, and with MLA_DEBUG_CHECKS=1 in the environment (or
 *     mla_set_debug_checks(1)) every decode call runs it first and returns
 *     MLA_ERR_BAD_INPUT without launching the decode.
 *   - Fixed sizes: d_qk = 576, dv = 512, page size 64, bf16 q / kvcache / o,
 *     fp32 lse.  All tensors are dense and row-major in the layouts below.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1)  /* null pointer, non-positive size, h_q % h_kv != 0, ... */
#define MLA_ERR_UNSUPPORTED (-2)  /* d_qk != 576, dv != 512, misaligned pointer, size limits */
#define MLA_ERR_WORKSPACE (-3)    /* workspace smaller than mla_workspace_bytes() */
#define MLA_ERR_METADATA (-4)     /* num_workers inconsistent with the launch */
#define MLA_ERR_HIP (-5)          /* the HIP runtime reported an error */
#define MLA_ERR_BAD_INPUT (-6)    /* debug checks: a block_table / cache_seqlens entry is out of range */

#define MLA_PAGE_SIZE 64
#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_METADATA_INTS 8       /* ints per worker row of tile_scheduler_metadata */
#define MLA_ROWS_PER_BLOCK 64     /* query rows one workgroup serves when rows_per_kv <= 128 ... */
#define MLA_ROWS_PER_WIDE_BLOCK 128  /* ... and when rows_per_kv > 128 */
#define MLA_MAX_WORKERS 4096

/* Text for a status code (static storage, never NULL). */
const char* mla_status_string(int status);

/* Number of scheduler workers W for a launch on `device` (-1 = current
 * device): W = max(1, CUs / (h_kv * ceil(rows_per_kv / rb))), capped at
 * MLA_MAX_WORKERS, where rows_per_kv = s_q * h_q / h_kv and rb, the query
 * rows of one workgroup, is 64 for rows_per_kv <= 128 and 128 above (one
 * workgroup per CU either way).  Host-only; reads the
 * device's compute-unit count once and caches it. */
int mla_num_workers(int device, int rows_per_kv, int h_kv, int* num_workers);

/* The split rule's fixed per-sequence overhead F, in page units. */
int mla_sched_fixed_overhead(void);

/* Split-KV tile scheduler (dolphin-ai.jp FlashMLA page, "FlashMLA の使用方法"
 * step 3; balance over variable lengths: deepseek.csdn.net article, section
 * 4.2(2)).  Each sequence is F overhead units followed by ceil(L_b/64) page
 * units on one cost line of total T; worker w owns units [w*Q, (w+1)*Q) with
 * Q = max(1, ceil(T / W)).  Writes, on the device, with one workgroup and no
 * host synchronisation:
 *   tile_scheduler_metadata [dev] int32 [num_workers][8]: per worker
 *       (begin_b, begin_page, end_b, end_page_exclusive, split ordinal of its
 *        first segment, 0, 0, 0); a worker with no pages gets
 *       (0, 0, -1, 0, 0, 0, 0, 0);
 *   num_splits [dev] int32 [batch + 1]: exclusive prefix sums of the number
 *       of splits of each sequence (num_splits[0] = 0).
 * cache_seqlens [dev] int32 [batch].  num_workers must be the value
 * mla_num_workers() gives for the same rows_per_kv and h_kv (any value in
 * [1, MLA_MAX_WORKERS] is accepted; mla_decode_paged must get the same). */
int mla_get_metadata(const int32_t* cache_seqlens, int batch, int rows_per_kv, int h_kv,
                     int num_workers, int32_t* tile_scheduler_metadata, int32_t* num_splits,
                     void* stream);

/* Bytes of workspace mla_decode_paged needs.  With slots = num_workers +
 * batch and rows = s_q*h_q/h_kv, the workspace holds, each part rounded up
 * to 256 bytes: fp32 split partials O_s [slots][h_kv][rows][dv], then fp32
 * lse_s [slots][h_kv][rows].  Returns 0 for invalid sizes.  Its contents
 * need no initialisation: every call writes what it later reads. */
size_t mla_workspace_bytes(int batch, int s_q, int h_q, int h_kv, int dv, int num_workers);

/* Paged MLA decode: split-KV attention over the paged latent cache followed
 * by the log-sum-exp merge of the splits (deepseek.csdn.net article, section
 * 4.2(1)).
 *   q              [dev] bf16 [batch][s_q][h_q][576], 16-byte aligned
 *   kvcache        [dev] bf16 [num_pages][64][h_kv][576], 16-byte aligned;
 *                  row = [c^KV (512); k^R (64)]; V = its first dv columns
 *   block_table    [dev] int32 [batch][max_pages_per_seq]; entries past
 *                  ceil(L_b/64) are never read (padding may be -1)
 *   cache_seqlens  [dev] int32 [batch], 0 <= L_b <= 64 * max_pages_per_seq
 *   d_qk, dv       must be 576 and 512
 *   tile_scheduler_metadata, num_splits, num_workers: from mla_get_metadata
 *                  with rows_per_kv = s_q*h_q/h_kv and the same h_kv
 *   causal         0 or 1; query token i sits at position L_b - s_q + i
 *   softmax_scale  <= 0 selects 1/sqrt(192)
 *   o              [dev] bf16 [batch][s_q][h_q][dv], 16-byte aligned
 *   lse            [dev] fp32 [batch][h_q][s_q], natural log, scale included
 *   workspace      [dev] >= mla_workspace_bytes(...) bytes, 256-byte aligned
 * Launches on `stream`: the decode kernel, then the combine kernel.  Each
 * workgroup of the decode kernel weighs keys against a per-row reference
 * taken from the first page of its split; should a later score rise more
 * than 48 (log2 units) above it, the workgroup runs that split again with
 * each row's maximum as the reference (ordinary inputs never need this). */
int mla_decode_paged(const void* q, const void* kvcache, const int32_t* block_table,
                     int max_pages_per_seq, int num_pages, const int32_t* cache_seqlens,
                     int batch, int s_q, int h_q, int h_kv, int d_qk, int dv,
                     const int32_t* tile_scheduler_metadata, const int32_t* num_splits,
                     int num_workers, int causal, float softmax_scale, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The first launch of mla_decode_paged alone: the split-KV decode kernel.
 * It writes o/lse of every sequence that has exactly one split and fp32
 * partials of the others into the workspace.  Same arguments and checks as
 * mla_decode_paged. */
int mla_decode_splitkv(const void* q, const void* kvcache, const int32_t* block_table,
                       int max_pages_per_seq, int num_pages, const int32_t* cache_seqlens,
                       int batch, int s_q, int h_q, int h_kv, int d_qk, int dv,
                       const int32_t* tile_scheduler_metadata, const int32_t* num_splits,
                       int num_workers, int causal, float softmax_scale, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* mla_decode_splitkv with its kernel timed: start_event and stop_event are
 * HIP events (hipEvent_t, created by the caller, not null) that the kernel
 * dispatch itself records when the decode kernel starts and when it ends, so
 * that the time between them is the kernel's own, without the dispatch gap
 * or end-of-launch cache write-back that events recorded on the stream
 * around the launch also span.  For measurement; same checks otherwise. */
int mla_decode_splitkv_timed(const void* q, const void* kvcache, const int32_t* block_table,
                             int max_pages_per_seq, int num_pages, const int32_t* cache_seqlens,
                             int batch, int s_q, int h_q, int h_kv, int d_qk, int dv,
                             const int32_t* tile_scheduler_metadata, const int32_t* num_splits,
                             int num_workers, int causal, float softmax_scale, void* o, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* start_event, void* stop_event);

/* The last launch alone: the log-sum-exp merge.  For each sequence with
 * n_b = num_splits[b+1] - num_splits[b] partials: n_b = 0 writes O = 0 and
 * LSE = -inf, n_b = 1 leaves what the decode kernel wrote, n_b > 1 writes
 * lse = M + ln sum_s exp(lse_s - M) (M = max_s lse_s) and
 * O = sum_s exp(lse_s - lse) * O_s in bf16.  The partials sit in the
 * workspace as fp32 O_s [slot][h_kv][rows][dv] followed by fp32 lse_s
 * [slot][h_kv][rows], slot = num_splits[b] + split ordinal. */
int mla_combine_splits(const int32_t* num_splits, int batch, int s_q, int h_q, int h_kv, int dv,
                       int num_workers, void* o, float* lse, const void* workspace,
                       size_t workspace_bytes, void* stream);

/* Maximum bytes of split partials mla_decode_paged_noalloc can hold: the
 * size of the library's static device scratch array. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* mla_decode_paged for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launches and results, with the split partials in a
 * static device array of MLA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on each GPU it runs on until the process ends, instead of a caller
 * workspace.  The caller still passes every input and the outputs o and lse.
 * The call allocates nothing; its first call on a device looks up the array's
 * address there.  Returns MLA_ERR_WORKSPACE, launching nothing, when
 * mla_workspace_bytes() of the call exceeds the array (e.g. 256 query rows per
 * latent head over more than ~250 workers plus sequences).  Every call on one
 * GPU shares that GPU's array: calls that may overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller.
 * Nothing in the array needs clearing: each call writes every partial it
 * reads.  Other arguments, checks and errors as mla_decode_paged. */
int mla_decode_paged_noalloc(const void* q, const void* kvcache, const int32_t* block_table,
                             int max_pages_per_seq, int num_pages, const int32_t* cache_seqlens,
                             int batch, int s_q, int h_q, int h_kv, int d_qk, int dv,
                             const int32_t* tile_scheduler_metadata, const int32_t* num_splits,
                             int num_workers, int causal, float softmax_scale, void* o, float* lse,
                             void* stream);

/* fp8 latent cache (the ruibaoantu.com page's outlook: BF16 mixed with
 * FP8; read here as fp8 storage of the cached rows with bf16 queries, bf16
 * MFMA products, fp32 accumulation and bf16 outputs).  The cache holds one
 * byte per value, OCP FP8 E4M3 ("E4M3FN": sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, 0x7F/0xFF NaN, largest finite 448), and
 * one fp32 scale kv_scale > 0 for the whole cache: a cached value is
 * e4m3_value(code) * kv_scale.
 *
 * mla_kvcache_append_fp8: mla_kvcache_append into such a cache
 *   (kvcache_fp8 [dev] uint8 [num_pages][64][h_kv][576], 16-byte aligned):
 *   each new bf16 value x is stored as the nearest E4M3 code, ties to even,
 *   of float(x) * (1 / kv_scale) (the reciprocal and the product in fp32)
 *   clamped to [-448, 448]; a NaN stays NaN (code 0xFF).  Other arguments,
 *   the bad_rows rule and errors as mla_kvcache_append; kv_scale must be a
 *   positive finite float (else MLA_ERR_INVALID_ARG).
 * mla_decode_paged_fp8: mla_decode_paged over such a cache, the result that
 *   of the cache's values e4m3_value(code) * kv_scale.  Heads of up to 128
 *   query rows (rows_per_kv = s_q*h_q/h_kv <= 128; MLA_ERR_UNSUPPORTED
 *   above).  The same metadata, workspace, outputs and errors as
 *   mla_decode_paged. */
int mla_kvcache_append_fp8(const void* kv_new, void* kvcache_fp8, float kv_scale, const int32_t* block_table,
                           int max_pages_per_seq, int num_pages, const int32_t* cache_seqlens, int batch, int s_new,
                           int h_kv, int d_qk, int32_t* bad_rows, void* stream);
int mla_decode_paged_fp8(const void* q, const void* kvcache_fp8, float kv_scale, const int32_t* block_table,
                         int max_pages_per_seq, int num_pages, const int32_t* cache_seqlens, int batch, int s_q,
                         int h_q, int h_kv, int d_qk, int dv, const int32_t* tile_scheduler_metadata,
                         const int32_t* num_splits, int num_workers, int causal, float softmax_scale, void* o,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Checker of the tables a decode reads (the paging contract of the
 * deepseek.csdn.net FlashMLA article, section 4.2(1): logical block j of
 * sequence b is physical page block_table[b][j]; the arguments of the call on
 * the dolphin-ai.jp FlashMLA page, "FlashMLA の使用方法" step 4).  One
 * workgroup checks, for every sequence b, that 0 <= L_b <= 64 *
 * max_pages_per_seq and that block_table[b][j] lies in [0, num_pages) for
 * every block j < ceil(L_b / 64) (padding past that is never read and not
 * checked), and writes
 *   result [dev] int32 [4]: number of bad entries, the first bad sequence
 *                (-1 if none), its first bad block (-1 when its length is
 *                bad), 0.
 * Asynchronous on `stream` like every launch; the caller reads result after
 * synchronising.  Errors: MLA_ERR_INVALID_ARG for null pointers or
 * non-positive sizes, MLA_ERR_UNSUPPORTED for misaligned pointers. */
int mla_check_inputs(const int32_t* block_table, int max_pages_per_seq, int num_pages,
                     const int32_t* cache_seqlens, int batch, int32_t* result, void* stream);

/* Turn the debug checks of every decode entry point on (1) or off (0) for
 * the process, overriding MLA_DEBUG_CHECKS.  With them on, mla_decode_paged,
 * mla_decode_splitkv and mla_decode_splitkv_timed run mla_check_inputs into
 * the first 16 bytes of their workspace, synchronise `stream` to read its
 * answer (so such calls cannot be captured into a graph), and return
 * MLA_ERR_BAD_INPUT without launching anything more if an entry is bad. */
void mla_set_debug_checks(int enable);

/* Whole-page allocator for the paged cache: memory goes out and comes back
 * only in whole pages of 64 token slots (the lukefan.com talk on FlashMLA, on
 * allocating and freeing in whole pages of 64; deepseek.csdn.net FlashMLA
 * article, section 4.2(2), paged KV cache management), and every call runs on
 * the stream with no host round trip.  Its state is caller memory:
 *   free_pages [dev] int32 [num_pages]: a stack of free page ids,
 *              free_pages[0 .. count) with the top at count - 1;
 *   state      [dev] int32 [4]: count; status of the last call (0 done,
 *              1 not enough free pages / the stack would overflow, 2 a
 *              length or page id out of range); pages the last call moved
 *              (or would have needed); 0.
 * A call that cannot be satisfied changes nothing but state[1..2]; the
 * caller reads state after synchronising.  Calls on one state must be
 * stream-ordered.
 *
 * mla_pages_init: every page free, free_pages[i] = num_pages - 1 - i (the
 *   first pages handed out are 0, 1, 2, ...).
 * mla_pages_reserve: before s_new tokens are appended to every sequence of
 *   lengths cache_seqlens (tokens cached now), sequence b needs
 *   ceil((L_b + s_new) / 64) - ceil(L_b / 64) more pages; sequences in batch
 *   order, and each one's blocks in ascending order, take pages popped from
 *   the top of the stack into block_table[b][ceil(L_b/64) ..].  Refused (1)
 *   if the free pages do not suffice, (2) if some L_b < 0 or
 *   ceil((L_b + s_new)/64) > max_pages_per_seq.
 * mla_pages_release: every sequence b with release[b] != 0 gives back its
 *   ceil(L_b / 64) mapped pages, pushed in the same order, and its entries
 *   become -1.  Refused (2) if a length or one of those page ids is out of
 *   range, (1) if the stack would hold more than num_pages (pages given back
 *   twice).  cache_seqlens is not changed by either call.
 * Errors (returned, nothing launched): MLA_ERR_INVALID_ARG for null pointers
 * or non-positive sizes (s_new may be 0), MLA_ERR_UNSUPPORTED for misaligned
 * pointers. */
int mla_pages_init(int32_t* free_pages, int32_t* state, int num_pages, void* stream);
int mla_pages_reserve(int32_t* free_pages, int32_t* state, int num_pages, const int32_t* cache_seqlens, int batch,
                      int s_new, int32_t* block_table, int max_pages_per_seq, void* stream);
int mla_pages_release(int32_t* free_pages, int32_t* state, int num_pages, const int32_t* cache_seqlens,
                      const int32_t* release, int batch, int32_t* block_table, int max_pages_per_seq, void* stream);

/* Measurement helper, not a step of the method: a plain streaming read of
 * `bytes` bytes at src (device memory; 16-byte aligned, bytes a multiple of
 * 16): one 512-thread workgroup per compute unit reading 64 KB runs, eight
 * 16-byte loads in flight per lane.  Timing it gives the achievable HBM read
 * rate that the decode's rooflines are reported beside.  sink [dev] 16 bytes, written only
 * in the (never expected) case that the folded data match a fixed pattern. */
int mla_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Measurement helper, not a step of the method: the rate at which one wave
 * reads LDS, the resource that feeds the decode's MFMAs their K, V and P
 * fragments.  Launches `blocks` workgroups of `waves` waves (4: one per SIMD,
 * as the 128-row decode workgroup; 8: two per SIMD, as the 64-row one); every
 * wave issues 64 * iters conflict-free reads of one kind from a 64 KB LDS
 * buffer, eight in flight, and each workgroup's first wave stores the shader
 * clock cycles (s_memtime) of its loop in cycles[block].  The rate per wave is
 * 64 * iters * (bytes per read) / cycles, bytes per read being 64 lanes
 * times 16, 8, 8 or 4 for kind 0 (ds_read_b128), 1 (ds_read_b64), 2
 * (ds_read_b64_tr_b16) or 3 (ds_read_b32).
 *   cycles [dev] int64 [blocks], written.  sink [dev] 16 bytes, written only
 *   in the (never expected) case that the folded data match a fixed pattern.
 * Errors (returned, nothing launched): MLA_ERR_INVALID_ARG for null pointers,
 * kind outside 0..3, waves other than 4 or 8, non-positive iters or blocks;
 * MLA_ERR_UNSUPPORTED for misaligned pointers. */
int mla_lds_read_rate(int kind, int waves, int iters, int blocks, int64_t* cycles, void* sink, void* stream);

/* The step before decode: write the latent rows of new tokens into the
 * paged cache.  The cache keeps the [c^KV (512); k^R (64)] row of every
 * token already seen, and a step computes only the new token's row and adds
 * it (deepseek.csdn.net FlashMLA article, section 4.1); pages of 64 slots
 * are mapped through block_table (same article, section 4.2(1)).
 *
 *   kv_new         [dev] bf16 [batch][s_new][h_kv][576]: rows to append.
 *   kvcache        [dev] bf16 [num_pages][64][h_kv][576], written in place.
 *   block_table    [dev] int32 [batch][max_pages_per_seq].
 *   cache_seqlens  [dev] int32 [batch]: tokens cached BEFORE this call.  New
 *                  token i of sequence b goes to position L_b + i, i.e. page
 *                  block_table[b][(L_b + i) / 64], slot (L_b + i) % 64.  The
 *                  call does not change cache_seqlens: the caller adds s_new
 *                  before the decode that reads the new rows.
 *   bad_rows       [dev] int32 counter or NULL: incremented once per
 *                  (token, latent head) row that is not written because its
 *                  position has no valid page (L_b < 0, position past the
 *                  block table, page id outside [0, num_pages)).  The caller
 *                  clears it.  Such rows are never written, so unlike the
 *                  decode's reads, a bad table entry cannot corrupt memory.
 *
 * The pages that receive rows must be owned by one sequence (a page shared
 * by two sequences that both append to it is a race), and kv_new must not
 * overlap kvcache.  Errors: MLA_ERR_INVALID_ARG for null pointers (other
 * than bad_rows) or non-positive sizes, MLA_ERR_UNSUPPORTED for d_qk != 576,
 * pointers not 16-byte (bf16 arrays) or 4-byte (int32) aligned, or sizes
 * past the library's limits. */
int mla_kvcache_append(const void* kv_new, void* kvcache, const int32_t* block_table, int max_pages_per_seq,
                       int num_pages, const int32_t* cache_seqlens, int batch, int s_new, int h_kv, int d_qk,
                       int32_t* bad_rows, void* stream);

/* The per-head projections on either side of the decode (deepseek.csdn.net
 * FlashMLA article, section 2.2, the matrix-absorption paragraph): the
 * decode works in the cache's latent space, so a head's query is absorbed
 * into it before, q~ = [W^UK^T q^C ; q^R] (q^C . W^UK c = W^UK^T q^C . c),
 * and its latent output is mapped to the head's value space after,
 * u = W^UV o (W^UV is linear and the attention weights are shared).
 * bf16 in and out, fp32 accumulation; d_h = 128, d_c = 512, RoPE part 64.
 *
 * mla_absorb_q:
 *   q_nope  [dev] bf16 [tokens][h_q][128]  (q^C of every head)
 *   q_rope  [dev] bf16 [tokens][h_q][64]   (q^R, copied unchanged)
 *   w_uk_t  [dev] bf16 [h_q][512][128]     (each head's W^UK, transposed)
 *   q_out   [dev] bf16 [tokens][h_q][576]  (the decode's q; tokens = B*s_q)
 * mla_absorb_o:
 *   o_latent [dev] bf16 [tokens][h_q][512] (the decode's o)
 *   w_uv     [dev] bf16 [h_q][128][512]    (each head's W^UV)
 *   out      [dev] bf16 [tokens][h_q][128]
 * Outputs must not overlap inputs.  Errors: MLA_ERR_INVALID_ARG for null
 * pointers or non-positive sizes, MLA_ERR_UNSUPPORTED for pointers that are
 * not 16-byte aligned or sizes past the library's limits. */
int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk_t, void* q_out, int tokens, int h_q,
                 void* stream);
int mla_absorb_o(const void* o_latent, const void* w_uv, void* out, int tokens, int h_q, void* stream);

/* The output projection over all heads (deepseek.csdn.net FlashMLA article,
 * section 2.2, second output equation): u_t = W^O [o_{t,1}; ...; o_{t,n_h}],
 * the per-head outputs (d_h = 128 each, the result of mla_absorb_o)
 * concatenated in head order and mapped by one matrix.  bf16 in and out,
 * fp32 accumulation.
 *   o_heads  [dev] bf16 [tokens][k]: row t = [o_{t,1}; ...; o_{t,n_h}],
 *            k = n_h * 128 (mla_absorb_o's output [tokens][h_q][128] is this
 *            layout)
 *   w_o      [dev] bf16 [n][k]: W^O, row-major (output column n's weights
 *            contiguous)
 *   out      [dev] bf16 [tokens][n]
 *   workspace [dev] fp32 scratch of mla_outproj_workspace_bytes(tokens, k, n)
 *            bytes (0 when the call needs none; then it may be NULL): the
 *            split-K partials, written before they are read.
 * k must be a multiple of 128 and n of 128; pointers 16-byte aligned.  The
 * result is deterministic (fixed summation order).  Errors:
 * MLA_ERR_INVALID_ARG (null pointers, non-positive sizes),
 * MLA_ERR_UNSUPPORTED (sizes or alignment), MLA_ERR_WORKSPACE. */
size_t mla_outproj_workspace_bytes(int tokens, int k, int n);
int mla_outproj(const void* o_heads, const void* w_o, void* out, int tokens, int k, int n, void* workspace,
                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
