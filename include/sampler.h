/*
 * sampler.h -- C ABI of the MI355X (gfx950) per-step batched sampler.
 *
 * One decode step of an LLM serving engine ends in a sampler: it turns the
 * [B, V] logits of the batch, plus per-request temperature / top_k / top_p,
 * into one int32 token per request; the token is written straight back into
 * the on-device token pool (the next step's input) and copied asynchronously
 * to pinned host memory (for the scheduler's finish checks).  The behaviour
 * follows the mini-sglang pages:
 *
 *   "The engine and the sampler", section "The sampler"   -- Sampler.prepare,
 *       Sampler.sample, sample_torch (temperature, top-k first, top-p second,
 *       one categorical draw; an all-greedy batch is a plain argmax);
 *   "The engine and the sampler", section "forward_batch" -- int32 tokens, a
 *       device copy, a non-blocking host copy and a completion event;
 *   "The scheduler skeleton and the offline interface", sections "Preparing a
 *       batch" (_make_write_tuple) and "_forward" -- token_pool[row, col] =
 *       token, a column of -1 lands in the last column; the step's input ids
 *       are gathered from the same pool at (row, position);
 *   "CacheManager: allocation, release and admission control" -- the page
 *       table rows of a step's newly allocated KV pages.
 *
 * Conventions for every entry point:
 *   - Return value: 0 (SAMPLER_OK) or a negative SAMPLER_E* code.  No C++
 *     exception crosses this boundary.  sampler_strerror() names a code;
 *     sampler_last_error() gives the detail of the handle's last failure.
 *   - "dev" pointers are device memory of the handle's device (e.g. from
 *     hipMalloc or torch); "host" pointers are host memory.  The caller owns
 *     every buffer it passes in; the library owns only the handle, a device
 *     workspace allocated once in sampler_create, a small pinned status word,
 *     pinned staging buffers for sampler_prepare and rings of events.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     sample_batch, write_tokens and gather_tokens only enqueue work on
 *     `stream`: they never allocate and never wait for the device
 *     (sampler_prepare and write_page_table may wait for their own staging
 *     buffers, see there).
 *   - Argument errors that the host can see are reported synchronously and
 *     nothing is enqueued.  Parameter *values* in device memory are never
 *     errors: they are clamped on the device as Sampler.prepare clamps them.
 *   - A handle is not thread-safe; use one handle per stream.  Calls on one
 *     handle share its workspace, so calls that overlap on different streams
 *     race.
 */
#ifndef DST_SAMPLER_H
#define DST_SAMPLER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define DST_API __attribute__((visibility("default")))
#else
#define DST_API
#endif

typedef struct dst_sampler dst_sampler;

enum sampler_dtype { SAMPLER_F32 = 0, SAMPLER_BF16 = 1 };

enum sampler_status {
    SAMPLER_OK = 0,
    SAMPLER_EINVAL = -1,      /* bad argument (null pointer, size, dtype, ...)      */
    SAMPLER_ENOMEM = -2,      /* workspace or event allocation failed               */
    SAMPLER_EHIP = -3,        /* a HIP runtime call or kernel launch failed         */
    SAMPLER_ENOTPINNED = -4,  /* host_pinned_out is not page-locked host memory     */
    SAMPLER_EDEVICE = -5,     /* a device-side bounds check fired (write/gather)     */
    SAMPLER_ETICKET = -6      /* unknown ticket                                      */
};

/* Largest top-k index list returned through sampler_debug.topk_idx_out. */
#define SAMPLER_DEBUG_TOPK 64

/* sampler_debug.flags: run every row through the exact multi-pass path
 * (re-reads each row several times) instead of the single-pass kernel. */
#define SAMPLER_DEBUG_FORCE_EXACT 1u
/* ... through the one-workgroup-per-row kernel (every batch with a
 * temperature array takes it by default). */
#define SAMPLER_DEBUG_FORCE_STREAM 2u
/* ... through the split-row kernel, the one sample_batch_static runs (a
 * misaligned logits pointer or row stride falls back to the per-row kernel). */
#define SAMPLER_DEBUG_FORCE_SPLIT 4u

/*
 * Optional per-call debug outputs (tests only; each field may be NULL; every
 * non-NULL field costs extra device traffic).  All are dev pointers.
 *   probs_out    [B, V] fp32, row-major: the final distribution r of each row
 *                (kept masses renormalised, zero elsewhere; one-hot for greedy
 *                rows).
 *   kept_out     [B] int32: length of the kept prefix of the descending order.
 *   topk_idx_out [B, 64] int32: the first min(k_eff, 64) token ids of the row
 *                in descending-logit order (ties by ascending id), -1 padded;
 *                for greedy rows the argmax then -1.
 *   rand_out     [B] uint64: the Philox word the row's uniform comes from
 *                (0 when the batch has no temperature array).
 *   flags        host value: 0, or one of SAMPLER_DEBUG_FORCE_EXACT,
 *                SAMPLER_DEBUG_FORCE_STREAM, SAMPLER_DEBUG_FORCE_SPLIT (all-greedy
 *                batches of fewer than 256 rows otherwise take the argmax kernel).
 */
typedef struct sampler_debug {
    float*    probs_out;
    int32_t*  kept_out;
    int32_t*  topk_idx_out;
    uint64_t* rand_out;
    uint32_t  flags;
} sampler_debug;

/*
 * sampler_create -- one sampler per engine ("The engine and the sampler",
 * section "The order of initialization": Sampler(device, vocab_size) is built
 * after the backends).
 *   out         host: receives the handle.
 *   device      HIP device ordinal the handle works on.
 *   max_batch   largest B any call will pass (1 .. 1<<20); sizes the workspace.
 *   vocab_size  V, the row length of every logits tensor (1 .. 1<<30).
 *   logits_dtype SAMPLER_F32 or SAMPLER_BF16 (raw bf16 bit patterns).
 *   seed        key of the counter-based generator (the engine seeds with 42).
 * Allocates the device workspace (hipMalloc), the pinned staging buffers
 * (hipHostMalloc, SAMPLER_PREP_SLOTS x (24 + 32) x max_batch bytes) and
 * events; the only call that allocates.  Errors: SAMPLER_EINVAL,
 * SAMPLER_ENOMEM, SAMPLER_EHIP.
 */
DST_API int sampler_create(dst_sampler** out, int device, int32_t max_batch, int32_t vocab_size,
                   int32_t logits_dtype, uint64_t seed);

/* sampler_destroy -- waits for the handle's outstanding tickets, frees its
 * resources.  NULL is a no-op. */
DST_API int sampler_destroy(dst_sampler* s);

/*
 * sample_batch -- one token per request ("The engine and the sampler", section
 * "The sampler": Sampler.sample and sample_torch, with Sampler.prepare's
 * clamps applied per row on the device).
 *   logits      dev [B, row_stride] of the handle's dtype, row-major; only the
 *               first V entries of each row are read.  Values must be finite.
 *   row_stride  elements between rows, >= V.
 *   B           rows, 0 .. max_batch (0 is a no-op).
 *   temperature dev [B] fp32, or NULL: the whole batch is greedy (plain
 *               row argmax, lowest index on ties).  A row whose temperature is
 *               not above 1e-6 (0, negative, NaN) is greedy: exact argmax.
 *   top_k       dev [B] int32 or NULL (disabled).  k < 1 or k >= V: disabled.
 *   top_p       dev [B] fp32 or NULL (disabled).  Clamped to [1e-6, 1];
 *               1 disables.  top-k is applied first, then top-p on the
 *               renormalised survivors; a rank is kept while the mass before
 *               it is < top_p (the top rank, with nothing before it, is
 *               never cut).
 *   min_p       dev [B] fp32 or NULL (disabled); the pages' exercise
 *               ("The engine and the sampler", section "Exercises"): keep
 *               the tokens whose probability (temperature applied, full
 *               distribution) is at least min_p times the largest, and
 *               intersect that with the top-k / top-p set.  A value not
 *               above 0 (or NaN) disables it; values above 1 act as 1.
 *   uid         dev [B] int64 request ids; required when temperature != NULL.
 *   step        decode-step counter.  The row's uniform u comes from
 *               Philox-4x64-10 with key (seed, 0) and counter
 *               (uid, step, 0, 0): u = (word0 >> 40) * 2^-24.  The token is the
 *               first id, in ascending id order, whose cumulative kept mass
 *               exceeds u times the total kept mass.
 *   tokens_out  dev [B] int32.
 *   dbg         NULL, or debug outputs (see sampler_debug).
 * Errors (synchronous, nothing enqueued): SAMPLER_EINVAL; launch failure:
 * SAMPLER_EHIP.
 */
DST_API int sample_batch(dst_sampler* s, void* stream, const void* logits, int64_t row_stride,
                 int32_t B, const float* temperature, const int32_t* top_k,
                 const float* top_p, const float* min_p, const int64_t* uid, uint64_t step,
                 int32_t* tokens_out, const sampler_debug* dbg);

/*
 * sample_batch_static -- sample_batch for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  No handle, no allocation of any kind: the split-row kernel's
 * workspace is a file-scope device array (18.5 MB, one copy per GPU,
 * held until the process ends), addressed through hipGetSymbolAddress on the
 * first call on each GPU.  Arguments as sample_batch, plus:
 *   device       HIP device ordinal the call runs on (made current for it).
 *   vocab_size   V, 1 .. 163840 for SAMPLER_F32, 1 .. 327680 for SAMPLER_BF16.
 *   logits_dtype SAMPLER_F32 or SAMPLER_BF16.
 *   seed         key of the counter-based generator (as sampler_create's).
 * B is limited to 0 .. 64; logits and every row start must be 16-byte
 * aligned.  No debug outputs.  Calls on one GPU share its workspace: calls
 * that overlap in time on one GPU (different streams, or threads) race and
 * must be serialised by the caller; consecutive calls on one stream are
 * safe.  Errors (synchronous, nothing enqueued): SAMPLER_EINVAL for sizes
 * beyond those limits or bad arguments, SAMPLER_EHIP; the message is
 * sampler_last_error(NULL) on the calling thread.
 */
DST_API int sample_batch_static(int device, void* stream, const void* logits, int64_t row_stride,
                        int32_t B, int32_t vocab_size, int32_t logits_dtype, uint64_t seed,
                        const float* temperature, const int32_t* top_k, const float* top_p,
                        const float* min_p, const int64_t* uid, uint64_t step,
                        int32_t* tokens_out);

/*
 * write_tokens -- token_pool[rows[b], cols[b]] = tokens[b], then an async copy
 * of tokens to host_pinned_out and a completion event ("The scheduler skeleton
 * and the offline interface", sections "Preparing a batch" and "_forward";
 * "The engine and the sampler", section "forward_batch").
 *   token_pool  dev [pool_rows, pool_cols] int32, row-major.
 *   rows, cols  dev [B] int64.  cols[b] == -1 means "do not write": it lands in
 *               the last column.  Any other out-of-range (row, col) skips that
 *               write and raises the handle's device flag (reported by
 *               sampler_wait / sampler_check as SAMPLER_EDEVICE).  Rows within
 *               one call must be distinct (one pool row per request;
 *               sampler_set_checks can verify it).
 *   tokens      dev [B] int32 (e.g. sample_batch's tokens_out).
 *   host_pinned_out  host [B] int32 page-locked (hipHostMalloc / torch
 *               pin_memory) or NULL (no host copy).  Must stay valid until the
 *               ticket completes.
 *   ticket_out  host, may be NULL: receives the ticket of this call.
 * Errors: SAMPLER_EINVAL, SAMPLER_ENOTPINNED (synchronous); SAMPLER_EHIP.
 */
DST_API int write_tokens(dst_sampler* s, void* stream, int32_t* token_pool, int64_t pool_rows,
                 int64_t pool_cols, const int64_t* rows, const int64_t* cols,
                 const int32_t* tokens, int32_t B, int32_t* host_pinned_out,
                 uint64_t* ticket_out);

/*
 * gather_tokens -- ids_out[i] = token_pool[rows[i], positions[i]]: the step's
 * input ids, gathered on the device so the host never sees token values
 * ("The scheduler skeleton and the offline interface", section "Preparing a
 * batch": input_tuple = (row, position) over each request's positions
 * [cached_len, device_len), packed one request after another; section
 * "_forward": input_ids = token_pool[input_tuple]).
 *   token_pool  dev [pool_rows, pool_cols] int32, row-major (read only).
 *   rows, positions  dev [n] int64, one (pool row, column) per input token.
 *               A decode batch has one entry per request, at device_len - 1.
 *               Indices are taken as given (no wrap of negative values): an
 *               entry outside [0, pool_rows) x [0, pool_cols) yields id -1 and
 *               raises the handle's device flag (SAMPLER_EDEVICE from the next
 *               sampler_wait / sampler_check).
 *   n           0 <= n <= INT32_MAX; n == 0 enqueues nothing.
 *   ids_out     dev [n] int32, written by the kernel; caller-owned.
 * Ordered on `stream` like every call: a gather after a write_tokens on the
 * same stream sees its tokens.  No ticket (no host side effect).
 * Errors: SAMPLER_EINVAL (synchronous); SAMPLER_EHIP.
 */
DST_API int gather_tokens(dst_sampler* s, void* stream, const int32_t* token_pool,
                          int64_t pool_rows, int64_t pool_cols, const int64_t* rows,
                          const int64_t* positions, int64_t n, int32_t* ids_out);

/*
 * write_page_table -- the cache manager's paged allocation write ("CacheManager:
 * allocation, release and admission control", sections "The free-page list"
 * and "Allocating pages for this step's tokens"): request r's new pages are
 * [ceil(cached_len[r] / page_size), ceil(device_len[r] / page_size)); going
 * through the requests in order, each new page takes the next entry of
 * page_starts, and every position p of the page gets
 * page_table[table_idx[r], p] = page_start + p % page_size.
 *   page_table  dev [table_rows, table_cols] int32, row-major.
 *   table_idx, cached_len, device_len  host [n_req] int64 (read before the
 *               call returns); 0 <= n_req <= max_batch; lengths >= 0.
 *   page_starts dev [n_pages] int32: the first token location of each newly
 *               allocated page, in request order (for example the front of
 *               a device free list).
 *   n_pages     the number of new pages; must equal the sum over requests of
 *               max(0, ceil(device_len / page_size) - ceil(cached_len /
 *               page_size)).
 *   page_size   >= 1.
 * The host stages one record per request with new pages in pinned memory
 * (SAMPLER_PREP_SLOTS buffers in rotation, as sampler_prepare) and one
 * kernel on `stream` expands them.  n_pages == 0 enqueues nothing.
 * Errors (synchronous, nothing enqueued): SAMPLER_EINVAL for bad arguments,
 * n_pages not matching, or a page range outside the table; SAMPLER_EHIP.
 */
DST_API int write_page_table(dst_sampler* s, void* stream, int32_t* page_table,
                             int64_t table_rows, int64_t table_cols, const int64_t* table_idx,
                             const int64_t* cached_len, const int64_t* device_len, int32_t n_req,
                             const int32_t* page_starts, int64_t n_pages, int32_t page_size);

/*
 * sampler_prepare -- Sampler.prepare moved into the library ("The engine and
 * the sampler", section "The sampler"): the batch's request-level sampling
 * parameters, given as host arrays, become the per-request device tensors
 * that sample_batch reads, through one pinned staging buffer and one
 * asynchronous upload on `stream` (a small kernel that reads the staging
 * buffer through its device mapping).
 *   B           requests, 0 .. max_batch.
 *   temperature host [B] fp32, or NULL (every request greedy).  A request is
 *               greedy iff its temperature is <= 0.  If every request is
 *               greedy nothing is copied and out->temperature is NULL
 *               (sample_batch then takes the plain argmax path).
 *   top_k       host [B] int32, or NULL (no request sets it).
 *   top_p       host [B] fp32, or NULL (no request sets it).
 *   min_p       host [B] fp32, or NULL (no request sets it).
 *   uid         host [B] int64; required unless every request is greedy.
 *   dev_block   dev, caller-owned, 8-byte aligned, at least
 *               SAMPLER_PREP_BYTES(B) bytes; receives, packed:
 *               uid int64[B] | temperature fp32[B] | top_k int32[B] |
 *               top_p fp32[B] | min_p fp32[B]
 *               with the pages' values: temperature max(0 if greedy else T,
 *               1e-6); top_k k if k >= 1 else vocab_size; top_p
 *               min(max(p, 1e-6), 1) (each computed in double, stored
 *               rounded to fp32); min_p as given (0 where not set).  The caller must not reuse it before the
 *               sample_batch that reads it has run (stream order suffices).
 *   out         host: device pointers into dev_block for sample_batch, each
 *               NULL where the pages pass None: temperature (all greedy),
 *               top_k (every entry equals vocab_size), top_p (no entry
 *               below 1), min_p (no entry above 0); uid NULL with
 *               temperature.
 * The host arrays are read before the call returns (pageable memory is
 * fine).  The library keeps SAMPLER_PREP_SLOTS pinned staging buffers in
 * rotation; a call waits on the host only if the upload issued from the same
 * buffer that many calls earlier has not finished.
 * Errors: SAMPLER_EINVAL (synchronous, nothing enqueued); SAMPLER_EHIP.
 */
#define SAMPLER_PREP_BYTES(B) ((int64_t)(B) * 24)
#define SAMPLER_PREP_SLOTS 8

typedef struct sampler_args {
    const float*   temperature;
    const int32_t* top_k;
    const float*   top_p;
    const float*   min_p;
    const int64_t* uid;
    int32_t        B;
} sampler_args;

DST_API int sampler_prepare(dst_sampler* s, void* stream, int32_t B, const float* temperature,
                            const int32_t* top_k, const float* top_p, const float* min_p,
                            const int64_t* uid, void* dev_block, int64_t block_bytes,
                            sampler_args* out);

/*
 * sampler_wait -- block until the ticket's work (and its host copy) is done:
 * copy_done_event.synchronize() of "The engine and the sampler", section
 * "forward_batch".  Returns SAMPLER_EDEVICE if a device bounds check has
 * fired since the last sampler_check, SAMPLER_ETICKET for a ticket never
 * issued.  Tickets older than the event ring (256) wait on a later ticket.
 */
DST_API int sampler_wait(dst_sampler* s, uint64_t ticket);

/* sampler_query -- 1 if the ticket is done, 0 if pending, <0 on error. */
DST_API int sampler_query(dst_sampler* s, uint64_t ticket);

/* sampler_check -- waits for the whole device, returns SAMPLER_EDEVICE if a
 * device bounds check (or an enabled debug check) fired since the last check,
 * and clears the flags. */
DST_API int sampler_check(dst_sampler* s);

/* sampler_set_checks flags. */
#define SAMPLER_CHECK_DUPLICATE_ROWS 1u

/*
 * sampler_set_checks -- debug checks for the handle's later calls (0: none,
 * the default).  SAMPLER_CHECK_DUPLICATE_ROWS: before each write_tokens, a
 * kernel compares every pair of requests that write (cols != -1) and raises
 * the handle's device flag if two name the same pool row -- each request owns
 * one row of the pool ("The scheduler skeleton and the offline interface",
 * section "Preparing a batch").  Reported by sampler_wait / sampler_check as
 * SAMPLER_EDEVICE; costs O(B^2) comparisons per call.  Errors: SAMPLER_EINVAL
 * for an unknown flag.
 */
DST_API int sampler_set_checks(dst_sampler* s, uint32_t flags);

/* sampler_strerror -- static string for a status code. */
DST_API const char* sampler_strerror(int code);

/* sampler_last_error -- detail of the handle's last failure ("" if none);
 * NULL: of the calling thread's last failed sample_batch_static. */
DST_API const char* sampler_last_error(dst_sampler* s);

#ifdef __cplusplus
}
#endif

#endif /* DST_SAMPLER_H */
