// C ABI of the batched sampler: handle, argument checks, launches, tickets.
//
// The handle stands for the engine's Sampler ("The engine and the sampler",
// section "The sampler"); sample_batch is Sampler.sample with prepare's clamps
// done on the device; write_tokens is the scheduler's token-pool write-back
// plus forward_batch's non-blocking host copy and completion event ("The
// scheduler skeleton and the offline interface", section "_forward"; "The
// engine and the sampler", section "forward_batch"); gather_tokens is
// _forward's input gather from the same pool; sampler_prepare is
// Sampler.prepare (host parameters -> pinned staging -> one copy);
// write_page_table is the cache manager's paged allocation write.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "sampler.h"
#include "kernels.hpp"

namespace {

constexpr int kRing = 256;
// Completion events only: what the host reads after a wait (the token copy,
// the status word) is written by the kernels straight into host memory with
// system-scope stores, each followed in its thread by a system-scope release
// fence, so those stores are performed before the dispatch ends and hence
// before the event is signalled; the event needs no cache write-back at
// system scope of its own -- and skipping it saves ~2 us of idle GPU per
// event.
constexpr unsigned kEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;
// page-table staging: (row, first position, positions, first page) per request
constexpr size_t kPageRecordBytes = 4 * sizeof(int64_t);
// one thread per gathered entry: a dispatch holds fewer than 2^32 work-items
constexpr int64_t kMaxGather = INT32_MAX;
// all-greedy batches with at least this many rows fill the GPU with one
// workgroup per row and take the single-pass kernel; smaller ones split rows
constexpr int kStreamGreedyMinRows = 256;

// Workspace of sample_batch_static, the entry point that allocates nothing:
// the split-row kernel's records, candidate blocks, histograms, decision
// words and flags for up to kStaticRows rows of up to kStaticChunks chunks
// (fp32 rows up to 163840 entries, bf16 up to 327680).  One copy per GPU,
// zero at load, held until the process ends; the host addresses it only
// through the device address hipGetSymbolAddress returns for that GPU.
constexpr int kStaticRows = 64;
constexpr int kStaticChunks = 20;
constexpr size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }
constexpr size_t kStaticRecBytes = align256(sizeof(dst::SplitRec) * kStaticRows * kStaticChunks);
constexpr size_t kStaticCandBytes =
    align256(sizeof(uint64_t) * dst::kSplitCandStride * kStaticRows * kStaticChunks);
constexpr size_t kStaticHistBytes = align256(sizeof(float) * dst::kSplitHistBins * kStaticRows * kStaticChunks);
constexpr size_t kStaticDecBytes = align256(sizeof(uint32_t) * 4 * kStaticRows);
constexpr size_t kStaticFlagBytes = align256(sizeof(uint32_t) * dst::kSplitMaxChunks * kStaticRows);
constexpr size_t kStaticScratchBytes =
    kStaticRecBytes + kStaticCandBytes + kStaticHistBytes + kStaticDecBytes + kStaticFlagBytes;
constexpr int kStaticMaxDevices = 64;

}  // namespace

// sample_batch_static's workspace (see above): a kernel reaches it only
// through the per-GPU device address kept in g_static.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

struct StaticDevice {
    void* scratch = nullptr;    // device address of this GPU's copy (null: not set up yet)
    uint32_t epoch = 0;         // last launch's publication epoch on it
};
StaticDevice g_static[kStaticMaxDevices];
std::mutex g_static_mu;
thread_local std::string g_static_error;

int static_fail(int code, const char* msg, hipError_t he = hipSuccess) {
    g_static_error = msg;
    if (he != hipSuccess) {
        g_static_error += ": ";
        g_static_error += hipGetErrorString(he);
    }
    return code;
}

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
            changed = hipSetDevice(dev) == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (changed) (void)hipSetDevice(prev);
    }
};

}  // namespace

struct dst_sampler {
    int device = 0;
    int max_batch = 0;
    int vocab = 0;
    int dtype = 0;
    uint64_t seed = 0;
    int cus = 0;                       // compute units: stream blocks resident at once
    void* argmax_ws = nullptr;         // device: argmax slots and counters
    uint64_t* slot = nullptr;
    uint32_t* count = nullptr;
    void* workspace = nullptr;       // device: split-row records, candidates, histograms, flags
    dst::SplitRec* rec = nullptr;
    uint64_t* cand = nullptr;
    float* hist = nullptr;
    uint32_t* dec = nullptr;
    uint32_t* flags = nullptr;
    int split_nl = 0;                  // loads per thread and chunk (0: rows go to the exact kernel)
    int split_chunks = 0;              // chunks per row
    uint32_t epoch = 0;                // last launch's publication epoch
    uint32_t* status_host = nullptr;  // pinned, mapped: [0] bounds-check flag, [1] duplicate rows
    uint32_t checks = 0;               // SAMPLER_CHECK_* flags
    uint32_t* status_dev = nullptr;
    hipEvent_t ring[kRing] = {};
    uint64_t ring_ticket[kRing] = {};
    uint64_t issued = 0;               // tickets are 1, 2, 3, ...
    char* prep_host = nullptr;         // pinned, mapped: SAMPLER_PREP_SLOTS staging buffers
    char* prep_mapped = nullptr;       // ... as the device addresses them
    hipEvent_t prep_ev[SAMPLER_PREP_SLOTS] = {};
    bool prep_used[SAMPLER_PREP_SLOTS] = {};
    uint32_t prep_next = 0;
    int64_t* pt_host = nullptr;        // pinned, mapped: page-table record staging
    int64_t* pt_mapped = nullptr;
    hipEvent_t pt_ev[SAMPLER_PREP_SLOTS] = {};
    bool pt_used[SAMPLER_PREP_SLOTS] = {};
    uint32_t pt_next = 0;
    std::string last_error;
};

static int fail(dst_sampler* s, int code, const char* what, hipError_t e = hipSuccess) {
    if (s) {
        char buf[256];
        if (e != hipSuccess)
            std::snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
        else
            std::snprintf(buf, sizeof(buf), "%s", what);
        s->last_error = buf;
    }
    return code;
}

extern "C" {

const char* sampler_strerror(int code) {
    switch (code) {
        case SAMPLER_OK: return "ok";
        case SAMPLER_EINVAL: return "invalid argument";
        case SAMPLER_ENOMEM: return "out of memory";
        case SAMPLER_EHIP: return "HIP runtime error";
        case SAMPLER_ENOTPINNED: return "host buffer is not pinned";
        case SAMPLER_EDEVICE: return "device bounds check fired (out-of-range token-pool index)";
        case SAMPLER_ETICKET: return "unknown ticket";
        default: return "unknown status";
    }
}

const char* sampler_last_error(dst_sampler* s) { return s ? s->last_error.c_str() : g_static_error.c_str(); }

int sampler_destroy(dst_sampler* s) {
    if (!s) return SAMPLER_OK;
    DeviceGuard g(s->device);
    if (s->issued) (void)hipEventSynchronize(s->ring[s->issued % kRing]);
    for (int i = 0; i < SAMPLER_PREP_SLOTS; ++i) {
        if (s->prep_used[i]) (void)hipEventSynchronize(s->prep_ev[i]);
        if (s->pt_used[i]) (void)hipEventSynchronize(s->pt_ev[i]);
    }
    for (auto& e : s->ring)
        if (e) (void)hipEventDestroy(e);
    for (auto& e : s->prep_ev)
        if (e) (void)hipEventDestroy(e);
    for (auto& e : s->pt_ev)
        if (e) (void)hipEventDestroy(e);
    if (s->workspace) (void)hipFree(s->workspace);
    if (s->argmax_ws) (void)hipFree(s->argmax_ws);
    if (s->status_host) (void)hipHostFree(s->status_host);
    if (s->prep_host) (void)hipHostFree(s->prep_host);
    if (s->pt_host) (void)hipHostFree(s->pt_host);
    delete s;
    return SAMPLER_OK;
}

int sampler_create(dst_sampler** out, int device, int32_t max_batch, int32_t vocab_size,
                   int32_t logits_dtype, uint64_t seed) {
    if (!out) return SAMPLER_EINVAL;
    *out = nullptr;
    if (max_batch < 1 || max_batch > (1 << 20) || vocab_size < 1 || vocab_size > (1 << 30) ||
        (logits_dtype != SAMPLER_F32 && logits_dtype != SAMPLER_BF16))
        return SAMPLER_EINVAL;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
        (void)hipGetLastError();
        return SAMPLER_EINVAL;
    }
    dst_sampler* s = new (std::nothrow) dst_sampler();
    if (!s) return SAMPLER_ENOMEM;
    s->device = device;
    s->max_batch = max_batch;
    s->vocab = vocab_size;
    s->dtype = logits_dtype;
    s->seed = seed;
    DeviceGuard g(device);
    if (hipDeviceGetAttribute(&s->cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
        (void)hipGetLastError();
        s->cus = 0;                    // unknown: rows keep their index order
    }

    // split-row workspace: per (row, chunk) a record, a candidate block and a
    // weight histogram; per row a decision word and one cache line of epoch
    // flags (zero: nothing published yet)
    s->split_nl = dst::split_plan(vocab_size, logits_dtype, &s->split_chunks);
    const size_t rows = static_cast<size_t>(max_batch);
    const size_t nrec = rows * static_cast<size_t>(s->split_nl ? s->split_chunks : 0);
    const size_t rec_bytes = nrec * sizeof(dst::SplitRec);
    const size_t cand_bytes = nrec * dst::kSplitCandStride * sizeof(uint64_t);
    const size_t hist_bytes = nrec * dst::kSplitHistBins * sizeof(float);
    const size_t dec_bytes = rows * 4 * sizeof(uint32_t);
    const size_t flag_bytes = rows * dst::kSplitMaxChunks * sizeof(uint32_t);
    const size_t slot_bytes = sizeof(uint64_t) * rows;
    const size_t count_bytes = sizeof(uint32_t) * rows;
    hipError_t e = hipMalloc(&s->argmax_ws, slot_bytes + count_bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        sampler_destroy(s);
        return SAMPLER_ENOMEM;
    }
    s->slot = static_cast<uint64_t*>(s->argmax_ws);
    s->count = reinterpret_cast<uint32_t*>(static_cast<char*>(s->argmax_ws) + slot_bytes);
    e = hipMemset(s->argmax_ws, 0, slot_bytes + count_bytes);
    if (e == hipSuccess && s->split_nl) {
        e = hipMalloc(&s->workspace, rec_bytes + cand_bytes + hist_bytes + dec_bytes + flag_bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            sampler_destroy(s);
            return SAMPLER_ENOMEM;
        }
        char* ws = static_cast<char*>(s->workspace);
        s->rec = reinterpret_cast<dst::SplitRec*>(ws);
        s->cand = reinterpret_cast<uint64_t*>(ws + rec_bytes);
        s->hist = reinterpret_cast<float*>(ws + rec_bytes + cand_bytes);
        s->dec = reinterpret_cast<uint32_t*>(ws + rec_bytes + cand_bytes + hist_bytes);
        s->flags = reinterpret_cast<uint32_t*>(ws + rec_bytes + cand_bytes + hist_bytes + dec_bytes);
        e = hipMemset(s->dec, 0, dec_bytes + flag_bytes);
    }
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&s->status_host), 2 * sizeof(uint32_t),
                                           hipHostMallocMapped);
    if (e == hipSuccess) {
        s->status_host[0] = 0;
        s->status_host[1] = 0;
        e = hipHostGetDevicePointer(reinterpret_cast<void**>(&s->status_dev), s->status_host, 0);
    }
    for (int i = 0; e == hipSuccess && i < kRing; ++i)
        e = hipEventCreateWithFlags(&s->ring[i], kEventFlags);
    if (e == hipSuccess)
        e = hipHostMalloc(reinterpret_cast<void**>(&s->prep_host),
                          static_cast<size_t>(SAMPLER_PREP_SLOTS) * SAMPLER_PREP_BYTES(max_batch),
                          hipHostMallocMapped);
    if (e == hipSuccess)
        e = hipHostGetDevicePointer(reinterpret_cast<void**>(&s->prep_mapped), s->prep_host, 0);
    for (int i = 0; e == hipSuccess && i < SAMPLER_PREP_SLOTS; ++i)
        e = hipEventCreateWithFlags(&s->prep_ev[i], kEventFlags);
    if (e == hipSuccess)
        e = hipHostMalloc(reinterpret_cast<void**>(&s->pt_host),
                          static_cast<size_t>(SAMPLER_PREP_SLOTS) * kPageRecordBytes * max_batch,
                          hipHostMallocMapped);
    if (e == hipSuccess)
        e = hipHostGetDevicePointer(reinterpret_cast<void**>(&s->pt_mapped), s->pt_host, 0);
    for (int i = 0; e == hipSuccess && i < SAMPLER_PREP_SLOTS; ++i)
        e = hipEventCreateWithFlags(&s->pt_ev[i], kEventFlags);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipGetLastError();
        sampler_destroy(s);
        return SAMPLER_EHIP;
    }
    *out = s;
    return SAMPLER_OK;
}

int sample_batch(dst_sampler* s, void* stream, const void* logits, int64_t row_stride, int32_t B,
                 const float* temperature, const int32_t* top_k, const float* top_p,
                 const float* min_p, const int64_t* uid, uint64_t step, int32_t* tokens_out,
                 const sampler_debug* dbg) {
    if (!s) return SAMPLER_EINVAL;
    if (B < 0 || B > s->max_batch) return fail(s, SAMPLER_EINVAL, "sample_batch: B out of range");
    if (B == 0) return SAMPLER_OK;
    if (!logits || !tokens_out) return fail(s, SAMPLER_EINVAL, "sample_batch: null logits or tokens_out");
    if (row_stride < s->vocab) return fail(s, SAMPLER_EINVAL, "sample_batch: row_stride < vocab_size");
    if (temperature && !uid) return fail(s, SAMPLER_EINVAL, "sample_batch: uid required with temperature");
    DeviceGuard g(s->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    const uint32_t flags = dbg ? dbg->flags : 0u;
    const uint32_t forced = flags & (SAMPLER_DEBUG_FORCE_EXACT | SAMPLER_DEBUG_FORCE_STREAM | SAMPLER_DEBUG_FORCE_SPLIT);
    // the split-row kernel reads rows with 16-byte loads: the logits and every
    // row start must be 16-byte aligned, and the vocabulary within its chunk count
    const int64_t esize = s->dtype == SAMPLER_F32 ? 4 : 2;
    const bool aligned = (reinterpret_cast<uintptr_t>(logits) & 15u) == 0 && ((row_stride * esize) & 15) == 0;
    const bool split_ok = s->split_nl && aligned;
    if (!forced && !temperature && B < kStreamGreedyMinRows) {
        dst::ArgmaxArgs a{};
        a.logits = logits;
        a.row_stride = row_stride;
        a.B = B;
        a.V = s->vocab;
        dst::argmax_plan(B, s->vocab, s->dtype, &a.chunks, &a.chunk_len);
        a.slot = s->slot;
        a.count = s->count;
        a.tokens_out = tokens_out;
        if (dbg) {
            a.probs_out = dbg->probs_out;
            a.kept_out = dbg->kept_out;
            a.topk_idx_out = dbg->topk_idx_out;
            a.rand_out = dbg->rand_out;
        }
        e = dst::launch_argmax(a, s->dtype, st);
    } else {
        dst::SampleArgs a{};
        a.logits = logits;
        a.row_stride = row_stride;
        a.B = B;
        a.V = s->vocab;
        a.temperature = temperature;
        a.top_k = top_k;
        a.top_p = top_p;
        a.min_p = min_p;
        a.uid = uid;
        a.step = step;
        a.seed = s->seed;
        a.resident = s->cus;
        a.tokens_out = tokens_out;
        if (dbg) {
            a.probs_out = dbg->probs_out;
            a.kept_out = dbg->kept_out;
            a.topk_idx_out = dbg->topk_idx_out;
            a.rand_out = dbg->rand_out;
        }
        // every sampled batch takes the one-workgroup-per-row kernel: measured
        // on B = 1 .. 127 rows of 1024 to 151936 entries it is faster than the
        // split-row kernel (which the entry point without allocations uses)
        if (flags & SAMPLER_DEBUG_FORCE_EXACT) {
            e = dst::launch_sample_exact(a, s->dtype, st);
        } else if (split_ok && (flags & SAMPLER_DEBUG_FORCE_SPLIT)) {
            a.rec = s->rec;
            a.cand = s->cand;
            a.hist = s->hist;
            a.dec = s->dec;
            a.flags = s->flags;
            a.rec_stride = s->split_chunks;
            a.chunks = s->split_chunks;
            s->epoch = s->epoch + 2u == 0u ? 2u : s->epoch + 2u;
            a.epoch = s->epoch;
            e = dst::launch_sample_split(a, s->dtype, s->split_nl, st);
        } else {
            e = dst::launch_sample_stream(a, s->dtype, st);
        }
    }
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "sample_batch: launch", e);
    return SAMPLER_OK;
}

int sample_batch_static(int device, void* stream, const void* logits, int64_t row_stride, int32_t B,
                        int32_t vocab_size, int32_t logits_dtype, uint64_t seed, const float* temperature,
                        const int32_t* top_k, const float* top_p, const float* min_p, const int64_t* uid,
                        uint64_t step, int32_t* tokens_out) {
    if (device < 0 || device >= kStaticMaxDevices)
        return static_fail(SAMPLER_EINVAL, "sample_batch_static: device out of range");
    if (B < 0 || B > kStaticRows)
        return static_fail(SAMPLER_EINVAL, "sample_batch_static: B outside 0 .. 64 (the static workspace)");
    if (logits_dtype != SAMPLER_F32 && logits_dtype != SAMPLER_BF16)
        return static_fail(SAMPLER_EINVAL, "sample_batch_static: unknown logits dtype");
    if (vocab_size < 1) return static_fail(SAMPLER_EINVAL, "sample_batch_static: vocab_size < 1");
    int chunks = 0;
    const int nl = dst::split_plan(vocab_size, logits_dtype, &chunks);
    if (!nl || chunks > kStaticChunks)
        return static_fail(SAMPLER_EINVAL,
                           "sample_batch_static: vocab_size beyond the static workspace "
                           "(163840 fp32 / 327680 bf16 entries)");
    if (row_stride < vocab_size) return static_fail(SAMPLER_EINVAL, "sample_batch_static: row_stride < vocab_size");
    if (B == 0) return SAMPLER_OK;
    if (!logits || !tokens_out) return static_fail(SAMPLER_EINVAL, "sample_batch_static: null logits or tokens_out");
    if (temperature && !uid) return static_fail(SAMPLER_EINVAL, "sample_batch_static: uid required with temperature");
    const int64_t esize = logits_dtype == SAMPLER_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(logits) & 15u) != 0 || ((row_stride * esize) & 15) != 0)
        return static_fail(SAMPLER_EINVAL, "sample_batch_static: logits and row starts must be 16-byte aligned");
    DeviceGuard g(device);
    char* base = nullptr;
    uint32_t epoch = 0;
    {
        std::lock_guard<std::mutex> lock(g_static_mu);
        StaticDevice& sd = g_static[device];
        if (!sd.scratch) {
            // once per GPU, with that GPU current: the device address of its copy
            void* p = nullptr;
            const hipError_t he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (he != hipSuccess || !p) {
                (void)hipGetLastError();
                return static_fail(SAMPLER_EHIP, "sample_batch_static: hipGetSymbolAddress", he);
            }
            sd.scratch = p;
        }
        sd.epoch = sd.epoch + 2u == 0u ? 2u : sd.epoch + 2u;
        base = static_cast<char*>(sd.scratch);
        epoch = sd.epoch;
    }
    dst::SampleArgs a{};
    a.logits = logits;
    a.row_stride = row_stride;
    a.B = B;
    a.V = vocab_size;
    a.temperature = temperature;
    a.top_k = top_k;
    a.top_p = top_p;
    a.min_p = min_p;
    a.uid = uid;
    a.step = step;
    a.seed = seed;
    a.tokens_out = tokens_out;
    a.rec = reinterpret_cast<dst::SplitRec*>(base);
    a.cand = reinterpret_cast<uint64_t*>(base + kStaticRecBytes);
    a.hist = reinterpret_cast<float*>(base + kStaticRecBytes + kStaticCandBytes);
    a.dec = reinterpret_cast<uint32_t*>(base + kStaticRecBytes + kStaticCandBytes + kStaticHistBytes);
    a.flags = reinterpret_cast<uint32_t*>(base + kStaticRecBytes + kStaticCandBytes + kStaticHistBytes +
                                          kStaticDecBytes);
    a.rec_stride = kStaticChunks;
    a.chunks = chunks;
    a.epoch = epoch;
    const hipError_t e = dst::launch_sample_split(a, logits_dtype, nl, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return static_fail(SAMPLER_EHIP, "sample_batch_static: launch", e);
    return SAMPLER_OK;
}

int write_tokens(dst_sampler* s, void* stream, int32_t* token_pool, int64_t pool_rows,
                 int64_t pool_cols, const int64_t* rows, const int64_t* cols, const int32_t* tokens,
                 int32_t B, int32_t* host_pinned_out, uint64_t* ticket_out) {
    if (!s) return SAMPLER_EINVAL;
    if (B < 0) return fail(s, SAMPLER_EINVAL, "write_tokens: B < 0");
    if (B > 0 && (!token_pool || !rows || !cols || !tokens))
        return fail(s, SAMPLER_EINVAL, "write_tokens: null pointer");
    if (pool_rows < 1 || pool_cols < 1) return fail(s, SAMPLER_EINVAL, "write_tokens: empty pool");
    DeviceGuard g(s->device);
    int32_t* host_dev = nullptr;     // the pinned buffer as the device addresses it
    if (host_pinned_out && B > 0) {
        hipPointerAttribute_t attr;
        std::memset(&attr, 0, sizeof(attr));
        const hipError_t pe = hipPointerGetAttributes(&attr, host_pinned_out);
        if (pe != hipSuccess) (void)hipGetLastError();
        if (pe != hipSuccess || attr.type != hipMemoryTypeHost || !attr.devicePointer)
            return fail(s, SAMPLER_ENOTPINNED, "write_tokens: host_pinned_out is not pinned host memory");
        host_dev = static_cast<int32_t*>(attr.devicePointer);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (B > 0) {
        // one kernel: pool scatter plus the tokens stored straight into the
        // pinned buffer (system-scope stores), no separate copy
        if (s->checks & SAMPLER_CHECK_DUPLICATE_ROWS)
            e = dst::launch_check_rows(rows, cols, B, s->status_dev + 1, st);
        dst::WriteArgs a{token_pool, pool_rows, pool_cols, rows, cols, tokens, B, s->status_dev, host_dev};
        if (e == hipSuccess) e = dst::launch_write_tokens(a, st);
    }
    const uint64_t ticket = s->issued + 1;
    if (e == hipSuccess) e = hipEventRecord(s->ring[ticket % kRing], st);
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "write_tokens: enqueue", e);
    s->issued = ticket;
    s->ring_ticket[ticket % kRing] = ticket;
    if (ticket_out) *ticket_out = ticket;
    return SAMPLER_OK;
}

int gather_tokens(dst_sampler* s, void* stream, const int32_t* token_pool, int64_t pool_rows,
                  int64_t pool_cols, const int64_t* rows, const int64_t* positions, int64_t n,
                  int32_t* ids_out) {
    if (!s) return SAMPLER_EINVAL;
    if (n < 0) return fail(s, SAMPLER_EINVAL, "gather_tokens: n < 0");
    if (n > kMaxGather) return fail(s, SAMPLER_EINVAL, "gather_tokens: n too large");
    if (n > 0 && (!token_pool || !rows || !positions || !ids_out))
        return fail(s, SAMPLER_EINVAL, "gather_tokens: null pointer");
    if (pool_rows < 1 || pool_cols < 1) return fail(s, SAMPLER_EINVAL, "gather_tokens: empty pool");
    if (n == 0) return SAMPLER_OK;
    DeviceGuard g(s->device);
    dst::GatherArgs a{token_pool, pool_rows, pool_cols, rows, positions, n, ids_out, s->status_dev};
    const hipError_t e = dst::launch_gather_tokens(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "gather_tokens: launch", e);
    return SAMPLER_OK;
}

int sampler_prepare(dst_sampler* s, void* stream, int32_t B, const float* temperature,
                    const int32_t* top_k, const float* top_p, const float* min_p,
                    const int64_t* uid, void* dev_block, int64_t block_bytes, sampler_args* out) {
    if (!s) return SAMPLER_EINVAL;
    if (!out) return fail(s, SAMPLER_EINVAL, "sampler_prepare: null out");
    *out = sampler_args{nullptr, nullptr, nullptr, nullptr, nullptr, B};
    if (B < 0 || B > s->max_batch) return fail(s, SAMPLER_EINVAL, "sampler_prepare: B out of range");
    // a request is greedy iff its temperature is <= 0 (NaN is not)
    bool all_greedy = true;
    for (int32_t b = 0; temperature && b < B && all_greedy; ++b) all_greedy = temperature[b] <= 0.0f;
    if (all_greedy) return SAMPLER_OK;
    if (!uid) return fail(s, SAMPLER_EINVAL, "sampler_prepare: uid required unless all greedy");
    if (!dev_block || (reinterpret_cast<uintptr_t>(dev_block) & 7u) != 0)
        return fail(s, SAMPLER_EINVAL, "sampler_prepare: dev_block null or not 8-byte aligned");
    const int64_t bytes = SAMPLER_PREP_BYTES(B);
    if (block_bytes < bytes) return fail(s, SAMPLER_EINVAL, "sampler_prepare: dev_block too small");
    DeviceGuard g(s->device);
    const uint32_t slot = s->prep_next;
    if (s->prep_used[slot]) {
        // the copy that last read this staging buffer must have finished
        const hipError_t we = hipEventSynchronize(s->prep_ev[slot]);
        if (we != hipSuccess) return fail(s, SAMPLER_EHIP, "sampler_prepare: staging wait", we);
    }
    char* h = s->prep_host + static_cast<size_t>(slot) * SAMPLER_PREP_BYTES(s->max_batch);
    int64_t* h_uid = reinterpret_cast<int64_t*>(h);
    float* h_t = reinterpret_cast<float*>(h + 8 * static_cast<size_t>(B));
    int32_t* h_k = reinterpret_cast<int32_t*>(h + 12 * static_cast<size_t>(B));
    float* h_p = reinterpret_cast<float*>(h + 16 * static_cast<size_t>(B));
    float* h_m = reinterpret_cast<float*>(h + 20 * static_cast<size_t>(B));
    // the pages' values, in double as Python computes them, stored as fp32;
    // max(a, b) and min(a, b) keep their first argument unless the second is
    // strictly larger (smaller), as Python's do
    const double kMin = 1e-6;
    bool any_k = false, any_p = false, any_m = false;
    for (int32_t b = 0; b < B; ++b) {
        const double t = temperature[b] <= 0.0f ? 0.0 : static_cast<double>(temperature[b]);
        h_t[b] = static_cast<float>(kMin > t ? kMin : t);
        const int32_t k = top_k ? top_k[b] : -1;
        h_k[b] = k >= 1 ? k : s->vocab;
        any_k = any_k || h_k[b] != s->vocab;
        const double p0 = top_p ? static_cast<double>(top_p[b]) : 1.0;
        const double p1 = kMin > p0 ? kMin : p0;
        const double p2 = 1.0 < p1 ? 1.0 : p1;
        h_p[b] = static_cast<float>(p2);
        any_p = any_p || p2 < 1.0;
        h_m[b] = min_p ? min_p[b] : 0.0f;
        any_m = any_m || h_m[b] > 0.0f;
        h_uid[b] = uid[b];
    }
    // the upload is a kernel reading the staging buffer through its mapping
    const char* hm = s->prep_mapped + static_cast<size_t>(slot) * SAMPLER_PREP_BYTES(s->max_batch);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = dst::launch_upload_words(reinterpret_cast<const uint32_t*>(hm),
                                            static_cast<uint32_t*>(dev_block),
                                            static_cast<int>(bytes / 4), st);
    if (e == hipSuccess) e = hipEventRecord(s->prep_ev[slot], st);
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "sampler_prepare: copy", e);
    s->prep_used[slot] = true;
    s->prep_next = (slot + 1) % SAMPLER_PREP_SLOTS;
    char* d = static_cast<char*>(dev_block);
    out->uid = reinterpret_cast<const int64_t*>(d);
    out->temperature = reinterpret_cast<const float*>(d + 8 * static_cast<size_t>(B));
    out->top_k = any_k ? reinterpret_cast<const int32_t*>(d + 12 * static_cast<size_t>(B)) : nullptr;
    out->top_p = any_p ? reinterpret_cast<const float*>(d + 16 * static_cast<size_t>(B)) : nullptr;
    out->min_p = any_m ? reinterpret_cast<const float*>(d + 20 * static_cast<size_t>(B)) : nullptr;
    return SAMPLER_OK;
}

int write_page_table(dst_sampler* s, void* stream, int32_t* page_table, int64_t table_rows,
                     int64_t table_cols, const int64_t* table_idx, const int64_t* cached_len,
                     const int64_t* device_len, int32_t n_req, const int32_t* page_starts,
                     int64_t n_pages, int32_t page_size) {
    if (!s) return SAMPLER_EINVAL;
    if (n_req < 0 || n_req > s->max_batch) return fail(s, SAMPLER_EINVAL, "write_page_table: n_req out of range");
    if (page_size < 1) return fail(s, SAMPLER_EINVAL, "write_page_table: page_size < 1");
    if (!page_table || table_rows < 1 || table_cols < 1 || table_cols > INT32_MAX)
        return fail(s, SAMPLER_EINVAL, "write_page_table: null, empty or too wide page table");
    if (n_req > 0 && (!table_idx || !cached_len || !device_len))
        return fail(s, SAMPLER_EINVAL, "write_page_table: null request arrays");
    if (n_pages < 0 || (n_pages > 0 && !page_starts))
        return fail(s, SAMPLER_EINVAL, "write_page_table: bad page_starts / n_pages");
    DeviceGuard g(s->device);
    const uint32_t slot = s->pt_next;
    if (s->pt_used[slot]) {
        const hipError_t we = hipEventSynchronize(s->pt_ev[slot]);
        if (we != hipSuccess) return fail(s, SAMPLER_EHIP, "write_page_table: staging wait", we);
    }
    const size_t slot_words = 4 * static_cast<size_t>(s->max_batch);
    int64_t* rec = s->pt_host + slot * slot_words;
    const int64_t ps = page_size;
    int64_t pages = 0;
    int n_rec = 0;
    for (int32_t r = 0; r < n_req; ++r) {
        const int64_t c = cached_len[r], d = device_len[r];
        if (c < 0 || d < 0) return fail(s, SAMPLER_EINVAL, "write_page_table: negative length");
        const int64_t first = c / ps + (c % ps != 0);     // ceil(c / ps)
        const int64_t last = d / ps + (d % ps != 0);
        if (last <= first) continue;
        if (table_idx[r] < 0 || table_idx[r] >= table_rows || last > table_cols / ps)
            return fail(s, SAMPLER_EINVAL, "write_page_table: page range outside the table");
        rec[4 * n_rec + 0] = table_idx[r];
        rec[4 * n_rec + 1] = first * ps;
        rec[4 * n_rec + 2] = (last - first) * ps;
        rec[4 * n_rec + 3] = pages;
        pages += last - first;
        ++n_rec;
    }
    if (pages != n_pages) return fail(s, SAMPLER_EINVAL, "write_page_table: n_pages differs from the pages needed");
    if (n_rec == 0) return SAMPLER_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    dst::PageTableArgs a{page_table, table_rows, table_cols, s->pt_mapped + slot * slot_words,
                         page_starts, ps, s->status_dev};
    hipError_t e = dst::launch_write_page_table(a, n_rec, st);
    if (e == hipSuccess) e = hipEventRecord(s->pt_ev[slot], st);
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "write_page_table: launch", e);
    s->pt_used[slot] = true;
    s->pt_next = (slot + 1) % SAMPLER_PREP_SLOTS;
    return SAMPLER_OK;
}

int sampler_wait(dst_sampler* s, uint64_t ticket) {
    if (!s) return SAMPLER_EINVAL;
    if (ticket == 0 || ticket > s->issued) return fail(s, SAMPLER_ETICKET, "sampler_wait: unknown ticket");
    DeviceGuard g(s->device);
    const hipError_t e = hipEventSynchronize(s->ring[ticket % kRing]);
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "sampler_wait", e);
    if (__atomic_load_n(s->status_host, __ATOMIC_ACQUIRE) != 0)
        return fail(s, SAMPLER_EDEVICE, "token-pool index out of range");
    if (__atomic_load_n(s->status_host + 1, __ATOMIC_ACQUIRE) != 0)
        return fail(s, SAMPLER_EDEVICE, "write_tokens: two requests name the same pool row");
    return SAMPLER_OK;
}

int sampler_query(dst_sampler* s, uint64_t ticket) {
    if (!s) return SAMPLER_EINVAL;
    if (ticket == 0 || ticket > s->issued) return fail(s, SAMPLER_ETICKET, "sampler_query: unknown ticket");
    DeviceGuard g(s->device);
    const hipError_t e = hipEventQuery(s->ring[ticket % kRing]);
    if (e == hipSuccess) return 1;
    if (e == hipErrorNotReady) return 0;
    return fail(s, SAMPLER_EHIP, "sampler_query", e);
}

int sampler_check(dst_sampler* s) {
    if (!s) return SAMPLER_EINVAL;
    DeviceGuard g(s->device);
    const hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "sampler_check", e);
    const uint32_t flag = __atomic_exchange_n(s->status_host, 0u, __ATOMIC_ACQ_REL);
    const uint32_t dup = __atomic_exchange_n(s->status_host + 1, 0u, __ATOMIC_ACQ_REL);
    if (flag) return fail(s, SAMPLER_EDEVICE, "token-pool index out of range");
    if (dup) return fail(s, SAMPLER_EDEVICE, "write_tokens: two requests name the same pool row");
    return SAMPLER_OK;
}

int sampler_set_checks(dst_sampler* s, uint32_t flags) {
    if (!s) return SAMPLER_EINVAL;
    if (flags & ~static_cast<uint32_t>(SAMPLER_CHECK_DUPLICATE_ROWS))
        return fail(s, SAMPLER_EINVAL, "sampler_set_checks: unknown flag");
    s->checks = flags;
    return SAMPLER_OK;
}

}  // extern "C"
