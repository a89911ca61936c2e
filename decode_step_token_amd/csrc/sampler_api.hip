// C ABI of the batched sampler: handle, argument checks, launches, tickets.
//
// The handle stands for the engine's Sampler ("The engine and the sampler",
// section "The sampler"); sample_batch is Sampler.sample with prepare's clamps
// done on the device; write_tokens is the scheduler's token-pool write-back
// plus forward_batch's non-blocking host copy and completion event ("The
// scheduler skeleton and the offline interface", section "_forward"; "The
// engine and the sampler", section "forward_batch"); gather_tokens is
// _forward's input gather from the same pool.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "sampler.h"
#include "kernels.hpp"

namespace {

constexpr int kRing = 256;
// one thread per gathered entry: a dispatch holds fewer than 2^32 work-items
constexpr int64_t kMaxGather = INT32_MAX;
// all-greedy batches with at least this many rows fill the GPU with one
// workgroup per row and take the single-pass kernel; smaller ones split rows
constexpr int kStreamGreedyMinRows = 256;

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
    void* workspace = nullptr;       // device: argmax slots and counters
    uint64_t* slot = nullptr;
    uint32_t* count = nullptr;
    uint32_t* status_host = nullptr;  // pinned, mapped: device bounds-check flag
    uint32_t* status_dev = nullptr;
    hipEvent_t ring[kRing] = {};
    uint64_t ring_ticket[kRing] = {};
    uint64_t issued = 0;               // tickets are 1, 2, 3, ...
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

const char* sampler_last_error(dst_sampler* s) { return s ? s->last_error.c_str() : ""; }

int sampler_destroy(dst_sampler* s) {
    if (!s) return SAMPLER_OK;
    DeviceGuard g(s->device);
    if (s->issued) (void)hipEventSynchronize(s->ring[s->issued % kRing]);
    for (auto& e : s->ring)
        if (e) (void)hipEventDestroy(e);
    if (s->workspace) (void)hipFree(s->workspace);
    if (s->status_host) (void)hipHostFree(s->status_host);
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

    const size_t slot_bytes = sizeof(uint64_t) * static_cast<size_t>(max_batch);
    const size_t count_bytes = sizeof(uint32_t) * static_cast<size_t>(max_batch);
    hipError_t e = hipMalloc(&s->workspace, slot_bytes + count_bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        sampler_destroy(s);
        return SAMPLER_ENOMEM;
    }
    s->slot = static_cast<uint64_t*>(s->workspace);
    s->count = reinterpret_cast<uint32_t*>(static_cast<char*>(s->workspace) + slot_bytes);
    e = hipMemset(s->workspace, 0, slot_bytes + count_bytes);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&s->status_host), sizeof(uint32_t),
                                           hipHostMallocMapped);
    if (e == hipSuccess) {
        *s->status_host = 0;
        e = hipHostGetDevicePointer(reinterpret_cast<void**>(&s->status_dev), s->status_host, 0);
    }
    for (int i = 0; e == hipSuccess && i < kRing; ++i)
        e = hipEventCreateWithFlags(&s->ring[i], hipEventDisableTiming);
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
                 const int64_t* uid, uint64_t step, int32_t* tokens_out, const sampler_debug* dbg) {
    if (!s) return SAMPLER_EINVAL;
    if (B < 0 || B > s->max_batch) return fail(s, SAMPLER_EINVAL, "sample_batch: B out of range");
    if (B == 0) return SAMPLER_OK;
    if (!logits || !tokens_out) return fail(s, SAMPLER_EINVAL, "sample_batch: null logits or tokens_out");
    if (row_stride < s->vocab) return fail(s, SAMPLER_EINVAL, "sample_batch: row_stride < vocab_size");
    if (temperature && !uid) return fail(s, SAMPLER_EINVAL, "sample_batch: uid required with temperature");
    DeviceGuard g(s->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (!temperature && B < kStreamGreedyMinRows) {
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
        a.uid = uid;
        a.step = step;
        a.seed = s->seed;
        a.tokens_out = tokens_out;
        if (dbg) {
            a.probs_out = dbg->probs_out;
            a.kept_out = dbg->kept_out;
            a.topk_idx_out = dbg->topk_idx_out;
            a.rand_out = dbg->rand_out;
        }
        if (dbg && (dbg->flags & SAMPLER_DEBUG_FORCE_EXACT))
            e = dst::launch_sample_exact(a, s->dtype, st);
        else
            e = dst::launch_sample_stream(a, s->dtype, st);
    }
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "sample_batch: launch", e);
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
        dst::WriteArgs a{token_pool, pool_rows, pool_cols, rows, cols, tokens, B, s->status_dev, host_dev};
        e = dst::launch_write_tokens(a, st);
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

int sampler_wait(dst_sampler* s, uint64_t ticket) {
    if (!s) return SAMPLER_EINVAL;
    if (ticket == 0 || ticket > s->issued) return fail(s, SAMPLER_ETICKET, "sampler_wait: unknown ticket");
    DeviceGuard g(s->device);
    const hipError_t e = hipEventSynchronize(s->ring[ticket % kRing]);
    if (e != hipSuccess) return fail(s, SAMPLER_EHIP, "sampler_wait", e);
    if (__atomic_load_n(s->status_host, __ATOMIC_ACQUIRE) != 0)
        return fail(s, SAMPLER_EDEVICE, "token-pool index out of range");
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
    if (flag) return fail(s, SAMPLER_EDEVICE, "token-pool index out of range");
    return SAMPLER_OK;
}

}  // extern "C"
