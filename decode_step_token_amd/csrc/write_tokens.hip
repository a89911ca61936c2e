// Token-pool write-back and input gather.
//
// "The scheduler skeleton and the offline interface", section "Preparing a
// batch": _make_write_tuple gives each request (row = table_idx, col =
// device_len), or col = -1 for a request whose token is not to be kept; -1
// indexes the pool's last column, a cell no request reads; section "_forward": the sampled
// tokens are scattered into token_pool[rows, cols] on the device, so the
// CPU never needs the token values.
//
// One thread per request; an out-of-range (row, col) skips the write and
// raises the handle's status word (mapped pinned host memory, system-scope
// store).
// The host copy of forward_batch is the same kernel: each thread also stores
// its token into the caller's pinned buffer through its device mapping, with
// system scope, then passes a system-scope release fence, so its stores are
// performed for the host before the thread ends; the dispatch ends after its
// last thread, and the completion event is signalled after the dispatch, so
// a host that has seen the event complete reads the tokens and the status
// word (the event itself then needs no system-scope release of its own).
//
// The input gather is the other side of the same pool: the step's input ids
// are token_pool[input_tuple] with input_tuple = (row, position) over each
// request's positions [cached_len, device_len), packed request after request
// (same page, sections "Preparing a batch" and "_forward").  One thread per
// packed entry; neighbouring entries of one request read neighbouring pool
// cells, so prefill spans coalesce and a decode batch (one entry per
// request) is one scattered 4-byte read per lane.  An out-of-range entry
// yields id -1 and raises the status word.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dst {

namespace {

constexpr int kWriteBlock = 256;

__global__ __launch_bounds__(kWriteBlock) void write_tokens_kernel(WriteArgs a) {
    const int b = blockIdx.x * kWriteBlock + threadIdx.x;
    if (b >= a.B) return;
    const int64_t r = a.rows[b];
    int64_t c = a.cols[b];
    const int32_t tok = a.tokens[b];
    if (c == -1) c = a.pool_cols - 1;
    const bool bad = !(r >= 0 && r < a.pool_rows && c >= 0 && c < a.pool_cols);
    if (!bad) a.pool[r * a.pool_cols + c] = tok;
    if (bad) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (a.host) __hip_atomic_store(a.host + b, tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (bad || a.host) __threadfence_system();
}

// Debug: one pool row per request within a call ("The scheduler skeleton and
// the offline interface", section "Preparing a batch": each request owns one
// row of the pool).  Thread b compares its row with every earlier request's
// that writes (col != -1).
__global__ __launch_bounds__(kWriteBlock) void check_rows_kernel(const int64_t* rows, const int64_t* cols,
                                                                 int B, uint32_t* dup_status) {
    const int b = blockIdx.x * kWriteBlock + threadIdx.x;
    if (b >= B || cols[b] == -1) return;
    const int64_t r = rows[b];
    bool dup = false;
    for (int o = 0; o < b && !dup; ++o) dup = rows[o] == r && cols[o] != -1;
    if (dup) {
        __hip_atomic_store(dup_status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __threadfence_system();    // performed for the host before the completion event
    }
}

constexpr int kGatherBlock = 256;

__global__ __launch_bounds__(kGatherBlock) void gather_tokens_kernel(GatherArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kGatherBlock + threadIdx.x;
    if (i >= a.n) return;
    const int64_t r = a.rows[i];
    const int64_t c = a.positions[i];
    int32_t id = -1;
    if (r >= 0 && r < a.pool_rows && c >= 0 && c < a.pool_cols) {
        id = a.pool[r * a.pool_cols + c];
    } else {
        __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __threadfence_system();    // performed for the host before the event (see above)
    }
    a.ids_out[i] = id;
}

}  // namespace

hipError_t launch_gather_tokens(const GatherArgs& args, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((args.n + kGatherBlock - 1) / kGatherBlock));
    hipLaunchKernelGGL(gather_tokens_kernel, grid, dim3(kGatherBlock), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_check_rows(const int64_t* rows, const int64_t* cols, int B, uint32_t* dup_status,
                             hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((B + kWriteBlock - 1) / kWriteBlock));
    hipLaunchKernelGGL(check_rows_kernel, grid, dim3(kWriteBlock), 0, stream, rows, cols, B, dup_status);
    return hipGetLastError();
}

hipError_t launch_write_tokens(const WriteArgs& args, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((args.B + kWriteBlock - 1) / kWriteBlock));
    hipLaunchKernelGGL(write_tokens_kernel, grid, dim3(kWriteBlock), 0, stream, args);
    return hipGetLastError();
}

}  // namespace dst
