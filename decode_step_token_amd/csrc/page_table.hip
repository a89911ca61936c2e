// Page-table write of the cache manager's paged allocation.
//
// "CacheManager: allocation, release and admission control", section
// "Allocating pages for this step's tokens": each request's new pages are
// [ceil(cached_len / page_size), ceil(device_len / page_size)); their
// positions in the request's page-table row receive, in order, the first
// token location of each newly allocated page plus the offset inside the
// page (section "The free-page list": a free slot is a page's first token
// location).  The pages build every (row, column) pair on the host and copy
// them over; here the host stages one 32-byte record per request with new
// pages -- (row, first position, positions, first page index) -- in mapped
// pinned memory, and each workgroup reads its record straight from there
// and expands it on the device.
//
// One 64-lane workgroup (one wave) per record; lanes stride over the record's
// positions, so a prefill span writes consecutive columns.  A position
// outside the table skips its store and raises the handle's status word.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dst {

namespace {

constexpr int kPageBlock = 64;

__global__ __launch_bounds__(kPageBlock) void write_page_table_kernel(PageTableArgs a) {
    // The record lives in host memory: lanes 0-3 read its four words with
    // coherent system-scope loads (one 32-byte request), then every lane
    // takes them from those lanes.
    const int64_t* rec = a.records + 4 * static_cast<int64_t>(blockIdx.x);
    const int q = threadIdx.x & 3;
    int64_t word = 0;
    if (threadIdx.x < 4) word = __hip_atomic_load(rec + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    auto lane_word = [&](int l) -> int64_t {
        const uint32_t lo = readlane_u32(static_cast<uint32_t>(word), l);
        const uint32_t hi = readlane_u32(static_cast<uint32_t>(static_cast<uint64_t>(word) >> 32), l);
        return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    };
    const int64_t row = lane_word(0);
    const int64_t first = lane_word(1);
    const int64_t npos = lane_word(2);
    const int64_t pbase = lane_word(3);
    const bool row_ok = row >= 0 && row < a.rows;
    bool bad = false;
    // positions and the page size fit 32 bits (the host keeps rows shorter
    // than 2^31 columns)
    const uint32_t ps = static_cast<uint32_t>(a.page_size);
    for (int64_t i = threadIdx.x; i < npos; i += kPageBlock) {
        const int64_t col = first + i;
        const uint32_t i32 = static_cast<uint32_t>(i);
        const uint32_t pg = ps == 1u ? i32 : i32 / ps;
        const int32_t loc = a.page_starts[pbase + pg] + static_cast<int32_t>(i32 - pg * ps);
        if (row_ok && col >= 0 && col < a.cols) {
            a.table[row * a.cols + col] = loc;
        } else {
            bad = true;
        }
    }
    if (bad) {
        __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __threadfence_system();    // performed for the host before the completion event
    }
}

}  // namespace

hipError_t launch_write_page_table(const PageTableArgs& args, int n_records, hipStream_t stream) {
    if (n_records <= 0) return hipSuccess;
    hipLaunchKernelGGL(write_page_table_kernel, dim3(static_cast<unsigned>(n_records)), dim3(kPageBlock),
                       0, stream, args);
    return hipGetLastError();
}

}  // namespace dst
