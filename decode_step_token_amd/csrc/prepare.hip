// Parameter upload of sampler_prepare.
//
// "The engine and the sampler", section "The sampler": prepare builds the
// batch's per-request temperature / top_k / top_p tensors on the host and
// copies them to the device without blocking.  Here the host packs them
// into a pinned staging buffer and this kernel, on the caller's stream,
// reads that buffer through its device mapping and writes the device block:
// a few microseconds in stream order, without the runtime's copy engine
// (whose launch leaves gaps of several microseconds on each side of a copy).
//
// One 4-byte word per thread.  The loads are relaxed atomics at system scope,
// so they read host memory coherently even when the same staging buffer
// comes round again.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dst {

namespace {

constexpr int kCopyBlock = 256;

__global__ __launch_bounds__(kCopyBlock) void upload_words_kernel(const uint32_t* src, uint32_t* dst,
                                                                  int n) {
    const int i = blockIdx.x * kCopyBlock + threadIdx.x;
    if (i >= n) return;
    dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

hipError_t launch_upload_words(const uint32_t* src_mapped, uint32_t* dst, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((n + kCopyBlock - 1) / kCopyBlock));
    hipLaunchKernelGGL(upload_words_kernel, grid, dim3(kCopyBlock), 0, stream, src_mapped, dst, n);
    return hipGetLastError();
}

}  // namespace dst
