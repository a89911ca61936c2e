// The exact multi-pass sampler as a kernel of its own: one 512-thread
// workgroup per row (see exact_path.hpp for the algorithm).  It serves rows
// the single-pass kernel does not take (unaligned rows) and is the reference
// point the single-pass kernel is measured against.
#include "exact_path.hpp"

namespace dst {

namespace {

constexpr int kExactBlock = 512;

template <int DT>
__global__ __launch_bounds__(kExactBlock) void sample_exact_kernel(SampleArgs a) {
    using S = typename Elem<DT>::scalar_t;
    __shared__ ExactSmem sm;
    const int b = blockIdx.x;
    const void* row = static_cast<const S*>(a.logits) + static_cast<int64_t>(b) * a.row_stride;
    const RowParams prm = row_params(a.temperature, a.top_k, a.top_p, a.min_p, b, a.V);
    const uint64_t word = request_word(a.seed, ld_global<int64_t>(a.uid + b), a.step);
    exact_row<DT, kExactBlock>(a, b, row, prm, word, uniform24(word), sm);
}

}  // namespace

hipError_t launch_sample_exact(const SampleArgs& args, int dtype, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.B));
    if (dtype == kDtypeF32)
        hipLaunchKernelGGL(sample_exact_kernel<kDtypeF32>, grid, dim3(kExactBlock), 0, stream, args);
    else
        hipLaunchKernelGGL(sample_exact_kernel<kDtypeBF16>, grid, dim3(kExactBlock), 0, stream, args);
    return hipGetLastError();
}

}  // namespace dst
