// Row argmax for all-greedy batches.
//
// "The engine and the sampler", section "The sampler": when every request of
// the batch is greedy, prepare() returns no temperature array and sample()
// goes straight to argmax over the logits, skipping the softmax.  The token
// is the lowest index holding the row maximum.
//
// Design (HBM-bound, no reuse): a row is split into chunks, one workgroup per
// chunk, so that even a 64-row batch fills the 256 CUs.  Each workgroup
// streams its chunk with 16-byte loads (four in flight per thread), keeps the
// best packed (key, ~index) per thread, reduces across the wave and the
// workgroup, and folds the result into the row's 64-bit slot with one
// atomicMax.  The last workgroup of the row to arrive (counted with an atomic
// ticket) reads the slot, writes the token and resets the slot and counter,
// so the workspace is clean for the next call without a memset.  Batches of
// at least 256 rows use the single-pass sampler kernel instead (one
// workgroup per row already fills the GPU).
#include "device_common.hpp"
#include "kernels.hpp"

namespace dst {

namespace {

constexpr int kArgmaxBlock = 256;
constexpr int kArgmaxUnroll = 4;

__device__ __forceinline__ uint64_t pack_key_index(uint32_t key, uint32_t idx) {
    // max over packed values = max key, then the lowest index
    return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xffffffffu - idx);
}

template <int DT>
__global__ __launch_bounds__(kArgmaxBlock) void argmax_rows_kernel(ArgmaxArgs a) {
    constexpr int VEC = Elem<DT>::kVec;
    using S = typename Elem<DT>::scalar_t;
    __shared__ uint64_t red[kArgmaxBlock / kWave + 1];
    __shared__ uint32_t last_flag;

    const int b = blockIdx.x / a.chunks;
    const int c = blockIdx.x - b * a.chunks;
    const int64_t lo = static_cast<int64_t>(c) * a.chunk_len;
    const int64_t hi = lo + a.chunk_len < a.V ? lo + a.chunk_len : a.V;
    const S* row = static_cast<const S*>(a.logits) + static_cast<int64_t>(b) * a.row_stride;

    uint64_t best = 0;
    if (lo < hi) {
        const bool aligned = (reinterpret_cast<uintptr_t>(row + lo) & 15u) == 0;
        int64_t i = lo;
        if (aligned) {
            const int64_t nvec = (hi - lo) / VEC;
            int64_t v = threadIdx.x;
            // four 16-byte loads in flight per thread
            for (; v + (kArgmaxUnroll - 1) * kArgmaxBlock < nvec; v += kArgmaxUnroll * kArgmaxBlock) {
                float x[kArgmaxUnroll][VEC];
#pragma unroll
                for (int u = 0; u < kArgmaxUnroll; ++u)
                    Elem<DT>::vec(row, lo + (v + u * kArgmaxBlock) * VEC, x[u]);
#pragma unroll
                for (int u = 0; u < kArgmaxUnroll; ++u) {
                    const int64_t base = lo + (v + u * kArgmaxBlock) * VEC;
#pragma unroll
                    for (int j = 0; j < VEC; ++j) {
                        const uint64_t pk = pack_key_index(f32_key(x[u][j]),
                                                           static_cast<uint32_t>(base + j));
                        best = pk > best ? pk : best;
                    }
                }
            }
            for (; v < nvec; v += kArgmaxBlock) {
                float x[VEC];
                Elem<DT>::vec(row, lo + v * VEC, x);
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    const uint64_t pk = pack_key_index(f32_key(x[j]),
                                                       static_cast<uint32_t>(lo + v * VEC + j));
                    best = pk > best ? pk : best;
                }
            }
            i = lo + nvec * VEC;
        }
        for (int64_t t = i + threadIdx.x; t < hi; t += kArgmaxBlock) {
            const uint64_t pk = pack_key_index(f32_key(Elem<DT>::at(row, t)), static_cast<uint32_t>(t));
            best = pk > best ? pk : best;
        }
    }
    best = block_max<kArgmaxBlock>(best, red);

    // debug: zero this chunk's slice of probs_out (the one-hot 1 comes last);
    // the zeros must reach memory before this chunk's ticket, since the last
    // chunk of the row may run on another XCD with its own L2
    if (a.probs_out) {
        float* pr = a.probs_out + static_cast<int64_t>(b) * a.V;
        for (int64_t t = lo + threadIdx.x; t < hi; t += kArgmaxBlock) pr[t] = 0.0f;
        __syncthreads();
        if (threadIdx.x == 0) __threadfence();
    }

    if (threadIdx.x == 0) {
        uint64_t final_best = best;
        bool last = true;
        if (a.chunks > 1) {
            // Device-scope atomics are performed where every XCD sees them;
            // consuming each returned value makes this thread wait for the
            // atomic to complete before issuing the next one, which is the
            // only ordering needed (no plain data is exchanged, so no L2
            // write-back / invalidate fence).
            const unsigned long long prev = atomicMax(reinterpret_cast<unsigned long long*>(a.slot + b),
                                                      static_cast<unsigned long long>(best));
            asm volatile("" ::"v"(prev));   // the returned value must have arrived
            const uint32_t arrived = atomicAdd(a.count + b, 1u);
            last = arrived == static_cast<uint32_t>(a.chunks - 1);
            if (last) {
                final_best = atomicExch(reinterpret_cast<unsigned long long*>(a.slot + b), 0ull);
                atomicExch(a.count + b, 0u);
            }
        }
        last_flag = last ? 1u : 0u;
        if (last) {
            const int32_t tok = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(final_best));
            a.tokens_out[b] = tok;
            if (a.kept_out) a.kept_out[b] = 1;
            if (a.rand_out) a.rand_out[b] = 0ull;
            if (a.probs_out) a.probs_out[static_cast<int64_t>(b) * a.V + tok] = 1.0f;
        }
    }
    __syncthreads();
    if (a.topk_idx_out && last_flag) {
        for (int t = threadIdx.x; t < kDebugTopK; t += kArgmaxBlock)
            a.topk_idx_out[static_cast<int64_t>(b) * kDebugTopK + t] = t == 0 ? a.tokens_out[b] : -1;
    }
}

}  // namespace

hipError_t launch_argmax(const ArgmaxArgs& args, int dtype, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.B * args.chunks));
    if (dtype == kDtypeF32)
        hipLaunchKernelGGL(argmax_rows_kernel<kDtypeF32>, grid, dim3(kArgmaxBlock), 0, stream, args);
    else
        hipLaunchKernelGGL(argmax_rows_kernel<kDtypeBF16>, grid, dim3(kArgmaxBlock), 0, stream, args);
    return hipGetLastError();
}

void argmax_plan(int B, int V, int dtype, int* chunks, int* chunk_len) {
    // aim for ~1024 workgroups over the batch (four per CU); chunks are whole
    // 16-byte vectors per thread-block pass so row alignment carries into
    // every chunk
    const int vec = dtype == kDtypeF32 ? 4 : 8;
    const int quantum = kArgmaxBlock * vec;
    int want = (1024 + B - 1) / (B > 0 ? B : 1);
    int len = (V + want - 1) / want;
    len = ((len + quantum - 1) / quantum) * quantum;
    if (len < quantum) len = quantum;
    *chunk_len = len;
    *chunks = (V + len - 1) / len;
}

}  // namespace dst
