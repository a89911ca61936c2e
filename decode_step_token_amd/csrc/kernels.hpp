// Launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dst {

constexpr int kDebugTopK = 64;

struct ArgmaxArgs {
    const void* logits;
    int64_t row_stride;       // elements
    int B, V;
    int chunks, chunk_len;    // chunks per row, elements per chunk
    uint64_t* slot;           // [B] workspace, zero between calls
    uint32_t* count;          // [B] workspace, zero between calls
    int32_t* tokens_out;
    float* probs_out;         // debug, may be null
    int32_t* kept_out;
    int32_t* topk_idx_out;
    uint64_t* rand_out;
};

struct SampleArgs {
    const void* logits;
    int64_t row_stride;
    int B, V;
    const float* temperature;  // null: every row greedy
    const int32_t* top_k;      // may be null
    const float* top_p;        // may be null
    const float* min_p;        // may be null
    const int64_t* uid;        // non-null unless temperature is null
    uint64_t step, seed;
    int resident;              // stream blocks resident at once (0: unknown)
    int32_t* tokens_out;
    float* probs_out;
    int32_t* kept_out;
    int32_t* topk_idx_out;
    uint64_t* rand_out;
};

struct WriteArgs {
    int32_t* pool;
    int64_t pool_rows, pool_cols;
    const int64_t* rows;
    const int64_t* cols;
    const int32_t* tokens;
    int B;
    uint32_t* status;          // mapped pinned host word; set to 1 on a bad (row, col)
    int32_t* host;             // device address of the pinned host copy, or null
};

struct GatherArgs {
    const int32_t* pool;
    int64_t pool_rows, pool_cols;
    const int64_t* rows;
    const int64_t* positions;
    int64_t n;
    int32_t* ids_out;
    uint32_t* status;          // mapped pinned host word; set to 1 on a bad (row, position)
};

struct PageTableArgs {
    int32_t* table;
    int64_t rows, cols;
    const int64_t* records;    // device address of mapped pinned records: row, first, npos, page base
    const int32_t* page_starts;
    int64_t page_size;
    uint32_t* status;          // mapped pinned host word; set to 1 on a bad (row, column)
};

hipError_t launch_argmax(const ArgmaxArgs& args, int dtype, hipStream_t stream);
void argmax_plan(int B, int V, int dtype, int* chunks, int* chunk_len);
hipError_t launch_sample_exact(const SampleArgs& args, int dtype, hipStream_t stream);
hipError_t launch_sample_stream(const SampleArgs& args, int dtype, hipStream_t stream);
hipError_t launch_write_tokens(const WriteArgs& args, hipStream_t stream);
hipError_t launch_gather_tokens(const GatherArgs& args, hipStream_t stream);
hipError_t launch_write_page_table(const PageTableArgs& args, int n_records, hipStream_t stream);
// copies n 4-byte words from mapped pinned host memory (its device address)
hipError_t launch_upload_words(const uint32_t* src_mapped, uint32_t* dst, int n, hipStream_t stream);

}  // namespace dst
