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

// Split-row sampler: per (row, chunk) record published by the chunk's
// workgroup and read by the row's finishing workgroup (128 bytes).
struct SplitRec {
    float m;           // chunk maximum
    uint32_t amax;     // lowest index holding it (argmax rows)
    float theta;       // every chunk element >= theta is among the candidates
    uint32_t cnt;      // candidates published; kSplitCap + 1: too many, none published
    double z;          // sum of the chunk's weights 2^(x c - rc)
    float rc;          // fl(m * c): the weights' reference
    uint32_t mode;
    // second publication of rows without a top-k filter, once the row's
    // boundary weight bin G* and min_p key are known
    double am_all;     // weight of the elements in bins above G*
    double am_kept;    // ... of those whose key passes min_p
    uint32_t an_all;   // their counts
    uint32_t an_kept;
    uint32_t bcnt;     // elements of bin G* published (after the candidates)
    uint32_t pad[17];
};
static_assert(sizeof(SplitRec) == 128, "record size");

constexpr int kSplitThreads = 256;
constexpr int kSplitCap = 256;        // candidates one chunk may publish
constexpr int kSplitBinCap = 1024;    // elements of bin G* one chunk may publish
constexpr int kSplitCandStride = kSplitCap + kSplitBinCap;   // entries per chunk block
constexpr int kSplitHistBins = 1024;  // weight histogram per chunk: 1/32 octave per bin
constexpr int kSplitMaxChunks = 64;   // chunks per row (one flag per lane of a wave)
constexpr int kSplitXcds = 8;         // rows are dealt to the XCDs round robin

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
    // split-row sampler workspace (see SplitRec)
    SplitRec* rec;             // [B][rec_stride]
    uint64_t* cand;            // [B][rec_stride][kSplitCandStride] (order key << 32 | index)
    float* hist;               // [B][rec_stride][kSplitHistBins]
    uint32_t* dec;             // [B][4] the finisher's decision: epoch, G*, min_p key, status
    uint32_t* flags;           // [B][kSplitMaxChunks] epoch of the last publication
    int rec_stride;            // chunks allocated per row
    int chunks;                // chunks per row in this launch
    uint32_t epoch;            // even, nonzero, different for every launch on a workspace;
                               // the second publication of a launch is flagged epoch + 1
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
// loads per thread and chunk for the split-row sampler (4, 8 or 16), 0 if V needs more
// than kSplitMaxChunks chunks even at 16; *chunks receives the chunk count
int split_plan(int V, int dtype, int* chunks);
// chunks per row the workspace must hold for a vocabulary (0: the split sampler is not used)
int split_chunks_alloc(int V, int dtype);
hipError_t launch_sample_split(const SampleArgs& args, int dtype, int nl, hipStream_t stream);
hipError_t launch_write_tokens(const WriteArgs& args, hipStream_t stream);
// debug check: sets *dup_status to 1 when two requests b != b' with cols != -1
// name the same pool row (O(B^2) comparisons)
hipError_t launch_check_rows(const int64_t* rows, const int64_t* cols, int B, uint32_t* dup_status,
                             hipStream_t stream);
hipError_t launch_gather_tokens(const GatherArgs& args, hipStream_t stream);
hipError_t launch_write_page_table(const PageTableArgs& args, int n_records, hipStream_t stream);
// copies n 4-byte words from mapped pinned host memory (its device address)
hipError_t launch_upload_words(const uint32_t* src_mapped, uint32_t* dst, int n, hipStream_t stream);

}  // namespace dst
