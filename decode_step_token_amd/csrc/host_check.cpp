// Host-code sanitizer driver: the C ABI exercised from a standalone program
// that is linked with the library's sources built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side only (the device code is the
// production code).  Without a GPU it runs the argument checks that fail
// before any HIP call; with one it also runs a short sequence of every entry
// point on small batches and checks the results it can check exactly
// (argmax tokens, pool writes, host copies, gathered ids, page-table cells,
// error codes).  Exit status 0 and the last line "host sanitizers: ok" mean
// no sanitizer report and every check held.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "sampler.h"

namespace {

int g_fail = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "host_check: FAILED %s\n", what);
        ++g_fail;
    }
}

template <typename T>
T* dev_copy(const std::vector<T>& h) {
    T* d = nullptr;
    if (hipMalloc(reinterpret_cast<void**>(&d), h.size() * sizeof(T)) != hipSuccess) std::abort();
    if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) std::abort();
    return d;
}

template <typename T>
std::vector<T> host_copy(const T* d, size_t n) {
    std::vector<T> h(n);
    if (hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) std::abort();
    return h;
}

void no_gpu_checks() {
    dst_sampler* s = nullptr;
    expect(sampler_create(nullptr, 0, 8, 100, SAMPLER_F32, 1) == SAMPLER_EINVAL, "create: null out");
    expect(sampler_create(&s, 0, 0, 100, SAMPLER_F32, 1) == SAMPLER_EINVAL, "create: max_batch 0");
    expect(sampler_create(&s, 0, 8, 0, SAMPLER_F32, 1) == SAMPLER_EINVAL, "create: vocab 0");
    expect(sampler_create(&s, 0, 8, 100, 7, 1) == SAMPLER_EINVAL, "create: dtype");
    expect(sample_batch(nullptr, nullptr, nullptr, 1, 1, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                        nullptr, nullptr) == SAMPLER_EINVAL, "sample: null handle");
    expect(sample_batch_static(0, nullptr, nullptr, 100, 65, 100, SAMPLER_F32, 1, nullptr, nullptr, nullptr,
                               nullptr, nullptr, 0, nullptr) == SAMPLER_EINVAL, "static: B 65");
    expect(std::strlen(sampler_last_error(nullptr)) > 0, "static: message");
    expect(sample_batch_static(0, nullptr, nullptr, 200000, 1, 200000, SAMPLER_F32, 1, nullptr, nullptr,
                               nullptr, nullptr, nullptr, 0, nullptr) == SAMPLER_EINVAL, "static: vocab");
    expect(sampler_destroy(nullptr) == SAMPLER_OK, "destroy null");
    for (int c = 0; c >= -6; --c) expect(sampler_strerror(c) != nullptr, "strerror");
}

void gpu_checks() {
    const int B = 48, V = 5000;
    dst_sampler* s = nullptr;
    expect(sampler_create(&s, 0, B, V, SAMPLER_F32, 42) == SAMPLER_OK, "create");
    if (!s) return;
    // logits with a known argmax per row; sampled rows from mixed parameters
    std::vector<float> x(static_cast<size_t>(B) * V);
    std::vector<int32_t> want(B);
    uint32_t st = 12345u;
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < V; ++i) {
            st = st * 1664525u + 1013904223u;
            x[static_cast<size_t>(b) * V + i] = static_cast<float>(st >> 8) * (1.0f / 16777216.0f);
        }
        want[b] = (b * 97) % V;
        x[static_cast<size_t>(b) * V + want[b]] = 3.0f;
    }
    float* dx = dev_copy(x);
    int32_t* dtok = dev_copy(std::vector<int32_t>(B, -1));
    expect(sample_batch(s, nullptr, dx, V, B, nullptr, nullptr, nullptr, nullptr, nullptr, 0, dtok, nullptr) ==
               SAMPLER_OK, "sample greedy");
    expect(host_copy(dtok, B) == want, "greedy tokens");
    // argument errors: nothing enqueued
    expect(sample_batch(s, nullptr, dx, V - 1, B, nullptr, nullptr, nullptr, nullptr, nullptr, 0, dtok,
                        nullptr) == SAMPLER_EINVAL, "sample: stride");
    expect(sample_batch(s, nullptr, dx, V, B + 1, nullptr, nullptr, nullptr, nullptr, nullptr, 0, dtok,
                        nullptr) == SAMPLER_EINVAL, "sample: B");
    // prepared parameters, sampled rows (every path)
    std::vector<float> T(B), P(B);
    std::vector<int32_t> K(B);
    std::vector<int64_t> U(B);
    for (int b = 0; b < B; ++b) {
        T[b] = (b % 4 == 0) ? 0.0f : 0.5f + 0.02f * b;
        K[b] = (b % 3 == 0) ? -1 : 1 + b;
        P[b] = (b % 5 == 0) ? 1.0f : 0.9f;
        U[b] = 1000 + b;
    }
    void* block = nullptr;
    if (hipMalloc(&block, SAMPLER_PREP_BYTES(B)) != hipSuccess) std::abort();
    sampler_args args{};
    expect(sampler_prepare(s, nullptr, B, T.data(), K.data(), P.data(), nullptr, U.data(), block,
                           SAMPLER_PREP_BYTES(B), &args) == SAMPLER_OK, "prepare");
    expect(sampler_prepare(s, nullptr, B, T.data(), K.data(), P.data(), nullptr, nullptr, block,
                           SAMPLER_PREP_BYTES(B), &args) == SAMPLER_EINVAL, "prepare: uid missing");
    expect(sampler_prepare(s, nullptr, B, T.data(), K.data(), P.data(), nullptr, U.data(), block,
                           SAMPLER_PREP_BYTES(B), &args) == SAMPLER_OK, "prepare again");
    for (uint32_t flags : {0u, static_cast<uint32_t>(SAMPLER_DEBUG_FORCE_STREAM),
                           static_cast<uint32_t>(SAMPLER_DEBUG_FORCE_SPLIT),
                           static_cast<uint32_t>(SAMPLER_DEBUG_FORCE_EXACT)}) {
        sampler_debug dbg{};
        dbg.flags = flags;
        expect(sample_batch(s, nullptr, dx, V, B, args.temperature, args.top_k, args.top_p, args.min_p,
                            args.uid, 7, dtok, &dbg) == SAMPLER_OK, "sample prepared");
        const std::vector<int32_t> got = host_copy(dtok, B);
        for (int b = 0; b < B; ++b) {
            expect(got[b] >= 0 && got[b] < V, "token in range");
            if (T[b] == 0.0f) expect(got[b] == want[b], "greedy row");
        }
    }
    // write-back with a pinned host copy, tickets, the duplicate-row check
    const int R = 64, C = 32;
    int32_t* dpool = dev_copy(std::vector<int32_t>(static_cast<size_t>(R) * C, 0));
    std::vector<int64_t> rows(B), cols(B);
    for (int b = 0; b < B; ++b) {
        rows[b] = b;
        cols[b] = (b % 7 == 0) ? -1 : b % C;
    }
    int64_t* drows = dev_copy(rows);
    int64_t* dcols = dev_copy(cols);
    int32_t* hout = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&hout), B * sizeof(int32_t), hipHostMallocDefault) != hipSuccess)
        std::abort();
    uint64_t ticket = 0;
    expect(sampler_set_checks(s, SAMPLER_CHECK_DUPLICATE_ROWS) == SAMPLER_OK, "set checks");
    expect(write_tokens(s, nullptr, dpool, R, C, drows, dcols, dtok, B, hout, &ticket) == SAMPLER_OK, "write");
    expect(sampler_wait(s, ticket) == SAMPLER_OK, "wait");
    expect(sampler_query(s, ticket) == 1, "query");
    const std::vector<int32_t> toks = host_copy(dtok, B);
    const std::vector<int32_t> pool = host_copy(dpool, static_cast<size_t>(R) * C);
    for (int b = 0; b < B; ++b) {
        expect(hout[b] == toks[b], "host copy");
        const int64_t c = cols[b] == -1 ? C - 1 : cols[b];
        expect(pool[static_cast<size_t>(rows[b]) * C + c] == toks[b], "pool cell");
    }
    std::vector<int32_t> stack_buf(B);
    expect(write_tokens(s, nullptr, dpool, R, C, drows, dcols, dtok, B, stack_buf.data(), &ticket) ==
               SAMPLER_ENOTPINNED, "write: pageable host buffer");
    expect(sampler_wait(s, 1u << 30) == SAMPLER_ETICKET, "wait: unknown ticket");
    expect(sampler_set_checks(s, 2u) == SAMPLER_EINVAL, "set checks: unknown flag");
    // gather of what was written
    std::vector<int64_t> gpos(B);
    for (int b = 0; b < B; ++b) gpos[b] = cols[b] == -1 ? C - 1 : cols[b];
    int64_t* dgpos = dev_copy(gpos);
    int32_t* dids = dev_copy(std::vector<int32_t>(B, -7));
    expect(gather_tokens(s, nullptr, dpool, R, C, drows, dgpos, B, dids) == SAMPLER_OK, "gather");
    expect(host_copy(dids, B) == toks, "gathered ids");
    // page table: request r gets pages for positions [cached, device)
    const int NR = 3, PS = 4;
    int32_t* dtable = dev_copy(std::vector<int32_t>(static_cast<size_t>(8) * 64, -1));
    const int64_t tidx[NR] = {5, 0, 7}, cached[NR] = {0, 4, 6}, devlen[NR] = {9, 8, 6};
    // new pages: ceil(9/4)-0 = 3, ceil(8/4)-1 = 1, ceil(6/4)-ceil(6/4) = 0
    int32_t* dstarts = dev_copy(std::vector<int32_t>{100, 200, 300, 400});
    expect(write_page_table(s, nullptr, dtable, 8, 64, tidx, cached, devlen, NR, dstarts, 4, PS) == SAMPLER_OK,
           "page table");
    expect(write_page_table(s, nullptr, dtable, 8, 64, tidx, cached, devlen, NR, dstarts, 3, PS) ==
               SAMPLER_EINVAL, "page table: page count");
    expect(sampler_check(s) == SAMPLER_OK, "check");
    const std::vector<int32_t> tab = host_copy(dtable, static_cast<size_t>(8) * 64);
    expect(tab[5 * 64 + 0] == 100 && tab[5 * 64 + 9] == 300 + 1 && tab[5 * 64 + 11] == 300 + 3,
           "page table cells (request 0)");
    expect(tab[0 * 64 + 4] == 400 && tab[0 * 64 + 7] == 403 && tab[0 * 64 + 3] == -1,
           "page table cells (request 1)");
    // the entry point that allocates nothing
    expect(sample_batch_static(0, nullptr, dx, V, B, V, SAMPLER_F32, 42, nullptr, nullptr, nullptr, nullptr,
                               nullptr, 0, dtok) == SAMPLER_OK, "static");
    expect(host_copy(dtok, B) == want, "static greedy tokens");
    expect(hipDeviceSynchronize() == hipSuccess, "synchronize");
    expect(sampler_destroy(s) == SAMPLER_OK, "destroy");
    for (void* p : {static_cast<void*>(dx), static_cast<void*>(dtok), block, static_cast<void*>(dpool),
                    static_cast<void*>(drows), static_cast<void*>(dcols), static_cast<void*>(dgpos),
                    static_cast<void*>(dids), static_cast<void*>(dtable), static_cast<void*>(dstarts)})
        (void)hipFree(p);
    (void)hipHostFree(hout);
}

}  // namespace

int main() {
    no_gpu_checks();
    int n = 0;
    const bool gpu = hipGetDeviceCount(&n) == hipSuccess && n > 0;
    if (!gpu) (void)hipGetLastError();
    if (gpu) gpu_checks();
    std::printf("host_check: %s part done, %d failures\n", gpu ? "GPU" : "no-GPU", g_fail);
    if (g_fail) return 1;
    std::printf("host sanitizers: ok\n");
    return 0;
}
