// Single-pass per-row sampler: one 1024-thread workgroup streams its row
// from HBM once and finishes the row from on-chip state.
//
// "The engine and the sampler", section "The sampler": temperature, top-k
// first, top-p on the renormalised survivors, one categorical draw (here an
// inverse CDF in token order with a keyed Philox uniform).  The kept set is
// always a prefix of the descending order, so it is held as a cut
// (key, last index): token i is kept iff key_i > key, or key_i == key and
// i <= last index.
//
// What one read of the row leaves behind:
//   * the row maximum and its lowest index, from per-tile lane maxima (the
//     argmax bookkeeping only runs when a lane's tile beats its running best);
//   * for rows without top-k: one softmax sum per tile (1024 fp32 or 2048
//     bf16 logits) relative to the tile's own maximum tref, with fp32
//     arguments (x - tref) * log2(e)/T through v_exp_f32, rescaled to the row
//     maximum in fp64 at the end.  (x - tref) is exact for every logit within
//     a factor two of tref, which carries the tile's mass, so the normaliser
//     stays within ~2e-7 of the fp64 sum on the workloads here (an argument
//     taken relative to the row maximum in one fp32 expression is off by up
//     to 2.5e-6);
//   * for rows with top-k or top-p: every logit >= theta, with its index, in a
//     wave-private LDS region (ballot + mbcnt compaction, a scalar counter, no
//     LDS atomics).  theta is fixed after the first tile of every wave: the
//     lower edge of the histogram bin that holds the j-th largest of the 1024
//     per-thread maxima.  j = k for top-k: j per-thread maxima are j distinct
//     logits >= theta, so the top-k set is always inside the regions.  For
//     top-p, j aims at a few thousand candidates.
//
// Finishing the row: all waves build 256-bin LDS histograms of their own
// entries; wave 0 scans them with DPP prefix sums and picks the bin; a bin of
// at most 64 entries is gathered and ranked exactly.
//   * full softmax (no top-k, top-p = 1): the tile sums are rescaled and
//     scanned; the one tile holding u * Z is read again and scanned;
//   * top-k: count descent over the keys;
//   * top-p: mass descent over the keys inside the top-k cut;
//   * the draw: mass descent over the token index of the kept entries.
// The candidates are every logit >= theta, a prefix of the descending order,
// so the result is exact whenever the kept prefix ends inside them.  When it
// does not (a flat top-p row whose nucleus reaches below theta, a full
// region, top-k above the thread count), or the row is not 16-byte aligned,
// the same descents run over the row itself, re-reading it from memory.
//
// Everything is inline and spill-free: a kernel that needs scratch memory
// pays ~10 us per launch on this GPU.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dst {

namespace {

constexpr int kBlock = 1024;
constexpr int kWaves = kBlock / kWave;
constexpr int kRegion = 512;               // candidate entries per wave
constexpr int kCap = kWaves * kRegion;     // 8192
constexpr int kMaxTiles = 512;
constexpr int kList = 64;
constexpr int kTopPTarget = 1500;          // aimed-at candidate count for top-p rows

enum Mode { kArgmax = 0, kTopK = 1, kTopP = 2, kFull = 3 };

struct Smem {
    uint32_t ckey[kCap];
    uint32_t cidx[kCap];
    float cw[kCap];
    float tref[kMaxTiles];
    double tsum[kMaxTiles];
    uint32_t hcnt[256];
    double hmass[256];
    uint64_t wbest[kWaves];
    uint32_t wcount[kWaves];
    uint32_t wu[kWaves];
    double wd[kWaves];
    uint32_t bu[8];        // wave-0 decisions broadcast to the block
    double bd[4];
    uint32_t list_n;       // gathered entries
    uint32_t lkey[kList];
    uint32_t lidx[kList];
    float lw[kList];
    uint32_t skey[kList];  // ... ranked
    uint32_t sidx[kList];
    float sw[kList];
};

// ------------------------------------------------------------ tile I/O --

template <int DT>
struct TileIO {
    static constexpr int VEC = Elem<DT>::kVec;
    static constexpr int U = DT == kDtypeF32 ? 4 : 2;  // 16-byte loads per lane per tile
    static constexpr int Q = U * VEC;                 // elements per lane per tile
    static constexpr int TILE = kWave * Q;            // contiguous elements per tile

    // Tile t for this lane: load u covers t*TILE + u*64*VEC + lane*VEC + [0, VEC).
    // Past the end of the row the values are -inf.
    __device__ static __forceinline__ void load(const void* row, int V, int t, int lane, uint4* raw) {
        const int64_t base = static_cast<int64_t>(t) * TILE;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t off = base + u * kWave * VEC + lane * VEC;
            if (off + VEC <= V) {
                raw[u] = ld_global_u4(static_cast<const char*>(row) + off * (DT == kDtypeF32 ? 4 : 2));
            } else {
                uint32_t w[4];
                if (DT == kDtypeF32) {
                    const float* r32 = static_cast<const float*>(row);
                    for (int e = 0; e < 4; ++e)
                        w[e] = off + e < V ? __float_as_uint(ld_global<float>(r32 + off + e)) : 0xff800000u;
                } else {
                    const uint16_t* r16 = static_cast<const uint16_t*>(row);
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = off + 2 * e < V ? ld_global<uint16_t>(r16 + off + 2 * e) : 0xff80u;
                        const uint32_t hi = off + 2 * e + 1 < V ? ld_global<uint16_t>(r16 + off + 2 * e + 1) : 0xff80u;
                        w[e] = lo | (hi << 16);
                    }
                }
                raw[u] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }

    // Element q of the lane's tile (increasing index order in q).
    __device__ static __forceinline__ float get(const uint4* raw, int q) {
        const int u = q / VEC, e = q % VEC;
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
        if (DT == kDtypeF32) return __uint_as_float(w[e]);
        const uint32_t v = w[e / 2];
        return __uint_as_float((e & 1) ? (v & 0xffff0000u) : (v << 16));
    }

    __device__ static __forceinline__ uint32_t index(int t, int lane, int q) {
        const int u = q / VEC, e = q % VEC;
        return static_cast<uint32_t>(t) * TILE + u * kWave * VEC + lane * VEC + e;
    }
};

// 2^((x - ref) * log2e / T) with the argument in fp64; refc = ref * c,
// c = log2(e) / T.  Exponents below -2000 (and -inf padding) give 0.
__device__ __forceinline__ double fast_weight(float x, double refc, double c) {
    double y = fma(static_cast<double>(x), c, -refc);
    y = fmax(y, -2000.0);
    const double n = rint(y);
    const float f = static_cast<float>(y - n);
    return ldexp(static_cast<double>(__builtin_amdgcn_exp2f(f)), static_cast<int>(n));
}

__device__ __forceinline__ double exp2_neg(double y) {
    y = fmax(y, -2000.0);
    const double n = rint(y);
    return ldexp(static_cast<double>(__builtin_amdgcn_exp2f(static_cast<float>(y - n))),
                 static_cast<int>(n));
}

// Smallest shift with (range >> shift) <= 255.
__device__ __forceinline__ int range_shift(uint32_t range) {
    return range > 255u ? (32 - __clz(static_cast<int>(range))) - 8 : 0;
}

// Upper end of digit bin d (shift sh) starting at lo, clipped to hi.
__device__ __forceinline__ uint32_t bin_hi(uint32_t lo_d, int sh, uint32_t hi) {
    const uint64_t e = static_cast<uint64_t>(lo_d) + ((1ull << sh) - 1ull);
    return e < hi ? static_cast<uint32_t>(e) : hi;
}

struct Cut {
    uint32_t key;
    uint32_t last;   // kept ties have index <= last
    __device__ __forceinline__ bool keep(uint32_t i, uint32_t k) const {
        return k > key || (k == key && i <= last);
    }
};

// ------------------------------------------------ wave-0 histogram scans --
// 256 bins, 4 per lane: lane l holds bins 4l .. 4l+3.

// Largest d with sum_{d' >= d} cnt[d'] >= r.  *above = sum_{d' > d}.  -1 if none.
__device__ __forceinline__ int w0_desc_count(const uint32_t* cnt, uint32_t r, uint32_t* above) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t b[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { b[i] = cnt[4 * lane + i]; s += b[i]; }
    const uint32_t incl = wave_scan_u32_dpp(s);
    const uint32_t total = readlane_u32(incl, kWave - 1);
    uint32_t pre = incl - s;
    int hit = -1;
    uint32_t hit_above = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t suffix = total - pre;
        if (suffix >= r) { hit = 4 * lane + i; hit_above = suffix - b[i]; }
        pre += b[i];
    }
    const uint64_t bal = __ballot(hit >= 0);
    if (!bal) return -1;
    const int top = 63 - __clzll(static_cast<long long>(bal));
    *above = readlane_u32(hit_above, top);
    return static_cast<int>(readlane_u32(static_cast<uint32_t>(hit), top));
}

// Largest non-empty d with base + sum_{d' >= d} m[d'] >= target.
// *above = base + sum_{d' > d} m[d'].  -1 if none.
__device__ __forceinline__ int w0_desc_mass(const uint32_t* cnt, const double* m, double base,
                                            double target, double* above) {
    const int lane = threadIdx.x & (kWave - 1);
    double b[4], s = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { b[i] = cnt[4 * lane + i] ? m[4 * lane + i] : 0.0; s += b[i]; }
    const double incl = wave_scan_f64_dpp(s);
    const double total = readlane_f64(incl, kWave - 1);
    double pre = incl - s;
    int hit = -1;
    double hit_above = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double suffix = total - pre;
        if (cnt[4 * lane + i] && base + suffix >= target) { hit = 4 * lane + i; hit_above = base + (suffix - b[i]); }
        pre += b[i];
    }
    const uint64_t bal = __ballot(hit >= 0);
    if (!bal) return -1;
    const int top = 63 - __clzll(static_cast<long long>(bal));
    *above = readlane_f64(hit_above, top);
    return static_cast<int>(readlane_u32(static_cast<uint32_t>(hit), top));
}

// Smallest d with sum_{d' <= d} cnt[d'] >= r.  *before = sum_{d' < d}.  -1 if none.
__device__ __forceinline__ int w0_asc_count(const uint32_t* cnt, uint32_t r, uint32_t* before) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t b[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { b[i] = cnt[4 * lane + i]; s += b[i]; }
    const uint32_t incl = wave_scan_u32_dpp(s);
    uint32_t pre = incl - s;
    int hit = -1;
    uint32_t hit_before = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (hit < 0 && pre + b[i] >= r) { hit = 4 * lane + i; hit_before = pre; }
        pre += b[i];
    }
    const uint64_t bal = __ballot(hit >= 0);
    if (!bal) return -1;
    const int first = __ffsll(static_cast<unsigned long long>(bal)) - 1;
    *before = readlane_u32(hit_before, first);
    return static_cast<int>(readlane_u32(static_cast<uint32_t>(hit), first));
}

// Smallest non-empty d with sum_{d' <= d} m[d'] > t.  *before = sum_{d' < d}.
// -1 if none; *last = largest non-empty bin.
__device__ __forceinline__ int w0_asc_mass(const uint32_t* cnt, const double* m, double t,
                                           double* before, int* last) {
    const int lane = threadIdx.x & (kWave - 1);
    double b[4], s = 0.0;
    int my_last = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b[i] = cnt[4 * lane + i] ? m[4 * lane + i] : 0.0;
        s += b[i];
        if (cnt[4 * lane + i]) my_last = 4 * lane + i;
    }
    const double incl = wave_scan_f64_dpp(s);
    double pre = incl - s;
    int hit = -1;
    double hit_before = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (hit < 0 && cnt[4 * lane + i] && pre + b[i] > t) { hit = 4 * lane + i; hit_before = pre; }
        pre += b[i];
    }
    const uint64_t nz = __ballot(my_last >= 0);
    *last = nz ? static_cast<int>(readlane_u32(static_cast<uint32_t>(my_last),
                                               63 - __clzll(static_cast<long long>(nz)))) : -1;
    const uint64_t bal = __ballot(hit >= 0);
    if (!bal) return -1;
    const int first = __ffsll(static_cast<unsigned long long>(bal)) - 1;
    *before = readlane_f64(hit_before, first);
    return static_cast<int>(readlane_u32(static_cast<uint32_t>(hit), first));
}

// ------------------------------------------------------------------ kernel --

template <int DT>
__global__ __launch_bounds__(kBlock) void sample_stream_kernel(SampleArgs a) {
    using IO = TileIO<DT>;
    using S = typename Elem<DT>::scalar_t;
    constexpr int Q = IO::Q;
    __shared__ Smem ss;

    const int b = blockIdx.x;
    const int V = a.V;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const void* row = static_cast<const S*>(a.logits) + static_cast<int64_t>(b) * a.row_stride;
    const RowParams prm = row_params(a.temperature, a.top_k, a.top_p, b, V);
    const uint64_t word = request_word(a.seed, ld_global<int64_t>(a.uid + b), a.step);
    const double u = uniform24(word);
    const int n_tiles = (V + IO::TILE - 1) / IO::TILE;

    int mode;
    if (prm.greedy || prm.k == 1) mode = kArgmax;
    else if (prm.k < V) mode = kTopK;
    else if (prm.top_p) mode = kTopP;
    else mode = kFull;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    // rows one read cannot serve go straight to the re-reading path
    bool use_row = !aligned || ((mode == kTopP || mode == kFull) && n_tiles > kMaxTiles);
    const bool want_z = !use_row && (mode == kTopP || mode == kFull);
    const bool want_cand = !use_row && (mode == kTopK || mode == kTopP);
    const double c = 1.4426950408889634 / static_cast<double>(prm.T);

    // ------------------------------------------------------------ stream --
    float best_x = -INFINITY;
    int best_t = -1, best_q = 0;
    float theta = INFINITY;
    const float c32 = static_cast<float>(c);
    uint32_t cnt = 0;                 // this wave's region fill (wave-uniform)

    auto process = [&](const uint4* raw, int t) {
        float tmax = IO::get(raw, 0);
#pragma unroll
        for (int q = 1; q < Q; ++q) tmax = fmaxf(tmax, IO::get(raw, q));
        if (tmax > best_x) {
            int qq = Q - 1;
#pragma unroll
            for (int q = Q - 1; q >= 0; --q) qq = IO::get(raw, q) == tmax ? q : qq;
            best_x = tmax;
            best_t = t;
            best_q = qq;
        }
        if (want_z) {
            // tile-local reference: (x - tref) is exact for the logits that
            // carry the tile's mass, so fp32 arguments are accurate here; the
            // tile sum is rescaled to the row maximum in fp64 at the end
            const float tref = wave_max_dpp(tmax);
            float s = 0.0f;
#pragma unroll
            for (int q = 0; q < Q; ++q) s += __builtin_amdgcn_exp2f((IO::get(raw, q) - tref) * c32);
            const double st = wave_sum_dpp(static_cast<double>(s));
            if (lane == 0) {
                ss.tref[t] = tref;
                ss.tsum[t] = st;
            }
        }
        if (want_cand && __ballot(tmax >= theta) != 0) {
            // lane masks, one DPP prefix scan for the slots, predicated writes
            uint32_t mask = 0;
#pragma unroll
            for (int q = 0; q < Q; ++q) mask |= IO::get(raw, q) >= theta ? (1u << q) : 0u;
            const uint32_t mine = static_cast<uint32_t>(__popc(mask));
            const uint32_t incl = wave_scan_u32_dpp(mine);
            const uint32_t tot = readlane_u32(incl, kWave - 1);
            if (cnt + tot <= static_cast<uint32_t>(kRegion)) {
                uint32_t pos = static_cast<uint32_t>(wid * kRegion) + cnt + incl - mine;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    if (mask & (1u << q)) {
                        ss.ckey[pos] = f32_key(IO::get(raw, q));
                        ss.cidx[pos] = IO::index(t, lane, q);
                        ++pos;
                    }
                }
            }
            cnt += tot;
        }
    };

    uint4 raw[IO::U], nxt[IO::U];
    int t = wid;
    if (!use_row) {
        if (t < n_tiles) IO::load(row, V, t, lane, raw);
        if (t + kWaves < n_tiles) IO::load(row, V, t + kWaves, lane, nxt);
    }
    if (want_cand) {
        // theta: lower edge of the histogram bin holding the j-th largest of
        // the per-thread maxima of the first tiles
        float lmax = -INFINITY;
        if (t < n_tiles) {
#pragma unroll
            for (int q = 0; q < Q; ++q) lmax = fmaxf(lmax, IO::get(raw, q));
        }
        const uint32_t key = lmax > -INFINITY ? f32_key(lmax) : 0u;
        const int first_elems = V < kWaves * IO::TILE ? V : kWaves * IO::TILE;
        uint32_t j;
        if (mode == kTopK) {
            j = static_cast<uint32_t>(prm.k < kBlock ? prm.k : kBlock);
        } else {
            const long long want = (static_cast<long long>(kTopPTarget) * first_elems + V - 1) / V;
            j = static_cast<uint32_t>(want < 64 ? 64 : (want > kBlock ? kBlock : want));
        }
        const uint32_t kmax = wave_max_u32_dpp(key);
        const uint32_t kmin_neg = wave_max_u32_dpp(key ? 0xffffffffu - key : 0u);
        const uint32_t nval = static_cast<uint32_t>(__popcll(__ballot(key != 0u)));
        if (threadIdx.x < 256) ss.hcnt[threadIdx.x] = 0;
        if (lane == 0) {
            ss.wbest[wid] = kmax;
            ss.wu[wid] = kmin_neg;
            ss.wcount[wid] = nval;
        }
        __syncthreads();
        uint32_t hi = 0, lo_neg = 0, nv = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            hi = max(hi, static_cast<uint32_t>(ss.wbest[w]));
            lo_neg = max(lo_neg, ss.wu[w]);
            nv += ss.wcount[w];
        }
        const uint32_t lo = 0xffffffffu - lo_neg;
        if (nv >= j) {
            const int sh = range_shift(hi - lo);
            if (key != 0u) atomicAdd(&ss.hcnt[(key - lo) >> sh], 1u);
            __syncthreads();
            if (wid == 0) {
                uint32_t above = 0;
                const int d = w0_desc_count(ss.hcnt, j, &above);
                if (lane == 0) ss.bu[0] = lo + (static_cast<uint32_t>(d < 0 ? 0 : d) << sh);
            }
            __syncthreads();
            theta = key_f32(ss.bu[0]);
        } else {
            theta = -INFINITY;
        }
    }
    if (!use_row) {
        if (t < n_tiles) process(raw, t);
        for (t += kWaves; t < n_tiles; t += kWaves) {
#pragma unroll
            for (int v = 0; v < IO::U; ++v) raw[v] = nxt[v];
            if (t + kWaves < n_tiles) IO::load(row, V, t + kWaves, lane, nxt);
            process(raw, t);
        }
    } else {
        // the re-reading path needs the maximum first
        for (int i = threadIdx.x; i < V; i += kBlock) {
            const float x = Elem<DT>::at(row, i);
            if (x > best_x) { best_x = x; best_t = i; }
        }
        best_q = -1;
    }

    // --------------------------------------------- row maximum and argmax --
    {
        uint64_t pk = 0;
        if (best_t >= 0) {
            const uint32_t idx = best_q >= 0 ? IO::index(best_t, lane, best_q) : static_cast<uint32_t>(best_t);
            pk = (static_cast<uint64_t>(f32_key(best_x)) << 32) | static_cast<uint64_t>(0xffffffffu - idx);
        }
        pk = wave_max_u64_dpp(pk);
        __syncthreads();
        if (lane == 0) {
            ss.wbest[wid] = pk;
            ss.wcount[wid] = cnt;
        }
    }
    __syncthreads();
    uint64_t best = 0;
    uint32_t n_total = 0;
    bool overflow = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        best = ss.wbest[w] > best ? ss.wbest[w] : best;
        n_total += ss.wcount[w] < kRegion ? ss.wcount[w] : kRegion;
        overflow |= ss.wcount[w] > kRegion;
    }
    const float m = key_f32(static_cast<uint32_t>(best >> 32));
    const uint32_t amax = 0xffffffffu - static_cast<uint32_t>(best);
    const double mc = static_cast<double>(m) * c;
    int32_t* topk_out = a.topk_idx_out ? a.topk_idx_out + static_cast<int64_t>(b) * kDebugTopK : nullptr;

    if (mode == kArgmax) {
        if (threadIdx.x == 0) {
            a.tokens_out[b] = static_cast<int32_t>(amax);
            if (a.kept_out) a.kept_out[b] = 1;
            if (a.rand_out) a.rand_out[b] = word;
        }
        if (a.probs_out) {
            float* probs = a.probs_out + static_cast<int64_t>(b) * V;
            for (int i = threadIdx.x; i < V; i += kBlock) probs[i] = static_cast<uint32_t>(i) == amax ? 1.0f : 0.0f;
        }
        if (topk_out && threadIdx.x < kDebugTopK) topk_out[threadIdx.x] = threadIdx.x == 0 ? static_cast<int32_t>(amax) : -1;
        return;
    }

    // ------------------------------------------------------ entry sources --
    // An entry is (key, index, weight).  The candidate source walks this
    // wave's LDS region; the row source walks this thread's share of the row
    // (read again from memory) within an index range.
    bool from_row = use_row;
    auto each = [&](uint32_t ilo, uint32_t ihi, auto&& f) {
        if (!from_row) {
            const int rbase = wid * kRegion;
            const uint32_t n = cnt < kRegion ? cnt : kRegion;
            for (uint32_t i = lane; i < n; i += kWave) {
                const uint32_t idx = ss.cidx[rbase + i];
                if (idx >= ilo && idx <= ihi) f(ss.ckey[rbase + i], idx, static_cast<int>(rbase + i));
            }
        } else {
            const uint32_t hi = ihi < static_cast<uint32_t>(V - 1) ? ihi : static_cast<uint32_t>(V - 1);
            for (uint32_t i = ilo + threadIdx.x; i <= hi; i += kBlock)
                f(f32_key(Elem<DT>::at(row, i)), i, -1);
        }
    };
    auto weight_of = [&](uint32_t k, int slot) -> double {
        return slot >= 0 ? static_cast<double>(ss.cw[slot]) : fast_weight(key_f32(k), mc, c);
    };

    // sum of weights (and count) over the entries inside `ct`
    auto sum_cut = [&](const Cut& ct, uint32_t* count_out) -> double {
        double s = 0.0;
        uint32_t n = 0;
        each(0u, 0xffffffffu, [&](uint32_t k, uint32_t i, int slot) {
            if (ct.keep(i, k)) { s += weight_of(k, slot); ++n; }
        });
        s = wave_sum_dpp(s);
        n = readlane_u32(wave_scan_u32_dpp(n), kWave - 1);
        __syncthreads();
        if (lane == 0) { ss.wd[wid] = s; ss.wu[wid] = n; }
        __syncthreads();
        double tot = 0.0;
        uint32_t nt = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) { tot += ss.wd[w]; nt += ss.wu[w]; }
        if (count_out) *count_out = nt;
        return tot;
    };

    // key range of the entries inside `ct`
    auto key_range = [&](const Cut& ct, uint32_t* lo, uint32_t* hi) {
        uint32_t mx = 0, mn = 0;
        each(0u, 0xffffffffu, [&](uint32_t k, uint32_t i, int) {
            if (ct.keep(i, k)) { mx = max(mx, k); mn = max(mn, 0xffffffffu - k); }
        });
        mx = wave_max_u32_dpp(mx);
        mn = wave_max_u32_dpp(mn);
        __syncthreads();
        if (lane == 0) { ss.wu[wid] = mx; ss.wcount[wid] = mn; }
        __syncthreads();
        uint32_t a1 = 0, a2 = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) { a1 = max(a1, ss.wu[w]); a2 = max(a2, ss.wcount[w]); }
        *hi = a1;
        *lo = 0xffffffffu - a2;
    };

    // Histogram of the entries with pred(key, index), by key digit (by_index
    // false) or index digit over [lo, hi] with shift sh; counts and masses.
    auto histogram = [&](auto&& pred, bool by_index, uint32_t lo, uint32_t hi, int sh, bool with_mass) {
        __syncthreads();
        if (threadIdx.x < 256) {
            ss.hcnt[threadIdx.x] = 0;
            ss.hmass[threadIdx.x] = 0.0;
        }
        __syncthreads();
        each(by_index ? lo : 0u, by_index ? hi : 0xffffffffu, [&](uint32_t k, uint32_t i, int slot) {
            if (!pred(k, i)) return;
            const uint32_t v = by_index ? i : k;
            if (v < lo || v > hi) return;
            const uint32_t d = (v - lo) >> sh;
            atomicAdd(&ss.hcnt[d], 1u);
            if (with_mass) atomicAdd(&ss.hmass[d], weight_of(k, slot));
        });
        __syncthreads();
    };

    // Gather the entries with pred(key, index) and key (or index) in [lo, hi]
    // (at most kList of them), ranked by (key desc, index asc) or index asc
    // into ss.skey/sidx/sw[0 .. list_n).
    auto gather = [&](auto&& pred, bool by_index, uint32_t lo, uint32_t hi) {
        __syncthreads();
        if (threadIdx.x == 0) ss.list_n = 0;
        __syncthreads();
        each(by_index ? lo : 0u, by_index ? hi : 0xffffffffu, [&](uint32_t k, uint32_t i, int slot) {
            if (!pred(k, i)) return;
            if (!by_index && (k < lo || k > hi)) return;
            const uint32_t p = atomicAdd(&ss.list_n, 1u);
            if (p < kList) {
                ss.lkey[p] = k;
                ss.lidx[p] = i;
                ss.lw[p] = static_cast<float>(weight_of(k, slot));
            }
        });
        __syncthreads();
        if (wid == 0) {
            const int n = ss.list_n < kList ? static_cast<int>(ss.list_n) : kList;
            if (lane < n) {
                const uint32_t k = ss.lkey[lane], i = ss.lidx[lane];
                int r = 0;
                for (int e = 0; e < n; ++e) {
                    const uint32_t k2 = ss.lkey[e], i2 = ss.lidx[e];
                    r += (by_index ? i2 < i : (k2 > k || (k2 == k && i2 < i))) ? 1 : 0;
                }
                ss.skey[r] = k;
                ss.sidx[r] = i;
                ss.sw[r] = ss.lw[lane];
            }
        }
        __syncthreads();
    };

    // Index of the r-th (1-based, token order) entry inside `ct` whose key is `key`.
    auto nth_tie = [&](const Cut& ct, uint32_t key, uint32_t r) -> uint32_t {
        auto pred = [&](uint32_t k, uint32_t i) { return k == key && ct.keep(i, k); };
        uint32_t ilo = 0, ihi = static_cast<uint32_t>(V - 1);
        for (;;) {
            const int sh = range_shift(ihi - ilo);
            histogram(pred, true, ilo, ihi, sh, false);
            if (wid == 0) {
                uint32_t before = 0;
                const int d = w0_asc_count(ss.hcnt, r, &before);
                if (lane == 0) {
                    ss.bu[2] = static_cast<uint32_t>(d < 0 ? 0 : d);
                    ss.bu[3] = before;
                    ss.bu[4] = ss.hcnt[d < 0 ? 0 : d];
                }
            }
            __syncthreads();
            const uint32_t d = ss.bu[2], before = ss.bu[3], cd = ss.bu[4];
            const uint32_t nlo = ilo + (d << sh);
            const uint32_t nhi = bin_hi(nlo, sh, ihi);
            r -= before;
            if (cd <= static_cast<uint32_t>(kList) || sh == 0) {
                gather(pred, true, nlo, nhi);
                return ss.sidx[r >= 1 && r <= kList ? r - 1 : 0];
            }
            ilo = nlo;
            ihi = nhi;
        }
    };

    // The cut ending at the r-th (1-based) entry of `ct` in descending order.
    auto select_desc = [&](const Cut& ct, uint32_t r) -> Cut {
        auto pred = [&](uint32_t k, uint32_t i) { return ct.keep(i, k); };
        uint32_t lo, hi;
        key_range(ct, &lo, &hi);
        for (;;) {
            const int sh = range_shift(hi - lo);
            histogram(pred, false, lo, hi, sh, false);
            if (wid == 0) {
                uint32_t above = 0;
                const int d = w0_desc_count(ss.hcnt, r, &above);
                if (lane == 0) {
                    ss.bu[2] = static_cast<uint32_t>(d < 0 ? 0 : d);
                    ss.bu[3] = above;
                    ss.bu[4] = ss.hcnt[d < 0 ? 0 : d];
                }
            }
            __syncthreads();
            const uint32_t d = ss.bu[2], above = ss.bu[3], cd = ss.bu[4];
            const uint32_t nlo = lo + (d << sh);
            const uint32_t nhi = bin_hi(nlo, sh, hi);
            r -= above;
            if (cd <= static_cast<uint32_t>(kList)) {
                gather(pred, false, nlo, nhi);
                const uint32_t e = r >= 1 && r <= kList ? r - 1 : 0;
                return Cut{ss.skey[e], ss.sidx[e]};
            }
            if (sh == 0) return Cut{nlo, nth_tie(ct, nlo, r)};
            lo = nlo;
            hi = nhi;
        }
    };

    // The top-p cut inside `ct`: the descending-order prefix up to the first
    // entry whose inclusive prefix mass reaches `target`.  false if the
    // entries' mass never reaches it.
    auto mass_cut = [&](const Cut& ct, double target, Cut* out) -> bool {
        auto pred = [&](uint32_t k, uint32_t i) { return ct.keep(i, k); };
        uint32_t lo, hi;
        key_range(ct, &lo, &hi);
        double above = 0.0;
        for (;;) {
            const int sh = range_shift(hi - lo);
            histogram(pred, false, lo, hi, sh, true);
            if (wid == 0) {
                double ab = 0.0;
                const int d = w0_desc_mass(ss.hcnt, ss.hmass, above, target, &ab);
                if (lane == 0) {
                    ss.bu[2] = static_cast<uint32_t>(d);
                    ss.bu[4] = d >= 0 ? ss.hcnt[d] : 0u;
                    ss.bd[1] = ab;
                }
            }
            __syncthreads();
            const int d = static_cast<int>(ss.bu[2]);
            const uint32_t cd = ss.bu[4];
            const double ab = ss.bd[1];
            if (d < 0) return false;
            above = ab;
            const uint32_t nlo = lo + (static_cast<uint32_t>(d) << sh);
            const uint32_t nhi = bin_hi(nlo, sh, hi);
            if (cd <= static_cast<uint32_t>(kList)) {
                gather(pred, false, nlo, nhi);
                if (wid == 0) {
                    const int n = ss.list_n < kList ? static_cast<int>(ss.list_n) : kList;
                    const double w = lane < n ? static_cast<double>(ss.sw[lane]) : 0.0;
                    const double incl = above + wave_scan_f64_dpp(w);
                    const uint64_t bal = __ballot(lane < n && incl >= target);
                    const int e = bal ? __ffsll(static_cast<unsigned long long>(bal)) - 1 : (n > 0 ? n - 1 : 0);
                    if (lane == 0) {
                        ss.bu[5] = ss.skey[e];
                        ss.bu[6] = ss.sidx[e];
                    }
                }
                __syncthreads();
                *out = Cut{ss.bu[5], ss.bu[6]};
                return true;
            }
            if (sh == 0) {
                // a run of equal keys: each weighs w and the j-th of them (token
                // order) has exclusive prefix above + j*w
                const double w = weight_of(nlo, -1);
                const double y = (target - above) / w;
                uint32_t keep = cd;
                if (y < static_cast<double>(cd)) {
                    const double cy = ceil(y);
                    keep = cy < 1.0 ? 1u : static_cast<uint32_t>(cy);
                }
                const uint32_t last = keep < cd ? nth_tie(ct, nlo, keep) : (ct.key == nlo ? ct.last : 0xffffffffu);
                *out = Cut{nlo, last};
                return true;
            }
            lo = nlo;
            hi = nhi;
        }
    };

    // ------------------------------------------------- softmax normaliser --
    if (want_z) {
        if (wid == 0) {
            const int per = (n_tiles + kWave - 1) / kWave;
            const int tlo = lane * per, thi = tlo + per < n_tiles ? tlo + per : n_tiles;
            double part = 0.0;
            for (int i = tlo; i < thi; ++i) {
                const double sc = ss.tsum[i] * exp2_neg((static_cast<double>(ss.tref[i]) - static_cast<double>(m)) * c);
                ss.tsum[i] = sc;
                part += sc;
            }
            const double incl = wave_scan_f64_dpp(part);
            const double z = readlane_f64(incl, kWave - 1);
            if (lane == 0) ss.bd[0] = z;
            if (mode == kFull) {
                // the tile holding u * Z, then that one tile read again
                const double target = u * z;
                const uint64_t bal = __ballot(part > 0.0 && incl > target);
                const uint64_t nz = __ballot(part > 0.0);
                const int owner = bal ? __ffsll(static_cast<unsigned long long>(bal)) - 1
                                      : (nz ? 63 - __clzll(static_cast<long long>(nz)) : 0);
                int ts = 0;
                double rem = 0.0;
                if (lane == owner) {
                    double cum = incl - part;
                    ts = -1;
                    int last_nz = tlo;
                    for (int i = tlo; i < thi; ++i) {
                        if (ss.tsum[i] > 0.0) last_nz = i;
                        if (ts < 0 && cum + ss.tsum[i] > target) { ts = i; rem = target - cum; }
                        if (ts < 0) cum += ss.tsum[i];
                    }
                    if (ts < 0) { ts = last_nz; rem = ss.tsum[last_nz] * 2.0 + 1.0; }
                }
                ts = static_cast<int>(readlane_u32(static_cast<uint32_t>(ts), owner));
                rem = readlane_f64(rem, owner);
                uint4 rr[IO::U];
                IO::load(row, V, ts, lane, rr);
                double run = 0.0;
                int tok = -1, last_pos = -1;
#pragma unroll
                for (int uu = 0; uu < IO::U; ++uu) {
                    double w[IO::VEC];
                    double ps = 0.0;
                    int my_last = -1;
#pragma unroll
                    for (int e = 0; e < IO::VEC; ++e) {
                        w[e] = fast_weight(IO::get(rr, uu * IO::VEC + e), mc, c);
                        ps += w[e];
                        if (w[e] > 0.0) my_last = static_cast<int>(IO::index(ts, lane, uu * IO::VEC + e));
                    }
                    const double pin = wave_scan_f64_dpp(ps);
                    const double tot = readlane_f64(pin, kWave - 1);
                    const uint64_t lastb = __ballot(my_last >= 0);
                    if (lastb)
                        last_pos = static_cast<int>(readlane_u32(static_cast<uint32_t>(my_last),
                                                                 63 - __clzll(static_cast<long long>(lastb))));
                    if (tok < 0 && run + tot > rem) {
                        const uint64_t ob = __ballot(ps > 0.0 && run + pin > rem);
                        if (ob) {
                            const int own = __ffsll(static_cast<unsigned long long>(ob)) - 1;
                            int mine = -1;
                            bool done = false;
                            double cum = run + (pin - ps);
#pragma unroll
                            for (int e = 0; e < IO::VEC; ++e) {
                                cum += w[e];
                                if (!done && w[e] > 0.0) mine = static_cast<int>(IO::index(ts, lane, uu * IO::VEC + e));
                                if (w[e] > 0.0 && cum > rem) done = true;
                            }
                            tok = static_cast<int>(readlane_u32(static_cast<uint32_t>(mine), own));
                        }
                    }
                    run += tot;
                }
                if (tok < 0) tok = last_pos;
                if (lane == 0) ss.bu[1] = static_cast<uint32_t>(tok);
            }
        }
        __syncthreads();
        if (mode == kFull) {
            const uint32_t tok = ss.bu[1];
            const double z = ss.bd[0];
            if (threadIdx.x == 0) {
                a.tokens_out[b] = static_cast<int32_t>(tok);
                if (a.kept_out) a.kept_out[b] = V;
                if (a.rand_out) a.rand_out[b] = word;
            }
            if (a.probs_out) {
                float* probs = a.probs_out + static_cast<int64_t>(b) * V;
                for (int i = threadIdx.x; i < V; i += kBlock)
                    probs[i] = static_cast<float>(fast_weight(Elem<DT>::at(row, i), mc, c) / z);
            }
            if (topk_out) {
                from_row = true;
                const Cut top = select_desc(Cut{0u, 0xffffffffu}, kDebugTopK < V ? kDebugTopK : V);
                gather([&](uint32_t k, uint32_t i) { return top.keep(i, k); }, false, 0u, 0xffffffffu);
                if (threadIdx.x < kDebugTopK)
                    topk_out[threadIdx.x] = threadIdx.x < ss.list_n ? static_cast<int32_t>(ss.sidx[threadIdx.x]) : -1;
            }
            return;
        }
    }
    const double Z = want_z ? ss.bd[0] : 0.0;

    // ------------------------------------------------- candidate weights --
    if (want_cand) {
        if (overflow || (mode == kTopK && n_total < static_cast<uint32_t>(prm.k)))
            use_row = true;
        else {
            const int rbase = wid * kRegion;
            for (uint32_t i = lane; i < cnt && i < kRegion; i += kWave)
                ss.cw[rbase + i] = static_cast<float>(fast_weight(key_f32(ss.ckey[rbase + i]), mc, c));
        }
    }

    // ------------------------------------------ top-k, then top-p, cuts --
    Cut cut{0u, 0xffffffffu};
    for (int pass = 0; pass < 2; ++pass) {
        from_row = use_row;
        cut = Cut{0u, 0xffffffffu};
        if (mode == kTopK) cut = select_desc(cut, static_cast<uint32_t>(prm.k));
        if (!prm.top_p) break;
        const double wk = (mode == kTopK || use_row) ? sum_cut(cut, nullptr) : Z;
        Cut pc;
        const bool found = mass_cut(cut, static_cast<double>(prm.p) * wk, &pc);
        if (found) {
            cut = pc;
            break;
        }
        // the mass never reached p * W inside the entries: top-k keeps all of
        // its set (rounding only); top-p over candidates must see the whole row
        if (mode == kTopK || use_row) break;
        use_row = true;
    }

    // ---- the draw: first index (token order) whose kept prefix exceeds u*W --
    uint32_t n_kept = 0;
    const double W = sum_cut(cut, &n_kept);
    double tgt = u * W;
    uint32_t token;
    {
        auto kept = [&](uint32_t k, uint32_t i) { return cut.keep(i, k); };
        uint32_t ilo = 0, ihi = static_cast<uint32_t>(V - 1);
        for (;;) {
            const int sh = range_shift(ihi - ilo);
            histogram(kept, true, ilo, ihi, sh, true);
            if (wid == 0) {
                double before = 0.0;
                int last = -1;
                const int d = w0_asc_mass(ss.hcnt, ss.hmass, tgt, &before, &last);
                if (lane == 0) {
                    ss.bu[2] = static_cast<uint32_t>(d);
                    ss.bu[3] = static_cast<uint32_t>(last);
                    ss.bu[4] = d >= 0 ? ss.hcnt[d] : (last >= 0 ? ss.hcnt[last] : 0u);
                    ss.bd[1] = before;
                }
            }
            __syncthreads();
            int d = static_cast<int>(ss.bu[2]);
            const int last = static_cast<int>(ss.bu[3]);
            const uint32_t cd = ss.bu[4];
            const double before = ss.bd[1];
            bool past = false;
            if (d < 0) {            // rounding: u * W at or past the kept total
                d = last < 0 ? 0 : last;
                past = true;
            } else {
                tgt -= before;
            }
            const uint32_t nlo = ilo + (static_cast<uint32_t>(d) << sh);
            const uint32_t nhi = bin_hi(nlo, sh, ihi);
            if (cd <= static_cast<uint32_t>(kList) || sh == 0) {
                gather(kept, true, nlo, nhi);
                if (wid == 0) {
                    const int n = ss.list_n < kList ? static_cast<int>(ss.list_n) : kList;
                    const double w = lane < n ? static_cast<double>(ss.sw[lane]) : 0.0;
                    const double incl = wave_scan_f64_dpp(w);
                    const uint64_t bal = past ? 0ull : __ballot(lane < n && w > 0.0 && incl > tgt);
                    const int e = bal ? __ffsll(static_cast<unsigned long long>(bal)) - 1 : (n > 0 ? n - 1 : 0);
                    if (lane == 0) ss.bu[7] = ss.sidx[e];
                }
                __syncthreads();
                token = ss.bu[7];
                break;
            }
            ilo = nlo;
            ihi = nhi;
        }
    }

    if (threadIdx.x == 0) {
        a.tokens_out[b] = static_cast<int32_t>(token);
        if (a.kept_out) a.kept_out[b] = static_cast<int32_t>(n_kept);
        if (a.rand_out) a.rand_out[b] = word;
    }
    if (a.probs_out) {
        float* probs = a.probs_out + static_cast<int64_t>(b) * V;
        for (int i = threadIdx.x; i < V; i += kBlock) {
            const float x = Elem<DT>::at(row, i);
            probs[i] = cut.keep(static_cast<uint32_t>(i), f32_key(x))
                           ? static_cast<float>(fast_weight(x, mc, c) / W) : 0.0f;
        }
    }
    if (topk_out) {
        // first min(k, 64) of the descending order, from the row itself
        from_row = true;
        const uint32_t nk = static_cast<uint32_t>(prm.k < kDebugTopK ? prm.k : kDebugTopK);
        const Cut top = select_desc(Cut{0u, 0xffffffffu}, nk);
        gather([&](uint32_t k, uint32_t i) { return top.keep(i, k); }, false, 0u, 0xffffffffu);
        if (threadIdx.x < kDebugTopK)
            topk_out[threadIdx.x] = threadIdx.x < nk && threadIdx.x < ss.list_n ? static_cast<int32_t>(ss.sidx[threadIdx.x]) : -1;
    }
}

}  // namespace

hipError_t launch_sample_stream(const SampleArgs& args, int dtype, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.B));
    if (dtype == kDtypeF32)
        hipLaunchKernelGGL(sample_stream_kernel<kDtypeF32>, grid, dim3(kBlock), 0, stream, args);
    else
        hipLaunchKernelGGL(sample_stream_kernel<kDtypeBF16>, grid, dim3(kBlock), 0, stream, args);
    return hipGetLastError();
}

}  // namespace dst
