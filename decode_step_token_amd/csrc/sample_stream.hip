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
// The row is read in tiles of 1024 logits (4 KB fp32, 2 KB bf16); tile t
// belongs to wave t mod 16.  What one read leaves behind:
//   * the row maximum and its lowest index, from per-tile lane maxima (the
//     argmax bookkeeping only runs when a lane's tile beats its running best);
//   * rows without top-k or top-p: one softmax sum per tile, relative to the
//     tile's own maximum tref, with fp32 arguments (x - tref) * log2(e)/T
//     through v_exp_f32, rescaled to the row maximum in fp64 at the end.
//     (x - tref) is exact for every logit within a factor two of tref, which
//     carries the tile's mass, so the normaliser stays within ~2e-7 of the
//     fp64 sum (an argument taken relative to the row maximum in one fp32
//     expression is off by up to 2.5e-6);
//   * top-p rows: the same sums per lane, against the lane's running maximum
//     (online rescaling when it grows), accumulated in fp64;
//   * rows with top-k or top-p: every logit >= theta, with its index, in a
//     wave-private LDS region in token order, with each tile's first slot and
//     count.  theta is fixed after the first tile of every wave: the lower
//     edge of the histogram bin that holds the j-th largest of the 1024
//     per-thread maxima.  j = k for top-k: j per-thread maxima are j distinct
//     logits >= theta, so the top-k set is always inside the regions.  For
//     top-p, j aims at about 900 candidates.
//
// Finishing the row from the candidates is a sequence of block-wide passes
// over the regions; after each one wave 0 reads what the pass produced and
// picks the next pass (see the candidate tail below).  Rows without top-k or
// top-p draw from the tile sums and read one tile again.  When the kept
// prefix does not end inside the candidates (a flat top-p row whose nucleus
// reaches below theta, a full region), or the row is not 16-byte aligned,
// exact block-wide descents run over the row itself, re-reading it.
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
constexpr int kTopKCands = 4096;          // top-k rows: candidate count the threshold aims below
constexpr int kTopPTarget = 900;           // aimed-at candidate count for top-p rows
constexpr int kBins = 1024;                // candidate histograms: 16 bins per lane of wave 0
// Rows whose candidates are few (top-p, min_p, top-k up to kStageMaxK) keep
// a lane's whole 16-byte load when it holds a candidate, two region slots
// per load at the top of the wave's region, and expand the loads into
// entries once, after the wave's stream.
constexpr int kStageCap = kRegion / 2;     // staged loads per wave
constexpr int kStageMaxK = 128;
// Flat top-p rows (the nucleus reaches far below the candidate threshold):
// a weight histogram of 1024 bins, 16 per octave of the weight from 2^-64 up
// (bin = the weight's fp32 exponent and top four mantissa bits), kept in
// kHistCopies interleaved copies (lane l adds to copy l mod kHistCopies) in
// the candidate regions.
constexpr int kWBinBase = (127 - 64) << 4;
constexpr int kHistCopies = 8;
// A top-p row is taken for flat when the first tiles' weight at or above the
// candidate threshold is below this fraction of p times their total weight;
// the estimate is made only when the threshold lies within 2^kFlatGap (in
// weight) of the first tiles' maximum, below which it cannot hold.
constexpr double kFlatFrac = 0.8;
constexpr float kFlatGap = 6.0f;
constexpr int kBinsPerLane = kBins / kWave;
constexpr int kTilesPerLane = kMaxTiles / kWave;
static_assert(kBins == kBlock, "one bin cleared per thread");

enum Mode { kArgmax = 0, kTopK = 1, kTopP = 2, kFull = 3 };

// One pass of the candidate tail over every wave's region (see below).
enum PassType : uint32_t {
    kPassHistW = 0,   // weights of all entries, then the key histogram
    kPassHist,        // key histogram of the entries in [lo, hi] kept by the restriction
    kPassGather,      // list the entries in [lo, hi] kept by the restriction
    kPassTieCount,    // per-tile counts of the entries with key == tie kept by the restriction
    kPassTileMass,    // per-tile weight of the entries kept by the restriction
    kPassDone,
    kPassFallback,    // the kept prefix reaches below theta: finish from the row
    kPassHistC,       // order keys and the count histogram only
    kPassWeights,     // weights of all entries
};

struct PassDesc {
    uint32_t type, lo, hi, sh;
    uint32_t rkey, rlast;   // restriction cut
    uint32_t tie;
    uint32_t pad;
};

// A bin picked by the block-parallel histogram scan.
struct BlockPick {
    int d;              // bin, -1 if the mass target is not reached
    uint32_t cnt;       // entries in the bin
    uint32_t above_c;   // entries in the bins above it
    uint32_t pad;
    double mass;        // weight of the bin
    double above_m;     // weight of the bins above it
};

struct Smem {
    alignas(16) uint2 cent[kCap + kBlock];  // candidates: (value bits, later the order key; token index);
                                  // the last kBlock entries: one discard slot per thread
    float cw[kCap];
    float tref[kMaxTiles];
    double tsum[kMaxTiles];
    double tacc[kMaxTiles];       // per-tile counts / weights of the candidate tail
    uint16_t tstart[kMaxTiles];   // a tile's first slot (in the region of the wave that read it)
    uint16_t tcnt[kMaxTiles];     // ... and its number of entries
    alignas(16) uint32_t hcnt[kBins];
    alignas(16) double hmass[kBins];
    PassDesc pass;
    unsigned long long mbest;     // merge: packed (key, ~index) maximum
    uint32_t mtotal, movf;        // merge: candidates stored, any region overflowed
    uint64_t word;                // the row's Philox word (written by wave 0)
    float minp;                   // the row's effective min_p (0: off)
    uint32_t kmin;                // min_p threshold as an order key (0: no min_p)
    double res_w;
    uint32_t res_token, res_kept;
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
    // block-parallel picks and ranks
    uint32_t wtc[kWaves];  // per-wave totals of a pick or tile scan
    double wtm[kWaves];
    BlockPick pick;
    uint32_t rankp[kList]; // rank of list entry i in descending order / in token order
    uint32_t ranki[kList];
    uint32_t xrp[kList];   // list in token order: its descending rank, weight, index
    float xw[kList];
    uint32_t xidx[kList];
    uint32_t cut_key, cut_last;
    uint32_t next_tile;    // the stream's next unclaimed tile
    uint32_t flat_bad;     // a flat row's weight reference had to be raised
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
        if (base + TILE <= V) {
            // a whole tile inside the row: no per-load bounds (the test is
            // wave-uniform)
            const char* p = static_cast<const char*>(row) + (base + lane * VEC) * (DT == kDtypeF32 ? 4 : 2);
#pragma unroll
            for (int u = 0; u < U; ++u)
                raw[u] = ld_global_u4_stream(p + u * kWave * VEC * (DT == kDtypeF32 ? 4 : 2));
            return;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t off = base + u * kWave * VEC + lane * VEC;
            if (off + VEC <= V) {
                raw[u] = ld_global_u4_stream(static_cast<const char*>(row) + off * (DT == kDtypeF32 ? 4 : 2));
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

// -------------------------------------- wave-0 scans of the 1024-bin tail --
// kBins bins, kBinsPerLane per lane: lane l holds bins l*kBinsPerLane + i.
// Each scan also clears the bins it has read (the next pass starts from 0).

struct BinPick {
    int d;            // chosen bin, -1 if none
    uint32_t cnt;     // its entry count
    double mass;      // ... and weight
    uint32_t above_c; // entries in the bins above it
    double above_m;   // weight of the bins above it (plus the base, for mass picks)
    bool reached;     // mass pick: the target was reached
};

// Per-lane sums of the lane's bins (one read), then wave scans.
struct BinScan {
    uint32_t total, pre;   // entries in all bins / in the bins before this lane's
    double totalm, prem;   // ... their weight
};

__device__ __forceinline__ BinScan w0_scan_bins(const uint32_t* cnt, const double* m) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint4* c4 = reinterpret_cast<const uint4*>(cnt + kBinsPerLane * lane);
    const double2* m2 = reinterpret_cast<const double2*>(m + kBinsPerLane * lane);
    uint32_t s = 0;
    double sm = 0.0;
#pragma unroll
    for (int i = 0; i < kBinsPerLane / 4; ++i) {
        const uint4 v = c4[i];
        s += v.x + v.y + v.z + v.w;
    }
#pragma unroll
    for (int i = 0; i < kBinsPerLane / 2; ++i) {
        const double2 v = m2[i];
        sm += v.x;
        sm += v.y;
    }
    const uint32_t incl = wave_scan_u32_dpp(s);
    const double inclm = wave_scan_f64_dpp(sm);
    return BinScan{readlane_u32(incl, kWave - 1), incl - s, readlane_f64(inclm, kWave - 1), inclm - sm};
}

__device__ __forceinline__ void w0_clear_bins(uint32_t* cnt, double* m) {
    const int lane = threadIdx.x & (kWave - 1);
    uint4* c4 = reinterpret_cast<uint4*>(cnt + kBinsPerLane * lane);
    double2* m2 = reinterpret_cast<double2*>(m + kBinsPerLane * lane);
#pragma unroll
    for (int i = 0; i < kBinsPerLane / 4; ++i) c4[i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kBinsPerLane / 2; ++i) m2[i] = make_double2(0.0, 0.0);
}

__device__ __forceinline__ BinPick w0_broadcast_pick(int hit_bin, uint32_t hcnt, double hmass, uint32_t hc,
                                                     double hm, int src) {
    BinPick out;
    out.d = static_cast<int>(readlane_u32(static_cast<uint32_t>(hit_bin), src));
    out.cnt = readlane_u32(hcnt, src);
    out.mass = readlane_f64(hmass, src);
    out.above_c = readlane_u32(hc, src);
    out.above_m = readlane_f64(hm, src);
    out.reached = true;
    return out;
}

// The bin holding the r-th entry in descending key order (r >= 1).
__device__ __forceinline__ BinPick w0_pick_count(uint32_t* cnt, double* m, uint32_t r) {
    const int lane = threadIdx.x & (kWave - 1);
    const BinScan bs = w0_scan_bins(cnt, m);
    uint32_t pre = bs.pre;
    double prem = bs.prem;
    int hit = -1;
    uint32_t hc = 0, hcnt = 0;
    double hm = 0.0, hmass = 0.0;
    const uint32_t* cl = cnt + kBinsPerLane * lane;
    const double* ml = m + kBinsPerLane * lane;
    for (int i = 0; i < kBinsPerLane; ++i) {
        const uint32_t b = cl[i];
        const double bm = ml[i];
        if (b != 0u && bs.total - pre >= r) {
            hit = kBinsPerLane * lane + i;
            hc = bs.total - pre - b;
            hm = bs.totalm - prem - bm;
            hcnt = b;
            hmass = bm;
        }
        pre += b;
        prem += bm;
    }
    w0_clear_bins(cnt, m);
    const uint64_t bal = __ballot(hit >= 0);
    if (!bal) return BinPick{-1, 0u, 0.0, 0u, 0.0, false};
    return w0_broadcast_pick(hit, hcnt, hmass, hc, hm, 63 - __clzll(static_cast<long long>(bal)));
}

// The bin where base + the descending-order weight first reaches target:
// the largest non-empty d with base + sum_{d' >= d} m[d'] >= target.  If no
// bin reaches it, the lowest non-empty bin with reached = false.
__device__ __forceinline__ BinPick w0_pick_mass(uint32_t* cnt, double* m, double base, double target) {
    const int lane = threadIdx.x & (kWave - 1);
    const BinScan bs = w0_scan_bins(cnt, m);
    uint32_t pre = bs.pre;
    double prem = bs.prem;
    int hit = -1, low = -1;
    uint32_t hc = 0, hcnt = 0, lc = 0, lcnt = 0;
    double hm = 0.0, hmass = 0.0, lm = 0.0, lmass = 0.0;
    const uint32_t* cl = cnt + kBinsPerLane * lane;
    const double* ml = m + kBinsPerLane * lane;
    for (int i = 0; i < kBinsPerLane; ++i) {
        const uint32_t b = cl[i];
        const double bm = ml[i];
        if (b != 0u) {
            const uint32_t ac = bs.total - pre - b;
            const double am = base + (bs.totalm - prem - bm);
            if (base + (bs.totalm - prem) >= target) {
                hit = kBinsPerLane * lane + i; hc = ac; hm = am; hcnt = b; hmass = bm;
            }
            if (low < 0) {
                low = kBinsPerLane * lane + i; lc = ac; lm = am; lcnt = b; lmass = bm;
            }
        }
        pre += b;
        prem += bm;
    }
    w0_clear_bins(cnt, m);
    const uint64_t bal = __ballot(hit >= 0);
    if (bal) return w0_broadcast_pick(hit, hcnt, hmass, hc, hm, 63 - __clzll(static_cast<long long>(bal)));
    const uint64_t nz = __ballot(low >= 0);
    if (!nz) return BinPick{-1, 0u, 0.0, 0u, 0.0, false};
    BinPick out = w0_broadcast_pick(low, lcnt, lmass, lc, lm, __ffsll(static_cast<unsigned long long>(nz)) - 1);
    out.reached = false;
    return out;
}

// Smallest shift with (range >> shift) < kBins.
__device__ __forceinline__ int range_shift_bins(uint32_t range) {
    return range >= static_cast<uint32_t>(kBins) ? (32 - __clz(static_cast<int>(range))) - 10 : 0;
}

// Orders the LDS accesses of one wave (the wave's lanes read what other lanes
// of the same wave wrote).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// --------------------------------------------------------------- row order --
// Sampled rows with top-k off and top-p or min_p on may take the flat-row or
// the re-reading path, several times longer than a stream.  One block of this
// kernel fills a compute unit (its LDS and registers), so a grid of more rows
// than compute units runs in rounds, blocks starting in index order as units
// free up.  Block g then takes the g-th row of the order "those long rows
// first, then the rest" (each part in index order): the long rows start in
// the first round instead of lengthening the last.  Every wave finds the same
// row by itself, from one read of the parameters; larger batches keep index
// order.

constexpr int kOrderChunks = 8;     // batches of up to 8 * 64 rows are reordered

__device__ __forceinline__ bool long_row(const SampleArgs& a, int r) {
    const RowParams p = row_params(a.temperature, a.top_k, a.top_p, a.min_p, r, a.V);
    return !p.greedy && p.k == a.V && (p.top_p || p.min_p > 0.0f);
}

__device__ __forceinline__ int long_rows_first(const SampleArgs& a, int g) {
    const int lane = threadIdx.x & (kWave - 1);
    // one coalesced read per parameter and 64 rows (rows past B read row
    // B - 1 and are masked off), the long-row masks kept per 64 rows
    uint64_t m[kOrderChunks];
    uint32_t n_long = 0;
#pragma unroll
    for (int c = 0; c < kOrderChunks; ++c) {
        const int r = c * kWave + lane;
        const bool lr = long_row(a, r < a.B ? r : a.B - 1);
        m[c] = __ballot(r < a.B && lr);
        n_long += static_cast<uint32_t>(__popcll(m[c]));
    }
    const bool want_long = static_cast<uint32_t>(g) < n_long;
    uint32_t left = want_long ? static_cast<uint32_t>(g) : static_cast<uint32_t>(g) - n_long;
    // the 64 rows holding the wanted one, and its rank among them
    uint64_t sm = 0ull;
    int sr0 = -1;
#pragma unroll
    for (int c = 0; c < kOrderChunks; ++c) {
        const int r0 = c * kWave;
        const int nv = a.B - r0;
        const uint64_t valid = nv <= 0 ? 0ull : (nv >= kWave ? ~0ull : (1ull << nv) - 1ull);
        const uint64_t mc = want_long ? m[c] : (~m[c] & valid);
        const uint32_t cnt = static_cast<uint32_t>(__popcll(mc));
        if (sr0 < 0) {
            if (left < cnt) { sm = mc; sr0 = r0; }
            else left -= cnt;
        }
    }
    if (sr0 < 0) return g;    // not reached: the wanted part holds more than left rows
    const uint64_t below = lane ? (sm & (~0ull >> (kWave - lane))) : 0ull;
    const uint64_t hit = __ballot(((sm >> lane) & 1ull) && static_cast<uint32_t>(__popcll(below)) == left);
    return sr0 + __ffsll(static_cast<unsigned long long>(hit)) - 1;
}

// ------------------------------------------------------------------ kernel --

template <int DT>
__global__ __launch_bounds__(kBlock) void sample_stream_kernel(SampleArgs a) {
    using IO = TileIO<DT>;
    using S = typename Elem<DT>::scalar_t;
    constexpr int Q = IO::Q;
    __shared__ Smem ss;

    const int b = a.resident > 0 && a.B > a.resident && a.B <= kOrderChunks * kWave && a.temperature != nullptr
        ? long_rows_first(a, static_cast<int>(blockIdx.x)) : static_cast<int>(blockIdx.x);
    const int V = a.V;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);  // wave-uniform
    const void* row = static_cast<const S*>(a.logits) + static_cast<int64_t>(b) * a.row_stride;
    const int n_tiles = (V + IO::TILE - 1) / IO::TILE;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    // The first tile is requested before anything waits on memory: its
    // address does not depend on the row's parameters, whose (scalar) loads
    // then overlap it.  Rows the re-reading path takes leave it unused.
    uint4 raw[IO::U], nxt[IO::U];
    int t = wid;
    if (aligned && t < n_tiles) IO::load(row, V, t, lane, raw);
    const RowParams prm = row_params(a.temperature, a.top_k, a.top_p, a.min_p, b, V);
    // The Philox word is wave-uniform scalar work (ten 64-bit multiply rounds);
    // only wave 0 uses it, so only wave 0 pays for it on the CU's scalar unit.
    uint64_t word = 0;
    if (wid == 0 && a.uid) word = request_word(a.seed, ld_global<int64_t>(a.uid + b), a.step);
    if (threadIdx.x == 0) {
        ss.word = word;                     // for the other waves, after the next barrier
        ss.minp = prm.min_p;
    }
    const double u = uniform24(word);       // valid in wave 0

    // min_p alone is a value cut on the same candidates as top-p: such rows
    // run as top-p rows (with p = 1)
    int mode;
    if (prm.greedy || prm.k == 1) mode = kArgmax;
    else if (prm.k < V) mode = kTopK;
    else if (prm.top_p || prm.min_p > 0.0f) mode = kTopP;
    else mode = kFull;
    // rows one read cannot serve go straight to the re-reading path
    bool use_row = !aligned || (mode != kArgmax && n_tiles > kMaxTiles);
    const bool want_tiles = !use_row && mode == kFull;    // per-tile softmax sums
    const bool want_lanez = !use_row && mode == kTopP;    // per-lane softmax sums
    const bool want_cand = !use_row && (mode == kTopK || mode == kTopP);
    const double c = 1.4426950408889634 / static_cast<double>(prm.T);

    // ------------------------------------------------------------ stream --
    float best_x = -INFINITY;
    int best_t = -1, best_q = 0;
    float theta = INFINITY;
    const float c32 = static_cast<float>(c);
    uint32_t cnt = 0;                 // this wave's region fill (wave-uniform)
    // Staged loads (wave-uniform count): load j of wave w in region slots
    // w*kRegion + kRegion - 2(j+1) and +1, the index of its first element in
    // cw[w*kRegion + j] (cw is unused until the stream ends).
    const bool stage = want_cand && (mode == kTopP || prm.k <= kStageMaxK);
    uint32_t nv = 0;
    bool stage_ovf = false;
    uint32_t* const stage_meta = reinterpret_cast<uint32_t*>(ss.cw) + wid * kRegion;
    auto stage_vec = [&](uint32_t j) -> uint4* {
        return reinterpret_cast<uint4*>(&ss.cent[wid * kRegion + kRegion - 2 * static_cast<int>(j) - 2]);
    };

    float lref = -INFINITY;           // top-p rows: this lane's running reference
    double lsum = 0.0;                // ... and its exponent sum relative to it
    // Each exponent is one fma, x * c32 - lrc with lrc = lref * c32 rounded;
    // that is (x - lref) * c32 + lrd, lrd = lref * c32 - lrc exactly, so the
    // sum carries a factor 2^lrd that is taken out in fp64.
    float lrc = INFINITY, lrd = 0.0f;
    // The candidate histogram is built by each wave right after its own
    // stream, before the row maximum is known: bins over [theta, m0] (m0 =
    // the largest value of the first tiles; keys above it land in the top
    // bin), top-p weights relative to m0.
    bool pre = false;
    uint32_t pre_lo = 0, pre_sh = 0;
    float m0 = -INFINITY;
    // Flat top-p rows build the weight histogram while they stream (relative
    // to m0, the weights the lane sums add), and collect no candidates.
    // (bf16 rows only: the fp32 kernel has no registers to spare for it)
    constexpr bool kFlatStream = DT == kDtypeBF16;
    bool flatp = false;               // block-uniform
    bool flat_bad = false;            // this lane raised its reference
    double* const fhist = reinterpret_cast<double*>(ss.cent);
    double* const fhl = fhist + (lane & (kHistCopies - 1));
    static_assert(sizeof(double) * kBins * kHistCopies <= sizeof(ss.cent), "histogram copies fit");
    auto wbin = [](float w) -> int {
        const int q = static_cast<int>(__float_as_uint(w) >> 19) - kWBinBase;
        return q < 0 ? 0 : (q > kBins - 1 ? kBins - 1 : q);
    };

    auto process = [&](const uint4* raw, int t) {
        // the maximum of each 16-byte load, then of the tile
        float lm[IO::U];
#pragma unroll
        for (int uu = 0; uu < IO::U; ++uu) {
            lm[uu] = IO::get(raw, uu * IO::VEC);
#pragma unroll
            for (int e = 1; e < IO::VEC; ++e) lm[uu] = fmaxf(lm[uu], IO::get(raw, uu * IO::VEC + e));
        }
        float tmax = lm[0];
#pragma unroll
        for (int uu = 1; uu < IO::U; ++uu) tmax = fmaxf(tmax, lm[uu]);
        if (tmax > best_x) {
            // the position inside the tile only matters to argmax rows
            if (mode == kArgmax) {
                int qq = Q - 1;
#pragma unroll
                for (int q = Q - 1; q >= 0; --q) qq = IO::get(raw, q) == tmax ? q : qq;
                best_q = qq;
            }
            best_x = tmax;
            best_t = t;
        }
        if (want_tiles) {
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
        if (want_lanez) {
            // the same argument per lane, against a reference that starts at
            // m0 (the first tiles' maximum) and is raised (the sum rescaled)
            // only when a value exceeds it by more than 2^30 in weight, so the
            // fp32 tile sums stay finite; accumulated in fp64
            // (a lane whose values so far are all padding (-inf) has no
            // reference yet; its lrc of +inf makes them add exactly 0)
            if (tmax > lref && (tmax - lref) * c32 > 30.0f) {
                if constexpr (kFlatStream) flat_bad = true;
                const float nrc = tmax * c32;
                const float nrd = fmaf(tmax, c32, -nrc);
                if (lsum > 0.0)
                    lsum *= exp2_neg((static_cast<double>(lref) - static_cast<double>(tmax)) * c
                                     - static_cast<double>(lrd) + static_cast<double>(nrd));
                lref = tmax;
                lrc = nrc;
                lrd = nrd;
            }
            float s = 0.0f;
            if (kFlatStream && flatp) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    // past the row's end the value is -inf: weight 0, bin 0
                    const float w = __builtin_amdgcn_exp2f(fmaf(IO::get(raw, q), c32, -lrc));
                    s += w;
                    atomicAdd(&fhl[wbin(w) * kHistCopies], static_cast<double>(w));
                }
            } else {
#pragma unroll
                for (int q = 0; q < Q; ++q) s += __builtin_amdgcn_exp2f(fmaf(IO::get(raw, q), c32, -lrc));
            }
            lsum += static_cast<double>(s);
        }
        if (stage && __ballot(tmax >= theta) != 0) {
            // a lane's load that holds a value >= theta is kept whole, in
            // (load, lane) order, which is token order
            const uint32_t vbase = IO::index(t, lane, 0);
#pragma unroll
            for (int uu = 0; uu < IO::U; ++uu) {
                const bool has = lm[uu] >= theta;
                const uint64_t bm = __ballot(has);
                if (bm == 0ull) continue;
                const uint32_t j = nv + lane_rank(bm);
                if (has && j < static_cast<uint32_t>(kStageCap)) {
                    *stage_vec(j) = raw[uu];
                    stage_meta[j] = vbase + static_cast<uint32_t>(uu * kWave * IO::VEC);
                }
                nv += static_cast<uint32_t>(__popcll(bm));
            }
        } else if (want_cand && __ballot(tmax >= theta) != 0) {
            // Slots in token order: the tile's index order is (load u, lane,
            // element), so each load needs its own prefix over the lanes.  The
            // per-load counts travel packed in one DPP scan (8-bit fields for
            // four loads: an exclusive prefix is at most 63 * 4; 16-bit fields
            // for two).  The values are stored as raw bits; the tail turns
            // them into order keys.
            constexpr int FB = 32 / IO::U;
            constexpr uint32_t FM = (1u << FB) - 1u;
            uint32_t packed = 0;
#pragma unroll
            for (int uu = 0; uu < IO::U; ++uu) {
                uint32_t cu = 0;
#pragma unroll
                for (int e = 0; e < IO::VEC; ++e) cu += IO::get(raw, uu * IO::VEC + e) >= theta ? 1u : 0u;
                packed |= cu << (FB * uu);
            }
            const uint32_t ex = wave_scan_u32_dpp(packed) - packed;
            const uint32_t ex_last = readlane_u32(ex, kWave - 1);
            const uint32_t pk_last = readlane_u32(packed, kWave - 1);
            uint32_t total = 0;
#pragma unroll
            for (int uu = 0; uu < IO::U; ++uu)
                total += ((ex_last >> (FB * uu)) & FM) + ((pk_last >> (FB * uu)) & FM);
            if (cnt + total <= static_cast<uint32_t>(kRegion)) {
                const uint32_t lanebase = IO::index(t, lane, 0);
                const uint32_t discard = (static_cast<uint32_t>(kCap) + threadIdx.x) * static_cast<uint32_t>(sizeof(uint2));
                uint32_t base = static_cast<uint32_t>(wid * kRegion) + cnt;
#pragma unroll
                for (int uu = 0; uu < IO::U; ++uu) {
                    // a load without candidates in any lane is skipped; otherwise
                    // every lane stores each element, non-candidates to its own
                    // discard slot, so the stores need no branches
                    const uint32_t cu_all = ((ex_last >> (FB * uu)) & FM) + ((pk_last >> (FB * uu)) & FM);
                    if (cu_all == 0u) continue;
                    uint32_t pos = (base + ((ex >> (FB * uu)) & FM)) * static_cast<uint32_t>(sizeof(uint2));
#pragma unroll
                    for (int e = 0; e < IO::VEC; ++e) {
                        const float x = IO::get(raw, uu * IO::VEC + e);
                        const bool is = x >= theta;
                        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(ss.cent) + (is ? pos : discard)) =
                            make_uint2(__float_as_uint(x), lanebase + uu * kWave * IO::VEC + e);
                        pos += is ? static_cast<uint32_t>(sizeof(uint2)) : 0u;
                    }
                    base += cu_all;
                }
                if (lane == 0) {
                    ss.tstart[t] = static_cast<uint16_t>(wid * kRegion + static_cast<int>(cnt));
                    ss.tcnt[t] = static_cast<uint16_t>(total);
                }
            }
            cnt += total;
        }
    };

    // One tile ahead.  Every row asks for its second tile only once the first
    // has arrived: with the whole grid's first requests half as large, the
    // first tiles come in sooner (the theta selection of candidate rows waits
    // for the first tiles of all waves), and the second tiles stream in while
    // the first are processed.
    if (threadIdx.x == 0) {
        ss.mbest = 0ull;
        ss.mtotal = 0u;
        ss.movf = 0u;
        ss.list_n = 0u;
        ss.next_tile = 2 * kWaves;
        ss.flat_bad = 0u;
    }
    if (want_cand) {
        if (threadIdx.x < kMaxTiles) {
            ss.tacc[threadIdx.x] = 0.0;
            ss.tcnt[threadIdx.x] = 0;
        }
        if (threadIdx.x < kList) {
            ss.rankp[threadIdx.x] = 0u;
            ss.ranki[threadIdx.x] = 0u;
        }
        // theta: lower edge of the histogram bin holding the j-th largest of
        // the per-thread maxima of the first tiles
        float lmax = -INFINITY;
        if (t < n_tiles) {
#pragma unroll
            for (int q = 0; q < Q; ++q) lmax = fmaxf(lmax, IO::get(raw, q));
        }
        // (the empty asm keeps the load below after the wait for the first tile)
        asm volatile("" :: "v"(lmax) : "memory");
        if (t + kWaves < n_tiles) IO::load(row, V, t + kWaves, lane, nxt);
        const uint32_t key = lmax > -INFINITY ? f32_key(lmax) : 0u;
        const int first_elems = V < kWaves * IO::TILE ? V : kWaves * IO::TILE;
        uint32_t j;
        if (mode == kTopK) {
            // j = k makes the top-k set always fit (j maxima are j distinct
            // logits >= theta); a large k would then keep far more candidates
            // than the regions hold, so j stops at about kTopKCands expected
            // candidates (the k-th largest is then almost always above theta;
            // when not, the row is finished from the row itself)
            const long long jcap = (static_cast<long long>(kTopKCands) * first_elems + V - 1) / V;
            const long long jc = jcap < 64 ? 64 : (jcap > kBlock ? kBlock : jcap);
            j = static_cast<uint32_t>(prm.k < jc ? prm.k : jc);
        } else {
            const long long want = (static_cast<long long>(kTopPTarget) * first_elems + V - 1) / V;
            j = static_cast<uint32_t>(want < 64 ? 64 : (want > kBlock ? kBlock : want));
        }
        const uint32_t kmax = wave_max_u32_dpp(key);
        const uint32_t kmin_neg = wave_max_u32_dpp(key ? 0xffffffffu - key : 0u);
        const uint32_t nval = static_cast<uint32_t>(__popcll(__ballot(key != 0u)));
        // all bins start empty; the rounds below leave them empty again
        ss.hcnt[threadIdx.x] = 0u;
        ss.hmass[threadIdx.x] = 0.0;
        if (lane == 0) {
            ss.wbest[wid] = kmax;
            ss.wu[wid] = kmin_neg;
            ss.wcount[wid] = nval;
        }
        lds_barrier();
        uint32_t hi = 0, lo_neg = 0, nv = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            hi = max(hi, static_cast<uint32_t>(ss.wbest[w]));
            lo_neg = max(lo_neg, ss.wu[w]);
            nv += ss.wcount[w];
        }
        const uint32_t lo = 0xffffffffu - lo_neg;
        if (nv >= j) {
            // a bin holding many more maxima than needed (a wide key range, e.g.
            // one negative lane maximum) is histogrammed again over its own range
            uint32_t tlo = lo, thi = hi, jr = j, tkey = lo;
            for (int round = 0; round < 3; ++round) {
                const int sh = range_shift(thi - tlo);
                if (key != 0u && key >= tlo && key <= thi) atomicAdd(&ss.hcnt[(key - tlo) >> sh], 1u);
                lds_barrier();
                if (wid == 0) {
                    uint32_t above = 0;
                    const int d = w0_desc_count(ss.hcnt, jr, &above);
                    const uint32_t dd = static_cast<uint32_t>(d < 0 ? 0 : d);
                    const uint32_t cd = ss.hcnt[dd];
#pragma unroll
                    for (int i = 0; i < 4; ++i) ss.hcnt[4 * lane + i] = 0u;
                    if (lane == 0) {
                        const uint32_t blo_t = tlo + (dd << sh);
                        ss.bu[0] = blo_t;
                        ss.bu[1] = bin_hi(blo_t, sh, thi);
                        ss.bu[2] = jr - above;
                        ss.bu[3] = (round < 2 && sh > 0 && above + cd > 2u * jr) ? 1u : 0u;
                    }
                }
                lds_barrier();
                tkey = ss.bu[0];
                if (ss.bu[3] == 0u) break;
                tlo = ss.bu[0];
                thi = ss.bu[1];
                jr = ss.bu[2];
            }
            theta = key_f32(tkey);
            pre = hi >= tkey;
            pre_lo = tkey;
            pre_sh = static_cast<uint32_t>(range_shift_bins(hi - tkey));
            m0 = key_f32(hi);
            lref = m0;
            lrc = m0 * c32;
            lrd = fmaf(m0, c32, -lrc);
            if (kFlatStream && mode == kTopP && !(prm.min_p > 0.0f) && aligned && (m0 - theta) * c32 <= kFlatGap) {
                // Is the row flat?  The first tiles' weight at or above theta
                // against their total (weights relative to m0, all <= 1).
                float zt = 0.0f, st = 0.0f;
                if (t < n_tiles) {
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        const float x = IO::get(raw, q);
                        const float w = __builtin_amdgcn_exp2f(fmaf(x, c32, -lrc));
                        zt += w;
                        st += x >= theta ? w : 0.0f;
                    }
                }
                const double zw = wave_sum_dpp(static_cast<double>(zt));
                const double sw = wave_sum_dpp(static_cast<double>(st));
                if (lane == 0) {
                    ss.tsum[wid] = zw;
                    ss.tsum[kWaves + wid] = sw;
                }
                lds_barrier();
                double z1 = 0.0, s1 = 0.0;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    z1 += ss.tsum[w];
                    s1 += ss.tsum[kWaves + w];
                }
                if (s1 < kFlatFrac * static_cast<double>(prm.p) * z1) {
                    flatp = true;
                    pre = false;
                    theta = INFINITY;          // no candidates
#pragma unroll
                    for (int cc = 0; cc < kHistCopies; ++cc) fhist[threadIdx.x * kHistCopies + cc] = 0.0;
                    lds_barrier();
                }
            }
        } else {
            theta = -INFINITY;
        }
    } else {
        lds_barrier();      // the merge slots above are set before any wave's merge
        if (!use_row) {
            // the second tile only once the first has arrived, as for
            // candidate rows: a smaller first burst of requests from the
            // whole grid brings every row's first tiles in sooner
            float x0 = -INFINITY;
            if (t < n_tiles) {
#pragma unroll
                for (int q = 0; q < Q; ++q) x0 = fmaxf(x0, IO::get(raw, q));
            }
            asm volatile("" :: "v"(x0) : "memory");
            if (t + kWaves < n_tiles) IO::load(row, V, t + kWaves, lane, nxt);
        }
    }
    if (!use_row) {
        // A wave's first two tiles are t and t + 16; after that each wave
        // claims the next unread tile as it starts on one, so the waves that
        // run ahead read more tiles and all finish close together.  Each
        // wave's tiles still come in increasing order.
        if (t < n_tiles) process(raw, t);
        int tn = t + kWaves;          // the tile in nxt
        while (tn < n_tiles) {
            const int tc = tn;
#pragma unroll
            for (int v = 0; v < IO::U; ++v) raw[v] = nxt[v];
            uint32_t cl = 0;
            if (lane == 0) cl = atomicAdd(&ss.next_tile, 1u);
            tn = __builtin_amdgcn_readfirstlane(static_cast<int>(cl));
            if (tn < n_tiles) IO::load(row, V, tn, lane, nxt);
            process(raw, tc);
        }
    } else {
        // the re-reading path needs the maximum first
        for (int i = threadIdx.x; i < V; i += kBlock) {
            const float x = Elem<DT>::at(row, i);
            if (x > best_x) { best_x = x; best_t = i; }
        }
        best_q = -1;
    }

    if (stage && !use_row) {
        // Expand the staged loads into entries: every value >= theta as
        // (value bits, index), in staging order (tiles in the order the wave
        // read them, token order inside a tile), with each tile's first slot
        // and count.  The loads are counted first, so that entries written
        // from the region's start never reach staged loads (at its end) that
        // are still to be read; a wave whose entries and staged loads would
        // not both fit marks the row as overflowing.
        constexpr int kTS = __builtin_ctz(IO::TILE);
        const int rbase = wid * kRegion;
        const uint32_t N = nv;
        bool ovf = N > static_cast<uint32_t>(kStageCap);
        uint32_t total = 0;
        if (!ovf) {
            for (uint32_t j0 = 0; j0 < N; j0 += kWave) {
                const uint32_t j = j0 + static_cast<uint32_t>(lane);
                uint32_t ce = 0;
                if (j < N) {
                    const uint4 v = *stage_vec(j);
#pragma unroll
                    for (int e = 0; e < IO::VEC; ++e) ce += IO::get(&v, e) >= theta ? 1u : 0u;
                }
                total += readlane_u32(wave_scan_u32_dpp(ce), kWave - 1);
            }
            ovf = total + 2u * N > static_cast<uint32_t>(kRegion);
        }
        if (ovf) {
            stage_ovf = true;
            cnt = 0;
        } else {
            uint32_t pos0 = 0;
            for (uint32_t j0 = 0; j0 < N; j0 += kWave) {
                const uint32_t j = j0 + static_cast<uint32_t>(lane);
                const bool in = j < N;
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                uint32_t meta = 0, ce = 0;
                if (in) {
                    v = *stage_vec(j);
                    meta = stage_meta[j];
#pragma unroll
                    for (int e = 0; e < IO::VEC; ++e) ce += IO::get(&v, e) >= theta ? 1u : 0u;
                }
                const uint32_t incl = wave_scan_u32_dpp(ce);
                const uint32_t pstart = pos0 + incl - ce;
                const uint32_t tl = meta >> kTS;
                const bool first = in && (j == 0u || (stage_meta[j - 1] >> kTS) != tl);
                const bool last = in && (j + 1u == N || (stage_meta[j + 1] >> kTS) != tl);
                uint32_t pw = pstart;
#pragma unroll
                for (int e = 0; e < IO::VEC; ++e) {
                    const float x = IO::get(&v, e);
                    if (in && x >= theta) {
                        ss.cent[rbase + static_cast<int>(pw)] = make_uint2(__float_as_uint(x), meta + static_cast<uint32_t>(e));
                        ++pw;
                    }
                }
                if (first) ss.tstart[tl] = static_cast<uint16_t>(rbase + static_cast<int>(pstart));
                wave_lds_sync();
                if (last) ss.tcnt[tl] = static_cast<uint16_t>(rbase + static_cast<int>(pw) - static_cast<int>(ss.tstart[tl]));
                pos0 += readlane_u32(incl, kWave - 1);
            }
            cnt = pos0;
        }
    }

    // ------------------------------- this wave's share of the candidate tail --
    // top-p: the lane sums relative to m0; every candidate row: order keys and
    // the count histogram of this wave's region, top-p rows also weights
    // relative to m0 and the mass histogram
    const double m0c = static_cast<double>(m0) * c;
    if (want_lanez && (pre || flatp)) {
        const double part = lsum > 0.0
            ? lsum * exp2_neg((static_cast<double>(lref) - static_cast<double>(m0)) * c - static_cast<double>(lrd)) : 0.0;
        const double ws = wave_sum_dpp(part);
        if (lane == 0) ss.wd[wid] = ws;
    }
    if (pre) {
        const int rbase = wid * kRegion;
        const uint32_t n = cnt < static_cast<uint32_t>(kRegion) ? cnt : static_cast<uint32_t>(kRegion);
        for (uint32_t i = lane; i < n; i += kWave) {
            const int sl = rbase + static_cast<int>(i);
            const float x = __uint_as_float(ss.cent[sl].x);
            const uint32_t key = f32_key(x);
            ss.cent[sl].x = key;
            const uint32_t d0 = (key - pre_lo) >> pre_sh;
            const uint32_t d = d0 < static_cast<uint32_t>(kBins - 1) ? d0 : static_cast<uint32_t>(kBins - 1);
            atomicAdd(&ss.hcnt[d], 1u);
            if (want_lanez) {
                const float w = static_cast<float>(fast_weight(x, m0c, c));
                ss.cw[sl] = w;
                atomicAdd(&ss.hmass[d], static_cast<double>(w));
            }
        }
    }

    // --------------------------------------------- row maximum and argmax --
    {
        uint64_t pk = 0;
        if (best_t >= 0) {
            const uint32_t idx = best_q >= 0 ? IO::index(best_t, lane, best_q) : static_cast<uint32_t>(best_t);
            pk = (static_cast<uint64_t>(f32_key(best_x)) << 32) | static_cast<uint64_t>(0xffffffffu - idx);
        }
        pk = wave_max_u64_dpp(pk);
        if (lane == 0) {
            atomicMax(reinterpret_cast<unsigned long long*>(&ss.mbest), static_cast<unsigned long long>(pk));
            atomicAdd(&ss.mtotal, cnt < static_cast<uint32_t>(kRegion) ? cnt : static_cast<uint32_t>(kRegion));
            if (cnt > static_cast<uint32_t>(kRegion) || stage_ovf) atomicOr(&ss.movf, 1u);
        }
        if constexpr (kFlatStream) {
            if (flatp && __ballot(flat_bad) != 0ull && lane == 0) atomicOr(&ss.flat_bad, 1u);
        }
    }
    __syncthreads();
    const uint64_t best = ss.mbest;
    const uint32_t n_total = ss.mtotal;
    const bool overflow = ss.movf != 0u;
    const float m = key_f32(static_cast<uint32_t>(best >> 32));
    const uint32_t amax = 0xffffffffu - static_cast<uint32_t>(best);
    // top-p rows keep m0 as the weight reference while every weight relative
    // to it stays far below the float range; otherwise the row maximum
    const bool pre_ok = (pre || flatp) && (mode != kTopP ||
                                          (static_cast<double>(m) - static_cast<double>(m0)) * c <= 64.0);
    // a flat row's histogram is complete unless some lane had to raise its
    // reference (weights relative to m0 no longer fit)
    const bool flat_ok = flatp && pre_ok && ss.flat_bad == 0u;
    const double mc = mode == kTopP && pre_ok ? m0c : static_cast<double>(m) * c;
    // min_p keeps p_i >= min_p * p_max, that is x >= m + T ln(min_p): the
    // threshold in fp64, as the order key of the smallest float at or above
    // it, kept in LDS (0: no min_p) and read where it is used
    const bool has_min = mode != kArgmax && ss.minp > 0.0f;
    if (has_min) {
        if (threadIdx.x == 0) {
            const double xm = static_cast<double>(m) + log2(static_cast<double>(ss.minp)) / c;
            const float xf = static_cast<float>(xm);
            ss.kmin = f32_key(xf) + (static_cast<double>(xf) < xm ? 1u : 0u);
        }
        __syncthreads();
    }
    auto kmin_now = [&]() -> uint32_t { return *reinterpret_cast<volatile uint32_t*>(&ss.kmin); };
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
                const uint2 en = ss.cent[rbase + i];
                if (en.y >= ilo && en.y <= ihi) f(en.x, en.y, static_cast<int>(rbase + i));
            }
        } else {
            const uint32_t hi = ihi < static_cast<uint32_t>(V - 1) ? ihi : static_cast<uint32_t>(V - 1);
            for (uint32_t i = ilo + threadIdx.x; i <= hi; i += kBlock)
                f(f32_key(Elem<DT>::at(row, i)), i, -1);
        }
    };
    // Weights of entries read from the row: one fma and one fp32 exp2,
    // 2^(x*c32 - Pf) with Pf = mref*c32 rounded, times G = 2^-(mref*c32 - Pf)
    // (the rounding, exact through fma) in fp64: the weight relative to the
    // reference mref (mc = mref*c) with c rounded to fp32; fp64 sums.
    const float mref = mode == kTopP && pre_ok ? m0 : m;
    const float Pf = mref * c32;
    const double G = exp2_neg(-static_cast<double>(fmaf(mref, c32, -Pf)));
    auto weight_of = [&](uint32_t k, int slot) -> double {
        return slot >= 0 ? static_cast<double>(ss.cw[slot])
                         : static_cast<double>(__builtin_amdgcn_exp2f(fmaf(key_f32(k), c32, -Pf))) * G;
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
    // entry whose inclusive prefix mass reaches `target`; also the kept
    // weight and count.  false if the entries' mass never reaches it.
    auto mass_cut = [&](const Cut& ct, double target, Cut* out, double* w_out, uint32_t* n_out) -> bool {
        auto pred = [&](uint32_t k, uint32_t i) { return ct.keep(i, k); };
        uint32_t lo, hi;
        key_range(ct, &lo, &hi);
        double above = 0.0;
        uint32_t above_n = 0;
        for (;;) {
            const int sh = range_shift(hi - lo);
            histogram(pred, false, lo, hi, sh, true);
            if (wid == 0) {
                double ab = 0.0;
                const int d = w0_desc_mass(ss.hcnt, ss.hmass, above, target, &ab);
                uint32_t ac = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) ac += 4 * lane + i > d ? ss.hcnt[4 * lane + i] : 0u;
                ac = readlane_u32(wave_scan_u32_dpp(ac), kWave - 1);
                if (lane == 0) {
                    ss.bu[2] = static_cast<uint32_t>(d);
                    ss.bu[4] = d >= 0 ? ss.hcnt[d] : 0u;
                    ss.bu[7] = ac;
                    ss.bd[1] = ab;
                }
            }
            __syncthreads();
            const int d = static_cast<int>(ss.bu[2]);
            const uint32_t cd = ss.bu[4];
            const double ab = ss.bd[1];
            if (d < 0) return false;
            above = ab;
            above_n += ss.bu[7];
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
                    const double we = readlane_f64(incl, e);
                    if (lane == 0) {
                        ss.bu[5] = ss.skey[e];
                        ss.bu[6] = ss.sidx[e];
                        ss.bu[3] = static_cast<uint32_t>(e) + 1u;
                        ss.bd[2] = we;
                    }
                }
                __syncthreads();
                *out = Cut{ss.bu[5], ss.bu[6]};
                *w_out = ss.bd[2];
                *n_out = above_n + ss.bu[3];
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
                *w_out = above + static_cast<double>(keep) * w;
                *n_out = above_n + keep;
                return true;
            }
            lo = nlo;
            hi = nhi;
        }
    };

    // ------------------- rows without top-k or top-p: draw from tile sums --
    if (want_tiles) {
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
    // top-p rows without the m0 reference: the per-lane sums rescaled to the
    // row maximum (read after the next barrier)
    if (want_lanez && !pre_ok) {
        const double part = lsum > 0.0
            ? lsum * exp2_neg((static_cast<double>(lref) - static_cast<double>(m)) * c - static_cast<double>(lrd)) : 0.0;
        const double ws = wave_sum_dpp(part);
        if (lane == 0) ss.wd[wid] = ws;
    }

    Cut cut{0u, 0xffffffffu};
    uint32_t n_kept = 0, token = 0;
    double W = 0.0;
    bool fast = false;
    bool cand_weights = false;    // the draw summed the candidates' fp32 weights

    // ------------------------------------------------------ candidate tail --
    // Passes over the candidates in the wave regions; after each pass wave 0
    // reads what the pass left (a 1024-bin key histogram, a list of at most
    // kList entries, per-tile counts or weights) and picks the next pass.
    //   top-k: the bin holding the k-th entry; a bin that is kept whole ends
    //     the search, a small bin is listed and ranked exactly, a bin of one
    //     key (a run of ties) is resolved in token order by per-tile counts,
    //     a larger bin is histogrammed again over its own key range;
    //   top-p: the same descent by weight, inside the top-k cut;
    //   the draw: per-tile kept weight, a scan over the tiles, then a scan of
    //     the one tile's entries in slot order, which is token order.
    if (want_cand && !flatp) {
        if (overflow || (mode == kTopK && n_total < static_cast<uint32_t>(prm.k))) {
            use_row = true;
        } else {
            constexpr int kTileShift = __builtin_ctz(IO::TILE);
            const uint32_t key_hi = f32_key(m);
            // wave-0 state (the other waves keep unused copies)
            int phase = mode == kTopK ? 0 : 1;      // 0 top-k, 1 top-p, 2 the draw
            bool first_p = mode == kTopP;
            uint32_t lo = f32_key(theta), hi = key_hi;
            uint32_t sh = static_cast<uint32_t>(range_shift_bins(hi - lo));
            uint32_t r = static_cast<uint32_t>(prm.k);
            uint32_t above_c = 0, nk = 0, tie = 0, tie_r = 0;
            double above_m = 0.0, wk = 0.0;
            double target = 0.0;
            Cut rc{0u, 0xffffffffu}, res{0u, 0xffffffffu};

            auto mk = [&](uint32_t type) {
                PassDesc x;
                x.type = type; x.lo = lo; x.hi = hi; x.sh = sh;
                x.rkey = rc.key; x.rlast = rc.last; x.tie = tie; x.pad = 0u;
                return x;
            };
            auto tie_weight = [&](uint32_t k) {
                return static_cast<double>(static_cast<float>(fast_weight(key_f32(k), mc, c)));
            };

            auto run_pass = [&](const PassDesc& pd) {
                const int rbase = wid * kRegion;
                const uint32_t n = cnt < static_cast<uint32_t>(kRegion) ? cnt : static_cast<uint32_t>(kRegion);
                const Cut rcut{pd.rkey, pd.rlast};
                for (uint32_t i = lane; i < n; i += kWave) {
                    const int sl = rbase + static_cast<int>(i);
                    if (pd.type == kPassHistW || pd.type == kPassHistC) {
                        // the stream stored raw value bits: turn them into order keys
                        const float x = __uint_as_float(ss.cent[sl].x);
                        const uint32_t key = f32_key(x);
                        ss.cent[sl].x = key;
                        const uint32_t d = (key - pd.lo) >> pd.sh;
                        atomicAdd(&ss.hcnt[d], 1u);
                        if (pd.type == kPassHistW) {
                            const float w = static_cast<float>(fast_weight(x, mc, c));
                            ss.cw[sl] = w;
                            atomicAdd(&ss.hmass[d], static_cast<double>(w));
                        }
                        continue;
                    }
                    if (pd.type == kPassWeights) {
                        ss.cw[sl] = static_cast<float>(fast_weight(key_f32(ss.cent[sl].x), mc, c));
                        continue;
                    }
                    const uint32_t key = ss.cent[sl].x;
                    if (pd.type == kPassHist || pd.type == kPassGather) {
                        if (key < pd.lo || key > pd.hi) continue;
                    } else if (pd.type == kPassTieCount) {
                        if (key != pd.tie) continue;
                    }
                    const uint32_t idx = ss.cent[sl].y;
                    if (!rcut.keep(idx, key)) continue;
                    if (pd.type == kPassHist) {
                        const uint32_t d = (key - pd.lo) >> pd.sh;
                        atomicAdd(&ss.hcnt[d], 1u);
                        atomicAdd(&ss.hmass[d], static_cast<double>(ss.cw[sl]));
                    } else if (pd.type == kPassGather) {
                        const uint32_t p = atomicAdd(&ss.list_n, 1u);
                        if (p < static_cast<uint32_t>(kList)) {
                            ss.lkey[p] = key;
                            ss.lidx[p] = idx;
                            ss.lw[p] = ss.cw[sl];
                        }
                    } else if (pd.type == kPassTieCount) {
                        atomicAdd(&ss.tacc[idx >> kTileShift], 1.0);
                    } else {
                        atomicAdd(&ss.tacc[idx >> kTileShift], static_cast<double>(ss.cw[sl]));
                    }
                }
            };

            // wave 0: the entry selected by per-tile counts (the want-th, 1-based,
            // in token order) or weights (first whose prefix exceeds want * total)
            auto tile_select = [&](bool by_mass, double want, double* total_out) -> uint32_t {
                double* tl = ss.tacc + lane * kTilesPerLane;   // zero past n_tiles
                double v[kTilesPerLane];
                double sl = 0.0;
#pragma unroll
                for (int i = 0; i < kTilesPerLane; ++i) {
                    v[i] = tl[i];
                    sl += v[i];
                }
#pragma unroll
                for (int i = 0; i < kTilesPerLane; ++i) tl[i] = 0.0;
                const double incl = wave_scan_f64_dpp(sl);
                const double total = readlane_f64(incl, kWave - 1);
                const double tgt = by_mass ? want * total : want;
                *total_out = total;
                const uint64_t hb = __ballot(sl > 0.0 && (by_mass ? incl > tgt : incl >= tgt));
                const uint64_t nzb = __ballot(sl > 0.0);
                if (!nzb) return 0u;
                const int owner = hb ? __ffsll(static_cast<unsigned long long>(hb)) - 1
                                     : 63 - __clzll(static_cast<long long>(nzb));
                int ts = -1, last_nz = -1;
                double rem = 0.0;
                if (lane == owner) {
                    double cum = incl - sl;
#pragma unroll
                    for (int i = 0; i < kTilesPerLane; ++i) {
                        if (ts < 0 && v[i] > 0.0) {
                            last_nz = lane * kTilesPerLane + i;
                            if (hb && (by_mass ? cum + v[i] > tgt : cum + v[i] >= tgt)) {
                                ts = last_nz;
                                rem = tgt - cum;
                            } else {
                                cum += v[i];
                            }
                        }
                    }
                    if (ts < 0) {            // rounding: take the last entry
                        ts = last_nz;
                        rem = INFINITY;
                    }
                }
                ts = static_cast<int>(readlane_u32(static_cast<uint32_t>(ts), owner));
                rem = readlane_f64(rem, owner);
                const int sb = ss.tstart[ts];
                const int n = ss.tcnt[ts];
                const Cut rcut = rc;
                double run = 0.0;
                uint32_t found = 0xffffffffu, last = 0xffffffffu;
                for (int j0 = 0; j0 < n; j0 += kWave) {
                    const int j = j0 + lane;
                    bool pr = false;
                    double val = 0.0;
                    uint32_t idx = 0;
                    if (j < n) {
                        const uint2 en = ss.cent[sb + j];
                        const uint32_t k2 = en.x;
                        idx = en.y;
                        pr = rcut.keep(idx, k2) && (by_mass || k2 == tie);
                        val = pr ? (by_mass ? static_cast<double>(ss.cw[sb + j]) : 1.0) : 0.0;
                    }
                    const double in2 = wave_scan_f64_dpp(val);
                    const uint64_t hit = __ballot(val > 0.0 && (by_mass ? run + in2 > rem : run + in2 >= rem));
                    const uint64_t pb = __ballot(val > 0.0);
                    if (pb) last = readlane_u32(idx, 63 - __clzll(static_cast<long long>(pb)));
                    if (hit) {
                        found = readlane_u32(idx, __ffsll(static_cast<unsigned long long>(hit)) - 1);
                        break;
                    }
                    run += readlane_f64(in2, kWave - 1);
                }
                return found != 0xffffffffu ? found : last;
            };

            auto enter_next = [&]() -> PassDesc {
                if (phase == 0 && prm.top_p) {
                    // top-p inside the top-k cut, against its weight
                    phase = 1;
                    rc = res;
                    target = static_cast<double>(prm.p) * wk;
                    lo = res.key;
                    hi = key_hi;
                    sh = static_cast<uint32_t>(range_shift_bins(hi - lo));
                    above_c = 0;
                    above_m = 0.0;
                    return mk(kPassHist);
                }
                phase = 2;
                rc = res;
                return mk(kPassTileMass);
            };

            auto step = [&](uint32_t done_type) -> PassDesc {
                if (first_p) {
                    // the softmax normaliser of a top-p row
                    const double z = wave_sum_dpp(lane < kWaves ? ss.wd[lane] : 0.0);
                    target = static_cast<double>(prm.p) * z;
                }
                if (done_type == kPassHistW || done_type == kPassHist) {
                    const BinPick bp = phase == 0 ? w0_pick_count(ss.hcnt, ss.hmass, r)
                                                  : w0_pick_mass(ss.hcnt, ss.hmass, above_m, target);
                    if (bp.d < 0 || (first_p && !bp.reached)) return mk(kPassFallback);
                    first_p = false;
                    above_c += bp.above_c;
                    if (phase == 0) {
                        above_m += bp.above_m;
                        r -= bp.above_c;
                    } else {
                        above_m = bp.above_m;
                    }
                    const uint32_t blo = lo + (static_cast<uint32_t>(bp.d) << sh);
                    const uint32_t bhi = bin_hi(blo, static_cast<int>(sh), hi);
                    if (phase == 0 && r == bp.cnt) {        // the bin is kept whole
                        res = Cut{blo, 0xffffffffu};
                        wk = above_m + bp.mass;
                        nk = above_c + bp.cnt;
                        return enter_next();
                    }
                    lo = blo;
                    hi = bhi;
                    if (bp.cnt <= static_cast<uint32_t>(kList)) return mk(kPassGather);
                    if (blo == bhi) {                       // a run of equal keys
                        tie = blo;
                        if (phase == 0) {
                            tie_r = r;
                            return mk(kPassTieCount);
                        }
                        // each weighs w: the j-th (token order) has exclusive prefix above + (j-1) w
                        const double w = tie_weight(blo);
                        uint32_t keep = bp.cnt;
                        if (bp.reached) {
                            const double y = (target - above_m) / w;
                            if (y < static_cast<double>(bp.cnt)) {
                                const double cy = ceil(y);
                                keep = cy < 1.0 ? 1u : static_cast<uint32_t>(cy);
                            }
                        }
                        if (keep == bp.cnt) {
                            res = rc.key == blo ? rc : Cut{blo, 0xffffffffu};
                            nk = above_c + bp.cnt;
                            return enter_next();
                        }
                        tie_r = keep;
                        return mk(kPassTieCount);
                    }
                    sh = static_cast<uint32_t>(range_shift_bins(hi - lo));
                    return mk(kPassHist);
                }
                if (done_type == kPassGather) {
                    const int n = ss.list_n < static_cast<uint32_t>(kList) ? static_cast<int>(ss.list_n) : kList;
                    if (lane < n) {
                        const uint32_t k = ss.lkey[lane], i = ss.lidx[lane];
                        int rr = 0;
                        for (int e = 0; e < n; ++e) {
                            const uint32_t k2 = ss.lkey[e], i2 = ss.lidx[e];
                            rr += (k2 > k || (k2 == k && i2 < i)) ? 1 : 0;
                        }
                        ss.skey[rr] = k;
                        ss.sidx[rr] = i;
                        ss.sw[rr] = ss.lw[lane];
                    }
                    wave_lds_sync();
                    if (lane == 0) ss.list_n = 0u;
                    const bool in = lane < n;
                    const uint32_t kk = in ? ss.skey[lane] : 0u, ii = in ? ss.sidx[lane] : 0u;
                    const double w = in ? static_cast<double>(ss.sw[lane]) : 0.0;
                    const double incl = wave_scan_f64_dpp(w);
                    int e;
                    if (phase == 0) {
                        e = static_cast<int>(r) - 1;
                        wk = above_m + readlane_f64(incl, e);
                    } else {
                        const uint64_t bal = __ballot(in && above_m + incl >= target);
                        e = bal ? __ffsll(static_cast<unsigned long long>(bal)) - 1 : n - 1;
                    }
                    res = Cut{readlane_u32(kk, e), readlane_u32(ii, e)};
                    nk = above_c + static_cast<uint32_t>(e) + 1u;
                    return enter_next();
                }
                if (done_type == kPassTieCount) {
                    double unused;
                    const uint32_t idx = tile_select(false, static_cast<double>(tie_r), &unused);
                    res = Cut{tie, idx};
                    if (phase == 0) wk = above_m + static_cast<double>(tie_r) * tie_weight(tie);
                    nk = above_c + tie_r;
                    return enter_next();
                }
                // the draw
                double total = 0.0;
                const uint32_t tok = tile_select(true, u, &total);
                if (lane == 0) {
                    ss.res_token = tok;
                    ss.res_kept = nk;
                    ss.res_w = total;
                }
                return mk(kPassDone);
            };

            // ------------------------------------------------ block-parallel routes --
            // The common cases finish with block-wide steps whose serial parts are
            // short: a single wave executes about one dependent instruction per
            // 10-15 cycles here, so long wave-0 sequences are what the tail costs.
            //   S (top-k <= 64, top-p optional): pick the bin of the k-th entry,
            //     list every entry at or above that bin (<= 64), rank the list in
            //     descending and in token order at once; cut, top-p and the draw
            //     are then scans over the list in wave 0.  A top-p row whose
            //     whole nucleus bin and the bins above it hold <= 64 entries
            //     takes this route too.
            //   P (top-p without top-k): pick the bin where the descending weight
            //     reaches p * Z; list that bin while adding the weight of the
            //     bins above it per tile; rank the list, cut, add the kept part;
            //     then wave 0 draws from the per-tile weights.
            // Anything else (a boundary bin of more than kList entries, top-k
            // above kList with top-p) goes to the pass-driven descent below.
            const int sh_tile = kTileShift;
            auto block_pick = [&](bool by_mass, uint32_t r, double tgt) -> BlockPick {
                const int d = wid * kWave + (kWave - 1 - lane);   // lane 0: the wave's top bin
                const uint32_t cb = ss.hcnt[d];
                const double mb = by_mass ? ss.hmass[d] : 0.0;
                const uint32_t sc = wave_scan_u32_dpp(cb);
                const double sm = by_mass ? wave_scan_f64_dpp(mb) : 0.0;
                if (lane == kWave - 1) {
                    ss.wtc[wid] = sc;
                    if (by_mass) ss.wtm[wid] = sm;
                }
                __syncthreads();
                // every wave scans the 16 wave totals the same way (lane l holds
                // wave 15 - l, from the top bins down), so all agree on the wave
                // that holds the pick
                const int wl = kWaves - 1 - lane;
                const uint32_t tc = lane < kWaves ? ss.wtc[wl] : 0u;
                const double tm = by_mass && lane < kWaves ? ss.wtm[wl] : 0.0;
                const uint32_t tci = wave_scan_u32_dpp(tc);
                const double tmi = by_mass ? wave_scan_f64_dpp(tm) : 0.0;
                const uint64_t wb = __ballot(lane < kWaves && tc != 0u && (by_mass ? tmi >= tgt : tci >= r));
                int cross = wb ? kWaves - 1 - (__ffsll(static_cast<unsigned long long>(wb)) - 1) : -1;
                if (cross < 0 && by_mass) {
                    // rounding at the very end: the lowest non-empty wave if the
                    // total reaches the target
                    const uint64_t nzw = __ballot(lane < kWaves && tc != 0u);
                    const double tot = readlane_f64(tmi, kWaves - 1);
                    if (nzw && tot >= tgt) cross = kWaves - 1 - (63 - __clzll(static_cast<long long>(nzw)));
                }
                const uint32_t acw = readlane_u32(tci - tc, kWaves - 1 - wid);
                const double amw = by_mass ? readlane_f64(tmi - tm, kWaves - 1 - wid) : 0.0;
                if (wid == cross) {
                    const bool hit = cb != 0u && (by_mass ? amw + sm >= tgt : acw + sc >= r);
                    uint64_t bal = __ballot(hit);
                    if (bal == 0ull) {      // rounding: the wave's lowest non-empty bin
                        const uint64_t nz = __ballot(cb != 0u);
                        bal = nz ? (1ull << (63 - __clzll(static_cast<long long>(nz)))) : 0ull;
                    }
                    if (lane == __ffsll(static_cast<unsigned long long>(bal)) - 1) {
                        ss.pick.d = d;
                        ss.pick.cnt = cb;
                        ss.pick.above_c = acw + sc - cb;
                        ss.pick.mass = mb;
                        ss.pick.above_m = amw + (sm - mb);
                    }
                }
                if (cross < 0 && threadIdx.x == 0) ss.pick.d = -1;
                __syncthreads();
                return ss.pick;
            };
            // list the entries with key in [glo, ghi]; entries with key > tabove
            // add their weight to their tile
            auto gather_pass = [&](uint32_t glo, uint32_t ghi, uint32_t tabove) {
                const int rbase = wid * kRegion;
                const uint32_t n = cnt < static_cast<uint32_t>(kRegion) ? cnt : static_cast<uint32_t>(kRegion);
                for (uint32_t i = lane; i < n; i += kWave) {
                    const int sl = rbase + static_cast<int>(i);
                    const uint2 en = ss.cent[sl];
                    if (en.x >= glo && en.x <= ghi) {
                        const uint32_t p = atomicAdd(&ss.list_n, 1u);
                        if (p < static_cast<uint32_t>(kList)) {
                            ss.lkey[p] = en.x;
                            ss.lidx[p] = en.y;
                            ss.lw[p] = static_cast<float>(fast_weight(key_f32(en.x), mc, c));
                        }
                    } else if (en.x > tabove) {
                        atomicAdd(&ss.tacc[en.y >> sh_tile], static_cast<double>(ss.cw[sl]));
                    }
                }
                __syncthreads();
            };
            // ranks of the listed entries: wave w compares every entry with
            // entries 4w .. 4w+3
            auto block_rank = [&]() {
                const int n = ss.list_n < static_cast<uint32_t>(kList) ? static_cast<int>(ss.list_n) : kList;
                if (lane < n && kWave / kWaves * wid < n) {
                    const uint32_t k0 = ss.lkey[lane], i0 = ss.lidx[lane];
                    uint32_t rp = 0, ri = 0;
                    const int j1 = kList / kWaves * (wid + 1) < n ? kList / kWaves * (wid + 1) : n;
                    for (int j = kList / kWaves * wid; j < j1; ++j) {
                        const uint32_t k2 = ss.lkey[j], i2 = ss.lidx[j];
                        rp += (k2 > k0 || (k2 == k0 && i2 < i0)) ? 1u : 0u;
                        ri += i2 < i0 ? 1u : 0u;
                    }
                    if (rp) atomicAdd(&ss.rankp[lane], rp);
                    if (ri) atomicAdd(&ss.ranki[lane], ri);
                }
                __syncthreads();
            };
            // wave 0: place the ranked list (descending order into skey/sidx/sw,
            // token order into xrp/xw/xidx) and clear the ranks and the list
            auto w0_place = [&](int n) {
                if (lane < n) {
                    const uint32_t rp = ss.rankp[lane], ri = ss.ranki[lane];
                    const uint32_t k0 = ss.lkey[lane], i0 = ss.lidx[lane];
                    const float w0 = ss.lw[lane];
                    ss.skey[rp] = k0;
                    ss.sidx[rp] = i0;
                    ss.sw[rp] = w0;
                    ss.xrp[ri] = rp;
                    ss.xw[ri] = w0;
                    ss.xidx[ri] = i0;
                    ss.rankp[lane] = 0u;
                    ss.ranki[lane] = 0u;
                }
                if (lane == 0) ss.list_n = 0u;
                wave_lds_sync();
            };
            // wave 0: the draw from the per-tile kept weights, with W the kept
            // mass the cut found: a scan over the tiles (64 at a time) finds
            // the first tile whose prefix exceeds u * W, then a scan of that
            // tile's entries kept by ct, in slot (token) order, the token
            auto w0_tile_draw = [&](const Cut& ct, double W) {
                const double tgt = u * W;
                double run = 0.0, rem = INFINITY;
                int ts = -1, last_t = -1;
                for (int c0 = 0; c0 < n_tiles; c0 += kWave) {
                    const int ti = c0 + lane;
                    const double v = ti < n_tiles ? ss.tacc[ti] : 0.0;
                    const double incl = wave_scan_f64_dpp(v);
                    const uint64_t nz = __ballot(v > 0.0);
                    if (nz) last_t = c0 + 63 - __clzll(static_cast<long long>(nz));
                    const uint64_t hb = __ballot(v > 0.0 && run + incl > tgt);
                    if (hb) {
                        const int lx = __ffsll(static_cast<unsigned long long>(hb)) - 1;
                        ts = c0 + lx;
                        rem = tgt - (run + readlane_f64(incl - v, lx));
                        break;
                    }
                    run += readlane_f64(incl, kWave - 1);
                }
                if (ts < 0) ts = last_t;        // rounding: u * W at or past the total
                uint32_t found = 0xffffffffu, last = 0xffffffffu;
                if (ts >= 0) {
                    const int sb = ss.tstart[ts];
                    const int n = ss.tcnt[ts];
                    double run2 = 0.0;
                    for (int j0 = 0; j0 < n; j0 += kWave) {
                        const int j = j0 + lane;
                        double val = 0.0;
                        uint32_t idx = 0;
                        if (j < n) {
                            const uint2 en = ss.cent[sb + j];
                            idx = en.y;
                            val = ct.keep(en.y, en.x) ? static_cast<double>(ss.cw[sb + j]) : 0.0;
                        }
                        const double in2 = wave_scan_f64_dpp(val);
                        const uint64_t hit = __ballot(val > 0.0 && run2 + in2 > rem);
                        const uint64_t pb = __ballot(val > 0.0);
                        if (pb) last = readlane_u32(idx, 63 - __clzll(static_cast<long long>(pb)));
                        if (hit) {
                            found = readlane_u32(idx, __ffsll(static_cast<unsigned long long>(hit)) - 1);
                            break;
                        }
                        run2 += readlane_f64(in2, kWave - 1);
                    }
                }
                if (lane == 0) {
                    ss.res_token = found != 0xffffffffu ? found : (last != 0xffffffffu ? last : amax);
                    ss.res_w = W;
                }
            };

            // The histogram the routes pick from: the one each wave built after
            // its stream (bins of width 2^pre_sh from theta, the top bin reaching
            // up to m), else one built now over [theta, m].  Top-k rows only
            // count; their weights are computed where they are needed.
            const bool small_k = mode == kTopK && prm.k <= kList;
            uint32_t hsh = pre_sh;
            bool top_ext = true;
            if (!pre_ok) {
                ss.hcnt[threadIdx.x] = 0u;
                ss.hmass[threadIdx.x] = 0.0;
                __syncthreads();
                if (pre) {
                    // keys are in place: weights relative to m, then the histogram
                    if (mode == kTopP) run_pass(mk(kPassWeights));
                    run_pass(mk(kPassHist));
                } else {
                    run_pass(mk(mode == kTopP ? kPassHistW : kPassHistC));
                }
                __syncthreads();
                hsh = sh;
                top_ext = false;
            }
            int route = 0;           // 0 general, 1 S, 2 P, 3 finish from the row, 4 min_p list
            double ptgt = 0.0;       // top-p rows: p * Z
            BlockPick bp{};
            // the softmax normaliser of a top-p row (same value wherever it is used)
            auto row_z = [&]() -> double {
                return wave_sum_dpp(lane < kWaves ? ss.wd[lane] : 0.0);
            };
            if (small_k) {
                bp = block_pick(false, static_cast<uint32_t>(prm.k), 0.0);
                if (bp.d >= 0 && bp.above_c + bp.cnt <= static_cast<uint32_t>(kList)) route = 1;
            } else if (mode == kTopP) {
                ptgt = static_cast<double>(prm.p) * row_z();
                bp = block_pick(true, 0u, ptgt);
                if (bp.d < 0) route = 3;
                else if (bp.above_c + bp.cnt <= static_cast<uint32_t>(kList)) route = 1;   // the whole nucleus listed
                else if (bp.cnt <= static_cast<uint32_t>(kList)) route = 2;
            }
            if (has_min && route != 1) {
                // min_p rows that the small list does not finish: when every
                // token min_p keeps is a candidate (and no top-p needs the
                // mass of a top-k above kList), list the tokens at or above its
                // threshold (route 4: route 1 over that list, if it holds at
                // most kList); otherwise finish from the row
                route = !small_k && kmin_now() >= lo && !(mode == kTopK && prm.top_p) ? 4 : 3;
            }
            const uint32_t key_lo0 = lo;
            const uint32_t blo = key_lo0 + (bp.d >= 0 ? static_cast<uint32_t>(bp.d) << hsh : 0u);
            const uint32_t bhi = top_ext && bp.d == kBins - 1 ? key_hi : bin_hi(blo, static_cast<int>(hsh), key_hi);
            if (route == 1 || route == 4) {
                gather_pass(route == 4 ? kmin_now() : blo, key_hi, 0xffffffffu);
            }
            if (route == 4 && ss.list_n > static_cast<uint32_t>(kList)) {
                // more than kList tokens at or above the min_p threshold: the
                // row path finishes the row
                __syncthreads();
                if (threadIdx.x == 0) ss.list_n = 0u;
                __syncthreads();
                route = 3;
            }
            if (route == 1 || route == 4) {
                block_rank();
                if (wid == 0) {
                    const int n = static_cast<int>(ss.list_n);
                    w0_place(n);
                    const bool in = lane < n;
                    const double w = in ? static_cast<double>(ss.sw[lane]) : 0.0;
                    const double incl = wave_scan_f64_dpp(w);
                    // top-k: the first k, then top-p inside them; top-p alone: the
                    // list holds every entry at or above the bin where the
                    // descending weight reaches p * Z
                    const int k = mode == kTopK && prm.k < n ? prm.k : n;
                    int e = k - 1;
                    if (prm.top_p) {
                        const double target_p = mode == kTopK
                            ? static_cast<double>(prm.p) * readlane_f64(incl, k - 1) : ptgt;
                        const uint64_t bal = __ballot(lane < k && incl >= target_p);
                        if (bal) e = __ffsll(static_cast<unsigned long long>(bal)) - 1;
                    }
                    if (has_min) {
                        // min_p's prefix: the listed entries at or above kmin
                        const int em = __popcll(__ballot(in && ss.skey[lane] >= kmin_now())) - 1;
                        e = em < e ? em : e;
                    }
                    const uint32_t ck = readlane_u32(in ? ss.skey[lane] : 0u, e);
                    const uint32_t cl = readlane_u32(in ? ss.sidx[lane] : 0u, e);
                    // the draw over the kept entries in token order
                    const double xv = in && ss.xrp[lane] <= static_cast<uint32_t>(e) ? static_cast<double>(ss.xw[lane]) : 0.0;
                    const double xin = wave_scan_f64_dpp(xv);
                    const double tot = readlane_f64(xin, kWave - 1);
                    const double tg = u * tot;
                    const uint64_t hit = __ballot(xv > 0.0 && xin > tg);
                    const uint64_t nzb = __ballot(xv > 0.0);
                    const int tl = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1
                                       : (nzb ? 63 - __clzll(static_cast<long long>(nzb)) : 0);
                    const uint32_t tok = readlane_u32(in ? ss.xidx[lane] : 0u, tl);
                    if (lane == 0) {
                        ss.res_token = tok;
                        ss.res_kept = static_cast<uint32_t>(e + 1);
                        ss.res_w = tot;
                        ss.cut_key = ck;
                        ss.cut_last = cl;
                    }
                }
                __syncthreads();
            } else if (route == 2) {
                gather_pass(blo, bhi, bhi);
                block_rank();
                if (wid == 0) {
                    const int n = static_cast<int>(ss.list_n);
                    w0_place(n);
                    const bool in = lane < n;
                    const double w = in ? static_cast<double>(ss.sw[lane]) : 0.0;
                    const double incl = wave_scan_f64_dpp(w);
                    const double target_p = ptgt;
                    const uint64_t bal = __ballot(in && bp.above_m + incl >= target_p);
                    const int e = bal ? __ffsll(static_cast<unsigned long long>(bal)) - 1 : n - 1;
                    if (in && lane <= e)
                        atomicAdd(&ss.tacc[ss.sidx[lane] >> sh_tile], static_cast<double>(ss.sw[lane]));
                    const uint32_t ck = readlane_u32(in ? ss.skey[lane] : 0u, e);
                    const uint32_t cl = readlane_u32(in ? ss.sidx[lane] : 0u, e);
                    if (lane == 0) {
                        ss.res_kept = bp.above_c + static_cast<uint32_t>(e) + 1u;
                        ss.cut_key = ck;
                        ss.cut_last = cl;
                    }
                    wave_lds_sync();        // this wave's weights are in the tile sums
                    w0_tile_draw(Cut{ck, cl}, bp.above_m + readlane_f64(incl, e));
                }
                __syncthreads();
            }
            if (route == 1 || route == 2 || route == 4) {
                fast = true;
                cand_weights = true;
                cut = Cut{ss.cut_key, ss.cut_last};
                token = ss.res_token;
                n_kept = ss.res_kept;
                W = ss.res_w;
            } else if (route == 3) {
                use_row = true;
            } else {
            // ------------------------------------------- pass-driven descent --
            // keys are in place (and weights, unless only counted so far):
            // start from a fresh histogram
            if (mode == kTopK) run_pass(mk(kPassWeights));
            ss.hcnt[threadIdx.x] = 0u;
            ss.hmass[threadIdx.x] = 0.0;
            __syncthreads();
            PassDesc pd = mk(kPassHist);
            for (;;) {
                run_pass(pd);
                __syncthreads();
                if (wid == 0) {
                    const PassDesc nx = step(pd.type);
                    if (lane == 0) ss.pass = nx;
                }
                __syncthreads();
                pd = ss.pass;
                if (pd.type == kPassDone || pd.type == kPassFallback) break;
            }
            if (pd.type == kPassDone) {
                fast = true;
                cand_weights = true;
                cut = Cut{pd.rkey, pd.rlast};
                token = ss.res_token;
                n_kept = ss.res_kept;
                W = ss.res_w;
            } else {
                use_row = true;
            }
            }
        }
    }

    // ------------------------------------------- flat top-p rows (row reads) --
    // The nucleus reaches below theta.  Two passes over the row in the stream's
    // tile layout: (A) a 1024-bin histogram of weight by depth below the
    // reference (1/16 octave per bin, the heaviest bin last), from which wave 0
    // picks the bin where the descending weight reaches p * Z; (B) per-tile
    // weight of the bins above it (each tile summed by its own wave) and the
    // entries of that bin gathered into the LDS regions.  The cut inside the
    // bin is then the mass descent over LDS entries, and the draw scans the
    // per-tile kept weights and reads the chosen tile once more.
    if (!fast && mode == kTopP && want_lanez && aligned && !has_min) {
        constexpr int kTS = __builtin_ctz(IO::TILE);
        __syncthreads();                       // every wave's share of Z is in ss.wd
        double z = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) z += ss.wd[w];
        const double ztgt = static_cast<double>(prm.p) * z;
        // The weight of a value relative to the reference, 2^(x*c32 - Pf) (times
        // G in fp64), and its bin: the weight's fp32 exponent and top four
        // mantissa bits, so 16 bins per octave from 2^-64 up (higher bin =
        // heavier); lighter weights and zero fall into bin 0, weights from
        // about 0.97 up into the top bin.  Bin edges are bit patterns of the
        // weight, so the second pass classifies a value with integer compares.
        // pass A's histogram: kHistCopies adjacent copies of each bin, lane l
        // adding to copy l mod kHistCopies (so lanes of a wave seldom meet on one
        // address), kept in the candidate regions, which pass B refills (fp64:
        // LDS fp32 atomic adds run an order of magnitude slower here)
        double* const hist = fhist;
        if (!flat_ok) {
#pragma unroll
            for (int c = 0; c < kHistCopies; ++c) hist[threadIdx.x * kHistCopies + c] = 0.0;
        }
        if (threadIdx.x == 0) { ss.movf = 0u; ss.mtotal = 0u; ss.next_tile = kWaves; }
        __syncthreads();
        // (A), unless the stream built the histogram
        if (!flat_ok) {
            double* const hl = hist + (lane & (kHistCopies - 1));
            uint4 ra[IO::U], rb[IO::U];
            int tt = wid;
            if (tt < n_tiles) IO::load(row, V, tt, lane, ra);
            for (; tt < n_tiles; tt += kWaves) {
#pragma unroll
                for (int v = 0; v < IO::U; ++v) rb[v] = ra[v];
                if (tt + kWaves < n_tiles) IO::load(row, V, tt + kWaves, lane, ra);
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    // past the row's end the value is -inf: weight 0, bin 0
                    const float w = __builtin_amdgcn_exp2f(fmaf(IO::get(rb, q), c32, -Pf));
                    atomicAdd(&hl[wbin(w) * kHistCopies], static_cast<double>(w));
                }
            }
        }
        __syncthreads();
        {
            double hs = 0.0;
#pragma unroll
            for (int c2 = 0; c2 < kHistCopies; ++c2) hs += hist[threadIdx.x * kHistCopies + c2];
            ss.hmass[threadIdx.x] = hs;
        }
        __syncthreads();
        if (wid == 0) {
            // a bin is non-empty iff it holds weight: every bin above the
            // deepest one has y > -64, so its entries weigh at least 2^-64; the
            // deepest bin's entries may weigh nothing and can never be kept
            // by a top-p cut (p < 1), so none is lost
#pragma unroll
            for (int i = 0; i < kBinsPerLane; ++i)
                ss.hcnt[kBinsPerLane * lane + i] = ss.hmass[kBinsPerLane * lane + i] > 0.0 ? 1u : 0u;
            const BinPick bq = w0_pick_mass(ss.hcnt, ss.hmass, 0.0, ztgt / G);
            if (lane == 0) ss.bu[2] = static_cast<uint32_t>(bq.d < 0 ? 0 : bq.d);
        }
        __syncthreads();
        const int dpick = static_cast<int>(ss.bu[2]);
        // bit patterns of the weights in bin dpick: [wlo, whi) (zero weights,
        // which no cut with p < 1 keeps, never count as inside)
        const uint32_t wlo = dpick == 0 ? 1u : static_cast<uint32_t>(dpick + kWBinBase) << 19;
        const uint32_t whi = dpick == kBins - 1 ? 0xffffffffu : static_cast<uint32_t>(dpick + 1 + kWBinBase) << 19;
        // (B)
        {
            uint4 ra[IO::U], rb[IO::U];
            uint32_t fill = 0, nabove = 0;
            const uint32_t rbeg = static_cast<uint32_t>(wid * kRegion);
            // a wave's first tile is its index; after that it claims the next
            // unread tile as it starts on one, as in the stream, so that the
            // waves finish close together
            int tn = wid;
            if (tn < n_tiles) IO::load(row, V, tn, lane, ra);
            while (tn < n_tiles) {
                const int tt = tn;
#pragma unroll
                for (int v = 0; v < IO::U; ++v) rb[v] = ra[v];
                uint32_t cl = 0;
                if (lane == 0) cl = atomicAdd(&ss.next_tile, 1u);
                tn = __builtin_amdgcn_readfirstlane(static_cast<int>(cl));
                if (tn < n_tiles) IO::load(row, V, tn, lane, ra);
                // the lane's weights above the bin: at most Q of them, summed
                // in fp32 (relative error below Q * 2^-24), then in fp64; its
                // entries inside the bin as a bit mask, stored after one scan
                // of the lanes' counts
                float part = 0.0f;
                float wq[Q];
                uint32_t inm = 0u;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float w = __builtin_amdgcn_exp2f(fmaf(IO::get(rb, q), c32, -Pf));
                    wq[q] = w;
                    const uint32_t wb = __float_as_uint(w);
                    const bool up = wb >= whi;
                    part += up ? w : 0.0f;
                    nabove += up ? 1u : 0u;
                    inm |= (wb >= wlo && wb < whi ? 1u : 0u) << q;
                }
                const uint32_t ln = static_cast<uint32_t>(__popc(inm));
                const uint32_t incl = wave_scan_u32_dpp(ln);
                const uint32_t tot = readlane_u32(incl, kWave - 1);
                if (tot != 0u) {
                    uint32_t pos = fill + incl - ln;
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        if ((inm >> q) & 1u) {
                            if (pos < static_cast<uint32_t>(kRegion)) {
                                ss.cent[rbeg + pos] = make_uint2(f32_key(IO::get(rb, q)), IO::index(tt, lane, q));
                                ss.cw[rbeg + pos] = static_cast<float>(static_cast<double>(wq[q]) * G);
                            }
                            ++pos;
                        }
                    }
                    fill += tot;
                }
                const double ts = wave_sum_dpp(static_cast<double>(part));
                if (lane == 0) ss.tacc[tt] = ts * G;
            }
            nabove = readlane_u32(wave_scan_u32_dpp(nabove), kWave - 1);
            if (lane == 0) {
                if (fill > static_cast<uint32_t>(kRegion)) atomicOr(&ss.movf, 1u);
                atomicAdd(&ss.mtotal, nabove);
            }
            cnt = fill;
        }
        __syncthreads();
        if (ss.movf == 0u) {
            // the weight above the bin (per tile, owner-summed) and its count
            if (wid == 0) {
                double a = 0.0;
                for (int i = lane; i < n_tiles; i += kWave) a += ss.tacc[i];
                a = wave_sum_dpp(a);
                if (lane == 0) ss.bd[1] = a;
            }
            __syncthreads();
            const double above = ss.bd[1];
            const uint32_t nabove = ss.mtotal;
            from_row = false;
            Cut pc{0u, 0xffffffffu};
            double wb = 0.0;
            uint32_t nb = 0;
            // the target must fall inside the bin pass A picked; a target that
            // rounding of the two passes' sums puts on the other side of a bin
            // edge leaves the row to the row path
            if (ztgt > above && mass_cut(Cut{0u, 0xffffffffu}, ztgt - above, &pc, &wb, &nb)) {
                cut = pc;
                W = above + wb;
                n_kept = nabove + nb;
                // the kept entries of the bin add their weight to their tile
                each(0u, 0xffffffffu, [&](uint32_t k, uint32_t i, int slot) {
                    if (cut.keep(i, k)) atomicAdd(&ss.tacc[i >> kTS], static_cast<double>(ss.cw[slot]));
                });
                __syncthreads();
                if (wid == 0) {
                    // the tile holding u * W (lane l: tiles l*per ..), then that tile again
                    const int per = (n_tiles + kWave - 1) / kWave;
                    const int tlo = lane * per, thi = tlo + per < n_tiles ? tlo + per : n_tiles;
                    double psum = 0.0;
                    for (int i = tlo; i < thi; ++i) psum += ss.tacc[i];
                    const double incl = wave_scan_f64_dpp(psum);
                    const double tot = readlane_f64(incl, kWave - 1);
                    const double target = u * tot;
                    const uint64_t bal = __ballot(psum > 0.0 && incl > target);
                    const uint64_t nz = __ballot(psum > 0.0);
                    const int owner = bal ? __ffsll(static_cast<unsigned long long>(bal)) - 1
                                          : (nz ? 63 - __clzll(static_cast<long long>(nz)) : 0);
                    int ts = tlo;
                    double rem = INFINITY;
                    if (lane == owner) {
                        double cum = incl - psum;
                        int found = -1, last_nz = tlo;
                        for (int i = tlo; i < thi; ++i) {
                            const double v = ss.tacc[i];
                            if (v > 0.0) last_nz = i;
                            if (found < 0 && v > 0.0 && cum + v > target) { found = i; rem = target - cum; }
                            if (found < 0) cum += v;
                        }
                        ts = found >= 0 ? found : last_nz;
                        if (found < 0) rem = INFINITY;
                    }
                    ts = static_cast<int>(readlane_u32(static_cast<uint32_t>(ts), owner));
                    rem = readlane_f64(rem, owner);
                    uint4 rr[IO::U];
                    IO::load(row, V, ts, lane, rr);
                    double run = 0.0;
                    int tok = -1, last_pos = -1;
    #pragma unroll
                    for (int uu = 0; uu < IO::U; ++uu) {
                        double wv[IO::VEC];
                        double ps = 0.0;
                        int my_last = -1;
    #pragma unroll
                        for (int e = 0; e < IO::VEC; ++e) {
                            const float x = IO::get(rr, uu * IO::VEC + e);
                            const uint32_t idx = IO::index(ts, lane, uu * IO::VEC + e);
                            const bool kp = idx < static_cast<uint32_t>(V) && cut.keep(idx, f32_key(x));
                            wv[e] = kp ? static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, c32, -Pf))) * G : 0.0;
                            ps += wv[e];
                            if (wv[e] > 0.0) my_last = static_cast<int>(idx);
                        }
                        const double pin = wave_scan_f64_dpp(ps);
                        const double tsum = readlane_f64(pin, kWave - 1);
                        const uint64_t lastb = __ballot(my_last >= 0);
                        if (lastb)
                            last_pos = static_cast<int>(readlane_u32(static_cast<uint32_t>(my_last),
                                                                     63 - __clzll(static_cast<long long>(lastb))));
                        if (tok < 0 && run + tsum > rem) {
                            const uint64_t ob = __ballot(ps > 0.0 && run + pin > rem);
                            if (ob) {
                                const int own = __ffsll(static_cast<unsigned long long>(ob)) - 1;
                                int mine = -1;
                                bool done_l = false;
                                double cum = run + (pin - ps);
    #pragma unroll
                                for (int e = 0; e < IO::VEC; ++e) {
                                    cum += wv[e];
                                    if (!done_l && wv[e] > 0.0) mine = static_cast<int>(IO::index(ts, lane, uu * IO::VEC + e));
                                    if (wv[e] > 0.0 && cum > rem) done_l = true;
                                }
                                tok = static_cast<int>(readlane_u32(static_cast<uint32_t>(mine), own));
                            }
                        }
                        run += tsum;
                    }
                    if (tok < 0) tok = last_pos;
                    if (lane == 0) ss.bu[7] = static_cast<uint32_t>(tok);
                }
                __syncthreads();
                token = ss.bu[7];
                fast = true;
            }
        }
    }

    if (!fast) {
        // ---------------------------- the row itself: top-k, then top-p --
        from_row = true;
        if (mode == kTopK) cut = select_desc(cut, static_cast<uint32_t>(prm.k));
        bool have_w = false;
        if (prm.top_p) {
            // top-p alone: the normaliser is the stream's (its lane sums, same
            // reference); after a top-k cut, the kept weight
            double wk = 0.0;
            if (mode == kTopP && want_lanez) {
                __syncthreads();        // every wave's share is in ss.wd
#pragma unroll
                for (int w = 0; w < kWaves; ++w) wk += ss.wd[w];
            } else {
                wk = sum_cut(cut, nullptr);
            }
            Cut pc;
            if (mass_cut(cut, static_cast<double>(prm.p) * wk, &pc, &W, &n_kept)) {
                cut = pc;
                have_w = true;
            }
        }
        // min_p's kept set is a prefix too, so the intersection is the shorter
        // prefix: it binds when the cut so far keeps keys below its threshold
        if (has_min && cut.key < kmin_now()) {
            cut = Cut{kmin_now(), 0xffffffffu};
            have_w = false;
        }

        // ---- the draw: first index (token order) whose kept prefix exceeds u*W --
        if (!have_w) W = sum_cut(cut, &n_kept);
        double tgt = u * W;
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
        // each kept token's weight as the draw summed it (over the same W):
        // the candidate routes' fp32 weights, or the row reads' fp32 exp2
        // times G
        float* probs = a.probs_out + static_cast<int64_t>(b) * V;
        for (int i = threadIdx.x; i < V; i += kBlock) {
            const float x = Elem<DT>::at(row, i);
            const double wt = cand_weights
                ? static_cast<double>(static_cast<float>(fast_weight(x, mc, c)))
                : static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, c32, -Pf))) * G;
            probs[i] = cut.keep(static_cast<uint32_t>(i), f32_key(x)) ? static_cast<float>(wt / W) : 0.0f;
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
