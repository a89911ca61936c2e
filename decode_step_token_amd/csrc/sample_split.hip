// Split-row sampler: many workgroups per row, each holding one chunk of the
// row in registers; the row's last workgroup finishes the row.
//
// "The engine and the sampler", section "The sampler": temperature, top-k
// first, top-p on the renormalised survivors, one categorical draw (here an
// inverse CDF in token order with a keyed Philox uniform).  The kept set is
// always a prefix of the descending order (value descending, ties by index
// ascending), so it is held as a cut (key, index): token i with order key k
// is kept iff k > key, or k == key and i <= index.
//
// Layout.  A row of V logits is cut into S chunks of 256 threads x NL
// 16-byte loads (thread t's load j covers chunk elements j*256*VEC + t*VEC +
// [0, VEC)).  One 256-thread workgroup per chunk issues all of its loads at
// once and keeps the chunk in registers, so every pass over the chunk after
// the first is free of memory traffic and a CU keeps several chunks in flight.
// The rows are dealt to the 8 XCDs round robin and a row's chunks are
// consecutive workgroups of its XCD; the chunk dispatched last (S - 1)
// finishes the row.
//
// Every chunk publishes a record (chunk maximum and its lowest index, the
// sum of its softmax weights per 16-byte-load slot, a candidate threshold)
// and, for rows that select, every element at or above the threshold with its
// index, in token order; then an epoch flag.  Publication uses device-scope
// stores (written through the XCD's L2) and the flag follows only once the
// data stores have completed (s_waitcnt), so a reader that sees the flag
// with a device-scope load and then loads the data with device-scope loads
// reads the published values.  The publishing workgroups never wait; only
// the finisher polls the flags of its row, whose other chunks were
// dispatched before it on the same XCD and therefore run.  Its wait is
// bounded: past the limit it finishes the row by the exact routine, which
// reads the row itself.
//
// Candidate thresholds.  For a rank target J (k for top-k rows, about 192
// for top-p rows, 64 for the debug top-64), the chunk histograms its 16-byte
// group maxima by distance below the chunk maximum (1/16 logit per bin) and
// takes theta = the smallest group maximum in the bins that hold the J
// largest.  J group maxima are J distinct elements >= theta, so the chunk's
// J largest elements are all candidates; the union over the chunks holds
// every element of the row at or above kappa = the largest chunk threshold,
// which is at least the row's J largest.
//
// The finisher loads the candidates >= kappa into LDS (in token order) and
// finds cuts by descents over key histograms (by count for top-k, by mass
// for top-p), resolving the boundary bin exactly; it draws by a block-wide
// scan of the kept weights in token order.  Rows with no filter draw from
// the per-slot weight sums and re-read one 16-byte-load slot of one chunk.
// Whatever the candidates cannot settle (a nucleus reaching below kappa, a
// chunk with too many candidates, a top-k too large to aim at) is finished
// by the exact multi-pass routine over the whole row.
#include "device_common.hpp"
#include "exact_path.hpp"
#include "kernels.hpp"

namespace dst {

namespace {

constexpr int kT = kSplitThreads;
constexpr int kNW = kT / kWave;
constexpr int kBins = 1024;
constexpr int kListMax = 2048;        // candidates the finisher holds
constexpr int kKList = 128;           // top-k rows up to this k aim their thresholds at k
constexpr int kJTopP = 192;           // rank aimed at by top-p / min_p rows
constexpr int kJMax = 224;            // largest rank aimed at (a chunk publishes <= kSplitCap)
constexpr int kJDebug = 64;           // debug: the row's 64 largest
constexpr float kGroupBinScale = 16.0f;
constexpr int kSpinLimit = 1 << 16;
constexpr int kSmall = 64;

enum : uint32_t { kModeArgmax = 0, kModeTopK = 1, kModeTopP = 2, kModeFull = 3, kModeExact = 4 };

static_assert(kT == 256 && kNW == 4, "the block layout below assumes 4 waves");
static_assert(kListMax == 8 * kT, "eight list entries per thread");

struct ChunkSmem {
    uint32_t hist[kBins];
    double wsum[kNW][16];
    uint32_t wtot[kNW][16];
    uint32_t off[kNW][16];
    float fseg[16];
    float fred[kNW];
    uint64_t ured[kNW];
    uint32_t bsel;
    uint32_t total;
};

struct FinSmem {
    uint32_t key[kListMax];
    uint32_t idx[kListMax];
    float w[kListMax];
    uint32_t hcnt[kBins];
    double hmass[kBins];
    float cm[kSplitMaxChunks];
    uint32_t camax[kSplitMaxChunks];
    float ctheta[kSplitMaxChunks];
    uint32_t ccnt[kSplitMaxChunks];
    double cz[kSplitMaxChunks];
    float crc[kSplitMaxChunks];
    uint32_t coff[kSplitMaxChunks + 1];
    uint32_t skey[kSmall];
    uint32_t sidx[kSmall];
    float sw[kSmall];
    uint32_t sn;
    // block scan scratch
    uint32_t wc[kNW];
    double wm[kNW];
    // decisions broadcast to the block
    int sel_bin;
    uint32_t sel_c, sel_cnt;
    double sel_m;
    uint32_t res_ok, res_key, res_idx, res_n;
    int32_t tok;
    int32_t last;
    uint32_t list_n, kappa, maxkey, bad;
    double zrow;
    int cstar, jstar;
    double before;
    int next;
};

union SplitSmem {
    ChunkSmem c;
    FinSmem f;
    ExactSmem e;
};

// ------------------------------------------------------------- helpers --

template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev_f32(float* p, float v) {
    st_dev(reinterpret_cast<uint32_t*>(p), __float_as_uint(v));
}
__device__ __forceinline__ float ld_dev_f32(const float* p) {
    return __uint_as_float(ld_dev(reinterpret_cast<const uint32_t*>(p)));
}
__device__ __forceinline__ void st_dev_f64(double* p, double v) {
    st_dev(reinterpret_cast<uint64_t*>(p), static_cast<uint64_t>(__double_as_longlong(v)));
}
__device__ __forceinline__ double ld_dev_f64(const double* p) {
    return __longlong_as_double(static_cast<long long>(ld_dev(reinterpret_cast<const uint64_t*>(p))));
}

// Waits until every memory operation this thread issued has completed.
__device__ __forceinline__ void wait_all_memory() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __asm__ __volatile__("" ::: "memory");
}

__device__ __forceinline__ float wave_min_dpp(float v) {
    v = fminf(v, dpp_f32<kDppXor1>(v, v));
    v = fminf(v, dpp_f32<kDppXor2>(v, v));
    v = fminf(v, dpp_f32<kDppHalfMirror>(v, v));
    v = fminf(v, dpp_f32<kDppMirror>(v, v));
    v = fminf(v, dpp_f32<kDppBcast15, 0xa>(INFINITY, v));
    v = fminf(v, dpp_f32<kDppBcast31, 0xc>(INFINITY, v));
    return __uint_as_float(readlane_u32(__float_as_uint(v), 63));
}

// Makes the compiler treat the chunk registers as changed: values derived
// from them in one pass (unpacked bf16, keys) are recomputed in the next
// instead of being kept live across it.
template <int NL>
__device__ __forceinline__ void opaque(uint4 (&d)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) __asm__ __volatile__("" : "+v"(d[j].x), "+v"(d[j].y), "+v"(d[j].z), "+v"(d[j].w));
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return static_cast<int>(threadIdx.x) >> 6; }

// Exclusive scan in thread order of a (count, mass) pair over the block;
// totals through the last two arguments.
__device__ __forceinline__ void block_scan2(uint32_t c, double m, uint32_t* ec, double* em, uint32_t* tc,
                                            double* tm, FinSmem& f) {
    const uint32_t ic = wave_scan_u32_dpp(c);
    const double im = wave_scan_f64_dpp(m);
    __syncthreads();
    if (lane_id() == kWave - 1) {
        f.wc[wave_id()] = ic;
        f.wm[wave_id()] = im;
    }
    __syncthreads();
    uint32_t bc = 0, ac = 0;
    double bm = 0.0, am = 0.0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
        const uint32_t xc = f.wc[w];
        const double xm = f.wm[w];
        if (w < wave_id()) {
            bc += xc;
            bm += xm;
        }
        ac += xc;
        am += xm;
    }
    *ec = bc + ic - c;
    *em = bm + (im - m);
    *tc = ac;
    *tm = am;
    __syncthreads();
}

// ----------------------------------------------------------- the chunk --

template <int DT>
__device__ __forceinline__ float elem(const uint4& v, int e) {
    if (DT == kDtypeF32) {
        const uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
        return __uint_as_float(w);
    }
    const int q = e >> 1;
    const uint32_t w = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// One 16-byte load slot of thread t: elements [off, off + VEC) of the row,
// -inf past V (the row is 16-byte aligned; a partial slot is read by element).
template <int DT>
__device__ __forceinline__ uint4 load_slot(const char* rowp, int V, int64_t off) {
    constexpr int VEC = Elem<DT>::kVec;
    if (off + VEC <= V) {
        return ld_global_u4_stream(rowp + off * (DT == kDtypeF32 ? 4 : 2));
    }
    uint32_t w[4];
    if (DT == kDtypeF32) {
        const float* r32 = reinterpret_cast<const float*>(rowp);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = off + e < V ? __float_as_uint(ld_global<float>(r32 + off + e)) : 0xff800000u;
    } else {
        const uint16_t* r16 = reinterpret_cast<const uint16_t*>(rowp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = off + 2 * e < V ? ld_global<uint16_t>(r16 + off + 2 * e) : 0xff80u;
            const uint32_t hi = off + 2 * e + 1 < V ? ld_global<uint16_t>(r16 + off + 2 * e + 1) : 0xff80u;
            w[e] = lo | (hi << 16);
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DT, int NL>
struct Geo {
    static constexpr int VEC = Elem<DT>::kVec;
    static constexpr int SLOT = kT * VEC;                  // elements per load slot
    static constexpr int64_t ELEMS = static_cast<int64_t>(NL) * SLOT;
    static constexpr int ES = DT == kDtypeF32 ? 4 : 2;
};

__device__ __forceinline__ const char* row_ptr(const SampleArgs& a, int b, int es) {
    return static_cast<const char*>(a.logits) + static_cast<int64_t>(b) * a.row_stride * es;
}

// The chunk's part of the row: loads it, reduces it and publishes its record
// and candidates (see the file comment).  mode is the row's route, cc the
// fp32 log2(e)/T, jrank the candidate rank target (0: none).
template <int DT, int NL>
__device__ __forceinline__ void chunk_phase(const SampleArgs& a, ChunkSmem& sm, int b, int c, uint32_t mode,
                                            float cc, int jrank, int jmin) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    const int t = static_cast<int>(threadIdx.x), lane = lane_id(), wid = wave_id();
    const char* rowp = row_ptr(a, b, G::ES);
    const int64_t base = static_cast<int64_t>(c) * G::ELEMS;
    uint4 d[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) d[j] = load_slot<DT>(rowp, a.V, base + static_cast<int64_t>(j) * G::SLOT + t * VEC);

    SplitRec* rec = a.rec + static_cast<int64_t>(b) * a.rec_stride + c;

    if (mode == kModeArgmax) {
        // thread maximum, then the lowest index holding it: walk down, keep the last hit
        float tm = -INFINITY;
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) tm = fmaxf(tm, elem<DT>(d[j], e));
        opaque(d);
        uint32_t ti = 0xffffffffu;
#pragma unroll
        for (int j = NL - 1; j >= 0; --j) {
#pragma unroll
            for (int e = VEC - 1; e >= 0; --e) {
                const uint32_t i = static_cast<uint32_t>(base + j * G::SLOT + t * VEC + e);
                ti = elem<DT>(d[j], e) == tm ? i : ti;
            }
        }
        const uint64_t pk = (static_cast<uint64_t>(f32_key(tm)) << 32) | static_cast<uint64_t>(0xffffffffu - ti);
        const uint64_t wb = wave_max_u64_dpp(pk);
        if (lane == 0) sm.ured[wid] = wb;
        __syncthreads();
        if (t == 0) {
            uint64_t best = sm.ured[0];
#pragma unroll
            for (int w = 1; w < kNW; ++w) best = sm.ured[w] > best ? sm.ured[w] : best;
            st_dev_f32(&rec->m, key_f32(static_cast<uint32_t>(best >> 32)));
            st_dev(&rec->amax, 0xffffffffu - static_cast<uint32_t>(best));
            st_dev(&rec->cnt, 0u);
            st_dev(&rec->mode, mode);
        }
        return;
    }

    // group (16-byte load) maxima, recomputed where needed rather than held
    auto group_max = [&](int j) {
        float g = elem<DT>(d[j], 0);
#pragma unroll
        for (int e = 1; e < VEC; ++e) g = fmaxf(g, elem<DT>(d[j], e));
        return g;
    };
    float tm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NL; ++j) tm = fmaxf(tm, group_max(j));
    opaque(d);

    // chunk maximum
    const float wmax = wave_max_dpp(tm);
    if (lane == 0) sm.fred[wid] = wmax;
    __syncthreads();
    const float mc = fmaxf(fmaxf(sm.fred[0], sm.fred[1]), fmaxf(sm.fred[2], sm.fred[3]));

    // softmax weights 2^(x c - rc) summed per load slot: fp32 over the
    // thread's VEC elements, fp64 across the block
    const float rc = mc * cc;
    if (mode == kModeTopP || mode == kModeFull) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) s += __builtin_amdgcn_exp2f(fmaf(elem<DT>(d[j], e), cc, -rc));
            const double ws = wave_sum_dpp(static_cast<double>(s));
            if (lane == 0) sm.wsum[wid][j] = ws;
        }
        __syncthreads();
        if (t < NL) {
            const double sj = sm.wsum[0][t] + sm.wsum[1][t] + sm.wsum[2][t] + sm.wsum[3][t];
            sm.fseg[t] = static_cast<float>(sj);
            st_dev_f32(&rec->seg[t], static_cast<float>(sj));
        }
        __syncthreads();
    }

    float theta = INFINITY;
    uint32_t total = 0;
    if (jrank > 0) {
        // histogram of the group maxima by distance below the chunk maximum
        for (int i = t; i < kBins; i += kT) sm.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const float g = group_max(j);
            if (g > -INFINITY) {
                const uint32_t bin = static_cast<uint32_t>(fminf((mc - g) * kGroupBinScale, 1023.0f));
                atomicAdd(&sm.hist[bin], 1u);
            }
        }
        opaque(d);
        __syncthreads();
        // the bin holding the jrank-th largest (thread t owns bins 4t .. 4t+3)
        uint32_t h[4], own = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h[q] = sm.hist[4 * t + q];
            own += h[q];
        }
        const uint32_t incl = wave_scan_u32_dpp(own);
        if (lane == kWave - 1) sm.wtot[wid][0] = incl;
        if (t == 0) sm.bsel = kBins - 1;
        __syncthreads();
        uint32_t excl = incl - own, groups = 0;
        for (int w = 0; w < kNW; ++w) {
            excl += w < wid ? sm.wtot[w][0] : 0u;
            groups += sm.wtot[w][0];
        }
        // the rank aimed at scales with the chunk's length (the last chunk of a
        // row may be short), never below jmin (a top-k set may lie in one chunk)
        const int64_t valid = a.V - base < G::ELEMS ? a.V - base : G::ELEMS;
        const int64_t scaled = (static_cast<int64_t>(jrank) * valid + G::ELEMS - 1) / G::ELEMS;
        const uint32_t J = static_cast<uint32_t>(scaled > jmin ? scaled : jmin);
        if (excl < J && excl + own >= J) {
            uint32_t cum = excl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cum += h[q];
                if (cum >= J) {
                    sm.bsel = static_cast<uint32_t>(4 * t + q);
                    break;
                }
            }
        }
        __syncthreads();
        const uint32_t bsel = sm.bsel;
        float tmin = INFINITY;
        if (groups < J) {
            // fewer groups than the rank aimed at: every element is a candidate
#pragma unroll
            for (int j = 0; j < NL; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float x = elem<DT>(d[j], e);
                    if (x > -INFINITY) tmin = fminf(tmin, x);
                }
        } else {
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const float g = group_max(j);
                if (g > -INFINITY) {
                    const uint32_t bin = static_cast<uint32_t>(fminf((mc - g) * kGroupBinScale, 1023.0f));
                    if (bin <= bsel) tmin = fminf(tmin, g);
                }
            }
        }
        const float wmin = wave_min_dpp(tmin);
        if (lane == 0) sm.fred[wid] = wmin;
        __syncthreads();
        theta = fminf(fminf(sm.fred[0], sm.fred[1]), fminf(sm.fred[2], sm.fred[3]));

        opaque(d);
        // ordered compaction: per slot, the candidates of lower threads first;
        // slot counts travel two to a register through the wave scan
        uint32_t exq[NL / 2];
#pragma unroll
        for (int q = 0; q < NL / 2; ++q) {
            opaque(d);
            uint32_t n0 = 0, n1 = 0;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                n0 += elem<DT>(d[2 * q], e) >= theta ? 1u : 0u;
                n1 += elem<DT>(d[2 * q + 1], e) >= theta ? 1u : 0u;
            }
            const uint32_t pk = n0 | (n1 << 16);
            const uint32_t in = wave_scan_u32_dpp(pk);
            exq[q] = in - pk;
            if (lane == kWave - 1) {
                sm.wtot[wid][2 * q] = in & 0xffffu;
                sm.wtot[wid][2 * q + 1] = in >> 16;
            }
        }
        __syncthreads();
        if (t == 0) {
            uint32_t run = 0;
            for (int j = 0; j < NL; ++j) {
                for (int w = 0; w < kNW; ++w) {
                    sm.off[w][j] = run;
                    run += sm.wtot[w][j];
                }
            }
            sm.total = run;
        }
        __syncthreads();
        total = sm.total;
        opaque(d);
        if (total <= static_cast<uint32_t>(kSplitCap)) {
            uint64_t* out = a.cand + (static_cast<int64_t>(b) * a.rec_stride + c) * kSplitCap;
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                opaque(d);
                uint32_t pos = sm.off[wid][j] + ((exq[j / 2] >> ((j & 1) * 16)) & 0xffffu);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float x = elem<DT>(d[j], e);
                    if (x >= theta) {
                        const uint32_t i = static_cast<uint32_t>(base + j * G::SLOT + t * VEC + e);
                        st_dev(out + pos, (static_cast<uint64_t>(f32_key(x)) << 32) | i);
                        ++pos;
                    }
                }
            }
        }
    }
    if (t == 0) {
        double z = 0.0;
        if (mode == kModeTopP || mode == kModeFull)
            for (int j = 0; j < NL; ++j) z += static_cast<double>(sm.fseg[j]);
        st_dev_f64(&rec->z, z);
        st_dev_f32(&rec->m, mc);
        st_dev(&rec->amax, 0u);
        st_dev_f32(&rec->theta, theta);
        st_dev(&rec->cnt, jrank > 0 ? (total <= static_cast<uint32_t>(kSplitCap) ? total : kSplitCap + 1u) : 0u);
        st_dev_f32(&rec->rc, rc);
        st_dev(&rec->mode, mode);
    }
}

// ------------------------------------------------------- the finisher --

struct DCut {
    uint32_t key, idx;   // kept iff k > key || (k == key && i <= idx)
};

__device__ __forceinline__ bool kept_by(const DCut& c, uint32_t k, uint32_t i) {
    return k > c.key || (k == c.key && i <= c.idx);
}

struct Found {
    bool ok;
    DCut cut;
    uint32_t n;       // entries kept (within the restriction)
};

// Sorts the small list (n <= 64 entries in f.skey/sidx/sw) into descending
// order in wave 0; lane r returns entry r (valid for r < n).
__device__ __forceinline__ void small_sorted(FinSmem& f, uint32_t n, uint32_t* k, uint32_t* i, float* w) {
    const int lane = lane_id();
    uint32_t mk = 0, mi = 0xffffffffu;
    float mw = 0.0f;
    if (lane < static_cast<int>(n)) {
        mk = f.skey[lane];
        mi = f.sidx[lane];
        mw = f.sw[lane];
    }
    uint32_t rank = 0;
    for (uint32_t q = 0; q < n; ++q) {
        const uint32_t ok = f.skey[q], oi = f.sidx[q];
        rank += (ok > mk || (ok == mk && oi < mi)) ? 1u : 0u;
    }
    // scatter by rank through the LDS list itself (wave 0 only; the
    // lanes read back in rank order)
    __builtin_amdgcn_wave_barrier();
    if (lane < static_cast<int>(n)) {
        f.skey[rank] = mk;
        f.sidx[rank] = mi;
        f.sw[rank] = mw;
    }
    __builtin_amdgcn_wave_barrier();
    *k = lane < static_cast<int>(n) ? f.skey[lane] : 0u;
    *i = lane < static_cast<int>(n) ? f.sidx[lane] : 0xffffffffu;
    *w = lane < static_cast<int>(n) ? f.sw[lane] : 0.0f;
}

// Cut after the first `target_n` entries (COUNT) or after the entries whose
// exclusive prefix mass is below `target_m` (MASS), in descending order,
// among the active entries (key >= lo0) kept by `res`.  Block-uniform.
template <bool MASS>
__device__ __forceinline__ Found descent(FinSmem& f, int L, uint32_t lo0, uint32_t hi0, DCut res, uint32_t target_n,
                         double target_m) {
    const int t = static_cast<int>(threadIdx.x);
    uint32_t lo = lo0, hi = hi0;
    uint32_t above_n = 0;
    double above_m = 0.0;
    for (int round = 0; round < 6; ++round) {
        const uint32_t span = hi - lo;
        int sh = 0;
        while ((span >> sh) >= static_cast<uint32_t>(kBins)) ++sh;
        for (int i = t; i < kBins; i += kT) {
            f.hcnt[i] = 0u;
            if (MASS) f.hmass[i] = 0.0;
        }
        if (t == 0) f.sel_bin = -1;
        __syncthreads();
        for (int i = t; i < L; i += kT) {
            const uint32_t k = f.key[i];
            if (k < lo || k > hi || !kept_by(res, k, f.idx[i])) continue;
            const uint32_t bin = (k - lo) >> sh;
            atomicAdd(&f.hcnt[bin], 1u);
            if (MASS) atomicAdd(&f.hmass[bin], static_cast<double>(f.w[i]));
        }
        __syncthreads();
        // thread t owns bins 1023 - 4t - q, q = 0..3 (descending)
        uint32_t hc[4], oc = 0;
        double hm[4], om = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int bin = kBins - 1 - 4 * t - q;
            hc[q] = f.hcnt[bin];
            hm[q] = MASS ? f.hmass[bin] : 0.0;
            oc += hc[q];
            om += hm[q];
        }
        uint32_t ec, tc;
        double em, tmass;
        block_scan2(oc, om, &ec, &em, &tc, &tmass, f);
        uint32_t cum_c = above_n + ec;
        double cum_m = above_m + em;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool hit = MASS ? (cum_m < target_m && cum_m + hm[q] >= target_m)
                                  : (cum_c < target_n && cum_c + hc[q] >= target_n);
            if (hit) {
                f.sel_bin = kBins - 1 - 4 * t - q;
                f.sel_c = cum_c;
                f.sel_m = cum_m;
                f.sel_cnt = hc[q];
            }
            cum_c += hc[q];
            cum_m += hm[q];
        }
        __syncthreads();
        const int sb = f.sel_bin;
        if (sb < 0) return Found{false, DCut{0u, 0u}, 0u};
        const uint32_t sel_c = f.sel_c, cnt = f.sel_cnt;
        const double sel_m = f.sel_m;
        const uint32_t blo = lo + (static_cast<uint32_t>(sb) << sh);
        const uint64_t bhi64 = static_cast<uint64_t>(blo) + ((1ull << sh) - 1ull);
        const uint32_t bhi = bhi64 < hi ? static_cast<uint32_t>(bhi64) : hi;
        __syncthreads();
        if (cnt <= static_cast<uint32_t>(kSmall)) {
            // the bin's entries, sorted in one wave
            if (t == 0) f.sn = 0u;
            __syncthreads();
            for (int i = t; i < L; i += kT) {
                const uint32_t k = f.key[i];
                if (k < blo || k > bhi || !kept_by(res, k, f.idx[i])) continue;
                const uint32_t pos = atomicAdd(&f.sn, 1u);
                if (pos < static_cast<uint32_t>(kSmall)) {
                    f.skey[pos] = k;
                    f.sidx[pos] = f.idx[i];
                    f.sw[pos] = f.w[i];
                }
            }
            __syncthreads();
            if (t < kWave) {
                const uint32_t n = f.sn < static_cast<uint32_t>(kSmall) ? f.sn : static_cast<uint32_t>(kSmall);
                uint32_t sk, si;
                float sw;
                small_sorted(f, n, &sk, &si, &sw);
                uint32_t n_in;
                if (MASS) {
                    const double wv = t < static_cast<int>(n) ? static_cast<double>(sw) : 0.0;
                    const double ex = wave_scan_f64_dpp(wv) - wv;
                    const bool kp = t < static_cast<int>(n) && sel_m + ex < target_m;
                    n_in = static_cast<uint32_t>(__popcll(__ballot(kp)));
                    if (n_in == 0) n_in = 1;   // the bin was picked because its first entry is kept
                } else {
                    n_in = target_n - sel_c;
                }
                if (n_in > n) n_in = n;
                const uint32_t ck = readlane_u32(sk, static_cast<int>(n_in) - 1);
                const uint32_t ci = readlane_u32(si, static_cast<int>(n_in) - 1);
                if (t == 0) {
                    f.res_ok = 1u;
                    f.res_key = ck;
                    f.res_idx = ci;
                    f.res_n = sel_c + n_in;
                }
            }
            __syncthreads();
            Found r{f.res_ok != 0u, DCut{f.res_key, f.res_idx}, f.res_n};
            __syncthreads();
            return r;
        }
        if (sh == 0) {
            // one key, many ties: their descending order is token order, which
            // is list order; walk the list in contiguous per-thread ranges
            const uint32_t K = blo;
            const int per = (L + kT - 1) / kT;
            const int i0 = t * per, i1 = (i0 + per < L) ? i0 + per : L;
            uint32_t oc2 = 0;
            double om2 = 0.0;
            for (int i = i0; i < i1; ++i) {
                if (f.key[i] == K && kept_by(res, K, f.idx[i])) {
                    ++oc2;
                    om2 += static_cast<double>(f.w[i]);
                }
            }
            uint32_t ec2, tc2;
            double em2, tm2;
            if (t == 0) {
                f.res_ok = 0u;
            }
            block_scan2(oc2, om2, &ec2, &em2, &tc2, &tm2, f);
            // COUNT: the (target_n - sel_c)-th tie; MASS: the last tie whose
            // exclusive prefix is below the target
            uint32_t run_c = ec2;
            double run_m = sel_m + em2;
            const uint32_t need = target_n - sel_c;
            for (int i = i0; i < i1; ++i) {
                if (!(f.key[i] == K && kept_by(res, K, f.idx[i]))) continue;
                const bool kp = MASS ? run_m < target_m : run_c < need;
                if (!kp) break;
                ++run_c;
                run_m += static_cast<double>(f.w[i]);
                const bool last = MASS ? !(run_m < target_m) : run_c == need;
                if (last) {
                    f.res_ok = 1u;
                    f.res_key = K;
                    f.res_idx = f.idx[i];
                    f.res_n = sel_c + run_c;
                }
            }
            __syncthreads();
            if (f.res_ok == 0u) {
                // every tie stays (rounding between the histogram and the walk)
                if (t == 0) {
                    f.res_ok = 1u;
                    f.res_key = K;
                    f.res_idx = 0xffffffffu;
                    f.res_n = sel_c + tc2;
                }
                __syncthreads();
            }
            Found r{true, DCut{f.res_key, f.res_idx}, f.res_n};
            __syncthreads();
            return r;
        }
        lo = blo;
        hi = bhi;
        above_n = sel_c;
        above_m = sel_m;
    }
    return Found{false, DCut{0u, 0u}, 0u};
}

// Writes the first n entries of the descending order (n <= 64) as the debug
// top-k index list: the n entries kept by the count cut, sorted in wave 0.
__device__ __forceinline__ void debug_topk_list(const SampleArgs& a, int b, FinSmem& f, int L, uint32_t kappa, uint32_t maxkey,
                                uint32_t n) {
    const int t = static_cast<int>(threadIdx.x);
    int32_t* o = a.topk_idx_out + static_cast<int64_t>(b) * kDebugTopK;
    const Found fc = descent<false>(f, L, kappa, maxkey, DCut{0u, 0xffffffffu}, n, 0.0);
    if (t == 0) f.sn = 0u;
    __syncthreads();
    if (fc.ok) {
        for (int i = t; i < L; i += kT) {
            const uint32_t k = f.key[i];
            if (k < kappa || !kept_by(fc.cut, k, f.idx[i])) continue;
            const uint32_t pos = atomicAdd(&f.sn, 1u);
            if (pos < static_cast<uint32_t>(kSmall)) {
                f.skey[pos] = k;
                f.sidx[pos] = f.idx[i];
                f.sw[pos] = 0.0f;
            }
        }
    }
    __syncthreads();
    if (t < kWave) {
        const uint32_t m = f.sn < n ? f.sn : n;
        uint32_t sk, si;
        float sw;
        small_sorted(f, m, &sk, &si, &sw);
        o[t] = t < static_cast<int>(m) ? static_cast<int32_t>(si) : -1;
    }
    __syncthreads();
}

// Debug: the final distribution over the whole row.  kept(c, i, key) says
// whether element i is kept; weight(c, x) returns its weight (divided by W).
template <int DT, int NL, typename K, typename Wt>
__device__ __forceinline__ void debug_probs(const SampleArgs& a, int b, K kept, Wt weight) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    const char* rowp = row_ptr(a, b, G::ES);
    float* pr = a.probs_out + static_cast<int64_t>(b) * a.V;
    const int t = static_cast<int>(threadIdx.x);
    for (int c = 0; c < a.chunks; ++c) {
        const int64_t base = static_cast<int64_t>(c) * G::ELEMS;
        uint4 d[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) d[j] = load_slot<DT>(rowp, a.V, base + static_cast<int64_t>(j) * G::SLOT + t * VEC);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int64_t i = base + static_cast<int64_t>(j) * G::SLOT + t * VEC + e;
                if (i >= a.V) continue;
                const float x = elem<DT>(d[j], e);
                const uint32_t k = f32_key(x);
                pr[i] = kept(c, static_cast<uint32_t>(i), k) ? weight(c, x) : 0.0f;
            }
        }
    }
}

template <int DT, int NL>
__device__ __forceinline__ void finish_row(const SampleArgs& a, SplitSmem& sm, int b, const RowParams& prm, uint32_t mode,
                           float cc, uint64_t word) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    FinSmem& f = sm.f;
    const int t = static_cast<int>(threadIdx.x), lane = lane_id();
    const int S = a.chunks;
    const double u = uniform24(word);
    const SplitRec* recs = a.rec + static_cast<int64_t>(b) * a.rec_stride;

    // the records
    if (t < S) {
        f.cm[t] = ld_dev_f32(&recs[t].m);
        f.camax[t] = ld_dev(&recs[t].amax);
        f.ctheta[t] = ld_dev_f32(&recs[t].theta);
        f.ccnt[t] = ld_dev(&recs[t].cnt);
        f.cz[t] = ld_dev_f64(&recs[t].z);
        f.crc[t] = ld_dev_f32(&recs[t].rc);
    }
    __syncthreads();

    if (mode == kModeArgmax) {
        if (t < kWave) {
            uint64_t pk = 0;
            if (t < S) pk = (static_cast<uint64_t>(f32_key(f.cm[t])) << 32) | (0xffffffffu - f.camax[t]);
            const uint64_t best = wave_max_u64_dpp(pk);
            if (t == 0) f.tok = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(best));
        }
        __syncthreads();
        finish_argmax_row<kT>(a, b, f.tok, word);
        return;
    }

    // row maximum, its weight reference, the chunks' scales and the row's mass
    if (t < kWave) {
        const float mv = t < S ? f.cm[t] : -INFINITY;
        const float m = wave_max_dpp(mv);
        const float rref = m * cc;
        const double sc = t < S ? exp2(static_cast<double>(f.crc[t]) - static_cast<double>(rref)) : 0.0;
        const double zc = t < S ? f.cz[t] * sc : 0.0;
        const double incl = wave_scan_f64_dpp(zc);
        const double zrow = readlane_f64(incl, S - 1);
        if (t == 0) {
            f.zrow = zrow;
            f.maxkey = f32_key(m);
        }
        if (mode == kModeFull) {
            // the chunk holding u * Z in token order
            const double target = u * zrow;
            const bool past = t < S && incl > target;
            const uint64_t bal = __ballot(past);
            const int cs = bal ? __ffsll(static_cast<long long>(bal)) - 1 : S - 1;
            const double before = readlane_f64(incl - zc, cs);
            if (t == 0) {
                f.cstar = cs;
                f.before = before;
            }
        }
    }
    __syncthreads();
    const float m = key_f32(f.maxkey);
    const float rref = m * cc;
    const double zrow = f.zrow;

    if (mode == kModeFull) {
        const int cs = f.cstar;
        const double sc = exp2(static_cast<double>(f.crc[cs]) - static_cast<double>(rref));
        const double target = u * zrow;
        // the load slot holding the target
        if (t < kWave) {
            const double sj = t < NL ? static_cast<double>(ld_dev_f32(&recs[cs].seg[t])) * sc : 0.0;
            const double incl = wave_scan_f64_dpp(sj);
            const double tb = f.before;
            const bool past = t < NL && tb + incl > target;
            const uint64_t bal = __ballot(past);
            // no slot passes the target (rounding): the last slot with elements
            int js;
            if (bal) {
                js = __ffsll(static_cast<long long>(bal)) - 1;
            } else {
                const int64_t left = a.V - static_cast<int64_t>(cs) * G::ELEMS;
                const int64_t nslots = (left + G::SLOT - 1) / G::SLOT;
                js = static_cast<int>((nslots < NL ? nslots : NL) - 1);
            }
            const double before = tb + readlane_f64(incl - sj, js);
            if (t == 0) {
                f.jstar = js;
                f.before = before;
                f.tok = -1;
                f.last = -1;
            }
        }
        __syncthreads();
        const int js = f.jstar;
        const double before = f.before;
        const char* rowp = row_ptr(a, b, G::ES);
        const int64_t sbase = static_cast<int64_t>(cs) * G::ELEMS + static_cast<int64_t>(js) * G::SLOT;
        const uint4 v = load_slot<DT>(rowp, a.V, sbase + t * VEC);
        const float rcs = f.crc[cs];
        float s32 = 0.0f;
        int my_last = -1;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float w = __builtin_amdgcn_exp2f(fmaf(elem<DT>(v, e), cc, -rcs));
            s32 += w;
            if (w > 0.0f) my_last = static_cast<int>(sbase + t * VEC + e);
        }
        const double own = static_cast<double>(s32) * sc;
        uint32_t ec, tc;
        double em, tm2;
        block_scan2(0u, own, &ec, &em, &tc, &tm2, f);
        if (before + em <= target && before + em + own > target) {
            double run = before + em;
            int tok = my_last;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float w = __builtin_amdgcn_exp2f(fmaf(elem<DT>(v, e), cc, -rcs));
                run += static_cast<double>(w) * sc;
                if (w > 0.0f && run > target) {
                    tok = static_cast<int>(sbase + t * VEC + e);
                    break;
                }
            }
            f.tok = tok;
        }
        atomicMax(&f.last, my_last);
        __syncthreads();
        const int32_t tok = f.tok >= 0 ? f.tok : f.last;
        if (t == 0) {
            a.tokens_out[b] = tok;
            if (a.kept_out) a.kept_out[b] = a.V;
            if (a.rand_out) a.rand_out[b] = word;
        }
        if (a.probs_out) {
            const double inv = 1.0 / zrow;
            debug_probs<DT, NL>(a, b, [](int, uint32_t, uint32_t) { return true; },
                                [&](int c, float x) {
                                    const double s = exp2(static_cast<double>(f.crc[c]) - static_cast<double>(rref));
                                    return static_cast<float>(
                                        static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, cc, -f.crc[c]))) * s * inv);
                                });
        }
        // the debug top-64 comes from the candidates (published with rank 64)
        if (!a.topk_idx_out) return;
    }

    // ---- candidate list: every published candidate >= kappa, in token order
    if (t < kWave) {
        const uint32_t cn = t < S ? f.ccnt[t] : 0u;
        const bool over = t < S && cn > static_cast<uint32_t>(kSplitCap);
        const uint32_t incl = wave_scan_u32_dpp(over ? 0u : cn);
        if (t < S) f.coff[t] = incl - cn;
        const uint32_t tot = readlane_u32(incl, S - 1);
        const uint32_t kap = wave_max_u32_dpp(t < S ? f32_key(f.ctheta[t]) : 0u);
        const bool any_over = __ballot(over) != 0ull;
        if (t == 0) {
            f.coff[S] = tot;
            f.list_n = tot;
            f.kappa = kap;
            f.bad = (any_over || tot > static_cast<uint32_t>(kListMax)) ? 1u : 0u;
        }
    }
    __syncthreads();
    const bool bad = f.bad != 0u;
    const int L = bad ? 0 : static_cast<int>(f.list_n);
    const uint32_t kappa = f.kappa, maxkey = f.maxkey;
    if (!bad) {
        uint64_t v[8];
        const uint64_t* cb = a.cand + static_cast<int64_t>(b) * a.rec_stride * kSplitCap;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int fi = t + q * kT;
            v[q] = 0ull;
            if (fi < L) {
                int lo = 0, hi = S - 1;       // the chunk c with coff[c] <= fi < coff[c + 1]
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (f.coff[mid] <= static_cast<uint32_t>(fi)) lo = mid; else hi = mid - 1;
                }
                v[q] = ld_dev(cb + static_cast<int64_t>(lo) * kSplitCap + (fi - static_cast<int>(f.coff[lo])));
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int fi = t + q * kT;
            if (fi < L) {
                uint32_t k = static_cast<uint32_t>(v[q] >> 32);
                const uint32_t i = static_cast<uint32_t>(v[q]);
                if (k < kappa) k = 0u;
                f.key[fi] = k;
                f.idx[fi] = i;
                f.w[fi] = k ? __builtin_amdgcn_exp2f(fmaf(key_f32(k), cc, -rref)) : 0.0f;
            }
        }
    }
    __syncthreads();

    if (mode == kModeFull) {
        // debug top-64 only (the token is written above)
        if (!bad) {
            debug_topk_list(a, b, f, L, kappa, maxkey,
                            static_cast<uint32_t>(prm.k < kDebugTopK ? prm.k : kDebugTopK));
        } else {
            __syncthreads();
            exact_debug_topk<DT, kT>(row_ptr(a, b, G::ES), a.V, kDebugTopK,
                                     a.topk_idx_out + static_cast<int64_t>(b) * kDebugTopK, sm.e);
        }
        return;
    }

    // ---- top-k, then top-p inside it, then min_p
    bool ok = !bad;
    DCut cut{0u, 0xffffffffu};
    bool kp_in_list = false;
    const bool has_k = prm.k < a.V;
    if (ok && has_k) {
        const Found fk = descent<false>(f, L, kappa, maxkey, cut, static_cast<uint32_t>(prm.k), 0.0);
        ok = fk.ok;
        cut = fk.cut;
        kp_in_list = fk.ok;
    }
    if (ok && prm.top_p) {
        double wk = zrow;
        if (has_k) {
            double own = 0.0;
            for (int i = t; i < L; i += kT) {
                const uint32_t k = f.key[i];
                if (k >= kappa && kept_by(cut, k, f.idx[i])) own += static_cast<double>(f.w[i]);
            }
            uint32_t ec, tc;
            double em, tm2;
            block_scan2(0u, own, &ec, &em, &tc, &tm2, f);
            wk = tm2;
        }
        const Found fp = descent<true>(f, L, kappa, maxkey, cut, 0u, static_cast<double>(prm.p) * wk);
        if (fp.ok) {
            cut = fp.cut;
            kp_in_list = true;
        } else if (!has_k) {
            kp_in_list = false;   // the nucleus reaches below kappa
        }
    }
    if (ok && prm.min_p > 0.0f) {
        const double xm = static_cast<double>(m) + static_cast<double>(prm.T) * log(static_cast<double>(prm.min_p));
        const float xf = static_cast<float>(xm);
        const uint32_t kmin = f32_key(xf) + (static_cast<double>(xf) < xm ? 1u : 0u);
        if (kp_in_list) {
            if (kmin > cut.key) cut = DCut{kmin, 0xffffffffu};
        } else if (kmin >= kappa) {
            cut = DCut{kmin, 0xffffffffu};
            kp_in_list = true;
        }
    }
    ok = ok && kp_in_list;
    if (!ok) {
        __syncthreads();
        exact_row<DT, kT>(a, b, row_ptr(a, b, G::ES), prm, word, u, sm.e);
        return;
    }

    // ---- kept count, kept mass and the draw in token order
    const int per = (L + kT - 1) / kT;
    const int i0 = t * per, i1 = i0 + per < L ? i0 + per : L;
    uint32_t oc = 0;
    double om = 0.0;
    int my_last = -1;
    for (int i = i0; i < i1; ++i) {
        const uint32_t k = f.key[i];
        if (k >= kappa && kept_by(cut, k, f.idx[i])) {
            ++oc;
            om += static_cast<double>(f.w[i]);
            my_last = static_cast<int>(f.idx[i]);
        }
    }
    if (t == 0) {
        f.tok = -1;
        f.last = -1;
    }
    uint32_t ec, kept_n;
    double em, W;
    block_scan2(oc, om, &ec, &em, &kept_n, &W, f);
    const double target = u * W;
    if (em <= target && em + om > target) {
        double run = em;
        int tok = my_last;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = f.key[i];
            if (k >= kappa && kept_by(cut, k, f.idx[i])) {
                run += static_cast<double>(f.w[i]);
                if (f.w[i] > 0.0f && run > target) {
                    tok = static_cast<int>(f.idx[i]);
                    break;
                }
            }
        }
        f.tok = tok;
    }
    atomicMax(&f.last, my_last);
    __syncthreads();
    const int32_t tok = f.tok >= 0 ? f.tok : f.last;
    if (t == 0) {
        a.tokens_out[b] = tok;
        if (a.kept_out) a.kept_out[b] = static_cast<int32_t>(kept_n);
        if (a.rand_out) a.rand_out[b] = word;
    }
    if (a.probs_out) {
        const double inv = 1.0 / W;
        const DCut fc = cut;
        debug_probs<DT, NL>(a, b,
                            [&](int, uint32_t i, uint32_t k) { return k >= kappa && kept_by(fc, k, i); },
                            [&](int, float x) {
                                return static_cast<float>(
                                    static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, cc, -rref))) * inv);
                            });
    }
    if (a.topk_idx_out) {
        __syncthreads();
        const uint32_t n = prm.k < kDebugTopK ? static_cast<uint32_t>(prm.k) : static_cast<uint32_t>(kDebugTopK);
        debug_topk_list(a, b, f, L, kappa, maxkey, n);
    }
}

template <int DT, int NL>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(4, 8))) void sample_split_kernel(SampleArgs a) {
    __shared__ SplitSmem sm;
    const int S = a.chunks;
    // workgroup -> (row, chunk): XCD x = blockIdx mod 8 takes rows x, x + 8, ...;
    // a row's chunks are consecutive on its XCD, chunk S - 1 last
    const int x = static_cast<int>(blockIdx.x) & (kSplitXcds - 1);
    const int kk = static_cast<int>(blockIdx.x) / kSplitXcds;
    const int rl = kk / S;
    const int c_own = kk - rl * S;
    const int b = rl * kSplitXcds + x;
    if (b >= a.B) return;
    const bool finisher = c_own == S - 1;

    const RowParams prm = row_params(a.temperature, a.top_k, a.top_p, a.min_p, b, a.V);
    const bool dbg_list = a.topk_idx_out != nullptr;
    // route; candidate rank aimed at (scaled by the chunk's length) and the
    // rank every chunk must cover whatever its length
    uint32_t mode;
    int jrank = 0, jmin = 0;
    if (prm.greedy || prm.k == 1) {
        mode = kModeArgmax;
    } else if (prm.k < a.V && prm.k <= kKList) {
        mode = kModeTopK;
        jrank = jmin = prm.k;
    } else if (prm.k < a.V) {
        mode = prm.k <= kJMax ? kModeTopP : kModeExact;
        jrank = kJTopP;
        jmin = prm.k;
    } else if (prm.top_p || prm.min_p > 0.0f) {
        mode = kModeTopP;
        jrank = kJTopP;
        jmin = dbg_list ? kJDebug : 1;
    } else {
        mode = kModeFull;
        jrank = jmin = dbg_list ? kJDebug : 0;
    }
    // log2(e) / T in fp32
    const float cc = static_cast<float>(1.4426950408889634 / static_cast<double>(prm.T));

    if (mode == kModeExact) {
        if (!finisher) return;
        const uint64_t word = a.temperature ? request_word(a.seed, ld_global<int64_t>(a.uid + b), a.step) : 0ull;
        exact_row<DT, kT>(a, b, row_ptr(a, b, Geo<DT, NL>::ES), prm, word, uniform24(word), sm.e);
        return;
    }

    chunk_phase<DT, NL>(a, sm.c, b, c_own, mode, cc, jrank, jmin);
    wait_all_memory();
    __syncthreads();
    if (!finisher) {
        if (threadIdx.x == 0) st_dev(a.flags + static_cast<int64_t>(b) * kSplitMaxChunks + c_own, a.epoch);
        return;
    }
    // the finisher waits for the row's other chunks (bounded)
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        const uint32_t* fl = a.flags + static_cast<int64_t>(b) * kSplitMaxChunks;
        int late = 0;
        for (int spin = 0;; ++spin) {
            const uint32_t fv = lane < S - 1 ? ld_dev(fl + lane) : a.epoch;
            if (__ballot(fv != a.epoch) == 0ull) break;
            if (spin >= kSpinLimit) {
                late = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) sm.f.next = late;
    }
    __syncthreads();
    const bool late = sm.f.next != 0;
    __syncthreads();
    const uint64_t word = a.temperature ? request_word(a.seed, ld_global<int64_t>(a.uid + b), a.step) : 0ull;
    if (late) {
        // a chunk never published within the wait: the exact routine reads the row itself
        exact_row<DT, kT>(a, b, row_ptr(a, b, Geo<DT, NL>::ES), prm, word, uniform24(word), sm.e);
        return;
    }
    finish_row<DT, NL>(a, sm, b, prm, mode, cc, word);
}

template <int DT>
hipError_t launch_dt(const SampleArgs& args, int nl, hipStream_t stream) {
    const int rows_per_xcd = (args.B + kSplitXcds - 1) / kSplitXcds;
    const dim3 grid(static_cast<unsigned>(kSplitXcds * rows_per_xcd * args.chunks));
    if (nl == 4)
        hipLaunchKernelGGL((sample_split_kernel<DT, 4>), grid, dim3(kT), 0, stream, args);
    else if (DT == kDtypeF32 && nl == 8)
        hipLaunchKernelGGL((sample_split_kernel<kDtypeF32, 8>), grid, dim3(kT), 0, stream, args);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int split_plan(int V, int dtype, int* chunks) {
    const int vec = dtype == kDtypeF32 ? 4 : 8;
    auto nchunks = [&](int nl) {
        const int64_t e = static_cast<int64_t>(kSplitThreads) * nl * vec;
        return static_cast<int64_t>((V + e - 1) / e);
    };
    // Eight 16-byte loads per thread at most for fp32 rows and four for bf16
    // rows: the chunk and the compaction state then fit in 128 VGPRs (four
    // waves per SIMD) with no scratch.  fp32 rows take eight unless that
    // leaves fewer than eight chunks per row.
    const int nl = (dtype == kDtypeF32 && nchunks(8) >= 8) ? 8 : 4;
    if (V < 1 || nchunks(nl) > kSplitMaxChunks) return 0;
    *chunks = static_cast<int>(nchunks(nl));
    return nl;
}

int split_chunks_alloc(int V, int dtype) {
    int ch = 0;
    return split_plan(V, dtype, &ch) ? ch : 0;
}

hipError_t launch_sample_split(const SampleArgs& args, int dtype, int nl, hipStream_t stream) {
    if (args.chunks < 1 || args.chunks > kSplitMaxChunks || args.chunks > args.rec_stride) return hipErrorInvalidValue;
    return dtype == kDtypeF32 ? launch_dt<kDtypeF32>(args, nl, stream) : launch_dt<kDtypeBF16>(args, nl, stream);
}

}  // namespace dst
