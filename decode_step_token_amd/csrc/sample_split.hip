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
// the first is free of memory traffic, and a CU keeps several chunks in
// flight.  The rows are dealt to the 8 XCDs round robin and a row's chunks
// are consecutive workgroups of its XCD; the chunk dispatched last (S - 1)
// finishes the row.  Everything is inline (no calls, no scratch) and sized
// for few registers, so that several workgroups share a CU.
//
// Every chunk publishes a record (its maximum and lowest index, the sum of
// its softmax weights, a candidate threshold) and, for rows that select,
// every element at or above the threshold with its index, in token order;
// then an epoch flag.  Publication uses device-scope stores (written through
// the XCD's L2), and the flag follows only once the data stores have
// completed (s_waitcnt), so a reader that sees the flag with a device-scope
// load and then loads the data with device-scope loads reads the published
// values.  The publishing workgroups never wait; only the finisher polls the
// flags of its row, whose other chunks were dispatched before it on the same
// XCD and therefore run.  Its wait is bounded: past the limit it finishes
// the row by the exact routine, which reads the row itself.
//
// Candidate thresholds.  For a rank target J (k for top-k rows, about
// 1200/S for top-p rows, 64 for the debug top-64), the chunk histograms its
// 16-byte group maxima by distance below the chunk maximum (1/16 logit per
// bin) and takes theta = the smallest group maximum in the bins that hold
// the J largest.  J group maxima are J distinct elements >= theta, so the
// chunk's J largest elements are all candidates; the union over the chunks
// holds every element of the row at or above kappa = the largest chunk
// threshold.
//
// Rows without a top-k filter (top-p and / or min_p).  Their nucleus can hold
// tens of thousands of tokens, far more than any candidate list, so they are
// cut through a weight histogram instead.  Every chunk of such a row also
// adds its weights into bins of 1/32 octave on a grid common to the whole row
// (floor(32 x log2(e) / T)) and publishes that histogram with its record.
// The finisher sums the chunks' histograms, finds the bin G* where the
// descending mass first reaches p of the row's (and the min_p key from the
// row maximum) and publishes that decision; the chunks, still holding their
// elements in registers, then publish the weight and count of everything
// above bin G* and the elements of bin G* itself in token order, and the
// finisher resolves the cut inside bin G* exactly.  The chunks of such a row
// wait for their finisher, which is dispatched after them on the same XCD:
// every earlier row's finisher is already resident, so the wait always ends
// (and it is bounded all the same).
//
// The finisher loads the candidates >= kappa into LDS (in token order) and
// finds cuts by descents over key histograms (by count for top-k, by mass
// for top-p), resolving the boundary bin exactly.  Rows whose kept set is in
// the list draw by a block-wide scan of the kept weights in token order;
// rows with no filter and rows cut through the histogram find the chunk
// holding the target from the published masses and re-read that one chunk.  Whatever the published
// data cannot settle is finished by the exact multi-pass routine over the
// whole row.
#include "device_common.hpp"
#include "exact_path.hpp"
#include "kernels.hpp"

#ifndef DST_SPLIT_NL_F32
#define DST_SPLIT_NL_F32 8      // 16-byte loads per thread and chunk, fp32 rows
#endif
#ifndef DST_SPLIT_NL_BF16
#define DST_SPLIT_NL_BF16 8     // ... bf16 rows
#endif
#ifndef DST_SPLIT_WAVES_PER_EU
#define DST_SPLIT_WAVES_PER_EU 4
#endif

namespace dst {

namespace {

constexpr int kT = kSplitThreads;
constexpr int kNW = kT / kWave;
constexpr int kGBins = 1024;          // group-maximum histogram: 1/16 logit per bin
constexpr int kDBins = 512;           // descent histograms
constexpr int kWBins = kSplitHistBins;   // weight histogram: 1/32 octave per bin
constexpr int kListMax = 1536;        // candidates the finisher holds
constexpr int kKList = 128;           // top-k rows up to this k aim their thresholds at k
constexpr int kPList = 1200;          // top-p / min_p rows: candidates aimed at per row
constexpr int kJMax = 224;            // largest rank aimed at (a chunk publishes <= kSplitCap)
constexpr int kJDebug = 64;           // debug: the row's 64 largest
constexpr float kGroupBinScale = 16.0f;
constexpr float kWeightBinScale = 32.0f;
constexpr int kSpinLimit = 1 << 16;
constexpr int kSmall = 64;

// kModeTopP: a top-k filter above kKList (cut through the candidates);
// kModeHist: top-p and / or min_p without a top-k filter (cut through the
// weight histogram)
enum : uint32_t { kModeArgmax = 0, kModeTopK = 1, kModeTopP = 2, kModeFull = 3, kModeExact = 4, kModeHist = 5 };

static_assert(kT == 256 && kNW == 4, "the block layout below assumes 4 waves");

struct ChunkSmem {
    uint32_t gh[kGBins];
    double wh[kWBins];
    uint32_t wtot[kNW][16];
    uint32_t off[kNW][16];
    double dred[kNW][8];
    uint32_t ured32[kNW][8];
    float fred[kNW];
    uint64_t ured[kNW];
    uint32_t bsel, total;
};

struct FinSmem {
    uint32_t key[kListMax];
    uint32_t idx[kListMax];
    float w[kListMax];
    uint32_t hcnt[kDBins];
    double hmass[kDBins];
    float cm[kSplitMaxChunks];
    uint32_t camax[kSplitMaxChunks];
    float ctheta[kSplitMaxChunks];
    uint32_t ccnt[kSplitMaxChunks];
    double cz[kSplitMaxChunks];
    float crc[kSplitMaxChunks];
    double csc[kSplitMaxChunks];       // 2^(rc_c - rref)
    double ckept[kSplitMaxChunks];     // histogram rows: kept mass per chunk
    uint32_t coff[kSplitMaxChunks + 1];
    uint32_t skey[kSmall];
    uint32_t sidx[kSmall];
    float sw[kSmall];
    uint32_t sn;
    double slot[kNW][16];
    double slott[16];
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
    double zrow, before, amass;
    uint32_t anum;
    float gstar;
    int cstar, jstar, next;
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

// Bulk reads of data published earlier in this launch (after its flag was
// seen): buffer loads with the sc1 cache policy, which read the L2 the
// publishing stores wrote through to, never a stale L1 line.  Plain loads,
// unlike the atomic ones above, so the compiler issues a batch before
// waiting; offsets past the buffer's size read 0 (kL2None).
constexpr int kSc1 = 16;
constexpr uint32_t kL2None = 0x7ffffff0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t l2_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(nbytes), 0x00020000);
}
__device__ __forceinline__ uint32_t l2_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1);
}
__device__ __forceinline__ float l2_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) { return __uint_as_float(l2_u32(r, off)); }
__device__ __forceinline__ uint64_t l2_u64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSc1);
    return static_cast<uint64_t>(v[0]) | (static_cast<uint64_t>(v[1]) << 32);
}
__device__ __forceinline__ double l2_f64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __longlong_as_double(static_cast<long long>(l2_u64(r, off)));
}
// byte offset of a record field
#define DST_REC_OFF(c, field) (static_cast<uint32_t>(c) * static_cast<uint32_t>(sizeof(SplitRec)) + \
                               static_cast<uint32_t>(offsetof(SplitRec, field)))

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

__device__ __forceinline__ uint32_t wave_sum_u32_dpp(uint32_t v) {
    return readlane_u32(wave_scan_u32_dpp(v), 63);
}

typedef uint32_t u32x4_t_ __attribute__((ext_vector_type(4)));

// Makes the compiler treat the chunk registers as changed: values derived
// from them in one pass (unpacked bf16, keys) are recomputed in the next
// instead of being kept live across it.
template <int NL>
__device__ __forceinline__ void opaque(u32x4_t_ (&d)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) __asm__ __volatile__("" : "+v"(d[j]));
}

// Keeps the scheduler from moving work across it: placed after each 16-byte
// slot of a pass, it bounds the values in flight to one slot's (without it
// the whole chunk's exponents are hoisted ahead of their sums and spill).
__device__ __forceinline__ void slot_fence() { __builtin_amdgcn_sched_barrier(0); }

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
__device__ __forceinline__ float elem(const u32x4_t_& v, int e) {
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

// The chunk into registers.  Every 16-byte slot is a buffer load through a
// descriptor bounded by the row, issued without a branch (a load past the row
// returns zeros and is replaced by -inf), so all NL loads are in flight
// before the first wait; the non-temporal hint keeps the row, read once,
// from displacing other lines.  The slot that straddles V (V not a multiple
// of VEC) is re-read element by element afterwards.
template <int DT, int NL>
__device__ __forceinline__ void load_chunk(const SampleArgs& a, int b, int c, u32x4_t_ (&d)[NL]) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    constexpr int kNonTemporal = 2;
    const char* rowp = row_ptr(a, b, G::ES);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(rowp), static_cast<short>(0), a.V * G::ES, 0x00020000);
    const uint32_t pad = DT == kDtypeF32 ? 0xff800000u : 0xff80ff80u;
    // element offsets fit 32 bits: a row has at most kSplitMaxChunks chunks.
    // One vector offset for the thread; slot j adds the constant j * SLOT,
    // passed as the scalar offset.  Slots 0 .. jfull lie inside the row.
    const int base = c * static_cast<int>(G::ELEMS) + static_cast<int>(threadIdx.x) * VEC;
    const int room = a.V - VEC - base;
    const int jfull = room < 0 ? -1 : room / G::SLOT;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const u32x4_t_ v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, base * G::ES, j * G::SLOT * G::ES,
                                                                 kNonTemporal);
        const bool full = j <= jfull;
        d[j] = full ? v : u32x4_t_{pad, pad, pad, pad};
    }
    if (a.V % VEC != 0) {
        // the one slot that straddles V, if it is this thread's
        const int rest = a.V - base;
        const int jp = rest > 0 && rest % G::SLOT < VEC && rest % G::SLOT > 0 ? rest / G::SLOT : -1;
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if (j == jp) {
                const uint4 v = load_slot<DT>(rowp, a.V, base + j * G::SLOT);
                d[j] = u32x4_t_{v.x, v.y, v.z, v.w};
            }
    }
}

// The common weight-bin grid of a row: floor(32 x log2(e) / T).
__device__ __forceinline__ float weight_bin(float x, float cc) {
    return floorf(x * cc * kWeightBinScale);
}

// Block sum of a double in a fixed order (wave trees, then the waves in
// order); `slot` picks the scratch column, which stays valid until reused.
__device__ __forceinline__ double block_sum_f64(double v, ChunkSmem& sm, int slot) {
    const double w = wave_sum_dpp(v);
    if (lane_id() == 0) sm.dred[wave_id()][slot] = w;
    __syncthreads();
    return sm.dred[0][slot] + sm.dred[1][slot] + sm.dred[2][slot] + sm.dred[3][slot];
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, ChunkSmem& sm, int slot) {
    const uint32_t w = wave_sum_u32_dpp(v);
    if (lane_id() == 0) sm.ured32[wave_id()][slot] = w;
    __syncthreads();
    return sm.ured32[0][slot] + sm.ured32[1][slot] + sm.ured32[2][slot] + sm.ured32[3][slot];
}

// Ordered compaction: the chunk's elements that pass keep(x), in token order
// (per slot, those of lower threads first; slot counts travel two to a
// register through the wave scan), written as (order key << 32 | index) to
// out[0, total) when total <= cap; each(x) sees every written element.
// Returns total, the same in every thread.
template <int DT, int NL, typename P, typename E>
__device__ __forceinline__ uint32_t ordered_publish(u32x4_t_ (&d)[NL], ChunkSmem& sm, uint32_t tbase, uint64_t* out,
                                                    uint32_t cap, P keep, E each) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    static_assert(NL % 2 == 0, "slot counts are paired");
    const int t = static_cast<int>(threadIdx.x), lane = lane_id(), wid = wave_id();
    uint32_t exq[NL / 2];
#pragma unroll
    for (int q = 0; q < NL / 2; ++q) {
        uint32_t n0 = 0, n1 = 0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            n0 += keep(elem<DT>(d[2 * q], e)) ? 1u : 0u;
            n1 += keep(elem<DT>(d[2 * q + 1], e)) ? 1u : 0u;
        }
        const uint32_t pk = n0 | (n1 << 16);
        const uint32_t in = wave_scan_u32_dpp(pk);
        exq[q] = in - pk;
        if (lane == kWave - 1) {
            sm.wtot[wid][2 * q] = in & 0xffffu;
            sm.wtot[wid][2 * q + 1] = in >> 16;
        }
    }
    opaque(d);
    __syncthreads();
    if (t == 0) {
        uint32_t run = 0;
        for (int j = 0; j < NL; ++j) {
            for (int w = 0; w < kNW; ++w) {
                sm.off[w][j] = run;
                run += sm.wtot[w][j];
            }
            slot_fence();
        }
        sm.total = run;
    }
    __syncthreads();
    const uint32_t total = sm.total;
    if (total <= cap) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            uint32_t pos = sm.off[wid][j] + ((exq[j / 2] >> ((j & 1) * 16)) & 0xffffu);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float x = elem<DT>(d[j], e);
                if (keep(x)) {
                    st_dev(out + pos, (static_cast<uint64_t>(f32_key(x)) << 32) | (tbase + j * G::SLOT + e));
                    ++pos;
                    each(x);
                }
            }
            slot_fence();
        }
    }
    opaque(d);
    __syncthreads();   // sm.total and sm.off may be reused
    return total;
}

// The first publication of a chunk (held in d): its record, its candidates
// when jrank > 0 (the rank aimed at, scaled by the chunk's length; jmin the
// rank every chunk covers), and its weight histogram when whist.  mode is
// the row's route, cc the fp32 log2(e)/T.  Returns rc.
template <int DT, int NL>
__device__ __forceinline__ float chunk_phase(const SampleArgs& a, ChunkSmem& sm, int b, int c, u32x4_t_ (&d)[NL],
                                             uint32_t mode, float cc, int jrank, int jmin, bool whist) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    const int t = static_cast<int>(threadIdx.x), lane = lane_id(), wid = wave_id();
    const int base = c * static_cast<int>(G::ELEMS);
    const uint32_t tbase = static_cast<uint32_t>(base + t * VEC);

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
                const uint32_t i = (tbase + j * G::SLOT + e);
                ti = elem<DT>(d[j], e) == tm ? i : ti;
            }
            slot_fence();
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
        return 0.0f;
    }

    // group (16-byte load) maxima, recomputed where needed rather than held
    auto group_max = [&](int j) {
        float g = elem<DT>(d[j], 0);
#pragma unroll
        for (int e = 1; e < VEC; ++e) g = fmaxf(g, elem<DT>(d[j], e));
        return g;
    };
    if (whist) {
#pragma unroll
        for (int q = 0; q < kWBins / kT; ++q) sm.wh[q * kT + t] = 0.0;
    }
    float tm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NL; ++j) tm = fmaxf(tm, group_max(j));
    opaque(d);
    const float wmax = wave_max_dpp(tm);
    if (lane == 0) sm.fred[wid] = wmax;
    __syncthreads();
    const float mc = fmaxf(fmaxf(sm.fred[0], sm.fred[1]), fmaxf(sm.fred[2], sm.fred[3]));

    // softmax weights 2^(x c - rc): fp32 over the thread's elements, fp64
    // across the block; with whist also by weight bin below the chunk's top
    // bin (fp64 in LDS, the deepest bin holding everything below)
    const float rc = mc > -INFINITY ? mc * cc : 0.0f;   // a chunk of -inf only: every weight 0
    double z = 0.0;
    if (mode == kModeTopP || mode == kModeFull || mode == kModeHist) {
        const float gtop = weight_bin(mc, cc);
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float x = elem<DT>(d[j], e);
                const float w = __builtin_amdgcn_exp2f(fmaf(x, cc, -rc));
                if (e & 1) s1 += w; else s0 += w;
                if (whist && x > -INFINITY) {
                    const int r = static_cast<int>(fminf(gtop - weight_bin(x, cc), kWBins - 1.0f));
                    atomicAdd(&sm.wh[r], static_cast<double>(w));
                }
            }
            slot_fence();
        }
        opaque(d);
        z = block_sum_f64(static_cast<double>(s0) + static_cast<double>(s1), sm, 0);   // also orders the histogram
        if (whist) {
            float* ho = a.hist + (static_cast<int64_t>(b) * a.rec_stride + c) * kWBins;
#pragma unroll
            for (int q = 0; q < kWBins / kT; ++q) st_dev_f32(ho + q * kT + t, static_cast<float>(sm.wh[q * kT + t]));
        }
    }

    float theta = INFINITY;
    uint32_t total = 0;
    if (jrank > 0) {
        const int64_t valid = a.V - base < G::ELEMS ? a.V - base : G::ELEMS;   // elements in the chunk
        const int64_t scaled = (static_cast<int64_t>(jrank) * valid + G::ELEMS - 1) / G::ELEMS;
        const uint32_t J = static_cast<uint32_t>(scaled > jmin ? scaled : jmin);
        // histogram of the group maxima by distance below the chunk maximum
        for (int i = t; i < kGBins; i += kT) sm.gh[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const float g = group_max(j);
            if (g > -INFINITY) {
                const uint32_t bin = static_cast<uint32_t>(fminf((mc - g) * kGroupBinScale, kGBins - 1.0f));
                atomicAdd(&sm.gh[bin], 1u);
            }
            slot_fence();
        }
        opaque(d);
        __syncthreads();
        // the bin holding the J-th largest (thread t owns bins 4t .. 4t+3)
        uint32_t h[4], own = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h[q] = sm.gh[4 * t + q];
            own += h[q];
        }
        const uint32_t incl = wave_scan_u32_dpp(own);
        if (lane == kWave - 1) sm.wtot[wid][0] = incl;
        if (t == 0) sm.bsel = kGBins - 1;
        __syncthreads();
        uint32_t excl = incl - own, groups = 0;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
            excl += w < wid ? sm.wtot[w][0] : 0u;
            groups += sm.wtot[w][0];
        }
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
                    const uint32_t bin = static_cast<uint32_t>(fminf((mc - g) * kGroupBinScale, kGBins - 1.0f));
                    if (bin <= bsel) tmin = fminf(tmin, g);
                }
                slot_fence();
            }
        }
        opaque(d);
        const float wmin = wave_min_dpp(tmin);
        if (lane == 0) sm.fred[wid] = wmin;
        __syncthreads();
        theta = fminf(fminf(sm.fred[0], sm.fred[1]), fminf(sm.fred[2], sm.fred[3]));

        total = ordered_publish<DT, NL>(d, sm, tbase,
                                       a.cand + (static_cast<int64_t>(b) * a.rec_stride + c) * kSplitCandStride,
                                       static_cast<uint32_t>(kSplitCap), [&](float x) { return x >= theta; },
                                       [](float) {});
    }

    if (t == 0) {
        st_dev_f64(&rec->z, z);
        st_dev_f32(&rec->m, mc);
        st_dev(&rec->amax, 0u);
        st_dev_f32(&rec->theta, theta);
        st_dev(&rec->cnt, jrank > 0 ? (total <= static_cast<uint32_t>(kSplitCap) ? total : kSplitCap + 1u) : 0u);
        st_dev_f32(&rec->rc, rc);
        st_dev(&rec->mode, mode);
    }
    return rc;
}

// The second publication of a histogram row's chunk, once the finisher has
// decided the boundary bin gstar (-inf: min_p alone) and the min_p key kmin
// (0: none): the weight and count of the elements in bins above gstar, all
// and those with key >= kmin, and (when bin) the elements of bin gstar in
// token order.
template <int DT, int NL>
__device__ __forceinline__ void hist_phase2(const SampleArgs& a, ChunkSmem& sm, int b, int c, u32x4_t_ (&d)[NL],
                                            float cc, float rc, float gstar, uint32_t kmin, bool bin) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    const int t = static_cast<int>(threadIdx.x);
    const uint32_t tbase = static_cast<uint32_t>(c * static_cast<int>(G::ELEMS) + t * VEC);
    SplitRec* rec = a.rec + static_cast<int64_t>(b) * a.rec_stride + c;
    float am = 0.0f, amk = 0.0f;
    uint32_t an = 0, ank = 0;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float x = elem<DT>(d[j], e);
            if (x > -INFINITY && weight_bin(x, cc) > gstar) {
                const float w = __builtin_amdgcn_exp2f(fmaf(x, cc, -rc));
                const bool k = f32_key(x) >= kmin;
                am += w;
                ++an;
                amk += k ? w : 0.0f;
                ank += k ? 1u : 0u;
            }
        }
        slot_fence();
    }
    opaque(d);
    const double am_b = block_sum_f64(static_cast<double>(am), sm, 0);
    const double amk_b = block_sum_f64(static_cast<double>(amk), sm, 1);
    const uint32_t an_b = block_sum_u32(an, sm, 2);
    const uint32_t ank_b = block_sum_u32(ank, sm, 3);
    uint32_t nb = 0;
    if (bin) {
        nb = ordered_publish<DT, NL>(
            d, sm, tbase, a.cand + (static_cast<int64_t>(b) * a.rec_stride + c) * kSplitCandStride + kSplitCap,
            static_cast<uint32_t>(kSplitBinCap),
            [&](float x) { return x > -INFINITY && weight_bin(x, cc) == gstar; }, [](float) {});
    }
    if (t == 0) {
        st_dev_f64(&rec->am_all, am_b);
        st_dev_f64(&rec->am_kept, amk_b);
        st_dev(&rec->an_all, an_b);
        st_dev(&rec->an_kept, ank_b);
        st_dev(&rec->bcnt, nb);
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
    uint32_t n;       // entries kept (within the restriction, plus above_n0)
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
// among the active entries (key >= lo0) kept by `res`; the prefix starts at
// (above_n0, above_m0), the count and mass of what lies above every entry.
// Block-uniform.
template <bool MASS>
__device__ __forceinline__ Found descent(FinSmem& f, int L, uint32_t lo0, uint32_t hi0, DCut res,
                                         uint32_t target_n, double target_m, uint32_t above_n0 = 0,
                                         double above_m0 = 0.0) {
    const int t = static_cast<int>(threadIdx.x);
    uint32_t lo = lo0, hi = hi0;
    uint32_t above_n = above_n0;
    double above_m = above_m0;
    for (int round = 0; round < 8; ++round) {
        const uint32_t span = hi - lo;
        int sh = 0;
        while ((span >> sh) >= static_cast<uint32_t>(kDBins)) ++sh;
        for (int i = t; i < kDBins; i += kT) {
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
        // thread t owns bins kDBins - 1 - 2t - q, q = 0, 1 (descending)
        uint32_t hc[2], oc = 0;
        double hm[2], om = 0.0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int bin = kDBins - 1 - 2 * t - q;
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
        for (int q = 0; q < 2; ++q) {
            const bool hit = MASS ? (cum_m < target_m && cum_m + hm[q] >= target_m)
                                  : (cum_c < target_n && cum_c + hc[q] >= target_n);
            if (hit) {
                f.sel_bin = kDBins - 1 - 2 * t - q;
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
            if (t == 0) f.res_ok = 0u;
            block_scan2(oc2, om2, &ec2, &em2, &tc2, &tm2, f);
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
__device__ __forceinline__ void debug_topk_list(const SampleArgs& a, int b, FinSmem& f, int L, uint32_t kappa,
                                                uint32_t maxkey, uint32_t n) {
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

// Debug: the final distribution over the whole row.  kept(i, x, key) says
// whether element i is kept; weight(c, x) returns its probability.
template <int DT, int NL, typename K, typename Wt>
__device__ __forceinline__ void debug_probs(const SampleArgs& a, int b, K kept, Wt weight) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    float* pr = a.probs_out + static_cast<int64_t>(b) * a.V;
    const int t = static_cast<int>(threadIdx.x);
    for (int c = 0; c < a.chunks; ++c) {
        const uint32_t tbase = static_cast<uint32_t>(c * static_cast<int>(G::ELEMS) + t * VEC);
        u32x4_t_ d[NL];
        load_chunk<DT, NL>(a, b, c, d);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t i = tbase + j * G::SLOT + e;
                if (i >= static_cast<uint32_t>(a.V)) continue;
                const float x = elem<DT>(d[j], e);
                pr[i] = kept(static_cast<uint32_t>(i), x, f32_key(x)) ? weight(c, x) : 0.0f;
            }
            slot_fence();
        }
    }
}

// The draw inside chunk cs: re-reads the chunk, weights its kept elements
// 2^(x c - rc) * sc, finds the first element whose inclusive prefix (in
// token order, starting at `before`) passes `target`.  Returns the token, or
// the chunk's last kept element when rounding leaves the target unreached.
template <int DT, int NL, typename K>
__device__ __forceinline__ int32_t draw_in_chunk(const SampleArgs& a, FinSmem& f, int b, int cs, float cc,
                                                 float rcs, double sc, double before, double target, K kept) {
    using G = Geo<DT, NL>;
    constexpr int VEC = G::VEC;
    const int t = static_cast<int>(threadIdx.x), lane = lane_id(), wid = wave_id();
    const uint32_t tbase = static_cast<uint32_t>(cs * static_cast<int>(G::ELEMS) + t * VEC);
    u32x4_t_ d[NL];
    load_chunk<DT, NL>(a, b, cs, d);
    auto wt = [&](int j, int e) {
        const float x = elem<DT>(d[j], e);
        const uint32_t i = (tbase + j * G::SLOT + e);
        return (x > -INFINITY && kept(i, x, f32_key(x))) ? __builtin_amdgcn_exp2f(fmaf(x, cc, -rcs)) : 0.0f;
    };
    // per-slot sums (fp32 per thread, fp64 across the block)
    int my_last = -1;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float w = wt(j, e);
            s += w;
            if (w > 0.0f) my_last = static_cast<int>(tbase + j * G::SLOT + e);
        }
        const double ws = wave_sum_dpp(static_cast<double>(s));
        if (lane == 0) f.slot[wid][j] = ws;
        slot_fence();
    }
    if (t == 0) {
        f.tok = -1;
        f.last = -1;
    }
    __syncthreads();
    if (t < NL) f.slott[t] = (f.slot[0][t] + f.slot[1][t] + f.slot[2][t] + f.slot[3][t]) * sc;
    atomicMax(&f.last, my_last);
    __syncthreads();
    if (t == 0) {
        double run = before;
        int js = -1;
        for (int j = 0; j < NL; ++j) {
            if (run + f.slott[j] > target) {
                js = j;
                break;
            }
            run += f.slott[j];
            slot_fence();
        }
        f.jstar = js;
        f.before = run;
    }
    __syncthreads();
    const int js = f.jstar;
    if (js >= 0) {
        float own = 0.0f;
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if (j == js)
#pragma unroll
                for (int e = 0; e < VEC; ++e) own += wt(j, e);
        uint32_t ec, tc;
        double em, tm2;
        block_scan2(0u, static_cast<double>(own) * sc, &ec, &em, &tc, &tm2, f);
        const double start = f.before + em;
        if (start <= target && start + static_cast<double>(own) * sc > target) {
            double run = start;
            int tok = -1;
#pragma unroll
            for (int j = 0; j < NL; ++j)
                if (j == js)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float w = wt(j, e);
                        run += static_cast<double>(w) * sc;
                        if (tok < 0 && w > 0.0f && run > target) tok = static_cast<int>(tbase + j * G::SLOT + e);
                    }
            if (tok >= 0) f.tok = tok;
        }
    }
    __syncthreads();
    const int32_t tok = f.tok >= 0 ? f.tok : f.last;
    __syncthreads();
    return tok;
}

// Finishes row b once every chunk has published (for histogram rows: both
// publications; gstar and kmin are the finisher's decision).
template <int DT, int NL>
__device__ __forceinline__ void finish_row(const SampleArgs& a, SplitSmem& sm, int b, const RowParams& prm,
                                           uint32_t mode, float cc, uint64_t word, float gstar, uint32_t kmin) {
    using G = Geo<DT, NL>;
    FinSmem& f = sm.f;
    const int t = static_cast<int>(threadIdx.x);
    const int S = a.chunks;
    const double u = uniform24(word);
    const SplitRec* recs = a.rec + static_cast<int64_t>(b) * a.rec_stride;

    // the records
    const __amdgpu_buffer_rsrc_t rr = l2_rsrc(recs, static_cast<uint32_t>(S) * sizeof(SplitRec));
    if (t < S) {
        f.cm[t] = l2_f32(rr, DST_REC_OFF(t, m));
        f.camax[t] = l2_u32(rr, DST_REC_OFF(t, amax));
        f.ctheta[t] = l2_f32(rr, DST_REC_OFF(t, theta));
        f.ccnt[t] = l2_u32(rr, DST_REC_OFF(t, cnt));
        f.cz[t] = l2_f64(rr, DST_REC_OFF(t, z));
        f.crc[t] = l2_f32(rr, DST_REC_OFF(t, rc));
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
        if (t < S) f.csc[t] = sc;
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
        const double tok_target = u * zrow;
        const int32_t tok = draw_in_chunk<DT, NL>(a, f, b, cs, cc, f.crc[cs], f.csc[cs], f.before, tok_target,
                                                  [](uint32_t, float, uint32_t) { return true; });
        if (t == 0) {
            a.tokens_out[b] = tok;
            if (a.kept_out) a.kept_out[b] = a.V;
            if (a.rand_out) a.rand_out[b] = word;
        }
        if (a.probs_out) {
            const double inv = 1.0 / zrow;
            debug_probs<DT, NL>(a, b, [](uint32_t, float, uint32_t) { return true; },
                                [&](int c, float x) {
                                    return static_cast<float>(
                                        static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, cc, -f.crc[c]))) *
                                        f.csc[c] * inv);
                                });
        }
        // the debug top-64 comes from the candidates (published with rank 64)
        if (!a.topk_idx_out) return;
    }

    // ---- candidate list: every published candidate >= kappa, in token order.
    if (t < kWave) {
        const uint32_t cn = t < S ? f.ccnt[t] : 0u;
        const bool over = t < S && cn > static_cast<uint32_t>(kSplitCap);
        const uint32_t cv = over ? 0u : cn;
        const uint32_t incl = wave_scan_u32_dpp(cv);
        if (t < S) f.coff[t] = incl - cv;
        const uint32_t tot = readlane_u32(incl, S - 1);
        const uint32_t kap = wave_max_u32_dpp(t < S ? f32_key(f.ctheta[t]) : 0u);
        const bool any_over = __ballot(over) != 0ull;
        if (t == 0) {
            f.coff[S] = tot;
            f.list_n = tot;
            f.kappa = kap;
            f.bad = any_over ? 1u : 0u;
        }
    }
    __syncthreads();
    const uint32_t kappa = f.kappa, maxkey = f.maxkey;
    bool bad = f.bad != 0u;
    // Loads the entries of the chunk blocks (at offset `region`; per-chunk
    // counts prefixed in f.coff, raw_n in all) that pass keep(key), in
    // order, into the LDS list, in batches of 8 entries per thread (thread t
    // takes 8 consecutive entries); returns how many passed.  side(chunk,
    // key) sees every entry once.
    auto load_list = [&](uint32_t raw_n, int region, auto keep, auto side) {
        const __amdgpu_buffer_rsrc_t cr =
            l2_rsrc(a.cand + static_cast<int64_t>(b) * a.rec_stride * kSplitCandStride,
                    static_cast<uint32_t>(S) * kSplitCandStride * sizeof(uint64_t));
        uint32_t L32 = 0;
        for (uint32_t batch = 0; batch < raw_n; batch += 8 * kT) {
            uint64_t v[8];
            int ch[8];
            uint32_t nk = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t fi = batch + 8 * static_cast<uint32_t>(t) + q;
                int lo = 0, hi = S - 1;       // the chunk c with coff[c] <= fi < coff[c + 1]
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (f.coff[mid] <= fi) lo = mid; else hi = mid - 1;
                }
                ch[q] = lo;
                const uint32_t e = static_cast<uint32_t>(lo) * kSplitCandStride + region + (fi - f.coff[lo]);
                v[q] = l2_u64(cr, fi < raw_n ? e * 8u : kL2None);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t fi = batch + 8 * static_cast<uint32_t>(t) + q;
                if (fi < raw_n) {
                    const uint32_t k = static_cast<uint32_t>(v[q] >> 32);
                    side(ch[q], k);
                    nk += keep(k) ? 1u : 0u;
                }
            }
            uint32_t ec, tc;
            double em, tm2;
            block_scan2(nk, 0.0, &ec, &em, &tc, &tm2, f);
            uint32_t pos = L32 + ec;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t fi = batch + 8 * static_cast<uint32_t>(t) + q;
                const uint32_t k = static_cast<uint32_t>(v[q] >> 32);
                if (fi < raw_n && keep(k)) {
                    if (pos < static_cast<uint32_t>(kListMax)) {
                        f.key[pos] = k;
                        f.idx[pos] = static_cast<uint32_t>(v[q]);
                        f.w[pos] = __builtin_amdgcn_exp2f(fmaf(key_f32(k), cc, -rref));
                    }
                    ++pos;
                }
            }
            L32 += tc;
        }
        __syncthreads();
        return L32;
    };
    uint32_t L32 = 0;
    if (!bad) {
        L32 = load_list(f.list_n, 0, [&](uint32_t k) { return k >= kappa; }, [](int, uint32_t) {});
        bad = L32 > static_cast<uint32_t>(kListMax);
    }
    const int L = bad ? 0 : static_cast<int>(L32);

    if (a.topk_idx_out) {
        const uint32_t n = prm.k < kDebugTopK ? static_cast<uint32_t>(prm.k) : static_cast<uint32_t>(kDebugTopK);
        if (!bad) {
            debug_topk_list(a, b, f, L, kappa, maxkey, n);
        } else {
            __syncthreads();
            exact_debug_topk<DT, kT>(row_ptr(a, b, G::ES), a.V, static_cast<int>(n),
                                     a.topk_idx_out + static_cast<int64_t>(b) * kDebugTopK, sm.e);
            __syncthreads();
        }
    }
    if (mode == kModeFull) return;

    if (mode == kModeHist) {
        // ---- top-p and / or min_p through the weight histogram: the bin G*
        // elements' cut, then the draw over the kept masses per chunk
        const bool bin = prm.top_p;
        const double target = static_cast<double>(prm.p) * zrow;
        if (t < kWave) {
            const bool has = t < S;
            const int tc = has ? t : 1 << 20;   // past the buffer: reads 0
            const double sc = has ? f.csc[t] : 0.0;
            const double aa = l2_f64(rr, DST_REC_OFF(tc, am_all)) * sc;
            const double ak = l2_f64(rr, DST_REC_OFF(tc, am_kept)) * sc;
            const uint32_t na = l2_u32(rr, DST_REC_OFF(tc, an_all));
            const uint32_t nk = l2_u32(rr, DST_REC_OFF(tc, an_kept));
            const uint32_t bc = l2_u32(rr, DST_REC_OFF(tc, bcnt));
            const bool over = has && bc > static_cast<uint32_t>(kSplitBinCap);
            const uint32_t bcv = over ? 0u : bc;
            const uint32_t incl = wave_scan_u32_dpp(bcv);
            if (has) {
                f.coff[t] = incl - bcv;
                f.ckept[t] = ak;
            }
            const double A = wave_sum_dpp(aa);
            const uint32_t NA = wave_sum_u32_dpp(na), NK = wave_sum_u32_dpp(nk);
            const bool any_over = __ballot(over) != 0ull;
            if (t == 0) {
                f.list_n = readlane_u32(incl, S - 1);
                f.amass = A;
                f.anum = NA;
                f.sel_c = NK;
                f.bad = any_over ? 1u : 0u;
            }
        }
        __syncthreads();
        const double A = f.amass;
        const uint32_t NA = f.anum, NK = f.sel_c;
        bool hok = f.bad == 0u;
        uint32_t Lb = 0;
        if (hok && bin) {
            Lb = load_list(f.list_n, kSplitCap, [](uint32_t) { return true; }, [](int, uint32_t) {});
            hok = Lb <= static_cast<uint32_t>(kListMax);
        }
        if (hok) {
            DCut cp{0u, 0xffffffffu};   // the top-p cut; without top-p the whole bin (it is empty)
            if (bin) {
                const Found fb = descent<true>(f, static_cast<int>(Lb), 0u, maxkey, DCut{0u, 0xffffffffu}, 0u,
                                               target, NA, A);
                if (fb.ok) cp = fb.cut;
                else if (A >= target) cp = DCut{0xffffffffu, 0u};   // rounding moved the crossing above the bin
                // else: rounding moved it below the bin, which is kept whole
            }
            const DCut fc = kmin > cp.key ? DCut{kmin, 0xffffffffu} : cp;
            // the bin's kept elements: their count, and their mass per chunk
            uint32_t bn = 0;
            for (int i = t; i < static_cast<int>(Lb); i += kT) {
                const uint32_t k = f.key[i];
                if (k >= kmin && kept_by(fc, k, f.idx[i])) {
                    ++bn;
                    atomicAdd(&f.ckept[f.idx[i] / G::ELEMS], static_cast<double>(f.w[i]));
                }
            }
            uint32_t ec, bn_all;
            double em, tm2;
            block_scan2(bn, 0.0, &ec, &em, &bn_all, &tm2, f);
            if (t < kWave) {
                const double kc = t < S ? f.ckept[t] : 0.0;
                const double incl = wave_scan_f64_dpp(kc);
                const double W = readlane_f64(incl, S - 1);
                const uint64_t bal = __ballot(t < S && incl > u * W);
                const int cs = bal ? __ffsll(static_cast<long long>(bal)) - 1 : S - 1;
                const double before = readlane_f64(incl - kc, cs);
                if (t == 0) {
                    f.cstar = cs;
                    f.before = before;
                    f.zrow = W;   // the kept mass, relative to rref
                }
            }
            __syncthreads();
            const int cs = f.cstar;
            const double W = f.zrow;
            auto keptf = [&](uint32_t i, float x, uint32_t k) {
                const float g = weight_bin(x, cc);
                return k >= kmin && (g > gstar || (g == gstar && kept_by(fc, k, i)));
            };
            const int32_t tok =
                draw_in_chunk<DT, NL>(a, f, b, cs, cc, f.crc[cs], f.csc[cs], f.before, u * W, keptf);
            if (t == 0) {
                a.tokens_out[b] = tok;
                if (a.kept_out) a.kept_out[b] = static_cast<int32_t>(NK + bn_all);
                if (a.rand_out) a.rand_out[b] = word;
            }
            if (a.probs_out) {
                const double inv = 1.0 / W;
                debug_probs<DT, NL>(a, b, keptf, [&](int c, float x) {
                    return static_cast<float>(
                        static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, cc, -f.crc[c]))) * f.csc[c] * inv);
                });
            }
            return;
        }
        __syncthreads();
        exact_row<DT, kT>(a, b, row_ptr(a, b, G::ES), prm, word, u, sm.e);
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
        kp_in_list = fp.ok;
        if (fp.ok) cut = fp.cut;
    }
    if (ok && prm.min_p > 0.0f) {
        const double xm = static_cast<double>(m) + static_cast<double>(prm.T) * log(static_cast<double>(prm.min_p));
        const float xf = static_cast<float>(xm);
        const uint32_t km = f32_key(xf) + (static_cast<double>(xf) < xm ? 1u : 0u);
        if (kp_in_list) {
            if (km > cut.key) cut = DCut{km, 0xffffffffu};
        } else if (km >= kappa) {
            cut = DCut{km, 0xffffffffu};
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
                            [&](uint32_t i, float, uint32_t k) { return k >= kappa && kept_by(fc, k, i); },
                            [&](int, float x) {
                                return static_cast<float>(
                                    static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x, cc, -rref))) * inv);
                            });
    }
}

// The min_p threshold as an order key: the smallest key whose value is
// >= m + T ln(min_p) (computed in fp64).
__device__ __forceinline__ uint32_t min_p_key(float m, const RowParams& prm) {
    const double xm = static_cast<double>(m) + static_cast<double>(prm.T) * log(static_cast<double>(prm.min_p));
    const float xf = static_cast<float>(xm);
    return f32_key(xf) + (static_cast<double>(xf) < xm ? 1u : 0u);
}

struct HistDec {
    float gstar;     // the row's boundary weight bin (-inf: no top-p)
    uint32_t kmin;   // min_p key (0: none)
    bool go;         // false: the histogram could not place the boundary
};

// The finisher's decision for a histogram row, from the chunks' first
// publication: the row's histogram (the chunks' bins shifted onto the row's
// grid, scaled to the row maximum; every chunk's deepest bin, which holds
// all its deeper weights, left out), the bin G* where the descending mass
// first reaches p of the row's, and the min_p key.  Published to the row's
// decision word (data, then the epoch once the data stores have completed).
template <int DT, int NL>
__device__ __forceinline__ HistDec hist_decide(const SampleArgs& a, FinSmem& f, int b, const RowParams& prm,
                                               float cc) {
    const int t = static_cast<int>(threadIdx.x);
    const int S = a.chunks;
    const SplitRec* recs = a.rec + static_cast<int64_t>(b) * a.rec_stride;
    if (t < kWave) {
        const bool has = t < S;
        const __amdgpu_buffer_rsrc_t rr = l2_rsrc(recs, static_cast<uint32_t>(S) * sizeof(SplitRec));
        const int tc = has ? t : 1 << 20;
        const float cm0 = l2_f32(rr, DST_REC_OFF(tc, m));
        const float crc = l2_f32(rr, DST_REC_OFF(tc, rc));
        const double cz = l2_f64(rr, DST_REC_OFF(tc, z));
        const float cm = has ? cm0 : -INFINITY;
        const float m = wave_max_dpp(cm);
        const float rref = m * cc;
        const double sc = has && cm > -INFINITY ? exp2(static_cast<double>(crc) - static_cast<double>(rref)) : 0.0;
        const double zrow = wave_sum_dpp(cz * sc);
        if (has) {
            f.csc[t] = sc;
            f.cm[t] = cm;
        }
        if (t == 0) {
            f.zrow = zrow;
            f.maxkey = f32_key(m);
            f.sel_bin = -1;
        }
    }
    __syncthreads();
    const float m = key_f32(f.maxkey);
    HistDec d{-INFINITY, 0u, true};
    if (prm.top_p) {
        const float gtop = weight_bin(m, cc);
        // thread t sums the row's bins q = 4t .. 4t + 3 (bin gtop - q), four
        // chunks' loads in flight at a time
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
        const __amdgpu_buffer_rsrc_t hr = l2_rsrc(a.hist + static_cast<int64_t>(b) * a.rec_stride * kWBins,
                                                  static_cast<uint32_t>(S) * kWBins * sizeof(float));
        for (int c0 = 0; c0 < S; c0 += 8) {
            float v[8][4];
#pragma unroll
            for (int cq = 0; cq < 8; ++cq) {
                const int c = c0 + cq;
                const float shf = c < S ? gtop - weight_bin(f.cm[c], cc) : INFINITY;
                const int sh = shf < static_cast<float>(kWBins) ? static_cast<int>(shf) : kWBins;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * t + j - sh;
                    const bool in = r >= 0 && r < kWBins - 1;
                    v[cq][j] = l2_f32(hr, in ? static_cast<uint32_t>(c * kWBins + r) * 4u : kL2None);
                }
            }
#pragma unroll
            for (int cq = 0; cq < 8; ++cq) {
                const double sc = c0 + cq < S ? f.csc[c0 + cq] : 0.0;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] += static_cast<double>(v[cq][j]) * sc;
            }
        }
        if (t == kT - 1) acc[3] = 0.0;   // the row's deepest bin
        const double own = acc[0] + acc[1] + acc[2] + acc[3];
        uint32_t ec, tc;
        double em, tm;
        block_scan2(0u, own, &ec, &em, &tc, &tm, f);
        const double target = static_cast<double>(prm.p) * f.zrow;
        double cum = em;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (cum < target && cum + acc[j] >= target) f.sel_bin = 4 * t + j;
            cum += acc[j];
        }
        __syncthreads();
        const int qs = f.sel_bin;
        d.go = qs >= 0;
        d.gstar = gtop - static_cast<float>(qs);
    }
    if (prm.min_p > 0.0f) d.kmin = min_p_key(m, prm);
    if (t == 0) {
        uint32_t* dw = a.dec + static_cast<int64_t>(b) * 4;
        st_dev(dw + 1, __float_as_uint(d.gstar));
        st_dev(dw + 2, d.kmin);
        st_dev(dw + 3, d.go ? 1u : 2u);
        wait_all_memory();
        st_dev(dw, a.epoch);
    }
    __syncthreads();
    return d;
}

// A histogram row's decision word, as a chunk reads it (thread 0 polls,
// bounded); go is false on an abort or when the wait runs out.
__device__ __forceinline__ HistDec wait_decision(const SampleArgs& a, int b, ChunkSmem& sm) {
    if (threadIdx.x == 0) {
        const uint32_t* dw = a.dec + static_cast<int64_t>(b) * 4;
        uint32_t st = 0, g = 0, km = 0;
        for (int spin = 0; spin < kSpinLimit; ++spin) {
            if (ld_dev(dw) == a.epoch) {
                asm volatile("" ::: "memory");   // the data loads stay after the epoch load
                const __amdgpu_buffer_rsrc_t r = l2_rsrc(dw, 16);
                g = l2_u32(r, 4);
                km = l2_u32(r, 8);
                st = l2_u32(r, 12);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        sm.wtot[0][0] = st;
        sm.wtot[0][1] = g;
        sm.wtot[0][2] = km;
    }
    __syncthreads();
    const HistDec d{__uint_as_float(sm.wtot[0][1]), sm.wtot[0][2], sm.wtot[0][0] == 1u};
    __syncthreads();
    return d;
}

// Waits (bounded) until the row's other chunks have flagged `value`; true
// when one of them never did.
__device__ __forceinline__ bool wait_flags(const SampleArgs& a, int b, uint32_t value, SplitSmem& sm) {
    const int S = a.chunks;
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        const uint32_t* fl = a.flags + static_cast<int64_t>(b) * kSplitMaxChunks;
        int late = 0;
        for (int spin = 0;; ++spin) {
            const uint32_t fv = lane < S - 1 ? ld_dev(fl + lane) : value;
            if (__ballot(fv != value) == 0ull) break;
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
    return late;
}

template <int DT, int NL>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(DST_SPLIT_WAVES_PER_EU, 8)))
void sample_split_kernel(SampleArgs a) {
    __shared__ SplitSmem sm;
    const int S = a.chunks;
    // workgroup -> (row, chunk): XCD x = blockIdx mod 8 takes rows x, x + 8, ...;
    // a row's chunks are consecutive on its XCD, chunk S - 1 last
    // (readfirstlane: the compiler cannot see through the division that
    // these are wave-uniform, and a row pointer in vector registers would
    // turn every buffer load into a loop over lanes)
    const int x = static_cast<int>(blockIdx.x) & (kSplitXcds - 1);
    const int kk = static_cast<int>(blockIdx.x) / kSplitXcds;
    const int rl = __builtin_amdgcn_readfirstlane(kk / S);
    const int c_own = __builtin_amdgcn_readfirstlane(kk - rl * S);
    const int b = __builtin_amdgcn_readfirstlane(rl * kSplitXcds + x);
    if (b >= a.B) return;
    const bool finisher = c_own == S - 1;

    const RowParams prm = row_params(a.temperature, a.top_k, a.top_p, a.min_p, b, a.V);
    const bool dbg_list = a.topk_idx_out != nullptr;
    // top-p rows aim at about kPList candidates over the whole row
    const int jtopp = kPList / S < kJMax ? (kPList / S > 1 ? kPList / S : 1) : kJMax;
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
        jrank = jtopp;
        jmin = prm.k;
    } else if (prm.top_p || prm.min_p > 0.0f) {
        mode = kModeHist;
        jrank = jmin = dbg_list ? kJDebug : 0;
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

    u32x4_t_ d[NL];
    load_chunk<DT, NL>(a, b, c_own, d);
    const float rc = chunk_phase<DT, NL>(a, sm.c, b, c_own, d, mode, cc, jrank, jmin,
                                         mode == kModeHist && prm.top_p);
    wait_all_memory();
    __syncthreads();
    uint32_t* own_flag = a.flags + static_cast<int64_t>(b) * kSplitMaxChunks + c_own;
    if (!finisher) {
        if (threadIdx.x == 0) st_dev(own_flag, a.epoch);
        if (mode != kModeHist) return;
        // a histogram row's chunk: the second publication, once decided
        const HistDec hd = wait_decision(a, b, sm.c);
        if (!hd.go) return;
        hist_phase2<DT, NL>(a, sm.c, b, c_own, d, cc, rc, hd.gstar, hd.kmin, prm.top_p);
        wait_all_memory();
        __syncthreads();
        if (threadIdx.x == 0) st_dev(own_flag, a.epoch + 1u);
        return;
    }
    // the finisher: waits for the row's other chunks (bounded); a chunk that
    // never published sends the row to the exact routine, which reads it
    const uint64_t word = a.temperature ? request_word(a.seed, ld_global<int64_t>(a.uid + b), a.step) : 0ull;
    bool late = wait_flags(a, b, a.epoch, sm);
    HistDec hd{-INFINITY, 0u, true};
    if (mode == kModeHist) {
        if (!late) {
            hd = hist_decide<DT, NL>(a, sm.f, b, prm, cc);
        } else if (threadIdx.x == 0) {
            uint32_t* dw = a.dec + static_cast<int64_t>(b) * 4;
            st_dev(dw + 3, 2u);   // abort: the other chunks stop waiting
            wait_all_memory();
            st_dev(dw, a.epoch);
        }
        if (!late && hd.go) {
            hist_phase2<DT, NL>(a, sm.c, b, c_own, d, cc, rc, hd.gstar, hd.kmin, prm.top_p);
            wait_all_memory();
            __syncthreads();
            late = wait_flags(a, b, a.epoch + 1u, sm);
        }
        late = late || !hd.go;
    }
    if (late) {
        exact_row<DT, kT>(a, b, row_ptr(a, b, Geo<DT, NL>::ES), prm, word, uniform24(word), sm.e);
        return;
    }
    finish_row<DT, NL>(a, sm, b, prm, mode, cc, word, hd.gstar, hd.kmin);
}

template <int DT, int NL>
hipError_t launch_nl(const SampleArgs& args, hipStream_t stream) {
    const int rows_per_xcd = (args.B + kSplitXcds - 1) / kSplitXcds;
    const dim3 grid(static_cast<unsigned>(kSplitXcds * rows_per_xcd * args.chunks));
    hipLaunchKernelGGL((sample_split_kernel<DT, NL>), grid, dim3(kT), 0, stream, args);
    return hipGetLastError();
}

}  // namespace

int split_plan(int V, int dtype, int* chunks) {
    const int vec = dtype == kDtypeF32 ? 4 : 8;
    auto nchunks = [&](int nl) {
        const int64_t e = static_cast<int64_t>(kSplitThreads) * nl * vec;
        return static_cast<int64_t>((V + e - 1) / e);
    };
    // the large chunk unless that leaves fewer than four chunks per row (short
    // rows fill the GPU with more, smaller chunks)
    const int big = dtype == kDtypeF32 ? DST_SPLIT_NL_F32 : DST_SPLIT_NL_BF16;
    const int nl = nchunks(big) >= 4 ? big : 4;
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
    if (dtype == kDtypeF32) {
        if (nl == 4) return launch_nl<kDtypeF32, 4>(args, stream);
        if (nl == DST_SPLIT_NL_F32) return launch_nl<kDtypeF32, DST_SPLIT_NL_F32>(args, stream);
    } else {
        if (nl == 4) return launch_nl<kDtypeBF16, 4>(args, stream);
        if (nl == DST_SPLIT_NL_BF16) return launch_nl<kDtypeBF16, DST_SPLIT_NL_BF16>(args, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dst
