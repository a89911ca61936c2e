// Exact per-row sampler, as device functions of one workgroup (BLOCK
// threads) that owns a row and re-reads it from memory as often as needed.
//
// "The engine and the sampler", section "The sampler" (sample_torch):
// softmax(logits / T), rank in descending order, zero the ranks >= top_k,
// renormalise, zero the ranks whose preceding mass is already >= top_p, put
// the probabilities back in token order, draw one token.  The same result
// is reached without sorting:
//   1. row maximum and lowest-index argmax (greedy rows and top_k = 1 stop);
//   2. top-k: 8-bit-digit radix selection of the k-th largest logit key, then
//      the index of the last kept tie (ties go to the lowest indices);
//   3. W_K = sum of exp((x - m) / T) over the top-k set (fp64);
//   4. top-p: the same radix descent weighted by mass: at each digit level it
//      finds the bucket where the exclusive prefix mass crosses p * W_K, and
//      finally how many equal-logit ties stay below the threshold;
//   4b. min_p (the pages' exercise: p_i >= min_p * p_max on the full
//      distribution, intersected with the top-k / top-p mask): the keys at
//      or above m + T ln(min_p), a prefix too, so the shorter prefix stays;
//   5. W = kept mass; the draw walks the row in token order in tiles,
//      scanning per-thread partial sums, until the prefix exceeds u * W.
// The kept set is always a prefix of the descending order, held as a cut
// (key, last index): token i is kept iff key_i > key, or key_i == key and
// i <= last index.
//
// This path handles any k, any p and any row (unaligned, ragged); it costs
// several passes over the row.  The single-pass kernel falls back to it for
// the rows it cannot finish from one read.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace dst {

struct Cut {
    uint32_t key;
    int64_t last;   // kept ties have index <= last
    __device__ __forceinline__ bool keep(int64_t i, uint32_t k) const {
        return k > key || (k == key && i <= last);
    }
};

// exp((x - m) / T) in fp64 (the oracle's weight, to fp64 rounding).
__device__ __forceinline__ double exact_weight(float x, float m, float T) {
    return exp((static_cast<double>(x) - static_cast<double>(m)) / static_cast<double>(T));
}

constexpr int kMaxWaves = 16;

struct ExactSmem {
    uint32_t cnt[256];
    double mass[256];
    double dscr[kMaxWaves + 1];
    uint64_t uscr[kMaxWaves + 1];
    int64_t iscr[kMaxWaves + 1];
    uint32_t sel_digit, sel_rem, sel_cnt;
    double sel_above;
    int64_t found;
    uint32_t list_key[kDebugTopK];
    int32_t list_idx[kDebugTopK];
    uint32_t list_n;
};

// Visits every element of the row (order across threads unspecified).
template <int DT, int BLOCK, typename F>
__device__ __forceinline__ void row_foreach(const void* row, int V, F&& f) {
    constexpr int VEC = Elem<DT>::kVec;
    int64_t start = 0;
    if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
        const int64_t nvec = V / VEC;
        for (int64_t v = threadIdx.x; v < nvec; v += BLOCK) {
            float x[VEC];
            Elem<DT>::vec(row, v * VEC, x);
#pragma unroll
            for (int j = 0; j < VEC; ++j) f(v * VEC + j, x[j]);
        }
        start = nvec * VEC;
    }
    for (int64_t i = start + threadIdx.x; i < V; i += BLOCK) f(i, Elem<DT>::at(row, i));
}

// Thread t's slice of the index-ordered tile starting at `base`:
// [base + t*VEC, base + t*VEC + VEC) clipped to V.  Returns the count.
template <int DT>
__device__ __forceinline__ int tile_slice(const void* row, int V, int64_t base, float* x) {
    constexpr int VEC = Elem<DT>::kVec;
    const int64_t s = base + static_cast<int64_t>(threadIdx.x) * VEC;
    if (s >= V) return 0;
    if (s + VEC <= V && (reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
        Elem<DT>::vec(row, s, x);
        return VEC;
    }
    const int n = static_cast<int>(V - s < VEC ? V - s : VEC);
    for (int j = 0; j < n; ++j) x[j] = Elem<DT>::at(row, s + j);
    return n;
}

// r-th largest key (1-based) among elements with pred(i, key); returns the
// key, and through *rem how many elements equal to it are taken and through
// *eq how many equal elements satisfy pred.
template <int DT, int BLOCK, typename P>
__device__ __forceinline__ uint32_t exact_select_kth(const void* row, int V, uint32_t r, P pred, ExactSmem& sm,
                                     uint32_t* rem, uint32_t* eq) {
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int t = threadIdx.x; t < 256; t += BLOCK) sm.cnt[t] = 0;
        __syncthreads();
        row_foreach<DT, BLOCK>(row, V, [&](int64_t i, float x) {
            const uint32_t k = f32_key(x);
            if ((k & mask) == prefix && pred(i, k)) atomicAdd(&sm.cnt[(k >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t cum = 0;
            int d = 255;
            for (; d > 0; --d) {
                if (cum + sm.cnt[d] >= r) break;
                cum += sm.cnt[d];
            }
            sm.sel_digit = static_cast<uint32_t>(d);
            sm.sel_rem = r - cum;
            sm.sel_cnt = sm.cnt[d];
        }
        __syncthreads();
        prefix |= sm.sel_digit << shift;
        mask |= 255u << shift;
        r = sm.sel_rem;
    }
    *rem = r;
    *eq = sm.sel_cnt;
    return prefix;
}

// Index of the n-th (1-based) element in token order with key == key and
// pred(i, key).  Returns -1 if there are fewer.
template <int DT, int BLOCK, typename P>
__device__ __forceinline__ int64_t exact_nth_equal(const void* row, int V, uint32_t key, uint32_t n, P pred,
                                   ExactSmem& sm) {
    constexpr int VEC = Elem<DT>::kVec;
    constexpr int64_t TILE = static_cast<int64_t>(BLOCK) * VEC;
    uint64_t running = 0;
    if (threadIdx.x == 0) sm.found = -1;
    __syncthreads();
    for (int64_t base = 0; base < V; base += TILE) {
        float x[VEC];
        const int cnt_n = tile_slice<DT>(row, V, base, x);
        const int64_t s = base + static_cast<int64_t>(threadIdx.x) * VEC;
        uint64_t mine = 0;
        for (int j = 0; j < cnt_n; ++j) {
            const uint32_t k = f32_key(x[j]);
            mine += (k == key && pred(s + j, k)) ? 1u : 0u;
        }
        uint64_t total;
        const uint64_t excl = block_excl_scan<BLOCK>(mine, sm.uscr, &total);
        if (running + total >= n) {
            if (running + excl < n && running + excl + mine >= n) {
                uint64_t c = running + excl;
                for (int j = 0; j < cnt_n; ++j) {
                    const uint32_t k = f32_key(x[j]);
                    if (k == key && pred(s + j, k) && ++c == n) { sm.found = s + j; break; }
                }
            }
            __syncthreads();
            return sm.found;
        }
        running += total;
    }
    return -1;
}

// Cut holding the r-th largest element (1-based) and everything above it.
template <int DT, int BLOCK, typename P>
__device__ __forceinline__ Cut exact_cut_by_count(const void* row, int V, uint32_t r, P pred, ExactSmem& sm) {
    uint32_t rem, eq;
    const uint32_t key = exact_select_kth<DT, BLOCK>(row, V, r, pred, sm, &rem, &eq);
    Cut c{key, INT64_MAX};
    if (rem < eq) c.last = exact_nth_equal<DT, BLOCK>(row, V, key, rem, pred, sm);
    return c;
}

// Top-p cut inside `base`: the shortest descending-order prefix whose
// exclusive prefix mass reaches `target` ends at the returned cut.  Returns
// `base` itself if the mass never reaches it (rounding only).
template <int DT, int BLOCK>
__device__ __forceinline__ Cut exact_cut_by_mass(const void* row, int V, const Cut& base, double target, float m,
                                 float T, ExactSmem& sm) {
    uint32_t prefix = 0, mask = 0;
    double above = 0.0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int t = threadIdx.x; t < 256; t += BLOCK) {
            sm.cnt[t] = 0;
            sm.mass[t] = 0.0;
        }
        __syncthreads();
        row_foreach<DT, BLOCK>(row, V, [&](int64_t i, float x) {
            const uint32_t k = f32_key(x);
            if ((k & mask) == prefix && base.keep(i, k)) {
                const uint32_t d = (k >> shift) & 255u;
                atomicAdd(&sm.cnt[d], 1u);
                atomicAdd(&sm.mass[d], exact_weight(x, m, T));
            }
        });
        __syncthreads();
        if (threadIdx.x == 0) {
            double cum = above, cum_before_last = above;
            int d = 255, last_nonempty = -1;
            for (; d >= 0; --d) {
                if (sm.cnt[d] == 0) continue;
                last_nonempty = d;
                cum_before_last = cum;
                if (cum + sm.mass[d] >= target) break;
                cum += sm.mass[d];
            }
            if (d < 0) {
                // The prefix mass never reached the target (rounding only).  At
                // the top level nothing is cut; deeper down the crossing stays
                // in the lowest bucket of the range.
                d = shift == 24 ? -1 : last_nonempty;
                cum = cum_before_last;
            }
            sm.sel_digit = static_cast<uint32_t>(d);
            sm.sel_above = cum;
            sm.sel_cnt = d >= 0 ? sm.cnt[d] : 0;
        }
        __syncthreads();
        if (static_cast<int>(sm.sel_digit) < 0) return base;
        prefix |= sm.sel_digit << shift;
        mask |= 255u << shift;
        above = sm.sel_above;
    }
    // prefix is the exact key of the crossing rank; every tie carries the same
    // weight w, and the j-th tie (token order) has exclusive prefix above + j*w
    const double w = exact_weight(key_f32(prefix), m, T);
    const uint32_t ties = sm.sel_cnt;
    const double y = (target - above) / w;
    uint32_t keep_ties = ties;
    if (y < static_cast<double>(ties)) {
        const double cy = ceil(y);
        keep_ties = cy < 1.0 ? 1u : static_cast<uint32_t>(cy);
    }
    Cut c{prefix, base.key == prefix ? base.last : INT64_MAX};
    if (keep_ties < ties)
        c.last = exact_nth_equal<DT, BLOCK>(
            row, V, prefix, keep_ties, [&](int64_t i, uint32_t k) { return base.keep(i, k); }, sm);
    return c;
}

// First n (<= 64) indices of the descending order into out[0..63], -1 padded.
template <int DT, int BLOCK>
__device__ __forceinline__ void exact_debug_topk(const void* row, int V, int n, int32_t* out, ExactSmem& sm) {
    const Cut c = exact_cut_by_count<DT, BLOCK>(row, V, static_cast<uint32_t>(n),
                                                 [](int64_t, uint32_t) { return true; }, sm);
    if (threadIdx.x == 0) sm.list_n = 0;
    __syncthreads();
    row_foreach<DT, BLOCK>(row, V, [&](int64_t i, float x) {
        const uint32_t k = f32_key(x);
        if (c.keep(i, k)) {
            const uint32_t slot = atomicAdd(&sm.list_n, 1u);
            if (slot < kDebugTopK) {
                sm.list_key[slot] = k;
                sm.list_idx[slot] = static_cast<int32_t>(i);
            }
        }
    });
    __syncthreads();
    const int len = sm.list_n < kDebugTopK ? static_cast<int>(sm.list_n) : kDebugTopK;
    if (threadIdx.x < kDebugTopK) out[threadIdx.x] = -1;
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < len) {
        const uint32_t k = sm.list_key[threadIdx.x];
        const int32_t i = sm.list_idx[threadIdx.x];
        int rank = 0;
        for (int e = 0; e < len; ++e) {
            const uint32_t k2 = sm.list_key[e];
            rank += (k2 > k || (k2 == k && sm.list_idx[e] < i)) ? 1 : 0;
        }
        if (rank < n) out[rank] = i;
    }
    __syncthreads();
}

// Debug outputs common to every path once the kept cut is known: the final
// distribution (one more pass) and the descending-order index list.
template <int DT, int BLOCK>
__device__ __forceinline__ void exact_debug_outputs(const SampleArgs& a, int b, const void* row,
                                    const RowParams& prm, const Cut& cut, float m, double W,
                                    ExactSmem& sm) {
    const int V = a.V;
    if (a.probs_out) {
        float* probs = a.probs_out + static_cast<int64_t>(b) * V;
        const double inv = 1.0 / W;
        for (int64_t i = threadIdx.x; i < V; i += BLOCK) {
            const float x = Elem<DT>::at(row, i);
            probs[i] = cut.keep(i, f32_key(x)) ? static_cast<float>(exact_weight(x, m, prm.T) * inv)
                                               : 0.0f;
        }
    }
    if (a.topk_idx_out) {
        const int nk = prm.k < kDebugTopK ? prm.k : kDebugTopK;
        exact_debug_topk<DT, BLOCK>(row, V, nk, a.topk_idx_out + static_cast<int64_t>(b) * kDebugTopK, sm);
    }
}

// Argmax row: token, and the debug outputs of a one-hot distribution.
template <int BLOCK>
__device__ __forceinline__ void finish_argmax_row(const SampleArgs& a, int b, int32_t amax, uint64_t word) {
    if (threadIdx.x == 0) {
        a.tokens_out[b] = amax;
        if (a.kept_out) a.kept_out[b] = 1;
        if (a.rand_out) a.rand_out[b] = word;
    }
    if (a.probs_out) {
        float* probs = a.probs_out + static_cast<int64_t>(b) * a.V;
        for (int64_t i = threadIdx.x; i < a.V; i += BLOCK) probs[i] = i == amax ? 1.0f : 0.0f;
    }
    if (a.topk_idx_out) {
        int32_t* o = a.topk_idx_out + static_cast<int64_t>(b) * kDebugTopK;
        for (int t = threadIdx.x; t < kDebugTopK; t += BLOCK) o[t] = t == 0 ? amax : -1;
    }
}

// The whole row by the exact multi-pass algorithm.  Inline like everything
// else: a call would give the calling kernel a scratch stack.
template <int DT, int BLOCK>
__device__ __forceinline__ void exact_row(const SampleArgs& a, int b, const void* row, const RowParams& prm,
                          uint64_t word, double u, ExactSmem& sm) {
    constexpr int VEC = Elem<DT>::kVec;
    constexpr int64_t TILE = static_cast<int64_t>(BLOCK) * VEC;
    const int V = a.V;

    // 1. maximum, lowest-index argmax
    uint64_t best = 0;
    row_foreach<DT, BLOCK>(row, V, [&](int64_t i, float x) {
        const uint64_t pk = (static_cast<uint64_t>(f32_key(x)) << 32) |
                            static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(i));
        best = pk > best ? pk : best;
    });
    best = block_max<BLOCK>(best, sm.uscr);
    const uint32_t mkey = static_cast<uint32_t>(best >> 32);
    const int32_t amax = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(best));
    const float m = key_f32(mkey);
    if (prm.greedy || prm.k == 1) {
        finish_argmax_row<BLOCK>(a, b, amax, word);
        return;
    }

    // 2. top-k cut
    const auto all = [](int64_t, uint32_t) { return true; };
    Cut cut{0u, INT64_MAX};
    if (prm.k < V) cut = exact_cut_by_count<DT, BLOCK>(row, V, static_cast<uint32_t>(prm.k), all, sm);

    // 3-4. top-p cut inside the top-k set
    if (prm.top_p) {
        double wk = 0.0;
        row_foreach<DT, BLOCK>(row, V, [&](int64_t i, float x) {
            if (cut.keep(i, f32_key(x))) wk += exact_weight(x, m, prm.T);
        });
        wk = block_sum<BLOCK>(wk, sm.dscr);
        cut = exact_cut_by_mass<DT, BLOCK>(row, V, cut, static_cast<double>(prm.p) * wk, m, prm.T, sm);
    }

    // 4b. min_p: p >= min_p * p_max, that is x >= m + T ln(min_p); its kept
    // set is a prefix of the same order, so the intersection is the shorter
    if (prm.min_p > 0.0f) {
        const double xm = static_cast<double>(m) + static_cast<double>(prm.T) * log(static_cast<double>(prm.min_p));
        const float xf = static_cast<float>(xm);
        const uint32_t kmin = f32_key(xf) + (static_cast<double>(xf) < xm ? 1u : 0u);
        if (cut.key < kmin) cut = Cut{kmin, INT64_MAX};
    }

    // 5. kept mass and size
    double W = 0.0;
    uint64_t n = 0;
    row_foreach<DT, BLOCK>(row, V, [&](int64_t i, float x) {
        if (cut.keep(i, f32_key(x))) {
            W += exact_weight(x, m, prm.T);
            ++n;
        }
    });
    W = block_sum<BLOCK>(W, sm.dscr);
    n = block_sum<BLOCK>(n, sm.uscr);

    // 6. inverse CDF in token order: first i with prefix(i) > u * W
    const double target = u * W;
    double running = 0.0;
    int64_t last_kept = -1;
    if (threadIdx.x == 0) sm.found = -1;
    __syncthreads();
    for (int64_t base = 0; base < V; base += TILE) {
        float x[VEC];
        const int cnt_n = tile_slice<DT>(row, V, base, x);
        const int64_t s = base + static_cast<int64_t>(threadIdx.x) * VEC;
        double mine = 0.0;
        int64_t my_last = -1;
        for (int j = 0; j < cnt_n; ++j) {
            if (cut.keep(s + j, f32_key(x[j]))) {
                mine += exact_weight(x[j], m, prm.T);
                my_last = s + j;
            }
        }
        double total;
        const double excl = block_excl_scan<BLOCK>(mine, sm.dscr, &total);
        const int64_t tile_last = block_max<BLOCK>(my_last, sm.iscr);
        last_kept = tile_last > last_kept ? tile_last : last_kept;
        // the first thread whose running prefix passes the target owns the token
        const bool passes = my_last >= 0 && running + excl + mine > target;
        const int64_t cand = passes ? static_cast<int64_t>(threadIdx.x) : INT64_MAX;
        const int64_t owner = -block_max<BLOCK>(-cand, sm.iscr);
        if (owner != INT64_MAX && owner >= 0 && owner < BLOCK) {
            if (static_cast<int64_t>(threadIdx.x) == owner) {
                double c = running + excl;
                int64_t tok = my_last;
                for (int j = 0; j < cnt_n; ++j) {
                    if (cut.keep(s + j, f32_key(x[j]))) {
                        c += exact_weight(x[j], m, prm.T);
                        if (c > target) { tok = s + j; break; }
                    }
                }
                sm.found = tok;
            }
            __syncthreads();
            break;
        }
        running += total;
    }
    __syncthreads();
    const int64_t tok = sm.found >= 0 ? sm.found : last_kept;

    if (threadIdx.x == 0) {
        a.tokens_out[b] = static_cast<int32_t>(tok);
        if (a.kept_out) a.kept_out[b] = static_cast<int32_t>(n);
        if (a.rand_out) a.rand_out[b] = word;
    }
    exact_debug_outputs<DT, BLOCK>(a, b, row, prm, cut, m, W, sm);
}

}  // namespace dst
