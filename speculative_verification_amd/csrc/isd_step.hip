// ISD verify-and-propose step kernels for gfx950.
//
// One kernel does the whole step ("Introspective Diffusion Language Models |
// Summary", section 3.2: verification of the previous proposals and the draw
// of the next ones come out of one forward).  Workgroup b does work item b,
// in this order:
//
//   [pq items]      for each sequence c, each verify row (anchor p_k and, in
//                   sample mode, proposal q_k) and each row segment: stream
//                   the segment once and write its softmax partial (sample)
//                   or argmax partial (greedy).  The workgroup that finishes
//                   the last pq item of sequence c takes the decision for c:
//                   ratios min(1, P(x)/Q(x)) in fp64, the accept test, the
//                   first rejection j by a wavefront ballot, alpha, and the
//                   outputs; it then publishes (j, row-j constants).
//   per sequence c: [mask-row items]  stream a segment of row qn[c, k] and
//                   record the mass of each 2048-element tile; the last
//                   segment of the row merges the tile masses, finds the tile
//                   where the running mass crosses u * S, re-reads that tile
//                   and picks the token (inverse CDF).
//                   [residual items]  wait until c's decision is published,
//                   then stream a segment of rows p[c, j], q[c, j] computing
//                   max(0, P - Q) per tile; the last one does the inverse-CDF
//                   draw over the residual the same way.
//
// A residual item only waits on pq items, which have smaller workgroup
// indices.  Each XCD dispatches its share of the grid in increasing index
// order, so by the time a residual workgroup is resident on an XCD every pq
// workgroup of that XCD has been dispatched; pq workgroups never wait, so all
// of them finish and every wait ends.  The wait is still bounded (spin_limit
// polls) and flags the device error word if it ever gives up.  No global
// atomic is taken per workgroup: completion is counted per row or sequence.
//
// Softmax partials use an integer reference e per wavefront so that
// rescaling is an exact power of two: terms are 2^(x*k2 - e) with
// k2 = log2(e)/T, summed in fp32 over each lane's 32 elements of a tile and
// accumulated in fp64.

#include "isd_device.h"
#include "isd_internal.h"

#include <math.h>

namespace isd {

namespace {

// ---------------------------------------------------------------------------
// Softmax and argmax partials
// ---------------------------------------------------------------------------

__device__ __forceinline__ void st_seg(SegRec *r, float ref, double sum) {
    st64(reinterpret_cast<uint64_t *>(r), pack2(ref, 0.0f));
    st64(reinterpret_cast<uint64_t *>(r) + 1, (uint64_t)__double_as_longlong(sum));
}
__device__ __forceinline__ void ld_seg(const SegRec *r, float &ref, double &sum) {
    ref = lo_f(ld64(reinterpret_cast<const uint64_t *>(r)));
    sum = __longlong_as_double((long long)ld64(reinterpret_cast<const uint64_t *>(r) + 1));
}
// Largest of a lane's 32 elements of a tile, read from the packed words:
// sixteen three-way maxima.
template <typename T>
__device__ __forceinline__ float tile_max(const TileRaw<T> &r) {
    float m = max3_hw(elem<T>(r, 0), elem<T>(r, 1), elem<T>(r, 2));
#pragma unroll
    for (int i = 3; i + 1 < kLaneElems; i += 2) m = max3_hw(m, elem<T>(r, i), elem<T>(r, i + 1));
    return max3_hw(m, elem<T>(r, kLaneElems - 1), elem<T>(r, kLaneElems - 1));
}

// Sum over a lane's 32 elements of 2^(x*k2 - ref): pairwise within each
// 8-element group, then over the four groups.
template <typename T>
__device__ __forceinline__ float tile_exp_sum(const TileRaw<T> &r, float k2, float ref) {
    float g[kGroupsPerTile];
#pragma unroll
    for (int q = 0; q < kGroupsPerTile; ++q) {
        float e[kGroupElems];
#pragma unroll
        for (int i = 0; i < kGroupElems; ++i) e[i] = fast_exp2(fmaf(elem<T>(r, q * kGroupElems + i), k2, -ref));
        g[q] = tree_sum(e);
    }
    return tree_sum(g);
}

struct LaneSoftmax {
    float ref = kNegInf;   // wavefront-uniform
    double acc = 0.0;      // lane sum relative to 2^ref

    // Folds one tile; returns the lane's fp32 tile sum (0 if nothing finite yet).
    template <typename T>
    __device__ __forceinline__ float add(const TileRaw<T> &r, float k2) {
        const float lm = tile_max<T>(r);
        if (__ballot(lm * k2 > ref)) {
            const float nref = ceilf(wave_max(lm) * k2);
            if (ref != kNegInf) acc *= pow2_int(ref - nref);
            ref = nref;
        }
        if (ref == kNegInf) return 0.0f;
        const float s = tile_exp_sum<T>(r, k2, ref);
        acc += (double)s;
        return s;
    }
};

// Merges (ref, sum) pairs in index order: ref = max ref, sum rescaled to it.
__device__ __forceinline__ void merge_refsum(const float *refs, const double *sums, int n,
                                             float &ref, double &sum) {
    ref = kNegInf;
    for (int i = 0; i < n; ++i) ref = fmaxf(ref, refs[i]);
    sum = 0.0;
    if (ref == kNegInf) return;
    for (int i = 0; i < n; ++i)
        if (refs[i] != kNegInf) sum += sums[i] * pow2_int(refs[i] - ref);
}

// Merges the n segment records of one row (loads issued four at a time) and
// clears them.
__device__ __forceinline__ void take_segrecs(SegRec *rec, int n, float &ref, double &sum) {
    ref = kNegInf;
    sum = 0.0;
    for (int i0 = 0; i0 < n; i0 += 4) {
        uint64_t lo[4], hi[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo[k] = i0 + k < n ? ld64(reinterpret_cast<const uint64_t *>(&rec[i0 + k])) : 0;
            hi[k] = i0 + k < n ? ld64(reinterpret_cast<const uint64_t *>(&rec[i0 + k]) + 1) : 0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (i0 + k >= n) continue;
            const float r = lo_f(lo[k]);
            if (r == kNegInf) continue;
            if (r > ref) {
                if (ref != kNegInf) sum *= pow2_int(ref - r);
                ref = r;
            }
            sum += __longlong_as_double((long long)hi[k]) * pow2_int(r - ref);
        }
    }
    for (int i = 0; i < n; ++i) st_seg(&rec[i], 0.0f, 0.0);
}

// Merges the n argmax records of one row (ties to the lowest index) and clears them.
__device__ __forceinline__ int take_argrecs(ArgRec *rec, int n) {
    float bv = kNegInf;
    int bi = INT_MAX;
    for (int i0 = 0; i0 < n; i0 += 4) {
        uint64_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = i0 + k < n ? ld_pair(&rec[i0 + k]) : 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (i0 + k < n && arg_better(lo_f(v[k]), hi_i(v[k]), bv, bi)) {
                bv = lo_f(v[k]);
                bi = hi_i(v[k]);
            }
    }
    for (int i = 0; i < n; ++i) st_pair(&rec[i], 0);
    return bi == INT_MAX ? 0 : bi;   // a row of -inf only: index 0, like numpy argmax
}

// Per-lane running argmax over the tiles a wavefront streams in vocab order;
// strict '>' keeps the first index of equal maxima.
template <typename T>
__device__ __forceinline__ void argmax_tile(const TileRaw<T> &r, int tile, int lane, float &bv,
                                            int &bi) {
    float v[kLaneElems];
    unpack<T>(r, v);
    const float lm = max32(v);
    if (__ballot(lm > bv)) {
        if (lm > bv) {
            int fi = 0;
#pragma unroll
            for (int i = kLaneElems - 1; i >= 0; --i) fi = (v[i] == lm) ? i : fi;
            bv = lm;
            bi = (int)elem_index(tile, lane, fi);
        }
    }
}

// ---------------------------------------------------------------------------
// Inverse-CDF search (one wavefront)
// ---------------------------------------------------------------------------
//
// A finisher runs at the tail of the work it completes, so its cost is the
// number of dependent memory round trips and the length of its dependent
// instruction chain, not bandwidth.  Tile records are visited in chunks of
// 128 tiles with lane l holding tiles 2l and 2l+1 of the chunk (loaded at
// once); the crossing tile is loaded once into registers.  A row of up to
// 128 tiles (V <= 262,144) costs two round trips, its records and then its
// crossing tile, and one wavefront scan over the records gives both the
// row's total and the crossing tile.

constexpr int kRecPerLane = 2;
constexpr int kRecChunk = kWave * kRecPerLane;

struct RecChunk {
    uint64_t r[kRecPerLane];
};

__device__ __forceinline__ void load_chunk(const uint64_t *recs, int n, int t0, int lane,
                                           RecChunk &c) {
#pragma unroll
    for (int i = 0; i < kRecPerLane; ++i) {
        const int t = t0 + lane * kRecPerLane + i;
        c.r[i] = t < n ? ld64(&recs[t]) : 0;
    }
}

// Lane masses of one chunk: m[i] = mass_of(record) for tiles < n, else 0.
template <typename MassOf>
__device__ __forceinline__ double chunk_masses(const RecChunk &c, int n, int t0, int lane,
                                               MassOf &&mass_of, double (&m)[kRecPerLane]) {
    double ls = 0.0;
#pragma unroll
    for (int i = 0; i < kRecPerLane; ++i) {
        const int t = t0 + lane * kRecPerLane + i;
        m[i] = t < n ? mass_of(c.r[i]) : 0.0;
        ls += m[i];
    }
    return ls;
}

template <typename Get, typename MassOf>
__device__ __forceinline__ double row_total(int n, Get &&get, int lane, MassOf &&mass_of) {
    double total = 0.0;
    for (int t0 = 0; t0 < n; t0 += kRecChunk) {
        RecChunk c;
        get(t0, c);
        double m[kRecPerLane];
        const double ls = chunk_masses(c, n, t0, lane, mass_of, m);
        total += __shfl(wave_incl_scan_d(ls, lane), kWave - 1);
    }
    return total;
}

// First tile whose running mass exceeds target (and the mass before it), or -1.
template <typename Get, typename MassOf>
__device__ __forceinline__ int row_find(int n, Get &&get, int lane, MassOf &&mass_of,
                                        double target, double &before) {
    double base = 0.0;
    for (int t0 = 0; t0 < n; t0 += kRecChunk) {
        RecChunk c;
        get(t0, c);
        double m[kRecPerLane];
        const double ls = chunk_masses(c, n, t0, lane, mass_of, m);
        const double inc = wave_incl_scan_d(ls, lane);
        double run = base + (inc - ls);
        int first = -1;
        double fb = 0.0;
#pragma unroll
        for (int i = 0; i < kRecPerLane; ++i) {
            if (first < 0 && run + m[i] > target) {
                first = i;
                fb = run;
            }
            run += m[i];
        }
        const unsigned long long hit = __ballot(first >= 0);
        if (hit) {
            const int l = wave_first(hit);
            before = __shfl(fb, l);
            return t0 + l * kRecPerLane + __shfl(first, l);
        }
        base += __shfl(inc, kWave - 1);
    }
    return -1;
}

template <typename Get, typename MassOf>
__device__ __forceinline__ int row_last_positive(int n, Get &&get, int lane, MassOf &&mass_of) {
    int best = -1;
    for (int t0 = 0; t0 < n; t0 += kRecChunk) {
        RecChunk c;
        get(t0, c);
        double m[kRecPerLane];
        chunk_masses(c, n, t0, lane, mass_of, m);
        int mine = -1;
#pragma unroll
        for (int i = 0; i < kRecPerLane; ++i)
            if (m[i] > 0.0) mine = t0 + lane * kRecPerLane + i;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mine = max(mine, __shfl_xor(mine, o));
        if (mine >= 0) best = mine;
    }
    return best;
}

// The tile where the running mass of the row first exceeds u * total, the
// mass before it and the target u * total; -1 if rounding leaves the target
// unreached.  total gets the row's mass.  A row of one chunk takes a single
// scan; longer rows take a pass for the total, then one to find the tile.
template <typename Get, typename MassOf>
__device__ __forceinline__ int row_draw(int n, Get &&get, int lane, MassOf &&mass_of, double u,
                                        double &total, double &before, double &target) {
    if (n > kRecChunk) {
        total = row_total(n, get, lane, mass_of);
        target = u * total;
        return row_find(n, get, lane, mass_of, target, before);
    }
    RecChunk c;
    get(0, c);
    double m[kRecPerLane];
    const double ls = chunk_masses(c, n, 0, lane, mass_of, m);
    const double inc = wave_incl_scan_d(ls, lane);
    total = lane_read_d(inc, kWave - 1);
    target = u * total;
    double run = inc - ls;
    int first = -1;
    double fb = 0.0;
#pragma unroll
    for (int i = 0; i < kRecPerLane; ++i) {
        if (first < 0 && run + m[i] > target) {
            first = i;
            fb = run;
        }
        run += m[i];
    }
    const unsigned long long hit = __ballot(first >= 0);
    if (!hit) return -1;
    const int l = wave_first(hit);
    before = lane_read_d(fb, l);
    return l * kRecPerLane + __builtin_amdgcn_readlane(first, l);
}

// Within one tile held in registers, finds the first vocab index where
// before + scale * (running weight) exceeds target; weight(i) is the fp32
// weight of the lane's element i (group-major, 0..31; 0 past the end of the
// row) and scale a power of two.  Groups are walked in vocab order, eight
// weights live at a time (a finisher shares the kernel's register budget).
// If rounding leaves the target unreached, returns the last index with
// positive weight (-1 if none).
template <typename W>
__device__ __forceinline__ long long search_tile(W &&weight, int tile, int lane, double before,
                                                 double target, double scale = 1.0) {
    double base = before;
#pragma unroll
    for (int g = 0; g < kGroupsPerTile; ++g) {
        float w[kGroupElems];
        double gs = 0.0;
#pragma unroll
        for (int e = 0; e < kGroupElems; ++e) {
            w[e] = weight(g * kGroupElems + e);
            gs += (double)w[e];
        }
        const double inc = wave_incl_scan_d(gs, lane);
        const double rel = (target - base) / scale;   // compared with unscaled running weights
        double c = inc - gs;
        int first = -1;
#pragma unroll
        for (int e = 0; e < kGroupElems; ++e) {
            c += (double)w[e];
            if (first < 0 && c > rel) first = e;
        }
        const unsigned long long hit = __ballot(first >= 0);
        if (hit) {
            const int l = wave_first(hit);
            return elem_index(tile, l, g * kGroupElems + __builtin_amdgcn_readlane(first, l));
        }
        base += lane_read_d(inc, kWave - 1) * scale;
    }
    long long last = -1;
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i)
        if (weight(i) > 0.0f) {
            const long long ei = elem_index(tile, lane, i);
            last = ei > last ? ei : last;
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const long long ol = __shfl_xor(last, o);
        last = ol > last ? ol : last;
    }
    return last;
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

// Element offset of logits row (c, k).
__device__ __forceinline__ long long row_offset(const StepArgs &a, int c, int k) {
    return (long long)c * a.ldc + (long long)k * a.ld;
}

// An item of at most this many tiles gathers its tile records in LDS and
// stores them with one instruction at its end (one lane per record) instead
// of one store per tile.
constexpr int kBatchTiles = kWave;

struct Shared {
    int ticket;
    int flag_ok;                  // a residual item's wait for its decision ended in time
    float refs[kWavesPerGroup];
    double sums[kWavesPerGroup];
    float vals[kWavesPerGroup];
    int idxs[kWavesPerGroup];
    float vals2[kWavesPerGroup];
    int idxs2[kWavesPerGroup];
    SeqInfo info;
    uint64_t trec[kBatchTiles];   // an item's tile records, stored together at its end
};

// Decision for sequence c from its merged verify rows (wavefront 0 of the
// workgroup that finished the sequence's last verify segment).
template <typename T, int MODE>
__device__ __forceinline__ void decide(const StepArgs &a, int c, int lane) {
    const int L = a.L;
    const int CL = a.C * L;
    const bool valid = lane < L;
    const int kk = valid ? lane : 0;
    const int xk = valid ? a.x[c * L + kk] : 0;
    const bool bad = valid && (xk < 0 || xk >= a.V);
    if (bad) atomicOr(&a.ws.ctl->error, kErrBadToken);
    float alpha;

    if (MODE == kSample) {
        float cp = kNegInf, cq = kNegInf;
        double sp = 0.0, sq = 0.0;
        double px = 0.0, qx = 0.0;
        if (valid) {
            // the logits at x_k first: their loads overlap the record loads
            float lp = 0.0f, lq = 0.0f;
            if (!bad) {
                const long long off = row_offset(a, c, kk) + xk;
                lp = load_value<T>(static_cast<const T *>(a.p), off);
                if (!a.q_onehot) lq = load_value<T>(static_cast<const T *>(a.q), off);
            }
            take_segrecs(&a.ws.seg[((size_t)c * L + kk) * a.S], a.S, cp, sp);
            if (!a.q_onehot) take_segrecs(&a.ws.seg[((size_t)CL + (size_t)c * L + kk) * a.S], a.S, cq, sq);
            if (sp <= 0.0 || (!a.q_onehot && sq <= 0.0)) atomicOr(&a.ws.ctl->error, kErrEmptyRow);
            if (!bad) {
                const double k2 = (double)a.k2;
                if (sp > 0.0) px = exp2((double)lp * k2 - (double)cp) / sp;
                if (a.q_onehot) {
                    qx = 1.0;   // the argmax pick's own law
                } else if (sq > 0.0) {
                    qx = exp2((double)lq * k2 - (double)cq) / sq;
                }
            }
        }
        // min(1, P(x)/Q(x)); Q(x) = 0 gives 1 if P(x) > 0, else 0.  The accept
        // test may use the relaxed ratio min(1, (1 + tau) P(x)/Q(x)); alpha
        // stays the plain rate.
        const double r = qx > 0.0 ? fmin(1.0, px / qx) : (px > 0.0 ? 1.0 : 0.0);
        const double ra = a.relax1p == 1.0
                              ? r
                              : (qx > 0.0 ? fmin(1.0, (a.relax1p * px) / qx) : (px > 0.0 ? 1.0 : 0.0));
        const bool accepted = !valid || (a.ua == nullptr || (double)a.ua[c * L + kk] < ra);
        const unsigned long long rej = __ballot(!accepted);
        const int j = rej ? wave_first(rej) : L;
        alpha = (float)(wave_sum_d(valid ? r : 0.0) / (double)L);
        if (valid) {
            if (a.p_x) a.p_x[c * L + kk] = (float)px;
            if (a.q_x) a.q_x[c * L + kk] = (float)qx;
            // position j (a rejection) is written by the residual draw
            if (a.verify_outputs && kk != j) a.out_tokens[c * L + kk] = kk < j ? xk : -1;
        }
        if (a.r_blk) {
            // publish the row-j constants, then the flag the residual items poll
            const int src = j < L ? j : 0;
            const float jcp = __shfl(cp, src), jcq = __shfl(cq, src);
            const double jsp = __shfl(sp, src), jsq = __shfl(sq, src);
            const int jx = __shfl(xk, src);
            const float ju = (j < L && a.ur) ? a.ur[c * L + j] : 0.0f;
            publish_decision(a, c, j, ju, jcp, jcq, jsp, jsq, jx, lane);
        }
        if (lane == 0 && a.verify_outputs) {
            a.accept_len[c] = j;
            a.n_emitted[c] = j + (j < L ? 1 : 0);
        }
    } else {
        int g = 0;
        if (valid) g = take_argrecs(&a.ws.arg[((size_t)c * L + kk) * a.S], a.S);
        const bool match = valid && !bad && xk == g;
        const unsigned long long mism = __ballot(valid && !match);
        const unsigned long long hits = __ballot(match);
        const int j = mism ? wave_first(mism) : L;
        alpha = (float)__popcll((long long)hits) / (float)L;
        if (valid) {
            if (a.p_x) a.p_x[c * L + kk] = match ? 1.0f : 0.0f;
            if (a.q_x) a.q_x[c * L + kk] = 1.0f;
            if (a.verify_outputs) a.out_tokens[c * L + kk] = kk < j ? xk : (kk == j ? g : -1);
        }
        if (lane == 0 && a.verify_outputs) {
            a.accept_len[c] = j;
            a.n_emitted[c] = j + (j < L ? 1 : 0);
        }
    }
    if (lane == 0 && a.alpha) a.alpha[c] = alpha;

    // batch mean of alpha, by the last sequence to be decided
    if (a.alpha_mean) {
        int last = 0;
        if (lane == 0) {
            st32(reinterpret_cast<uint32_t *>(&a.ws.info[c].alpha), __float_as_uint(alpha));
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_s_waitcnt(0);
            last = __hip_atomic_fetch_add(&a.ws.ctl->seq_done, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) + 1 == (uint32_t)a.C;
        }
        last = __shfl(last, 0);
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            double s = 0.0;
            for (int c0 = 0; c0 < a.C; c0 += kWave) {
                const int cc = c0 + lane;
                uint32_t* ap = reinterpret_cast<uint32_t *>(&a.ws.info[cc < a.C ? cc : 0].alpha);
                s += wave_sum_d(cc < a.C ? (double)__uint_as_float(ld32(ap)) : 0.0);
            }
            for (int cc = lane; cc < a.C; cc += kWave)
                st32(reinterpret_cast<uint32_t *>(&a.ws.info[cc].alpha), 0u);
            if (lane == 0) {
                a.alpha_mean[0] = (float)(s / (double)a.C);
                st32(&a.ws.ctl->seq_done, 0u);
            }
        }
    }
}

// Outputs of a sequence that verifies nothing in a masked step.
__device__ __forceinline__ void write_idle_verify(const StepArgs &a, int c) {
    const int L = a.L;
    for (int k = threadIdx.x; k < L; k += kThreads) {
        if (a.verify_outputs) a.out_tokens[c * L + k] = -1;
        if (a.p_x) a.p_x[c * L + k] = 0.0f;
        if (a.q_x) a.q_x[c * L + k] = 0.0f;
    }
    if (threadIdx.x == 0) {
        if (a.verify_outputs) {
            a.accept_len[c] = -1;
            a.n_emitted[c] = 0;
        }
        if (a.alpha) a.alpha[c] = 0.0f;
    }
}

template <typename T, bool VEC, int MODE>
__device__ __forceinline__ void pq_item(const StepArgs &a, int t, Shared &sh, int wave, int lane) {
    const int per_seq = a.rows_pq * a.S;
    const int c = t / per_seq;
    const int rem = t - c * per_seq;
    const int slot = rem / a.S;
    const int seg = rem - slot * a.S;
    const int CL = a.C * a.L;
    // sample mode verifies (p, q) row pairs, unless the proposals were argmax
    // picks whose law is one-hot at x (no q row to read)
    const bool pairs = MODE == kSample && !a.q_onehot;
    const int k = pairs ? slot >> 1 : slot;
    const int which = pairs ? (slot & 1) : 0;
    const T *row = static_cast<const T *>(which ? a.q : a.p) + row_offset(a, c, k);
    const int tb = seg * a.tps;
    const int te = min(a.tiles_row, tb + a.tps);
    const size_t rec = ((size_t)which * CL + (size_t)c * a.L + k) * a.S + seg;

    if (a.vmask && a.vmask[c] == 0) {
        // sequence c verifies nothing this step: its first item writes the
        // defined outputs of an idle sequence, and no other item of c runs
        if (slot == 0 && seg == 0) write_idle_verify(a, c);
        return;
    }

    if (MODE == kSample) {
        LaneSoftmax sm;
        stream_row<T, VEC>(row, tb, te, a.V, wave, lane, [&](const TileRaw<T> &r, int) {
            sm.add<T>(r, a.k2);
        });
        const double ws = wave_sum_d(sm.acc);
        if (lane == 0) {
            sh.refs[wave] = sm.ref;
            sh.sums[wave] = ws;
        }
        __syncthreads();
        if (threadIdx.x < 2) {
            // the record's two words in one store instruction (lanes 0 and 1)
            float ref;
            double sum;
            merge_refsum(sh.refs, sh.sums, kWavesPerGroup, ref, sum);
            st64(reinterpret_cast<uint64_t *>(&a.ws.seg[rec]) + threadIdx.x,
                 threadIdx.x == 0 ? pack2(ref, 0.0f) : (uint64_t)__double_as_longlong(sum));
        }
    } else {
        float bv = kNegInf;
        int bi = INT_MAX;
        stream_row<T, VEC>(row, tb, te, a.V, wave, lane, [&](const TileRaw<T> &r, int tile) {
            argmax_tile<T>(r, tile, lane, bv, bi);
        });
        wave_argmax(bv, bi);
        if (lane == 0) {
            sh.vals[wave] = bv;
            sh.idxs[wave] = bi;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float v = kNegInf;
            int i = INT_MAX;
            for (int w = 0; w < kWavesPerGroup; ++w)
                if (arg_better(sh.vals[w], sh.idxs[w], v, i)) {
                    v = sh.vals[w];
                    i = sh.idxs[w];
                }
            st_pair(&a.ws.arg[rec], pack2(v, i));
        }
    }

    if (!arrive(counter(a.ws.seq_cnt, c), (uint32_t)per_seq)) return;
    if (wave == 0) decide<T, MODE>(a, c, lane);
}

template <typename T, bool VEC, int MODE>
__device__ __forceinline__ void qn_item(const StepArgs &a, int c, int k, int seg, Shared &sh,
                                        int wave, int lane) {
    const int rowid = c * a.L + k;
    const T *row = static_cast<const T *>(a.qn) + row_offset(a, c, k);
    const int tb = seg * a.tpsq;
    const int te = min(a.tiles_row, tb + a.tpsq);
    if (a.pmask && a.pmask[c] == 0) {
        // no proposal for sequence c this step; its row is not read
        if (seg == 0 && threadIdx.x == 0) {
            a.next_tokens[rowid] = -1;
            if (a.qnext_x) a.qnext_x[rowid] = 0.0f;
        }
        return;
    }

    if (MODE == kSample) {
        TileRec *tr = a.ws.tiles + (size_t)rowid * a.tiles_row;
        const bool batch = te - tb <= kBatchTiles;
        LaneSoftmax sm;
        stream_row<T, VEC>(row, tb, te, a.V, wave, lane, [&](const TileRaw<T> &r, int tile) {
            const float s = sm.add<T>(r, a.k2);
            const float ts = wave_sum(s);
            if (lane == 0) {
                if (batch) sh.trec[tile - tb] = pack2(sm.ref, ts);
                else st_pair(&tr[tile], pack2(sm.ref, ts));
            }
        });
        if (batch) {
            __syncthreads();
            if (wave == 0 && lane < te - tb) st_pair(&tr[tb + lane], sh.trec[lane]);
        }
        if (!arrive(counter(a.ws.row_cnt, rowid), (uint32_t)a.Sq)) return;
        if (wave != 0) return;

        // ---- inverse-CDF draw over the whole row ----
        const uint64_t *recs = reinterpret_cast<const uint64_t *>(tr);
        const int nt = a.tiles_row;
        RecChunk first;
        load_chunk(recs, nt, 0, lane, first);
        auto get = [&](int t0, RecChunk &c) {
            if (t0 == 0) c = first;
            else load_chunk(recs, nt, t0, lane, c);
        };
        float cr = kNegInf;
        for (int t0 = 0; t0 < nt; t0 += kRecChunk) {
            RecChunk ch;
            get(t0, ch);
#pragma unroll
            for (int i = 0; i < kRecPerLane; ++i)
                if (t0 + lane * kRecPerLane + i < nt) cr = fmaxf(cr, lo_f(ch.r[i]));
        }
        cr = wave_max(cr);
        auto mass = [&](uint64_t rc) -> double {
            const float ref = lo_f(rc);
            return ref == kNegInf ? 0.0 : (double)hi_f(rc) * pow2_int(ref - cr);
        };
        int token = 0;
        double S = 0.0;
        double q_tok = 0.0;   // Qn(token) * S
        if (cr == kNegInf) {
            if (lane == 0) atomicOr(&a.ws.ctl->error, kErrEmptyRow);
        } else {
            double before = 0.0, target = 0.0;
            int tile = row_draw(nt, get, lane, mass, (double)a.up[rowid], S, before, target);
            double tile_target = target;
            if (tile < 0) {
                // rounding left the target unreached: clamp to the last positive weight
                tile = max(0, row_last_positive(nt, get, lane, mass));
                tile_target = __builtin_inf();
            }
            RecChunk tc;
            get(tile - tile % kRecChunk, tc);
            const int owner = (tile % kRecChunk) / kRecPerLane;
            uint64_t trec = 0;
#pragma unroll
            for (int i = 0; i < kRecPerLane; ++i)
                if (i == tile % kRecPerLane) trec = tc.r[i];
            const float tref = __uint_as_float(__builtin_amdgcn_readlane((int)(uint32_t)trec, owner));
            const double scale = pow2_int(tref - cr);
            TileRaw<T> raw;
            load_tile<T, VEC>(row, tile, a.V, lane, raw);
            const float k2 = a.k2;
            auto weight = [&](int i) -> float { return fast_exp2(fmaf(elem<T>(raw, i), k2, -tref)); };
            const long long tok = search_tile(weight, tile, lane, before, tile_target, scale);
            if (tok >= 0) {
                token = (int)tok;
                // the token lies in the crossing tile: its weight comes from
                // the lane that holds it (a select over the lane's words:
                // indexing the array with a run-time value would move it out
                // of registers)
                const int off = (int)(tok - (long long)tile * kTileElems);
                const int holder = (off % (kWave * kGroupElems)) / kGroupElems;
                const int pos = off / (kWave * kGroupElems) * kGroupElems + off % kGroupElems;
                float mine = 0.0f;
#pragma unroll
                for (int q = 0; q < kLaneElems; ++q) mine = q == pos ? elem<T>(raw, q) : mine;
                const float lv = __uint_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), holder));
                q_tok = (double)fast_exp2(fmaf(lv, k2, -tref)) * scale;
            } else {
                q_tok = (double)fast_exp2(fmaf(load_value<T>(row, 0), k2, -cr));
            }
        }
        // the tile masses are consumed: return them to zero
        for (int t = lane; t < a.tiles_row; t += kWave) st_pair(&tr[t], 0);
        if (lane == 0) {
            a.next_tokens[rowid] = token;
            if (a.qnext_x) a.qnext_x[rowid] = S > 0.0 ? (float)(q_tok / S) : 0.0f;
        }
    } else {
        float bv = kNegInf;
        int bi = INT_MAX;
        stream_row<T, VEC>(row, tb, te, a.V, wave, lane, [&](const TileRaw<T> &r, int tile) {
            argmax_tile<T>(r, tile, lane, bv, bi);
        });
        wave_argmax(bv, bi);
        if (lane == 0) {
            sh.vals[wave] = bv;
            sh.idxs[wave] = bi;
        }
        __syncthreads();
        ArgRec *recs = &a.ws.arg[(size_t)a.C * a.L * a.smax + (size_t)rowid * a.Sq];
        if (threadIdx.x == 0) {
            float v = kNegInf;
            int i = INT_MAX;
            for (int w = 0; w < kWavesPerGroup; ++w)
                if (arg_better(sh.vals[w], sh.idxs[w], v, i)) {
                    v = sh.vals[w];
                    i = sh.idxs[w];
                }
            st_pair(&recs[seg], pack2(v, i));
        }
        if (!arrive(counter(a.ws.row_cnt, rowid), (uint32_t)a.Sq)) return;
        if (threadIdx.x == 0) {
            a.next_tokens[rowid] = take_argrecs(recs, a.Sq);
            if (a.qnext_x) a.qnext_x[rowid] = 1.0f;
        }
    }
}

// ---------------------------------------------------------------------------
// Gumbel-max correction
// ---------------------------------------------------------------------------
//
// The correction of the pages' fused kernel is a Gumbel-max draw
// ("Introspective Diffusion Language Models | Summary", section 3.3): the
// token is argmax_i ln w_i + G_i with G_i = -ln(-ln U_i).  Since exp is
// increasing, that is argmax_i w_i / E_i with E_i = -ln U_i, which costs one
// logarithm and one reciprocal per entry instead of two logarithms; the
// ratio's relative error is a few fp32 ulps.  The noise comes from
// Philox4x32-10 (isd_device.h) under key (bits of u_resid[c, j], c).

// Running per-lane argmax of a score over entries visited in increasing index
// order: strict '>' keeps the first of equal scores; zero scores never win.
__device__ __forceinline__ void gumbel_take(float s, int i, float &bv, int &bi) {
    if (s > bv) {
        bv = s;
        bi = i;
    }
}

// Block-wide merge of the per-wave argmax pairs (v, i) and (v2, i2); thread 0
// writes them to rec[0] and rec[1].
__device__ __forceinline__ void gumbel_publish(Shared &sh, int wave, int lane, float v, int i,
                                               float v2, int i2, ArgRec *rec) {
    wave_argmax(v, i);
    wave_argmax(v2, i2);
    if (lane == 0) {
        sh.vals[wave] = v;
        sh.idxs[wave] = i;
        sh.vals2[wave] = v2;
        sh.idxs2[wave] = i2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bv = 0.0f, bv2 = 0.0f;
        int bi = INT_MAX, bi2 = INT_MAX;
        for (int w = 0; w < kWavesPerGroup; ++w) {
            if (arg_better(sh.vals[w], sh.idxs[w], bv, bi)) {
                bv = sh.vals[w];
                bi = sh.idxs[w];
            }
            if (arg_better(sh.vals2[w], sh.idxs2[w], bv2, bi2)) {
                bv2 = sh.vals2[w];
                bi2 = sh.idxs2[w];
            }
        }
        st_pair(&rec[0], pack2(bv, bi));
        st_pair(&rec[1], pack2(bv2, bi2));
    }
}

// Merges the n segment records (pairs of R and P partials) of one correction
// and clears them (one wavefront).  Returns the Gumbel-max token over R if
// any R entry is positive, else over P.
__device__ __forceinline__ int gumbel_finish(ArgRec *rec, int n, int lane) {
    float vr = 0.0f, vp = 0.0f;
    int ir = INT_MAX, ip = INT_MAX;
    if (lane < n) {
        const uint64_t r = ld_pair(&rec[2 * lane]), q = ld_pair(&rec[2 * lane + 1]);
        vr = lo_f(r);
        ir = hi_i(r);
        vp = lo_f(q);
        ip = hi_i(q);
        st_pair(&rec[2 * lane], 0);
        st_pair(&rec[2 * lane + 1], 0);
    }
    wave_argmax(vr, ir);
    wave_argmax(vp, ip);
    const int tok = vr > 0.0f ? ir : ip;
    return tok == INT_MAX ? 0 : tok;
}

constexpr int kVarGumbel = 1;   // correction by Gumbel-max (else inverse CDF)
constexpr int kVarOnehot = 2;   // proposals were argmax picks: Q = onehot(x)

// ---------------------------------------------------------------------------
// Residual weights
// ---------------------------------------------------------------------------
//
// The correction draws from max(0, P - Q) over row j.  In units of the anchor
// row's denominator Sp the weight of entry i is d_i = a_i - rho * b_i, with
// a_i = 2^(p_i*k2 - cp), b_i = 2^(q_i*k2 - cq) and rho = Sp / Sq; a_i is the
// entry's weight under P.  Where P and Q nearly agree, d_i is a small
// difference of two large terms, and a rounding of the row constant would
// shift every entry of the residual the same way: rho enters as
// rho_hi + rho_lo (two fused multiply-adds), so no row-wide rounding is left
// and the error of d_i is that of the entry's own two exponentials.

struct ResidForm {
    float k2, cp, cq, rho_hi, rho_lo;
};

__device__ __forceinline__ ResidForm resid_form(const SeqInfo &inf, float k2) {
    return ResidForm{k2, inf.cp, inf.cq, inf.rho_hi, inf.rho_lo};
}

// Residual weight max(0, d) of one entry; a_out gets its P weight a.
__device__ __forceinline__ float resid_weight(float vp, float vq, const ResidForm &f, float &a_out) {
    const float a = fast_exp2(fmaf(vp, f.k2, -f.cp));
    const float b = fast_exp2(fmaf(vq, f.k2, -f.cq));
    a_out = a;
    return fmaxf(fmaf(-f.rho_lo, b, fmaf(-f.rho_hi, b, a)), 0.0f);
}

// VAR bit 0: Gumbel-max correction; bit 1: one-hot proposal law (q not read).
template <typename T, bool VEC, int VAR>
__device__ __forceinline__ void res_item(const StepArgs &a, int c, int seg, Shared &sh, int wave,
                                         int lane) {
    constexpr bool GUMBEL = (VAR & kVarGumbel) != 0, ONEHOT = (VAR & kVarOnehot) != 0;
    if (a.vmask && a.vmask[c] == 0) return;   // no decision is taken for c
    // wait for sequence c's decision
    if (threadIdx.x == 0) {
        uint32_t polls = 0;
        bool ok = true;
        uint32_t *flag = counter(a.ws.flag, c);
        while (ld32(flag) != a.epoch) {
            __builtin_amdgcn_s_sleep(4);
            if (++polls > a.spin_limit) {
                atomicOr(&a.ws.ctl->error, kErrWaitExpired);
                ok = false;
                break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        sh.flag_ok = ok;
    }
    __syncthreads();
    if (threadIdx.x < 10) {
        // the decision record, one word per lane in one load instruction
        const uint32_t w = ld32(reinterpret_cast<const uint32_t *>(&a.ws.info[c]) + threadIdx.x);
        reinterpret_cast<uint32_t *>(&sh.info)[threadIdx.x] =
            (threadIdx.x == 0 && !sh.flag_ok) ? (uint32_t)a.L : w;
    }
    __syncthreads();
    const SeqInfo inf = sh.info;
    const int L = a.L;
    const int j = inf.j;
    ResTile *rt = a.ws.rtiles + (size_t)c * a.tiles_row;
    const T *prow = static_cast<const T *>(a.p) + row_offset(a, c, j < L ? j : 0);
    const T *qrow = static_cast<const T *>(a.q) + row_offset(a, c, j < L ? j : 0);

    if (GUMBEL && j < L) {
        // Gumbel-max partials of this segment: best R / E and best P / E
        const uint32_t k0 = __float_as_uint(inf.u), k1 = (uint32_t)c;
        float br = 0.0f, bp = 0.0f;
        int ir = INT_MAX, ip = INT_MAX;
        auto take = [&](const float (&P)[kGroupElems], const float (&R)[kGroupElems], int tile,
                        int g) {
            const long long first = elem_index(tile, lane, g * kGroupElems);
            float inv_e[kGroupElems];
            inv_exp_noise8((uint32_t)first, (uint32_t)j, k0, k1, inv_e);
#pragma unroll
            for (int e = 0; e < kGroupElems; ++e) {
                gumbel_take(R[e] * inv_e[e], (int)first + e, br, ir);
                gumbel_take(P[e] * inv_e[e], (int)first + e, bp, ip);
            }
        };
        const int tb = seg * a.tpsr;
        const int te = min(a.tiles_row, tb + a.tpsr);
        if (ONEHOT) {
            stream_row<T, VEC>(prow, tb, te, a.V, wave, lane, [&](const TileRaw<T> &rp, int tile) {
#pragma unroll
                for (int g = 0; g < kGroupsPerTile; ++g) {
                    float P[kGroupElems], R[kGroupElems];
#pragma unroll
                    for (int e = 0; e < kGroupElems; ++e) {
                        const int i = g * kGroupElems + e;
                        P[e] = fast_exp2(fmaf(elem<T>(rp, i), a.k2, -inf.cp)) * inf.inv_sp;
                        R[e] = elem_index(tile, lane, i) == (long long)inf.xj ? 0.0f : P[e];
                    }
                    take(P, R, tile, g);
                }
            });
        } else {
            const ResidForm rf = resid_form(inf, a.k2);
            auto body = [&](const TileRaw<T> &rp, const TileRaw<T> &rq, int tile) {
#pragma unroll
                for (int g = 0; g < kGroupsPerTile; ++g) {
                    float P[kGroupElems], R[kGroupElems];
#pragma unroll
                    for (int e = 0; e < kGroupElems; ++e) {
                        const int i = g * kGroupElems + e;
                        R[e] = resid_weight(elem<T>(rp, i), elem<T>(rq, i), rf, P[e]);
                    }
                    take(P, R, tile, g);
                }
            };
            stream_rows2<T, VEC, false>(prow, qrow, tb, te, a.V, wave, lane, body);
        }
        gumbel_publish(sh, wave, lane, br, ir, bp, ip,
                       a.ws.garg + ((size_t)c * kMaxResidSegments + seg) * 2);
    } else if (ONEHOT && j < L) {
        // Q is one-hot at x_j: the residual is P with x_j removed
        const int tb = seg * a.tpsr;
        const int te = min(a.tiles_row, tb + a.tpsr);
        const bool batch = te - tb <= kBatchTiles;
        stream_row<T, VEC>(prow, tb, te, a.V, wave, lane, [&](const TileRaw<T> &rp, int tile) {
            float lr = 0.0f, lp = 0.0f;
#pragma unroll
            for (int g = 0; g < kGroupsPerTile; ++g) {
                float er[kGroupElems], ep[kGroupElems];
#pragma unroll
                for (int e = 0; e < kGroupElems; ++e) {
                    const int i = g * kGroupElems + e;
                    const float P = fast_exp2(fmaf(elem<T>(rp, i), a.k2, -inf.cp)) * inf.inv_sp;
                    er[e] = elem_index(tile, lane, i) == (long long)inf.xj ? 0.0f : P;
                    ep[e] = P;
                }
                lr += tree_sum(er);
                lp += tree_sum(ep);
            }
            const float sr = wave_sum(lr);
            const float spp = wave_sum(lp);
            if (lane == 0) {
                if (batch) sh.trec[tile - tb] = pack2(sr, spp);
                else st_pair(&rt[tile], pack2(sr, spp));
            }
        });
        if (batch) {
            __syncthreads();
            if (wave == 0 && lane < te - tb) st_pair(&rt[tb + lane], sh.trec[lane]);
        }
    } else if (j < L) {
        const int tb = seg * a.tpsr;
        const int te = min(a.tiles_row, tb + a.tpsr);
        const bool batch = te - tb <= kBatchTiles;
        const ResidForm rf = resid_form(inf, a.k2);
        stream_rows2<T, VEC>(prow, qrow, tb, te, a.V, wave, lane,
                             [&](const TileRaw<T> &rp, const TileRaw<T> &rq, int tile) {
            float lr = 0.0f, lp = 0.0f;
#pragma unroll
            for (int g = 0; g < kGroupsPerTile; ++g) {
                float er[kGroupElems], ep[kGroupElems];
#pragma unroll
                for (int e = 0; e < kGroupElems; ++e) {
                    const int i = g * kGroupElems + e;
                    er[e] = resid_weight(elem<T>(rp, i), elem<T>(rq, i), rf, ep[e]);
                }
                lr += tree_sum(er);
                lp += tree_sum(ep);
            }
            const float sr = wave_sum(lr);
            const float spp = wave_sum(lp);
            if (lane == 0) {
                if (batch) sh.trec[tile - tb] = pack2(sr, spp);
                else st_pair(&rt[tile], pack2(sr, spp));
            }
        });
        if (batch) {
            __syncthreads();
            if (wave == 0 && lane < te - tb) st_pair(&rt[tb + lane], sh.trec[lane]);
        }
    }

    if (!arrive(counter(a.ws.res_cnt, c), (uint32_t)a.r_blk)) return;
    if (wave != 0) return;
    if (GUMBEL && j < L) {
        const int tok = gumbel_finish(a.ws.garg + (size_t)c * kMaxResidSegments * 2, a.Sr, lane);
        if (lane == 0 && a.verify_outputs) a.out_tokens[c * L + j] = tok;
    } else if (j < L) {
        // ---- inverse-CDF draw over max(0, P - Q) (P if that is empty) ----
        const uint64_t *recs = reinterpret_cast<const uint64_t *>(rt);
        const int nt = a.tiles_row;
        RecChunk first;
        load_chunk(recs, nt, 0, lane, first);
        auto get = [&](int t0, RecChunk &c) {
            if (t0 == 0) c = first;
            else load_chunk(recs, nt, t0, lane, c);
        };
        auto mass_r = [&](uint64_t rc) -> double { return (double)lo_f(rc); };
        auto mass_p = [&](uint64_t rc) -> double { return (double)hi_f(rc); };
        double Z = 0.0, before = 0.0, target = 0.0;
        int tile = row_draw(nt, get, lane, mass_r, (double)inf.u, Z, before, target);
        const bool use_p = !(Z > 0.0);
        if (use_p) tile = row_draw(nt, get, lane, mass_p, (double)inf.u, Z, before, target);
        double tile_target = target;
        if (tile < 0) {
            tile = use_p ? row_last_positive(nt, get, lane, mass_p)
                         : row_last_positive(nt, get, lane, mass_r);
            tile_target = __builtin_inf();
        }
        long long tok = 0;
        if (tile >= 0) {
            TileRaw<T> rp, rq;
            load_tile<T, VEC>(prow, tile, a.V, lane, rp);
            if (!ONEHOT) load_tile<T, VEC>(qrow, tile, a.V, lane, rq);
            const float k2 = a.k2;
            const ResidForm rf = resid_form(inf, k2);
            // the weights the tile masses summed, entry by entry
            auto weight = [&](int i) -> float {
                if (ONEHOT) {
                    const float P = fast_exp2(fmaf(elem<T>(rp, i), k2, -inf.cp)) * inf.inv_sp;
                    if (use_p) return P;
                    return elem_index(tile, lane, i) == (long long)inf.xj ? 0.0f : P;
                }
                float P;
                const float R = resid_weight(elem<T>(rp, i), elem<T>(rq, i), rf, P);
                return use_p ? P : R;
            };
            tok = search_tile(weight, tile, lane, before, tile_target);
            if (tok < 0) tok = 0;
        }
        for (int t = lane; t < a.tiles_row; t += kWave) st_pair(&rt[t], 0);
        if (lane == 0 && a.verify_outputs) a.out_tokens[c * L + j] = (int)tok;
    }
    if (lane == 0) {
        // every residual item of c has read the decision: clear it for the next launch
        SeqInfo *si = &a.ws.info[c];
        st32(reinterpret_cast<uint32_t *>(&si->j), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->u), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->cp), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->cq), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->inv_sp), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->inv_sq), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->xj), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->rho_hi), 0u);
        st32(reinterpret_cast<uint32_t *>(&si->rho_lo), 0u);
        st32(counter(a.ws.flag, c), 0u);
    }
}

// VAR selects the correction's variant (sample mode): the Gumbel-max draw
// and the one-hot proposal law are separate instantiations, so that the
// default kernel carries neither their code nor their registers.
template <typename T, bool VEC, int MODE, int VAR>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs a) {
    __shared__ Shared sh;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    int t = (int)blockIdx.x;
    if (t >= a.n_static) {
        // The last items go to whichever workgroups reach them first, so that
        // an XCD running ahead takes more of them: each takes a ticket from a
        // launch-wide counter.  The grid holds spare workgroups, which find
        // the items gone and exit; the last one to take a ticket re-arms the
        // counter.
        if (threadIdx.x == 0) {
            const uint32_t k =
                __hip_atomic_fetch_add(&a.ws.ctl->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (k + 1 == gridDim.x - (uint32_t)a.n_static) st32(&a.ws.ctl->ticket, 0u);
            sh.ticket = a.n_static + (int)k;
        }
        __syncthreads();
        t = sh.ticket;
        if (t >= a.n_items) return;
    }

    if (t < a.n_pq) {
        pq_item<T, VEC, MODE>(a, t, sh, wave, lane);
    } else if (t < a.n_items) {
        const int t2 = t - a.n_pq;
        int c, w;
        if (a.order == 0) {
            // per sequence: its mask-row items, then its residual items
            const int blk = a.q_blk + a.r_blk;
            c = t2 / blk;
            w = t2 - c * blk;
        } else {
            // every mask-row item, then every residual item
            const int nq = a.C * a.q_blk;
            if (t2 < nq) {
                c = t2 / a.q_blk;
                w = t2 - c * a.q_blk;
            } else {
                c = (t2 - nq) / a.r_blk;
                w = a.q_blk + (t2 - nq) - c * a.r_blk;
            }
        }
        if (w < a.q_blk) {
            const int k = w / a.Sq;
            qn_item<T, VEC, MODE>(a, c, k, w - k * a.Sq, sh, wave, lane);
        } else if (MODE == kSample) {
            res_item<T, VEC, VAR>(a, c, w - a.q_blk, sh, wave, lane);
        }
    }
}

}  // namespace

// Items at the end of the launch that take tickets, and spare workgroups in
// percent of them.
constexpr int kTicketItems = 256;
constexpr int kSpareGroupsPct = 25;

template <typename T, bool VEC, int MODE, int VAR>
hipError_t launch_one(const StepArgs &a, hipStream_t stream) {
    // Items that wait (residual items wait for their sequence's decision) wait
    // only on verify items, which take their items by index and never wait;
    // each XCD dispatches its workgroups in index order, so every verify item
    // is dispatched before any ticket is taken on its XCD, and every wait ends.
    // A launch small enough to be resident at once gains nothing from tickets.
    StepArgs b = a;
    const int dyn = a.n_items >= 4 * kTicketItems ? min(kTicketItems, a.n_items - a.n_pq) : 0;
    b.n_static = a.n_items - max(dyn, 0);
    long long grid = a.n_items;
    if (dyn > 0) grid += ((long long)dyn * kSpareGroupsPct + 99) / 100;
    hipLaunchKernelGGL((step_kernel<T, VEC, MODE, VAR>), dim3((unsigned)grid), dim3(kThreads), 0, stream, b);
    return hipGetLastError();
}

template <typename T, bool VEC>
hipError_t launch_typed(const StepArgs &a, int mode, hipStream_t stream) {
    if (mode != kSample) return launch_one<T, VEC, kGreedy, 0>(a, stream);
    switch ((a.sampler ? kVarGumbel : 0) | (a.q_onehot ? kVarOnehot : 0)) {
    case 0: return launch_one<T, VEC, kSample, 0>(a, stream);
    case kVarGumbel: return launch_one<T, VEC, kSample, kVarGumbel>(a, stream);
    case kVarOnehot: return launch_one<T, VEC, kSample, kVarOnehot>(a, stream);
    default: return launch_one<T, VEC, kSample, kVarGumbel | kVarOnehot>(a, stream);
    }
}

hipError_t launch_step(const StepArgs &a, int dtype, int mode, bool vec, hipStream_t stream) {
    if (dtype == kBf16)
        return vec ? launch_typed<uint16_t, true>(a, mode, stream) : launch_typed<uint16_t, false>(a, mode, stream);
    return vec ? launch_typed<float, true>(a, mode, stream) : launch_typed<float, false>(a, mode, stream);
}

}  // namespace isd
