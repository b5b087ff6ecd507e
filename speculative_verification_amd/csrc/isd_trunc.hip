// ISD step with top-k / top-p truncated sampling laws, for gfx950.
//
// The pages' quality runs sample with top-k 50 and top-p 0.95
// ("Introspective Diffusion Language Models | Summary", section 4.1), and the
// acceptance test must use the law of the proposal mechanism actually used
// (section 3.3).  With truncation the anchor law P, the proposal law Q and the
// law of the next proposals are each supported on at most k <= 64 entries of
// their row, so the whole step reduces to one top-k selection per row; every
// later stage works on those k entries.
//
// Ranking: entries are ordered by logit, larger first, ties to the lower
// vocabulary index (-0 ranks as +0).  Each entry gets a unique 64-bit key
// (order-preserving bits of the value, then the complemented index), so the
// ranking is the order of the keys and the top k are the k largest keys.
// top-k keeps the first k ranks; top-p then keeps a rank while the mass of the
// ranks before it, in the top-k renormalised law, is below p; the survivors
// are renormalised.  All probabilities and decisions are in fp64.
//
// Work items, in dispatch order:
//   [verify-row items]  for each sequence c, each verify row (p_0..p_{L-1},
//       then q_0..q_{L-1} unless the proposals are one-hot) and each row
//       segment;
//   [mask-row items]    for each sequence c, each mask row qn_k and segment.
// An item streams its segment with four wavefronts and records, in LDS, the
// best entry of each lane's 32 entries of a tile (a group); it then picks the
// k best group keys, re-reads those k groups and keeps their best k entries:
// the segment's top k, recorded for the row.  Keys are kept in lane-
// distributed sorted lists (lane t holds rank t), merged with a bitonic sort
// and a bitonic merge across lanes.  The item that completes a row merges its
// segment records, applies top-k and top-p and then either draws the next
// proposal (mask row; inverse CDF over the survivors in vocabulary order) or
// stores P'(x_k) or Q'(x_k) and the row's survivors sorted by index (verify
// row).  The item that completes the last verify row of sequence c decides:
// ratios, accept test, first rejection j, alpha, and the correction from
// max(0, P' - Q') over the survivors of p_j (inverse CDF, or Gumbel-max).
// No item ever waits for another.

#include "isd_device.h"
#include "isd_internal.h"

#include <math.h>

namespace isd {

namespace {

// ---------------------------------------------------------------------------
// Keys and lane-distributed sorted lists
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t ord_bits(float v) {
    const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);   // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Unique key of entry idx with value v; larger key = earlier rank.  0 is below
// every real key and marks an empty slot.
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
    return ((uint64_t)ord_bits(v) << 32) | (uint64_t)(uint32_t)~idx;
}

__device__ __forceinline__ float key_value(uint64_t k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~(uint32_t)k; }

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Bitonic sort of one key per lane across the wavefront, largest first.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int lane) {
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t y = xor_lane_n(x, j, lane);
            const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
            x = keep_max ? umax64(x, y) : umin64(x, y);
        }
    }
    return x;
}

// The 64 largest keys of two lists sorted largest first, sorted largest first:
// the lane-wise max of one list and the other reversed is bitonic and holds
// them; a bitonic merge sorts it.
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t a, uint64_t b, int lane) {
    uint64_t x = umax64(a, reverse_lanes(b, lane));
#pragma unroll
    for (int j = kWave / 2; j > 0; j >>= 1) {
        const uint64_t y = xor_lane_n(x, j, lane);
        x = ((lane & j) == 0) ? umax64(x, y) : umin64(x, y);
    }
    return x;
}

// ---------------------------------------------------------------------------
// Selection of a segment's top k (one workgroup)
// ---------------------------------------------------------------------------
//
// A lane's 32 entries of a tile form a group.  Every top-k entry lies in a
// group whose best key is among the k best group keys: if it did not, k
// group maxima would beat it.  So the selection takes three passes:
//
//   1. stream the segment and record each group's best entry in LDS: the
//      order bits of its value and its position in the lane (32 + 8 bits),
//      nothing else, so the stream never waits on selection work;
//   2. from LDS: a threshold from the column maxima (below) leaves few
//      records, which are compacted; when more than 64 remain (or the
//      segment spans several chunks) they are sorted and merged, and ranks
//      0..k-1 of the result are the candidate groups;
//   3. re-read the candidate groups (at most 64 * 32 entries, one tile's
//      worth) and keep the best k of their entries.
// Passes 1 and 2 run over chunks of kMaxSegTiles tiles, so LDS bounds no
// segment length.

constexpr int kMaxSegTiles = 80;   // tiles per chunk of group records in LDS

// Candidate records per chunk: at most k columns (below) hold one, and a column
// holds kMaxSegTiles / kWavesPerGroup records.
constexpr int kMaxCand = kMaxSegTiles / kWavesPerGroup * kMaxTopK;

template <typename T>
struct TruncShared {
    int ncand;
    uint64_t lists[kWavesPerGroup][kWave];
    // Each group's record (0: empty group): the order bits of its best value
    // and that entry's position among the lane's 32.  For bf16 the low 16
    // order bits follow from the sign, so the position takes their place; for
    // fp32 it has an array of its own.
    uint32_t grec[kMaxSegTiles * kWave];
    uint8_t gpos[sizeof(T) == 2 ? 1 : kMaxSegTiles * kWave];
    uint16_t cand[kMaxCand];               // records of a chunk that reach the threshold
};

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Key held by lane `l` (wave-uniform l).
__device__ __forceinline__ uint64_t lane_key(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

template <typename T>
__device__ __forceinline__ void put_record(TruncShared<T> &sh, int at, uint32_t ord, int pos) {
    if constexpr (sizeof(T) == 2) {
        sh.grec[at] = ord ? (ord & 0xFFFF0000u) | (uint32_t)pos : 0u;
    } else {
        sh.grec[at] = ord;
        sh.gpos[at] = (uint8_t)pos;
    }
}

// Order bits of a record (0 for an empty group).  A bf16 value's order bits
// end in 0x0000 when it is positive and 0xFFFF when it is negative; no bf16
// value has order bits that start 0x0000.
template <typename T>
__device__ __forceinline__ uint32_t record_ord(uint32_t rec) {
    if constexpr (sizeof(T) == 2) {
        if (rec == 0u) return 0u;
        return (rec & 0xFFFF0000u) | ((rec & 0x80000000u) ? 0u : 0xFFFFu);
    } else {
        return rec;
    }
}

// Key of the group record at position `at` of the chunk starting at tile cb
// (0 for an empty group).
template <typename T>
__device__ __forceinline__ uint64_t record_key(const TruncShared<T> &sh, int cb, int at) {
    const uint32_t rec = sh.grec[at];
    if (rec == 0u) return 0;
    const int pos = sizeof(T) == 2 ? (int)(rec & 31u) : (int)sh.gpos[sizeof(T) == 2 ? 0 : at];
    const uint32_t idx = (uint32_t)elem_index(cb + at / kWave, at % kWave, pos);
    return ((uint64_t)record_ord<T>(rec) << 32) | (uint64_t)(uint32_t)~idx;
}

// Sorted list (largest first) of up to 64 keys, N offered per lane
// (key(e) for e < N; 0 is not offered): the candidates are packed through
// this wavefront's row of `stage` and sorted once; more than 64 are taken
// 64 at a time and merged.  Uniform control flow.
template <int N, typename Key>
__device__ __forceinline__ uint64_t gather_sorted(Key &&key, uint64_t *stage, int lane) {
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) cnt += key(e) != 0 ? 1u : 0u;
    const uint32_t incl = wave_incl_scan_u32(cnt);
    const int total = __builtin_amdgcn_readlane((int)incl, kWave - 1);
    uint64_t list = 0;
    for (int b0 = 0; b0 < total; b0 += kWave) {
        // candidates b0 .. b0 + 63 of the wavefront's order (lane, then entry)
        int slot = (int)(incl - cnt) - b0;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const uint64_t ke = key(e);
            if (ke != 0) {
                if (slot >= 0 && slot < kWave) stage[slot] = ke;
                ++slot;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint64_t sorted = wave_sort_desc(b0 + lane < total ? stage[lane] : 0, lane);
        list = b0 == 0 ? sorted : wave_merge_desc(list, sorted, lane);
        __builtin_amdgcn_wave_barrier();   // the stage is rewritten next round
    }
    return list;
}

constexpr int kColRecs = kMaxSegTiles / kWavesPerGroup;   // records per column and chunk

// Top k keys of tiles [tb, te) of `row`, largest first (0 past the end),
// returned to wavefront 0 (the others get 0).  All threads call it.
template <typename T, bool VEC>
__device__ __forceinline__ uint64_t select_segment(const T *__restrict__ row, int tb, int te, int V,
                                               int k, int wave, int lane, TruncShared<T> &sh) {
    uint64_t groups = 0;   // the best group keys of the chunks so far (same in every wavefront)
    bool direct = false;   // one chunk with at most 64 candidate records: re-read them all
    uint64_t thr = 0;      // pass 3 keeps entries whose key reaches it
    int ngroups = 0;
    for (int cb = tb; cb < te; cb += kMaxSegTiles) {
        const int ce = min(te, cb + kMaxSegTiles);
        // ---- 1. stream: each group's best entry into LDS; the column maximum ----
        // A thread's records (lane `lane` of its wavefront's tiles) form a column.
        uint64_t colmax = 0;
        stream_row<T, VEC>(row, cb, ce, V, wave, lane, [&](const TileRaw<T> &r, int tile) {
            // the lane's maximum and its first position (the lowest index
            // among equals: a later entry replaces it only if larger)
            float vmax = elem<T>(r, 0);
            int fi = 0;
#pragma unroll
            for (int i = 1; i < kLaneElems; ++i) {
                const float x = elem<T>(r, i);
                fi = x > vmax ? i : fi;
                vmax = fmaxf(vmax, x);
            }
            const long long idx = elem_index(tile, lane, fi);
            const uint32_t o = idx < V ? ord_bits(vmax) : 0u;
            const int at = (tile - cb) * kWave + lane;
            put_record(sh, at, o, fi);
            if (o) colmax = umax64(colmax, ((uint64_t)o << 32) | (uint64_t)(uint32_t)~(uint32_t)idx);
        });
        if (threadIdx.x == 0) sh.ncand = 0;
        sh.lists[wave][lane] = wave_sort_desc(colmax, lane);
        __syncthreads();

        // ---- 2. the candidate groups ----
        // theta0, the k-th best of the column maxima and of the earlier
        // chunks' best keys, is reached by at least k keys, so every top-k key
        // reaches it; and at most k columns hold a key that does.
        uint64_t m = sh.lists[0][lane];
#pragma unroll
        for (int w = 1; w < kWavesPerGroup; ++w) m = wave_merge_desc(m, sh.lists[w][lane], lane);
        if (cb != tb) m = wave_merge_desc(m, groups, lane);
        const uint64_t theta0 = uniform64(lane_key(m, k - 1));
        // the chunk's records that reach theta0, packed into sh.cand
        uint32_t cmask = 0;
        if (colmax != 0 && colmax >= theta0) {
            // order bits first; the position only where they equal theta0's
            const uint32_t tord = (uint32_t)(theta0 >> 32);
#pragma unroll
            for (int i = 0; i < kColRecs; ++i) {
                const int t = cb + wave + kWavesPerGroup * i;
                if (t < ce) {
                    const int at = (t - cb) * kWave + lane;
                    const uint32_t o = record_ord<T>(sh.grec[at]);
                    if (o > tord || (o == tord && o != 0u && record_key(sh, cb, at) >= theta0))
                        cmask |= 1u << i;
                }
            }
        }
        const uint32_t cnt = (uint32_t)__popc(cmask);
        const uint32_t incl = wave_incl_scan_u32(cnt);
        const int wtotal = __builtin_amdgcn_readlane((int)incl, kWave - 1);
        if (wtotal > 0) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&sh.ncand, wtotal);
            base = __builtin_amdgcn_readfirstlane(base) + (int)(incl - cnt);
            for (uint32_t mm = cmask; mm; mm &= mm - 1) {
                const int i = __ffs((int)mm) - 1;
                sh.cand[base++] = (uint16_t)((wave + kWavesPerGroup * i) * kWave + lane);
            }
        }
        __syncthreads();
        const int n = sh.ncand;
        if (cb == tb && ce == te && n <= kWavesPerGroup * (kWave / 4)) {
            // Every top-k entry reaches theta0 and lies in a group whose best
            // key does: pass 3 can take all n candidate groups as they are,
            // without sorting them first.
            direct = true;
            thr = theta0;
            ngroups = n;
            break;
        }
        // sort them, 64 per wavefront at a time, and merge with the earlier best
        uint64_t wl = 0;
        for (int b = wave * kWave; b < n; b += kThreads) {
            const uint64_t sorted =
                wave_sort_desc(b + lane < n ? record_key(sh, cb, sh.cand[b + lane]) : 0, lane);
            wl = b == wave * kWave ? sorted : wave_merge_desc(wl, sorted, lane);
        }
        sh.lists[wave][lane] = wl;
        __syncthreads();
        const int used = min(kWavesPerGroup, (n + kWave - 1) / kWave);   // n >= 1 when any key is real
        for (int w = 0; w < used; ++w)
            groups = (w == 0 && cb == tb) ? sh.lists[0][lane] : wave_merge_desc(groups, sh.lists[w][lane], lane);
        __syncthreads();   // the next chunk or pass overwrites the records and lists
    }

    // ---- 3. re-read the candidate groups; keep the best k entries ----
    // wavefront w takes candidate groups 16w .. 16w + 15; lane j reads run
    // j % 4 (8 consecutive entries, one 16-byte load for bf16) of group 16w + j / 4
    const int gi = wave * (kWave / 4) + lane / 4;
    int gtile = 0, glane = 0;
    bool mine;
    if (direct) {
        mine = gi < ngroups;
        if (mine) {
            const int at = sh.cand[gi];
            gtile = tb + at / kWave;
            glane = at % kWave;
        }
    } else {
        // the k best group keys; every top-k entry's key is at least the k-th
        thr = uniform64(lane_key(groups, k - 1));
        const uint64_t gk = __shfl(groups, gi);
        mine = gi < k && gk != 0;
        if (mine) {
            const uint32_t e0 = key_index(gk);
            gtile = (int)(e0 / kTileElems);
            glane = (int)(e0 % (kWave * kGroupElems)) / kGroupElems;
        }
    }
    uint32_t w[kGroupElems * (int)sizeof(T) / 4] = {};
    long long first = 0;
    if (mine) {
        first = (long long)gtile * kTileElems + (lane % 4) * (kWave * kGroupElems) + glane * kGroupElems;
        load_group<T, VEC>(row, first, V, first + kGroupElems <= (long long)V, w);
    }
    auto entry_key = [&](int e) -> uint64_t {
        float val;
        if constexpr (sizeof(T) == 2)
            val = (e & 1) ? __uint_as_float(w[e >> 1] & 0xFFFF0000u) : __uint_as_float(w[e >> 1] << 16);
        else
            val = __uint_as_float(w[e]);
        const uint64_t key = make_key(val, (uint32_t)(first + e));
        return (mine && first + e < V && key >= thr) ? key : 0;
    };
    const uint64_t out = gather_sorted<kGroupElems>(entry_key, sh.lists[wave], lane);   // lists are free here
    sh.lists[wave][lane] = out;
    __syncthreads();
    uint64_t x = 0;
    if (wave == 0) {
        x = out;
#pragma unroll
        for (int w2 = 1; w2 < kWavesPerGroup; ++w2) x = wave_merge_desc(x, sh.lists[w2][lane], lane);
    }
    return x;
}

// ---------------------------------------------------------------------------
// Truncated law of one row from its top keys (one wavefront)
// ---------------------------------------------------------------------------

struct RowLaw {
    uint32_t idx;      // lane s < n: the s-th survivor in increasing vocabulary index
    double w;          // its probability under the truncated law (0 for s >= n)
    int n;             // survivors
    bool empty;        // no finite logit among the top keys
};

// `top` holds the row's keys sorted largest first (lane t = rank t, 0 past the
// row's end); ranks >= k are ignored.
__device__ __forceinline__ RowLaw truncated_law(uint64_t top, int k, double temp, double top_p,
                                                int lane) {
    const bool real = lane < k && top != 0;
    const float v = key_value(top);
    const float v0 = __shfl(v, 0);
    RowLaw law;
    law.empty = __shfl(top, 0) == 0 || !(v0 > -__builtin_inff());
    double w = 0.0;
    if (real && !law.empty && v > -__builtin_inff())
        w = exp((double)v / temp - (double)v0 / temp);
    bool keep = real;
    if (top_p < 1.0) {
        const double W = wave_sum_d(w);
        const double pi = W > 0.0 ? w / W : 0.0;
        const double incl = wave_incl_scan_d(pi, lane);
        double before = dpp_d<0x138>(incl);   // wave_shr:1
        if (lane == 0) before = 0.0;
        keep = real && before < top_p;
    }
    const double Wk = wave_sum_d(keep ? w : 0.0);
    const double P = (keep && Wk > 0.0) ? w / Wk : 0.0;
    // survivors in increasing vocabulary index: sort (index, rank) ascending
    const uint64_t key2 = keep ? (((uint64_t)key_index(top) << 32) | (uint64_t)lane) : ~0ull;
    const uint64_t asc = ~wave_sort_desc(~key2, lane);
    const int src = (int)(uint32_t)asc;
    const bool live = asc != ~0ull;
    law.n = __popcll(__ballot(keep));
    law.idx = live ? (uint32_t)(asc >> 32) : 0u;
    const double Ps = __shfl(P, live ? src : 0);
    law.w = live ? Ps : 0.0;
    return law;
}

// Inverse-CDF draw over weights held one per lane in increasing vocabulary
// index: the first lane whose running sum exceeds u times the total, else the
// last lane with positive weight, else lane 0.
__device__ __forceinline__ int lane_inverse_cdf(double w, double u, int lane) {
    const double Z = wave_sum_d(w);
    const double inc = wave_incl_scan_d(w, lane);
    const unsigned long long hit = __ballot(w > 0.0 && inc > u * Z);
    if (hit) return wave_first(hit);
    const unsigned long long pos = __ballot(w > 0.0);
    return pos ? 63 - __clzll((long long)pos) : 0;
}

// ---------------------------------------------------------------------------
// Workspace records
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t *seg_keys(const StepArgs &a, int row, int seg) {
    return a.tws.keys + ((size_t)row * a.St + seg) * kWave;
}
// survivors of verify row `slot` (0..2L-1) of sequence c: (index, weight) pairs
__device__ __forceinline__ uint64_t *row_list(const StepArgs &a, int c, int slot) {
    return a.tws.lists + ((size_t)c * 2 * a.L + slot) * kWave * 2;
}

__device__ __forceinline__ double ld_f64(const uint64_t *p) {
    return __longlong_as_double((long long)ld64(p));
}
__device__ __forceinline__ void st_f64(uint64_t *p, double v) {
    st64(p, (uint64_t)__double_as_longlong(v));
}

// Counts one arrival of a single wavefront on `counter` (total arrivals
// `total`) after its own record stores; returns, to every lane, whether it was
// the last.  The last one resets the counter for the next launch.
__device__ __forceinline__ bool arrive_wave(uint32_t *counter, uint32_t total, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    int last = 0;
    if (lane == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = prev + 1 == total;
        if (last) st32(counter, 0u);
    }
    last = __shfl(last, 0);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return last != 0;
}

// ---------------------------------------------------------------------------
// Decision of one sequence (wavefront 0 of the item completing its rows)
// ---------------------------------------------------------------------------

__device__ __forceinline__ void trunc_decide(const StepArgs &a, int c, int lane) {
    const int L = a.L;
    const bool valid = lane < L;
    const int kk = valid ? lane : 0;
    const int xk = valid ? a.x[c * L + kk] : 0;
    const bool bad = valid && (xk < 0 || xk >= a.V);
    if (bad) atomicOr(&a.ws.ctl->error, kErrBadToken);
    uint64_t *pxq = a.tws.pxq + (size_t)c * 2 * L;
    double px = 0.0, qx = 0.0;
    if (valid) {
        px = ld_f64(&pxq[kk]);
        qx = a.q_onehot ? (bad ? 0.0 : 1.0) : ld_f64(&pxq[L + kk]);
        st64(&pxq[kk], 0);
        if (!a.q_onehot) st64(&pxq[L + kk], 0);
    }
    // min(1, P'(x)/Q'(x)); Q'(x) = 0 gives 1 if P'(x) > 0, else 0.  The accept
    // test may use the relaxed ratio; alpha stays the plain rate.
    const double r = qx > 0.0 ? fmin(1.0, px / qx) : (px > 0.0 ? 1.0 : 0.0);
    const double ra = a.relax1p == 1.0
                          ? r
                          : (qx > 0.0 ? fmin(1.0, (a.relax1p * px) / qx) : (px > 0.0 ? 1.0 : 0.0));
    const bool accepted = !valid || (a.ua == nullptr || (double)a.ua[c * L + kk] < ra);
    const unsigned long long rej = __ballot(!accepted);
    const int j = rej ? wave_first(rej) : L;
    const float alpha = (float)(wave_sum_d(valid ? r : 0.0) / (double)L);
    if (valid) {
        if (a.p_x) a.p_x[c * L + kk] = (float)px;
        if (a.q_x) a.q_x[c * L + kk] = (float)qx;
        if (a.verify_outputs && kk != j) a.out_tokens[c * L + kk] = kk < j ? xk : -1;
    }
    if (lane == 0 && a.alpha) a.alpha[c] = alpha;
    if (lane == 0 && a.verify_outputs) {
        a.accept_len[c] = j;
        a.n_emitted[c] = j + (j < L ? 1 : 0);
    }

    if (a.verify_outputs && j < L) {
        // correction from max(0, P' - Q') over the survivors of p_j (P' if that is empty)
        const uint64_t *pl = row_list(a, c, j);
        const uint32_t idx = (uint32_t)ld64(&pl[2 * lane]);
        const double P = ld_f64(&pl[2 * lane + 1]);
        double Q = 0.0;
        const int xj = __shfl(xk, j);
        if (a.q_onehot) {
            Q = (int)idx == xj ? 1.0 : 0.0;
        } else {
            const uint64_t *ql = row_list(a, c, L + j);
            const uint32_t qidx = (uint32_t)ld64(&ql[2 * lane]);
            const double qw = ld_f64(&ql[2 * lane + 1]);
            for (int t = 0; t < kWave; ++t) {
                const uint32_t ti = __shfl(qidx, t);
                const double tw = __shfl(qw, t);
                if (ti == idx) Q += tw;    // unused slots carry weight 0
            }
        }
        const double R = fmax(P - Q, 0.0);
        const bool use_p = !(wave_sum_d(R) > 0.0);
        const double wgt = use_p ? P : R;
        const float ur = a.ur[c * L + j];
        int tok;
        if (a.sampler) {
            // Gumbel-max: argmax of w / E over the survivors (ties to the lower index)
            const float e = inv_exp_noise1(idx, (uint32_t)j, __float_as_uint(ur), (uint32_t)c);
            float bv = 0.0f;
            int bi = INT_MAX;
            const float s = (float)wgt * e;
            if (wgt > 0.0 && s > 0.0) {
                bv = s;
                bi = (int)idx;
            }
            wave_argmax(bv, bi);
            tok = bi == INT_MAX ? 0 : bi;
        } else {
            const int l = lane_inverse_cdf(wgt, (double)ur, lane);
            tok = (int)__shfl(idx, l);
        }
        if (lane == 0) a.out_tokens[c * L + j] = tok;
    }
    // the survivor lists of c are consumed: return them to zero
    for (int slot = 0; slot < 2 * L; ++slot) {
        uint64_t *l = row_list(a, c, slot);
        st64(&l[2 * lane], 0);
        st64(&l[2 * lane + 1], 0);
    }

    // batch mean of alpha, by the last sequence to be decided
    if (a.alpha_mean) {
        int last = 0;
        if (lane == 0) {
            st32(&a.tws.alpha[c], __float_as_uint(alpha));
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_s_waitcnt(0);
            last = __hip_atomic_fetch_add(&a.ws.ctl->seq_done, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) + 1 == (uint32_t)a.C;
        }
        last = __shfl(last, 0);
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            double sum = 0.0;
            for (int c0 = 0; c0 < a.C; c0 += kWave) {
                const int cc = c0 + lane;
                sum += wave_sum_d(cc < a.C ? (double)__uint_as_float(ld32(&a.tws.alpha[cc])) : 0.0);
            }
            for (int cc = lane; cc < a.C; cc += kWave) st32(&a.tws.alpha[cc], 0u);
            if (lane == 0) {
                a.alpha_mean[0] = (float)(sum / (double)a.C);
                st32(&a.ws.ctl->seq_done, 0u);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

__device__ __forceinline__ long long trunc_row_offset(const StepArgs &a, int c, int k) {
    return (long long)c * a.ldc + (long long)k * a.ld;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void trunc_kernel(StepArgs a) {
    __shared__ TruncShared<T> sh;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int t = (int)blockIdx.x;
    const int L = a.L;
    const int n_v = a.C * a.rows_pq * a.St;

    // which row and segment this item streams
    int c, slot, seg;
    bool verify;
    if (t < n_v) {
        const int per = a.rows_pq * a.St;
        c = t / per;
        const int rem = t - c * per;
        slot = rem / a.St;       // 0..L-1: p rows; L..2L-1: q rows
        seg = rem - slot * a.St;
        verify = true;
    } else {
        const int t2 = t - n_v;
        const int per = L * a.St;
        c = t2 / per;
        const int rem = t2 - c * per;
        slot = 2 * L + rem / a.St;
        seg = rem % a.St;
        verify = false;
    }
    const int k_row = verify ? (slot < L ? slot : slot - L) : slot - 2 * L;
    const int rowid = c * 3 * L + slot;

    if (verify && a.vmask && a.vmask[c] == 0) {
        if (slot == 0 && seg == 0) {
            for (int kk = threadIdx.x; kk < L; kk += kThreads) {
                if (a.verify_outputs) a.out_tokens[c * L + kk] = -1;
                if (a.p_x) a.p_x[c * L + kk] = 0.0f;
                if (a.q_x) a.q_x[c * L + kk] = 0.0f;
            }
            if (threadIdx.x == 0) {
                if (a.verify_outputs) {
                    a.accept_len[c] = -1;
                    a.n_emitted[c] = 0;
                }
                if (a.alpha) a.alpha[c] = 0.0f;
            }
        }
        return;
    }
    if (!verify && a.pmask && a.pmask[c] == 0) {
        if (seg == 0 && threadIdx.x == 0) {
            a.next_tokens[c * L + k_row] = -1;
            if (a.qnext_x) a.qnext_x[c * L + k_row] = 0.0f;
        }
        return;
    }

    const void *base = verify ? (slot < L ? a.p : a.q) : a.qn;
    const T *row = static_cast<const T *>(base) + trunc_row_offset(a, c, k_row);
    const int k = a.top_k;

    // ---- this segment's top k ----
    const int tb = seg * a.tpst;
    const int te = min(a.tiles_row, tb + a.tpst);
    const uint64_t seg_top = select_segment<T, VEC>(row, tb, te, a.V, k, wave, lane, sh);

    // ---- the row's top k, truncated law ----
    uint64_t top = 0;
    if (a.St == 1) {
        // the item holds the whole row
        if (wave != 0) return;
        top = lane < k ? seg_top : 0;
    } else {
        if (wave == 0 && lane < k) st64(&seg_keys(a, rowid, seg)[lane], seg_top);
        if (!arrive(counter(a.tws.row_cnt, rowid), (uint32_t)a.St)) return;
        if (wave != 0) return;
        uint64_t rec[kMaxTruncSegments];
#pragma unroll
        for (int s = 0; s < kMaxTruncSegments; ++s)
            rec[s] = (s < a.St && lane < k) ? ld64(&seg_keys(a, rowid, s)[lane]) : 0;
#pragma unroll
        for (int s = 0; s < kMaxTruncSegments; ++s)
            if (s < a.St && lane < k) st64(&seg_keys(a, rowid, s)[lane], 0);
        top = rec[0];
#pragma unroll
        for (int s = 1; s < kMaxTruncSegments; ++s)
            if (s < a.St) top = wave_merge_desc(top, rec[s], lane);
    }
    const RowLaw law = truncated_law(top, k, a.temp, a.top_p, lane);
    if (law.empty && lane == 0) atomicOr(&a.ws.ctl->error, kErrEmptyRow);

    if (!verify) {
        const int r = c * L + k_row;
        const int l = lane_inverse_cdf(law.w, (double)a.up[r], lane);
        const int tok = (int)__shfl(law.idx, l);
        const double pw = __shfl(law.w, l);
        if (lane == 0) {
            a.next_tokens[r] = tok;
            if (a.qnext_x) a.qnext_x[r] = (float)pw;
        }
        return;
    }

    // verify row: P'(x_k) or Q'(x_k), and the survivors for a correction
    const int xk = a.x[c * L + k_row];
    const unsigned long long hit = __ballot(lane < law.n && (int)law.idx == xk);
    const double wx = hit ? __shfl(law.w, wave_first(hit)) : 0.0;
    if (lane == 0) st_f64(&a.tws.pxq[(size_t)c * 2 * L + slot], wx);
    if (a.verify_outputs) {
        uint64_t *l = row_list(a, c, slot);
        st64(&l[2 * lane], lane < law.n ? (uint64_t)law.idx : 0);
        st_f64(&l[2 * lane + 1], lane < law.n ? law.w : 0.0);
    }
    if (!arrive_wave(counter(a.tws.seq_cnt, c), (uint32_t)a.rows_pq, lane)) return;
    trunc_decide(a, c, lane);
}

}  // namespace

hipError_t launch_trunc(const StepArgs &a, int dtype, bool vec, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_items), block(kThreads);
    if (dtype == kBf16) {
        if (vec) hipLaunchKernelGGL((trunc_kernel<uint16_t, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((trunc_kernel<uint16_t, false>), grid, block, 0, stream, a);
    } else {
        if (vec) hipLaunchKernelGGL((trunc_kernel<float, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((trunc_kernel<float, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace isd
