// Device building blocks shared by the ISD kernels: wavefront reductions,
// vectorised tile loads of logits rows, the records and completion counters
// that workgroups of one launch exchange, and the Philox4x32-10 generator of
// the Gumbel-max draws.
#pragma once

#include "isd_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace isd {
namespace {

constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Wavefront primitives
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}

// Lane exchanges in the VALU: DPP row operations and the permlane16/32 swaps
// move data between lanes in a few cycles, where ds_bpermute takes a round
// trip through the LDS crossbar.  xor_lane<J>(v, lane) is v of lane lane ^ J:
//   J = 1, 2   quad_perm [1,0,3,2] and [2,3,0,1];
//   J = 4      row_ror:4 gives lane - 4 (mod 16), row_ror:12 lane + 4;
//   J = 8      row_ror:8;
//   J = 16, 32 the permlane swap of odd and even rows (or row pairs): with
//              both operands v, the first result holds lane - J on the lanes
//              with bit J set, the second lane + J on the others.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
    static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "lane mask");
    if constexpr (J == 1) {
        return dpp_u32<0xB1>(v);
    } else if constexpr (J == 2) {
        return dpp_u32<0x4E>(v);
    } else if constexpr (J == 4) {
        const uint32_t down = dpp_u32<0x124>(v), up = dpp_u32<0x12C>(v);
        return (lane & 4) ? down : up;
    } else if constexpr (J == 8) {
        return dpp_u32<0x128>(v);
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane(uint64_t v, int lane) {
    const uint32_t lo = xor_lane<J>((uint32_t)v, lane), hi = xor_lane<J>((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

template <int J>
__device__ __forceinline__ double xor_lane(double v, int lane) {
    return __longlong_as_double((long long)xor_lane<J>((uint64_t)__double_as_longlong(v), lane));
}

template <int J>
__device__ __forceinline__ float xor_lane(float v, int lane) {
    return __uint_as_float(xor_lane<J>(__float_as_uint(v), lane));
}

// The same with a mask known only after unrolling.
template <typename V>
__device__ __forceinline__ V xor_lane_n(V v, int j, int lane) {
    switch (j) {
    case 1: return xor_lane<1>(v, lane);
    case 2: return xor_lane<2>(v, lane);
    case 4: return xor_lane<4>(v, lane);
    case 8: return xor_lane<8>(v, lane);
    case 16: return xor_lane<16>(v, lane);
    default: return xor_lane<32>(v, lane);
    }
}

// v of lane 63 - lane: row_mirror reverses each row of 16, then rows r and
// 3 - r (lane ^ 48) are exchanged.
__device__ __forceinline__ uint64_t reverse_lanes(uint64_t v, int lane) {
    const uint32_t lo = dpp_u32<0x140>((uint32_t)v), hi = dpp_u32<0x140>((uint32_t)(v >> 32));
    return xor_lane<16>(xor_lane<32>(((uint64_t)hi << 32) | lo, lane), lane);
}

// row_ror:n rotates within each row of 16 lanes; four rotations give every
// lane its row's result, two cross-row exchanges finish the wavefront.  All
// lanes end with bitwise-identical results.
__device__ __forceinline__ float wave_max(float v) {
    const int lane = (int)__lane_id();
    v = fmaxf(v, dpp<0x128>(v));
    v = fmaxf(v, dpp<0x124>(v));
    v = fmaxf(v, dpp<0x122>(v));
    v = fmaxf(v, dpp<0x121>(v));
    v = fmaxf(v, xor_lane<16>(v, lane));
    v = fmaxf(v, xor_lane<32>(v, lane));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    const int lane = (int)__lane_id();
    v += dpp<0x128>(v);
    v += dpp<0x124>(v);
    v += dpp<0x122>(v);
    v += dpp<0x121>(v);
    v += xor_lane<16>(v, lane);
    v += xor_lane<32>(v, lane);
    return v;
}

// Butterfly sum: every lane ends with the same bits (each exchange adds the
// same two values in the same order on both lanes of a pair).
__device__ __forceinline__ double wave_sum_d(double v) {
    const int lane = (int)__lane_id();
    v += xor_lane<32>(v, lane);
    v += xor_lane<16>(v, lane);
    v += xor_lane<8>(v, lane);
    v += xor_lane<4>(v, lane);
    v += xor_lane<2>(v, lane);
    v += xor_lane<1>(v, lane);
    return v;
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)u), hi = dpp_u32<CTRL, ROWS>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over the lanes: row_shr:1,2,4,8 scan each row of 16
// (lanes with no source read 0), then row_bcast:15 adds row 0's total to
// row 1 and row 2's to row 3, and row_bcast:31 adds the total of rows 0-1 to
// rows 2-3.
__device__ __forceinline__ double wave_incl_scan_d(double v, int lane) {
    (void)lane;
    v += dpp_d<0x111>(v);
    v += dpp_d<0x112>(v);
    v += dpp_d<0x114>(v);
    v += dpp_d<0x118>(v);
    v += dpp_d<0x142, 0xA>(v);
    v += dpp_d<0x143, 0xC>(v);
    return v;
}

// Four independent inclusive prefix sums over the lanes, step by step, so
// that their DPP chains overlap.
__device__ __forceinline__ void wave_incl_scan4_d(double (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += dpp_d<0x111>(v[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += dpp_d<0x112>(v[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += dpp_d<0x114>(v[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += dpp_d<0x118>(v[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += dpp_d<0x142, 0xA>(v[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += dpp_d<0x143, 0xC>(v[i]);
}

// v of lane l (l wave-uniform), read through the scalar unit.
__device__ __forceinline__ double lane_read_d(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum of 32-bit counts over the lanes (same DPP pattern).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    v += dpp_u32<0x111>(v);
    v += dpp_u32<0x112>(v);
    v += dpp_u32<0x114>(v);
    v += dpp_u32<0x118>(v);
    v += dpp_u32<0x142, 0xA>(v);
    v += dpp_u32<0x143, 0xC>(v);
    return v;
}

__device__ __forceinline__ int wave_first(unsigned long long mask) {
    return __ffsll((long long)mask) - 1;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^n for an integer-valued float n, saturating far below the fp64 range.
__device__ __forceinline__ double pow2_int(float n) {
    return ldexp(1.0, (int)fmaxf(n, -2000.0f));
}

// ---------------------------------------------------------------------------
// Tile loads
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct TileRaw {
    static constexpr int kWords = kLaneElems * (int)sizeof(T) / 4;
    uint32_t w[kWords];
};

template <typename T>
__device__ __forceinline__ uint32_t neg_inf_bits();
template <>
__device__ __forceinline__ uint32_t neg_inf_bits<uint16_t>() { return 0xFF80u; }
template <>
__device__ __forceinline__ uint32_t neg_inf_bits<float>() { return 0xFF800000u; }

template <typename T>
__device__ __forceinline__ uint32_t load_bits(const T *p) {
    if constexpr (sizeof(T) == 2) return (uint32_t)(*reinterpret_cast<const uint16_t *>(p));
    else return *reinterpret_cast<const uint32_t *>(p);
}

// One lane's 8-element group at element offset i of `row` (8 consecutive
// elements); elements at or past V read as -inf and are never loaded.  With
// VEC the group is one or two 16-byte non-temporal loads: the logits are
// streamed once, and non-temporal loads keep them from displacing useful
// cache lines and measurably raise the read rate.  The VEC form is used only
// for rows whose length V is a multiple of 8, so a group lies either wholly
// below V (`whole`) or wholly at or past it and needs no element-wise bound
// checks, whose code would otherwise be inlined at every tile load.
template <typename T, bool VEC>
__device__ __forceinline__ void load_group(const T *__restrict__ row, long long i, int V, bool whole,
                                           uint32_t *w) {
    constexpr int kVecPerGroup = kGroupElems * (int)sizeof(T) / 16;   // 1 (bf16) or 2 (fp32)
    constexpr int kWordsPerGroup = kGroupElems * (int)sizeof(T) / 4;
    if constexpr (VEC) {
        if (whole) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(row + i);
#pragma unroll
            for (int h = 0; h < kVecPerGroup; ++h) {
                const u32x4 v = __builtin_nontemporal_load(&src[h]);
                w[h * 4 + 0] = v.x;
                w[h * 4 + 1] = v.y;
                w[h * 4 + 2] = v.z;
                w[h * 4 + 3] = v.w;
            }
        } else {
            const uint32_t ninf = sizeof(T) == 2 ? (neg_inf_bits<T>() | (neg_inf_bits<T>() << 16))
                                                 : neg_inf_bits<T>();
#pragma unroll
            for (int k = 0; k < kWordsPerGroup; ++k) w[k] = ninf;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kGroupElems; ++e) {
            const uint32_t b = (i + e < (long long)V) ? load_bits<T>(row + i + e) : neg_inf_bits<T>();
            if constexpr (sizeof(T) == 2) {
                if (e & 1) w[e >> 1] |= b << 16;
                else w[e >> 1] = b;
            } else {
                w[e] = b;
            }
        }
    }
}

// Lane `lane`'s 32 elements of a tile that lies wholly below V, on the vector
// path: four (bf16) or eight (fp32) unconditional 16-byte non-temporal loads.
template <typename T>
__device__ __forceinline__ void load_tile_full(const T *__restrict__ row, int tile, int lane,
                                               TileRaw<T> &r) {
    constexpr int kWordsPerGroup = kGroupElems * (int)sizeof(T) / 4;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(row + (long long)tile * kTileElems +
                                                       lane * kGroupElems);
#pragma unroll
    for (int g = 0; g < kGroupsPerTile; ++g)
#pragma unroll
        for (int h = 0; h < kWordsPerGroup / 4; ++h) {
            const u32x4 v = __builtin_nontemporal_load(&src[g * (kWave * kGroupElems * (int)sizeof(T) / 16) + h]);
            r.w[g * kWordsPerGroup + h * 4 + 0] = v.x;
            r.w[g * kWordsPerGroup + h * 4 + 1] = v.y;
            r.w[g * kWordsPerGroup + h * 4 + 2] = v.z;
            r.w[g * kWordsPerGroup + h * 4 + 3] = v.w;
        }
}

// Lane `lane`'s 32 elements of tile `tile` of `row`; elements at or past V
// read as -inf and are never loaded.  In the last, partial tile of a row the
// groups wholly below V still take the vector path, so that tile costs about
// what a full one does.
template <typename T, bool VEC>
__device__ __forceinline__ void load_tile(const T *__restrict__ row, int tile, int V, int lane,
                                          TileRaw<T> &r) {
    constexpr int kWordsPerGroup = kGroupElems * (int)sizeof(T) / 4;
    const long long base = (long long)tile * kTileElems + lane * kGroupElems;
    const bool full = (long long)(tile + 1) * kTileElems <= (long long)V;
#pragma unroll
    for (int g = 0; g < kGroupsPerTile; ++g) {
        const long long i = base + g * (kWave * kGroupElems);
        load_group<T, VEC>(row, i, V, full || i + kGroupElems <= (long long)V,
                           &r.w[g * kWordsPerGroup]);
    }
}

// Element idx (0..31, group-major) of a lane's tile as fp32.
template <typename T>
__device__ __forceinline__ float elem(const TileRaw<T> &r, int idx) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t w = r.w[idx >> 1];
        return (idx & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    } else {
        return __uint_as_float(r.w[idx]);
    }
}

// max(a, b, c) by the hardware instruction.  fmaxf would first quiet each
// operand that does not come from arithmetic (one extra max per element of a
// tile, since the elements come from bit operations); NaN logits are
// undefined input, so the quieting buys nothing here.
__device__ __forceinline__ float max3_hw(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Vocab index of element idx of lane `lane` in tile `tile`.
__device__ __forceinline__ long long elem_index(int tile, int lane, int idx) {
    return (long long)tile * kTileElems + (idx / kGroupElems) * (kWave * kGroupElems) +
           lane * kGroupElems + (idx % kGroupElems);
}

template <typename T>
__device__ __forceinline__ float load_value(const T *row, long long i) {
    const uint32_t b = load_bits<T>(row + i);
    if constexpr (sizeof(T) == 2) return __uint_as_float(b << 16);
    else return __uint_as_float(b);
}

template <typename T>
__device__ __forceinline__ void unpack(const TileRaw<T> &r, float (&v)[kLaneElems]) {
#pragma unroll
    for (int i = 0; i < kLaneElems; ++i) v[i] = elem<T>(r, i);
}

__device__ __forceinline__ float max32(const float (&v)[kLaneElems]) {
    float m[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) m[i] = fmaxf(v[i], v[i + 16]);
#pragma unroll
    for (int s = 8; s >= 1; s >>= 1)
#pragma unroll
        for (int i = 0; i < s; ++i) m[i] = fmaxf(m[i], m[i + s]);
    return m[0];
}

template <int N>
__device__ __forceinline__ float tree_sum(float (&e)[N]) {
#pragma unroll
    for (int s = N / 2; s >= 1; s >>= 1)
#pragma unroll
        for (int i = 0; i < s; ++i) e[i] += e[i + s];
    return e[0];
}

// Streams tiles tile_begin + wave, + kWavesPerGroup, ... < tile_end of `row`
// (wave is wavefront-uniform), keeping the next tile's loads in flight while
// `f` consumes the current one.  On the vector path the tiles wholly below V
// run in a loop whose loads are all unconditional and whose two tile buffers
// alternate roles (the loop is unrolled twice): a load under a branch the
// wavefront might skip, or a copy of a buffer still being loaded, would make
// the compiler wait for every load in flight, the prefetch included, before
// the current tile is used.  A row's last, partial tile is taken on its own.
// SPLIT = false keeps the single loop with per-group load checks, which holds
// fewer registers (for a heavy f) but keeps only one tile in flight.
template <typename T, bool VEC, bool SPLIT = true, typename F>
__device__ __forceinline__ void stream_row(const T *__restrict__ row, int tile_begin, int tile_end,
                                           int V, int wave, int lane, F &&f) {
    int t = tile_begin + wave;
    if (t >= tile_end) return;
    if constexpr (VEC && SPLIT) {
        const int full_end = min(tile_end, V / kTileElems);   // tiles below it are whole
        if (t < full_end) {
            TileRaw<T> a, b;
            load_tile_full<T>(row, t, lane, a);
            for (;;) {
                if (t + kWavesPerGroup >= full_end) {
                    f(a, t);
                    t += kWavesPerGroup;
                    break;
                }
                load_tile_full<T>(row, t + kWavesPerGroup, lane, b);
                f(a, t);
                t += kWavesPerGroup;
                if (t + kWavesPerGroup >= full_end) {
                    f(b, t);
                    t += kWavesPerGroup;
                    break;
                }
                load_tile_full<T>(row, t + kWavesPerGroup, lane, a);
                f(b, t);
                t += kWavesPerGroup;
            }
        }
        if (t < tile_end) {   // the row's partial last tile
            TileRaw<T> a;
            load_tile<T, VEC>(row, t, V, lane, a);
            f(a, t);
        }
    } else {
        TileRaw<T> cur;
        load_tile<T, VEC>(row, t, V, lane, cur);
        for (;;) {
            const int tn = t + kWavesPerGroup;
            const bool more = tn < tile_end;
            TileRaw<T> nxt;
            if (more) load_tile<T, VEC>(row, tn, V, lane, nxt);
            f(cur, t);
            if (!more) break;
            cur = nxt;
            t = tn;
        }
    }
}

// Lane `lane`'s 32 elements of the same whole tile of two rows, the loads of
// the two rows interleaved group by group (the first group of both is needed
// first).
template <typename T>
__device__ __forceinline__ void load_tile_pair_full(const T *__restrict__ ra, const T *__restrict__ rb,
                                                    int tile, int lane, TileRaw<T> &ca,
                                                    TileRaw<T> &cb) {
    constexpr int kWordsPerGroup = kGroupElems * (int)sizeof(T) / 4;
    const long long off = (long long)tile * kTileElems + lane * kGroupElems;
    const u32x4 *sa = reinterpret_cast<const u32x4 *>(ra + off);
    const u32x4 *sb = reinterpret_cast<const u32x4 *>(rb + off);
    constexpr int kStride = kWave * kGroupElems * (int)sizeof(T) / 16;   // u32x4 per group row
#pragma unroll
    for (int g = 0; g < kGroupsPerTile; ++g)
#pragma unroll
        for (int h = 0; h < kWordsPerGroup / 4; ++h) {
            const u32x4 va = __builtin_nontemporal_load(&sa[g * kStride + h]);
            const u32x4 vb = __builtin_nontemporal_load(&sb[g * kStride + h]);
            uint32_t *wa = &ca.w[g * kWordsPerGroup + h * 4];
            uint32_t *wb = &cb.w[g * kWordsPerGroup + h * 4];
            wa[0] = va.x; wa[1] = va.y; wa[2] = va.z; wa[3] = va.w;
            wb[0] = vb.x; wb[1] = vb.y; wb[2] = vb.z; wb[3] = vb.w;
        }
}

// Streams the same tiles of two rows together (one tile of each in flight);
// on the vector path the whole tiles take unconditional loads and a row's
// partial last tile is taken on its own.
// SPLIT = false keeps one loop with per-group load checks (fewer registers
// live at once, for a heavy f).
template <typename T, bool VEC, bool SPLIT = true, typename F>
__device__ __forceinline__ void stream_rows2(const T *__restrict__ ra, const T *__restrict__ rb,
                                             int tile_begin, int tile_end, int V, int wave,
                                             int lane, F &&f) {
    int t = tile_begin + wave;
    if constexpr (VEC && SPLIT) {
        const int full_end = min(tile_end, V / kTileElems);
        for (; t < full_end; t += kWavesPerGroup) {
            TileRaw<T> ca, cb;
            load_tile_pair_full<T>(ra, rb, t, lane, ca, cb);
            f(ca, cb, t);
        }
    }
    for (; t < tile_end; t += kWavesPerGroup) {
        TileRaw<T> ca, cb;
        load_tile<T, VEC>(ra, t, V, lane, ca);
        load_tile<T, VEC>(rb, t, V, lane, cb);
        f(ca, cb, t);
    }
}

// ---------------------------------------------------------------------------
// Data exchanged between workgroups of one launch
// ---------------------------------------------------------------------------
//
// Records that one workgroup writes and another reads in the same launch
// (segment partials, tile masses, the per-sequence decision) are written and
// read with agent-scope atomic stores and loads, which are coherent across
// the XCDs and never served from a stale per-XCD L2 line.  Each wave waits
// for its own record stores to complete (s_waitcnt) before the workgroup
// barrier; thread 0 then counts the workgroup with one relaxed atomic on a
// counter that has a 128-byte line to itself.  No agent-scope fence is
// issued: on this part such a fence writes back or invalidates the L2 and,
// issued by thousands of workgroups, serialises the launch.

__device__ __forceinline__ void st32(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld32(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld64(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
    return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}
__device__ __forceinline__ uint64_t pack2(float lo, int hi) {
    return (uint64_t)__float_as_uint(lo) | ((uint64_t)(uint32_t)hi << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }
__device__ __forceinline__ int hi_i(uint64_t v) { return (int)(uint32_t)(v >> 32); }

__device__ __forceinline__ void st_pair(void *r, uint64_t v) { st64(static_cast<uint64_t *>(r), v); }
__device__ __forceinline__ uint64_t ld_pair(const void *r) {
    return ld64(static_cast<const uint64_t *>(r));
}

// Counts the workgroup's arrival on `counter` (total arrivals `total`) once
// every wavefront's record stores have completed, and returns true, on
// wavefront 0 only, to the last arrival, which also resets the counter.  The
// other wavefronts return false at once, without waiting for the count: every
// finisher runs on wavefront 0.
__device__ __forceinline__ bool arrive(uint32_t *counter, uint32_t total) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x >= kWave) return false;
    int last = 0;
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = prev + 1 == total;
        if (last) st32(counter, 0u);
    }
    last = __builtin_amdgcn_readfirstlane(last);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return last != 0;
}

__device__ __forceinline__ bool arg_better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float &bv, int &bi) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const int lane = (int)__lane_id();
        const float ov = xor_lane_n(bv, o, lane);
        const int oi = (int)xor_lane_n((uint32_t)bi, o, lane);
        if (arg_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
}

__device__ __forceinline__ uint32_t *counter(uint32_t *base, int i) {
    return base + (size_t)i * kCounterStride;
}

// Publishes sequence c's decision for its residual items (one lane): j, the
// residual draw's uniform, the references and denominators of rows p[c, j]
// and q[c, j], and their ratio Sp / Sq as rho_hi + rho_lo (both fp32, the
// second holding what the first rounds away), then the flag.  The flag holds
// the launch's epoch, so a flag left over from an earlier launch never
// releases a wait of this one.
__device__ __forceinline__ void publish_decision(const StepArgs &a, int c, int j, float u, float cp, float cq,
                                 double sp, double sq, int xj, int lane) {
    // one store instruction: lane w writes word w of the record (the alpha
    // word is not part of the decision)
    uint32_t *si = reinterpret_cast<uint32_t *>(&a.ws.info[c]);
    const double rho = sq > 0.0 ? sp / sq : 0.0;
    const float rho_hi = (float)rho;
    const float rho_lo = (float)(rho - (double)rho_hi);
    static_assert(sizeof(SeqInfo) == 10 * sizeof(uint32_t), "SeqInfo is ten words");
    uint32_t w = 0;
    switch (lane) {
    case 0: w = (uint32_t)j; break;
    case 1: w = __float_as_uint(u); break;
    case 2: w = __float_as_uint(cp); break;
    case 3: w = __float_as_uint(cq); break;
    case 4: w = __float_as_uint(sp > 0.0 ? (float)(1.0 / sp) : 0.0f); break;
    case 5: w = __float_as_uint(sq > 0.0 ? (float)(1.0 / sq) : 0.0f); break;
    case 7: w = (uint32_t)xj; break;
    case 8: w = __float_as_uint(rho_hi); break;
    case 9: w = __float_as_uint(rho_lo); break;
    default: break;
    }
    if (lane < 10 && lane != 6) st32(&si[lane], w);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) st32(counter(a.ws.flag, c), a.epoch);
}

// ---------------------------------------------------------------------------
// Philox4x32-10
// ---------------------------------------------------------------------------
//
// Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
// (SC 2011), implemented from that definition: ten rounds of two 32x32->64-bit
// products, the key bumped by the Weyl constants between rounds.  The Gumbel
// noise of vocabulary entry i at correction position j under key (k0, k1) is
// word i % 4 of the block at counter (i / 4, j, 0x15D, 0), turned into
// U = (2 * (w >> 9) + 1) / 2^24 (exact in fp32, strictly inside (0, 1)).

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;
constexpr uint32_t kGumbelStream = 0x15Du;

__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        // one 32 x 32 -> 64 product each (a single v_mad_u64_u32)
        const uint64_t p0 = (uint64_t)kPhiloxM0 * c[0], p1 = (uint64_t)kPhiloxM1 * c[2];
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

// 1 / E for the 8 consecutive entries first, first + 1, ... (first % 8 == 0)
// of correction position j under key (k0, k1).  E is taken in units of
// ln 2 (E = -log2 U, the hardware logarithm; U is a normal number): every
// candidate's w / E then carries the same factor ln 2, which leaves the
// argmax unchanged.
__device__ __forceinline__ void inv_exp_noise8(uint32_t first, uint32_t j, uint32_t k0,
                                               uint32_t k1, float (&inv_e)[kGroupElems]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        uint32_t w[4] = {(first >> 2) + (uint32_t)b, j, kGumbelStream, 0u};
        philox4x32_10(w, k0, k1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // U = (2 * (w >> 9) + 1) / 2^24: exact in fp32, strictly inside (0, 1)
            const float u = (float)(((w[e] >> 9) << 1) | 1u) * 0x1p-24f;
            inv_e[b * 4 + e] = __builtin_amdgcn_rcpf(-__builtin_amdgcn_logf(u));
        }
    }
}

// 1 / E for the single entry i (same noise as inv_exp_noise8).
__device__ __forceinline__ float inv_exp_noise1(uint32_t i, uint32_t j, uint32_t k0, uint32_t k1) {
    uint32_t w[4] = {i >> 2, j, kGumbelStream, 0u};
    philox4x32_10(w, k0, k1);
    const uint32_t sel = i & 3u;
    const uint32_t word = sel == 0 ? w[0] : sel == 1 ? w[1] : sel == 2 ? w[2] : w[3];
    const float u = (float)(((word >> 9) << 1) | 1u) * 0x1p-24f;
    return __builtin_amdgcn_rcpf(-__builtin_amdgcn_logf(u));
}

}  // namespace
}  // namespace isd
