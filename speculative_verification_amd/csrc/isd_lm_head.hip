// LM-head projection on the matrix cores: logits[M, N] = h[M, K] @ w[K, N].
//
// bf16 operands, fp32 accumulation with v_mfma_f32_32x32x16_bf16, bf16 output
// rounded to nearest even.  The projection produces every anchor and mask
// row that the ISD step consumes ("Introspective Diffusion Language Models |
// Summary", section 3.3: one extend forward yields both).
//
// Tiling: a 256-thread workgroup owns a 256 x 128 output tile and walks K in
// steps of 64 through two LDS buffers (the next step's global loads are in
// flight while the current one is multiplied).  Its four wavefronts form a
// 2 x 2 grid of 128 x 64 sub-tiles, each 4 x 2 MFMA tiles of 32 x 32.
//
// The MFMA operands need 8 consecutive k per lane.  h is k-contiguous; w is
// n-contiguous, so its tile is transposed on the way into LDS ([n][k]).
// Tiles are ordered so that one XCD owns a contiguous range of N-tiles with
// all their M-tiles: the M-tiles that share a w tile read it through the same
// L2, and w streams from HBM about once.

#include "isd_internal.h"

namespace isd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 128, kBK = 64;
constexpr int kLdsPad = 8;              // bf16 of padding per LDS row
constexpr int kLdA = kBK + kLdsPad;     // A tile row (m) length in LDS
constexpr int kLdB = kBK + kLdsPad;     // transposed B tile row (n) length in LDS
constexpr int kXcds = 8;
constexpr int kThreadsG = 256;
constexpr int kAVecRow = kBK / 8;                       // 16-byte vectors per A row per step
constexpr int kAPerThread = kBM * kBK / 8 / kThreadsG;  // A vectors each thread moves per step
constexpr int kBVecRow = kBN / 8;                       // 16-byte vectors per w row per step
constexpr int kBPerThread = kBK * kBN / 8 / kThreadsG;  // w vectors each thread moves per step

// fp32 -> bf16, round to nearest even, in integer arithmetic (a NaN keeps its
// payload, made quiet)
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// The same rounding in one v_cvt_pk_bf16_f32 (equal for every finite value and
// infinity; a NaN comes out as the canonical quiet NaN).  The wide kernel's
// epilogue converts 128 values per lane, so the instruction count matters
// there.
__device__ __forceinline__ uint16_t bf16_cvt(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__global__ __launch_bounds__(256) void lm_head_kernel(const uint16_t *__restrict__ h,
                                                      const uint16_t *__restrict__ w, int M, int K,
                                                      int N, uint16_t *__restrict__ out,
                                                      int m_tiles, int total, int per_xcd) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdA];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLdB];

    const int b = blockIdx.x;
    const int idx = (b % kXcds) * per_xcd + b / kXcds;
    if (idx >= total) return;
    const int m0 = (idx % m_tiles) * kBM;
    const int n0 = (idx / m_tiles) * kBN;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave / 2, wn = wave % 2;

    // global -> register mapping of one K step: A is kBM rows of kAVecRow
    // vectors of 8 k, w is kBK rows of kBVecRow vectors of 8 n; thread tid
    // moves vectors tid, tid + 256, ...
    uint4 ra[kAPerThread], rb[kBPerThread];
    auto load_step = [&](int k0) {
#pragma unroll
        for (int r = 0; r < kAPerThread; ++r) {
            const int v = tid + kThreadsG * r;
            const int row = m0 + v / kAVecRow, kk = k0 + (v % kAVecRow) * 8;
            ra[r] = row < M ? *reinterpret_cast<const uint4 *>(h + (size_t)row * K + kk)
                            : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < kBPerThread; ++r) {
            const int v = tid + kThreadsG * r;
            const int kk = k0 + v / kBVecRow, col = n0 + (v % kBVecRow) * 8;
            rb[r] = col < N ? *reinterpret_cast<const uint4 *>(w + (size_t)kk * N + col)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_step = [&](int s) {
#pragma unroll
        for (int r = 0; r < kAPerThread; ++r) {
            const int v = tid + kThreadsG * r;
            *reinterpret_cast<uint4 *>(&As[s][(v / kAVecRow) * kLdA + (v % kAVecRow) * 8]) = ra[r];
        }
#pragma unroll
        for (int r = 0; r < kBPerThread; ++r) {
            const int v = tid + kThreadsG * r;
            const int kk = v / kBVecRow, nb = (v % kBVecRow) * 8;
            const uint32_t wd[4] = {rb[r].x, rb[r].y, rb[r].z, rb[r].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Bs[s][(nb + e) * kLdB + kk] = (uint16_t)(wd[e / 2] >> (16 * (e % 2)));
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

    const int nk = K / kBK;
    load_step(0);
    store_step(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < nk) load_step((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kk = ks * 16 + 8 * (lane / 32);
            bf16x8 af[4], bfr[2];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8 *>(
                    &As[s][(wm * 128 + mi * 32 + lane % 32) * kLdA + kk]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bfr[ni] = *reinterpret_cast<const bf16x8 *>(
                    &Bs[s][(wn * 64 + ni * 32 + lane % 32) * kLdB + kk]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < nk) store_step(s ^ 1);
        __syncthreads();
    }

    // D layout of a 32 x 32 tile: lane holds column lane % 32, rows
    // 8 * (i / 4) + 4 * (lane / 32) + i % 4 for its 16 values i.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const int col = n0 + wn * 64 + ni * 32 + lane % 32;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * 128 + mi * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
                if (row < M && col < N) out[(size_t)row * N + col] = bf16_rne(acc[mi][ni][i]);
            }
        }
}

// ---------------------------------------------------------------------------
// Pre-packed head: logits[M, N] = h[M, K] @ wt[N, K]^T
// ---------------------------------------------------------------------------
//
// With the head stored k-contiguous per vocabulary row (wt = w^T, packed
// once), both MFMA operands are 8 consecutive k of one row: every global
// load and every LDS store is one 16-byte vector, with no transposition.
//
// Small projections (fewer 256-wide tiles than CUs) run on 256 x 128 tiles:
// four wavefronts, a single 55 KB LDS buffer with the next K step's tiles held
// in registers while the current one is multiplied, and two workgroups per CU
// whose barrier phases interleave.  Larger ones use the ping-pong kernel
// further down.

constexpr int kPBM = 256, kPBN = 128, kPBK = 64;
constexpr int kPLd = kPBK + 8;                              // LDS row length (bf16), padded
constexpr int kPVecRow = kPBK / 8;                          // 16-byte vectors per row per step

// The A operand may come in two K segments: columns [0, K1) from h [M, K1]
// and [K1, K1 + K2) from h2 [M, K2] (K2 = 0: none); wt is [N, K1 + K2].  Both
// K1 and K2 are multiples of 64, so a K step never straddles the two.
__global__ __launch_bounds__(256, 2) void lm_head_packed_kernel(
    const uint16_t *__restrict__ h, int K1, const uint16_t *__restrict__ h2, int K2,
    const uint16_t *__restrict__ wt, int M, int N, uint16_t *__restrict__ out, int m_tiles,
    int total, int per_xcd) {
    constexpr int BN = kPBN;
    constexpr int kThr = BN * 2;                       // 4 wavefronts
    constexpr int kWN = BN / 64;                       // wavefronts along N
    constexpr int kAPer = kPBM * kPVecRow / kThr;      // A vectors per thread per step
    constexpr int kBPer = BN * kPVecRow / kThr;        // B vectors per thread per step
    __shared__ __attribute__((aligned(16))) uint16_t smem[(kPBM + BN) * kPLd];
    uint16_t *As = smem;
    uint16_t *Bs = smem + kPBM * kPLd;

    const int b = blockIdx.x;
    const int idx = (b % kXcds) * per_xcd + b / kXcds;
    if (idx >= total) return;
    const int m0 = (idx % m_tiles) * kPBM;
    const int n0 = (idx / m_tiles) * BN;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave / kWN, wn = wave % kWN;

    // thread tid moves the 16-byte vectors tid, tid + kThr, ... of each tile
    const int K = K1 + K2;
    uint4 ra[kAPer], rb[kBPer];
    auto load_step = [&](int k0) {
        const bool first = k0 < K1;
        const uint16_t *src = first ? h : h2;
        const int lda = first ? K1 : K2;
        const int ka = first ? k0 : k0 - K1;
#pragma unroll
        for (int r = 0; r < kAPer; ++r) {
            const int v = tid + kThr * r;
            const int row = m0 + v / kPVecRow, kk = ka + (v % kPVecRow) * 8;
            ra[r] = row < M ? *reinterpret_cast<const uint4 *>(src + (size_t)row * lda + kk)
                            : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < kBPer; ++r) {
            const int v = tid + kThr * r;
            const int col = n0 + v / kPVecRow, kk = k0 + (v % kPVecRow) * 8;
            rb[r] = col < N ? *reinterpret_cast<const uint4 *>(wt + (size_t)col * K + kk)
                            : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_step = [&]() {
#pragma unroll
        for (int r = 0; r < kAPer; ++r) {
            const int v = tid + kThr * r;
            *reinterpret_cast<uint4 *>(&As[(v / kPVecRow) * kPLd + (v % kPVecRow) * 8]) = ra[r];
        }
#pragma unroll
        for (int r = 0; r < kBPer; ++r) {
            const int v = tid + kThr * r;
            *reinterpret_cast<uint4 *>(&Bs[(v / kPVecRow) * kPLd + (v % kPVecRow) * 8]) = rb[r];
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

    const int nk = K / kPBK;
    load_step(0);
    for (int kt = 0; kt < nk; ++kt) {
        store_step();
        __syncthreads();
        if (kt + 1 < nk) load_step((kt + 1) * kPBK);
#pragma unroll
        for (int ks = 0; ks < kPBK / 16; ++ks) {
            const int kk = ks * 16 + 8 * (lane / 32);
            bf16x8 af[4], bfr[2];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8 *>(
                    &As[(wm * 128 + mi * 32 + lane % 32) * kPLd + kk]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bfr[ni] = *reinterpret_cast<const bf16x8 *>(
                    &Bs[(wn * 64 + ni * 32 + lane % 32) * kPLd + kk]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
        __syncthreads();
    }

#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const int col = n0 + wn * 64 + ni * 32 + lane % 32;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * 128 + mi * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
                if (row < M && col < N) out[(size_t)row * N + col] = bf16_rne(acc[mi][ni][i]);
            }
        }
}

// ---------------------------------------------------------------------------
// Wide heads: 256 x 256 tiles, two wavefront groups in ping-pong
// ---------------------------------------------------------------------------
//
// Eight wavefronts, two per SIMD, form two groups of four (group g holds
// wavefronts 4g .. 4g + 3, one per SIMD).  Each wavefront owns a 128 x 64
// sub-tile: rows 128 g .. + 127, columns 64 (wave % 4) .. + 63, 4 x 2 MFMA
// 32x32x16 tiles.  The K loop runs in phases that end on a workgroup barrier.
// In every phase one group reads its fragments from LDS and issues global
// loads while the other group multiplies (16 MFMAs per wavefront, half a K
// step of 64); the groups swap at each barrier, group 1 one phase behind, so
// each SIMD's matrix pipe is fed by one wavefront while its partner waits on
// memory.  Both groups pass the same number of barriers: group 1 takes one
// extra before its first phase and group 0 one after its last.
//
// Operands go from global memory straight into LDS with global_load_lds_dwordx4
// (one wavefront instruction fills 1 KiB of LDS; lane i writes its 16 bytes at
// offset 16 i).  Group 0 moves the h tile, group 1 the head tile.  Two stages
// of 64 KiB hold K steps j and j + 1: step j + 1's loads are issued in the
// first phase of step j and waited for at the end of its third (group 0) or
// fourth (group 1) phase, before either group reads them.  Rows past M or N
// re-read the last valid row; their results are never stored.
//
// LDS rows are 128 bytes (64 k) without padding.  The 16-byte chunk c of tile
// row r sits in slot c ^ f(r) with f(r) = (r & 6) | ((r ^ (r >> 3)) & 1): the
// fragment reads (32 consecutive rows, one chunk) then touch every bank once
// per cycle whether the LDS serves 8 lanes of 16 bytes (32 banks) or 16 lanes
// (64 banks).  Lane i of a load fetches the chunk that belongs in slot i % 8,
// so the DMA's linear fill produces that layout.
//
// With STATS the epilogue also emits, for every output row and every
// 128-column tile, the softmax partial of the bf16 logits it writes: an integer
// reference e = ceil(max * k2) and s = sum 2^(x * k2 - e) (k2 = log2(e) / T),
// stored as two floats at stats[(row * ceil(N / 128) + tile) * 2].  The ISD
// step can then take its row statistics from these instead of reading the
// logits back.  The output tile is staged through the two LDS stages (rows of
// group g in stage g, 16-byte chunks XOR-swizzled by row).  Then each row of
// 16 lanes takes one (row, 128-column tile) at a time: every lane reads one
// 16-byte chunk of it once, stores it to the logits and reduces it, and the
// 16 lanes combine their maxima, then their sums, with DPP exchanges.

constexpr int kWBM = 256, kWBN = 256, kWBK = 64;
constexpr int kStage = (kWBM + kWBN) * kWBK * 2;     // 64 KiB: A rows, then B rows
constexpr int kStageB = kWBM * kWBK * 2;             // byte offset of the B rows

__device__ __forceinline__ int chunk_swz(int r) { return (r & 6) | ((r ^ (r >> 3)) & 1); }

// All-reduce over each row of 16 lanes: quad_perm [1,0,3,2] and [2,3,0,1]
// within quads, then row_half_mirror (lane i <-> 7 - i) and row_mirror
// (i <-> 15 - i); every lane ends with the same value (the pairs combine in
// either order, and max and + are commutative).
template <int CTRL>
__device__ __forceinline__ float dpp16(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp16<0xB1>(v));
    v = fmaxf(v, dpp16<0x4E>(v));
    v = fmaxf(v, dpp16<0x141>(v));
    return fmaxf(v, dpp16<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp16<0xB1>(v);
    v += dpp16<0x4E>(v);
    v += dpp16<0x141>(v);
    return v + dpp16<0x140>(v);
}

// With SEG2 the A operand has a second K segment, as in the 128-wide kernel:
// columns [K, K + K2) come from h2 [M, K2], and wt is [N, K + K2].
//
// With SPLIT (with or without STATS) the tiles past the last whole round over
// the CUs are cut in two along K, so that the last round is half as long:
// workgroups 0 .. n_full - 1 take the whole tiles 0 .. n_full - 1 (in the same
// XCD-aware order as without the split), and the rest take the K steps
// [0, ks) or [ks, n) of one remaining tile.  Each half stores its fp32 tile
// in the workspace (agent-scope atomic stores, coherent across the XCDs) and
// counts itself on the tile's counter; the second to arrive adds the other
// half's tile to its own (fp32 addition is commutative, so the result does
// not depend on which half comes last), stores the output (and, with STATS,
// its partials) and resets the counter.  No half waits for the other.
struct SplitArgs {
    int n_full;                // whole tiles (a multiple of 8)
    int ks;                    // K steps of the first half
    float *part;               // [tiles - n_full][2][256 * 256] fp32 halves
    uint32_t *cnt;             // [tiles - n_full] counters, 128 bytes apart, zero between launches
};

template <bool STATS, bool SEG2, bool SPLIT>
__global__ __launch_bounds__(512) void lm_head_pp_kernel(const uint16_t *__restrict__ h,
                                                         const uint16_t *__restrict__ wt, int M,
                                                         int K, int N, uint16_t *__restrict__ out,
                                                         int m_tiles, int total, int per_xcd,
                                                         float k2, float *__restrict__ stats,
                                                         const uint16_t *__restrict__ h2, int K2,
                                                         SplitArgs sp) {
    // two separate arrays, so that loads into one stage are known not to
    // alias fragment reads from the other
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStage];

    const int b = blockIdx.x;
    int idx, half = -1;
    if constexpr (SPLIT) {
        if (b < sp.n_full) {
            idx = (b % kXcds) * (sp.n_full / kXcds) + b / kXcds;
        } else {                               // the two halves of a tile share an XCD
            const int u = b - sp.n_full, nu = (int)gridDim.x - sp.n_full;
            const int q = (u % kXcds) * (nu / kXcds) + u / kXcds;
            idx = sp.n_full + q / 2;
            half = q % 2;
        }
    } else {
        idx = (b % kXcds) * per_xcd + b / kXcds;
        if (idx >= total) return;
    }
    const int m0 = (idx % m_tiles) * kWBM;
    const int n0 = (idx / m_tiles) * kWBN;
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int g = wave / 4;                    // ping-pong group
    const int wm = g, wn = wave % 4;           // 128 x 64 sub-tile

    // loads: instruction t of this wavefront fills tile rows 64 (wave % 4) + 8 t
    // .. + 7 of its group's operand; lane i takes row + i / 8, slot i % 8
    const int Kt = SEG2 ? K + K2 : K;          // row length of wt, extent of the K loop
    const int lim = g == 0 ? M : N;
    const int gbase = g == 0 ? m0 : n0;
    const uint16_t *src = g == 0 ? h : wt;
    const int ldsoff = g == 0 ? 0 : kStageB;
    const uint16_t *gp[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int r = (wave % 4) * 64 + 8 * t + lane / 8;
        const int grow = min(gbase + r, lim - 1);
        gp[t] = src + (size_t)grow * (g == 0 ? K : Kt) + ((lane % 8) ^ chunk_swz(r)) * 8;
    }
    auto load_step = [&](uint8_t *stage, int k0) {
        if constexpr (SEG2) {
            if (g == 0 && k0 >= K) {           // A columns from h2: rare, addresses made here
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int r = (wave % 4) * 64 + 8 * t + lane / 8;
                    const int grow = min(m0 + r, M - 1);
                    __builtin_amdgcn_global_load_lds(
                        h2 + (size_t)grow * K2 + ((lane % 8) ^ chunk_swz(r)) * 8 + (k0 - K),
                        stage + ((wave % 4) * 64 + 8 * t) * 128, 16, 0, 0);
                }
                return;
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
            __builtin_amdgcn_global_load_lds(gp[t] + k0,
                                             stage + ldsoff + ((wave % 4) * 64 + 8 * t) * 128, 16, 0, 0);
    };

    // fragments: the lane's rows are base + lane % 32 with base a multiple of
    // 32, so the slot swizzle depends on lane % 16 only
    const int sw = chunk_swz(lane & 15);
    int aoff[4], boff[2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) aoff[mi] = (wm * 128 + mi * 32 + lane % 32) * 128;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) boff[ni] = kStageB + (wn * 64 + ni * 32 + lane % 32) * 128;

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;
    bf16x8 af[2][4], bfr[2][2];
    auto read_frags = [&](const uint8_t *stage, int half) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int co = (((half * 2 + q) * 2 + lane / 32) ^ sw) * 16;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[q][mi] = *reinterpret_cast<const bf16x8 *>(stage + aoff[mi] + co);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bfr[q][ni] = *reinterpret_cast<const bf16x8 *>(stage + boff[ni] + co);
        }
    };
    auto multiply = [&]() {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[q][mi], bfr[q][ni],
                                                                         acc[mi][ni], 0, 0, 0);
    };
    // a phase boundary: nothing is scheduled across it
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // s_waitcnt operands (gfx9 encoding): lgkmcnt(0) only; vmcnt(0) only;
    // vmcnt(0) and lgkmcnt(0)
    constexpr int kWaitLds = 0xC07F, kWaitVm = 0x0F70, kWaitBoth = 0x0070;

    // K steps [j0, j1) of the tile
    int j0 = 0, j1 = Kt / kWBK;
    if constexpr (SPLIT) {
        if (half == 0) j1 = sp.ks;
        if (half == 1) j0 = sp.ks;
    }
    load_step(stage0, j0 * kWBK);
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    phase_end();
    if (g == 1) phase_end();
    auto step = [&](uint8_t *cur, uint8_t *nxt, int j) {
        read_frags(cur, 0);                    // phase 4j (+ g): fragments, next step's loads
        if (j + 1 < j1) load_step(nxt, (j + 1) * kWBK);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        phase_end();
        multiply();                            // phase 4j + 1 (+ g)
        phase_end();
        read_frags(cur, 1);                    // phase 4j + 2 (+ g): step j + 1 has landed
        __builtin_amdgcn_s_waitcnt(kWaitBoth);
        phase_end();
        multiply();                            // phase 4j + 3 (+ g)
        phase_end();
    };
    for (int j = j0; j < j1; j += 2) {
        step(stage0, stage1, j);
        if (j + 1 < j1) step(stage1, stage0, j + 1);
    }
    if (g == 0) phase_end();

    if constexpr (SPLIT) {
        if (half >= 0) {
            // this half's tile, wavefront-major: 64-bit word ((wave * 8 + mi * 2 + ni) * 8
            // + i / 2) * 64 + lane holds elements i, i + 1 of accumulator (mi, ni)
            const int si = idx - sp.n_full;
            uint64_t *mine = reinterpret_cast<uint64_t *>(sp.part + ((size_t)si * 2 + half) * (kWBM * kWBN));
            const uint64_t *other =
                reinterpret_cast<const uint64_t *>(sp.part + ((size_t)si * 2 + (1 - half)) * (kWBM * kWBN));
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        const uint64_t w = (uint64_t)__float_as_uint(acc[mi][ni][i]) |
                                           ((uint64_t)__float_as_uint(acc[mi][ni][i + 1]) << 32);
                        __hip_atomic_store(&mine[((wave * 8 + mi * 2 + ni) * 8 + i / 2) * 64 + lane], w,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
            // every wavefront's stores complete, then one count per half
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            uint32_t *cnt = sp.cnt + (size_t)si * kCounterStride;
            volatile uint32_t *flag = reinterpret_cast<volatile uint32_t *>(stage0);
            if (tid == 0) {
                const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (prev == 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *flag = prev;
            }
            __syncthreads();
            const uint32_t arrived = *flag;
            __syncthreads();                   // every wavefront has the word before LDS is reused
            if (arrived != 1) return;          // the first half: the other one finishes the tile
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        const uint64_t w = __hip_atomic_load(
                            const_cast<uint64_t *>(&other[((wave * 8 + mi * 2 + ni) * 8 + i / 2) * 64 + lane]),
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        acc[mi][ni][i] += __uint_as_float((uint32_t)w);
                        acc[mi][ni][i + 1] += __uint_as_float((uint32_t)(w >> 32));
                    }
        }
    }

    if constexpr (!STATS) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int col = n0 + wn * 64 + ni * 32 + lane % 32;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = m0 + wm * 128 + mi * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
                    if (row < M && col < N) out[(size_t)row * N + col] = bf16_cvt(acc[mi][ni][i]);
                }
            }
    } else {
        // stage the bf16 tile: local row rl of group g at byte rl * 512 of
        // stage g, its 16-byte chunk c at slot c ^ (rl & 31)
        uint8_t *mine = g == 0 ? stage0 : stage1;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rl = mi * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
                    const int cl = wn * 64 + ni * 32 + lane % 32;
                    *reinterpret_cast<uint16_t *>(mine + rl * 512 + (((cl >> 3) ^ (rl & 31)) << 4) +
                                                  (cl & 7) * 2) = bf16_cvt(acc[mi][ni][i]);
                }
        __syncthreads();
        auto staged = [&](int r, int c8) -> const uint8_t * {   // tile row r, chunk c8
            const uint8_t *s = r < 128 ? stage0 : stage1;
            const int rl = r & 127;
            return s + rl * 512 + ((c8 ^ (rl & 31)) << 4);
        };
        // round j: lanes 16 q .. 16 q + 15 of wavefront w take pair
        // 32 j + 4 w + q, i.e. tile row (pair / 2) and column tile (pair % 2);
        // lane 16 q + i holds its 16-byte chunk i
        const bool vec_out = (N % 8) == 0 && ((uintptr_t)out % 16) == 0;
        const int nt = (N + 127) / 128;
        const int sl = lane % 16;
        const float neg = -__builtin_inff();
#pragma unroll 2
        for (int j = 0; j < 16; ++j) {
            const int pair = 32 * j + 4 * wave + lane / 16;
            const int r = pair / 2, sub = pair % 2;
            const int grow = m0 + r, c0 = n0 + sub * 128, gcol = c0 + sl * 8;
            const uint4 w4 = *reinterpret_cast<const uint4 *>(staged(r, sub * 16 + sl));
            if (grow < M && gcol < N) {
                uint16_t *dp = out + (size_t)grow * N + gcol;
                if (vec_out && gcol + 8 <= N) {
                    *reinterpret_cast<uint4 *>(dp) = w4;
                } else {
                    const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
                    for (int e = 0; e < 8 && gcol + e < N; ++e)
                        dp[e] = (uint16_t)(wd[e / 2] >> (16 * (e % 2)));
                }
            }
            const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = __uint_as_float(w[e] << 16);
                x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
            float m = neg;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (gcol + e < N) m = fmaxf(m, x[e]);
            m = row16_max(m);
            const float ref = m == neg ? neg : ceilf(m * k2);
            float sum = 0.0f;
            if (ref != neg) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (gcol + e < N) sum += __builtin_amdgcn_exp2f(fmaf(x[e], k2, -ref));
            }
            sum = row16_sum(sum);
            if (sl == 0 && grow < M && c0 < N) {
                const size_t at = ((size_t)grow * nt + c0 / 128) * 2;
                stats[at] = ref;
                stats[at + 1] = sum;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Segment-gated LoRA shrink: t[M, r] = gate_j * (x_j A^T), bf16
// ---------------------------------------------------------------------------
//
// The adapter acts only at mask positions ("Introspective Diffusion Language
// Models | Summary", appendix G), so t is zero on the other rows; the expand
// B t then rides on the base projection as a second K segment (x | t) times
// (W | B)^T.  The shrink has only r columns, so what bounds it is the length
// of each wavefront's K loop, not the MFMA rate: a workgroup of sixteen
// wavefronts owns 32 rows x 32 adapter channels, the wavefronts take every
// sixteenth 16-wide K step each (reading both operands straight from global
// memory as the 8-element k-runs the MFMA takes), and wavefront 0 sums the
// sixteen partial tiles through LDS in a fixed order.

constexpr int kSRows = 32, kSCols = 32, kSWaves = 16;

__global__ __launch_bounds__(kSWaves * 64) void lora_shrink_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a,
    const int32_t *__restrict__ mask, int M, int K, int r, uint16_t *__restrict__ t) {
    __shared__ float part[kSWaves - 1][16][64];
    const int m0 = blockIdx.x * kSRows, n0 = blockIdx.y * kSCols;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int row = m0 + lane % 32;
    const uint16_t *xr = x + (size_t)(row < M ? row : 0) * K + 8 * (lane / 32);
    const uint16_t *ar = a + (size_t)(n0 + lane % 32) * K + 8 * (lane / 32);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    // rows past M read row 0 and are never stored; the K steps of this
    // wavefront are loaded eight at a time so that their loads overlap
    constexpr int kBatch = 8;
    const int stride = 16 * kSWaves;
    for (int k0 = 16 * wave; k0 < K; k0 += kBatch * stride) {
        bf16x8 xa[kBatch], av[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int k = k0 + b * stride;
            if (k < K) {
                xa[b] = *reinterpret_cast<const bf16x8 *>(xr + k);
                av[b] = *reinterpret_cast<const bf16x8 *>(ar + k);
            } else {
                xa[b] = bf16x8{};
                av[b] = bf16x8{};
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[b], av[b], acc, 0, 0, 0);
    }
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) part[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll 1
    for (int w = 0; w < kSWaves - 1; ++w)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += part[w][i][lane];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int rr = m0 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
        if (rr >= M) continue;
        const bool gate = mask == nullptr || mask[rr] != 0;
        t[(size_t)rr * r + n0 + lane % 32] = gate ? bf16_rne(acc[i]) : (uint16_t)0;
    }
}

// Split-K form of the shrink, for calls whose output buffer can hold the
// partial sums.  Workgroup (b, s, z) multiplies rows 64b .. 64b + 63 of x by
// adapter channels 128z .. 128z + 127 of A over K slice s, both staged in LDS
// with row-contiguous 16-byte loads, and writes the fp32 partial tile to
// part[s][row][channel]; a second kernel adds the slices in order, applies the
// gate and rounds to bf16.  The partials live in the projection's output
// buffer, which the GEMM that follows overwrites.

constexpr int kSpRows = 64, kSpCh = 128, kSpSlice = 256;
constexpr int kSpLd = kSpSlice + 8;                         // LDS row length (bf16), padded

__global__ __launch_bounds__(256) void lora_shrink_part_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a, int M, int K, int r,
    float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[kSpRows * kSpLd];
    __shared__ __attribute__((aligned(16))) uint16_t as[kSpCh * kSpLd];
    const int m0 = blockIdx.x * kSpRows, s = blockIdx.y, c0 = blockIdx.z * kSpCh;
    const int k0 = s * kSpSlice;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    constexpr int kVec = kSpSlice / 8;                      // 16-byte vectors per row
    // every load is issued before the first LDS store, so their latencies
    // overlap; x rows past M and k past K read as zeros
    constexpr int kXPer = kSpRows * kVec / 256, kAPer = kSpCh * kVec / 256;
    uint4 vx[kXPer], va[kAPer];
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
        const int v = tid + 256 * j;
        const int row = m0 + v / kVec, k = k0 + (v % kVec) * 8;
        vx[j] = (row < M && k < K) ? *reinterpret_cast<const uint4 *>(x + (size_t)row * K + k)
                                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int v = tid + 256 * j;
        const int k = k0 + (v % kVec) * 8;
        va[j] = k < K ? *reinterpret_cast<const uint4 *>(a + (size_t)(c0 + v / kVec) * K + k)
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
        const int v = tid + 256 * j;
        *reinterpret_cast<uint4 *>(&xs[(v / kVec) * kSpLd + (v % kVec) * 8]) = vx[j];
    }
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int v = tid + 256 * j;
        *reinterpret_cast<uint4 *>(&as[(v / kVec) * kSpLd + (v % kVec) * 8]) = va[j];
    }
    __syncthreads();
    // wavefront w: rows 32 (w % 2) .., channels 64 (w / 2) .. as two 32 x 32 tiles
    const int mt = wave % 2, nb = (wave / 2) * 2;
    f32x16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
#pragma unroll 4
    for (int ks = 0; ks < kSpSlice / 16; ++ks) {
        const int kk = ks * 16 + 8 * (lane / 32);
        const bf16x8 af = *reinterpret_cast<const bf16x8 *>(&xs[(mt * 32 + lane % 32) * kSpLd + kk]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x8 bfr =
                *reinterpret_cast<const bf16x8 *>(&as[((nb + j) * 32 + lane % 32) * kSpLd + kk]);
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = m0 + mt * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
            const int ch = c0 + (nb + j) * 32 + lane % 32;
            if (row < M) part[((size_t)s * M + row) * r + ch] = acc[j][i];
        }
}

// t[row, ch] = gate(row) * bf16(sum over the slices, in slice order).
__global__ __launch_bounds__(256) void lora_shrink_sum_kernel(const float *__restrict__ part,
                                                              const int32_t *__restrict__ mask,
                                                              int M, int r, int slices,
                                                              uint16_t *__restrict__ t) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)M * r) return;
    const int row = (int)(i / r);
    float acc = 0.0f;
    int s = 0;
    for (; s + 4 <= slices; s += 4) {   // four loads in flight, added in slice order
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = part[(size_t)(s + j) * M * r + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc += v[j];
    }
    for (; s < slices; ++s) acc += part[(size_t)s * M * r + i];
    const bool gate = mask == nullptr || mask[row] != 0;
    t[i] = gate ? bf16_rne(acc) : (uint16_t)0;
}

// wt[N, K] = w[K, N]^T through 64 x 64 LDS tiles (bit copies).
__global__ __launch_bounds__(256) void pack_wt_kernel(const uint16_t *__restrict__ w,
                                                      uint16_t *__restrict__ wt, int K, int N) {
    __shared__ uint16_t t[64][65];
    const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int kk = i / 64, nn = i % 64;
        const int k = k0 + kk, n = n0 + nn;
        t[kk][nn] = (k < K && n < N) ? w[(size_t)k * N + n] : 0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int nn = i / 64, kk = i % 64;
        const int k = k0 + kk, n = n0 + nn;
        if (k < K && n < N) wt[(size_t)n * K + k] = t[kk][nn];
    }
}

}  // namespace

hipError_t launch_lm_head(const uint16_t *h, const uint16_t *w, int M, int K, int N, uint16_t *out,
                          hipStream_t stream) {
    const int m_tiles = (M + kBM - 1) / kBM;
    const int n_tiles = (N + kBN - 1) / kBN;
    const long long total = (long long)m_tiles * n_tiles;
    if (total >= (1LL << 31) / kXcds) return hipErrorInvalidValue;
    const int per_xcd = (int)((total + kXcds - 1) / kXcds);
    hipLaunchKernelGGL(lm_head_kernel, dim3((unsigned)(per_xcd * kXcds)), dim3(256), 0, stream, h,
                       w, M, K, N, out, m_tiles, (int)total, per_xcd);
    return hipGetLastError();
}

namespace {

// Projections with at least one 256-wide tile per CU (the LM head's 2376, the
// MLP projection's 384) run on the ping-pong kernel; smaller ones, which
// would leave CUs idle, on the 128-wide tiles of the single-group kernel.
constexpr int kWideTilesMin = 256;

hipError_t launch_packed(const uint16_t *h, int K1, const uint16_t *h2, int K2, const uint16_t *wt,
                         int M, int N, uint16_t *out, hipStream_t stream) {
    const int m_tiles = (M + kPBM - 1) / kPBM;
    const int n_tiles = (N + kPBN - 1) / kPBN;
    const long long total = (long long)m_tiles * n_tiles;
    if (total >= (1LL << 31) / kXcds) return hipErrorInvalidValue;
    const int per_xcd = (int)((total + kXcds - 1) / kXcds);
    hipLaunchKernelGGL(lm_head_packed_kernel, dim3((unsigned)(per_xcd * kXcds)), dim3(256), 0,
                       stream, h, K1, h2, K2, wt, M, N, out, m_tiles, (int)total, per_xcd);
    return hipGetLastError();
}

// h2 / K2: the second A segment (nullptr / 0 for none)
template <bool STATS, bool SEG2, bool SPLIT = false>
hipError_t launch_pp(const uint16_t *h, int K, const uint16_t *h2, int K2, const uint16_t *wt, int M,
                     int N, uint16_t *out, float k2, float *stats, hipStream_t stream,
                     SplitArgs sp = SplitArgs{0, 0, nullptr, nullptr}, int n_split = 0) {
    const int m_tiles = (M + kWBM - 1) / kWBM;
    const int n_tiles = (N + kWBN - 1) / kWBN;
    const long long total = (long long)m_tiles * n_tiles;
    if (total >= (1LL << 31) / kXcds) return hipErrorInvalidValue;
    const int per_xcd = (int)((total + kXcds - 1) / kXcds);
    const unsigned grid = SPLIT ? (unsigned)(sp.n_full + 2 * n_split) : (unsigned)(per_xcd * kXcds);
    hipLaunchKernelGGL((lm_head_pp_kernel<STATS, SEG2, SPLIT>), dim3(grid), dim3(512), 0, stream, h, wt,
                       M, K, N, out, m_tiles, (int)total, per_xcd, k2, stats, h2, K2, sp);
    return hipGetLastError();
}

long long wide_tiles(int M, int N) {
    return (long long)((M + kWBM - 1) / kWBM) * ((N + kWBN - 1) / kWBN);
}

// The K split of the last partial round: it applies when the tiles past the
// whole rounds over the CUs fill at most half a round (their halves then fill
// at most one), their number is a multiple of 4 (the halves spread evenly over
// the XCDs), and the first K segment has at least two steps.  The workspace
// holds one 128-byte counter per split tile, then its two fp32 halves.
constexpr int kCUs = 256;

struct SplitPlan {
    int n_full, n_split, ks;
    size_t bytes;
};

SplitPlan split_plan(int M, int K1, int N) {
    SplitPlan p{0, 0, 0, 0};
    const long long tiles = wide_tiles(M, N);
    const long long rem = tiles % kCUs;
    if (tiles < kCUs || rem == 0 || 2 * rem > kCUs || rem % 4 != 0 || K1 / kWBK < 2) return p;
    p.n_full = (int)(tiles - rem);
    p.n_split = (int)rem;
    p.ks = K1 / kWBK / 2;
    p.bytes = (size_t)rem * kCounterStride * sizeof(uint32_t) + (size_t)rem * 2 * kWBM * kWBN * sizeof(float);
    return p;
}

// The ping-pong GEMM, split when the plan applies and the workspace is large enough.
template <bool SEG2>
hipError_t launch_pp_maybe_split(const uint16_t *h, int K, const uint16_t *h2, int K2, const uint16_t *wt,
                                 int M, int N, uint16_t *out, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
    const SplitPlan p = split_plan(M, K, N);
    if (p.n_split == 0 || ws == nullptr || ws_bytes < p.bytes)
        return launch_pp<false, SEG2>(h, K, h2, K2, wt, M, N, out, 0.0f, nullptr, stream);
    uint32_t *cnt = static_cast<uint32_t *>(ws);
    float *part = reinterpret_cast<float *>(cnt + (size_t)p.n_split * kCounterStride);
    return launch_pp<false, SEG2, true>(h, K, h2, K2, wt, M, N, out, 0.0f, nullptr, stream,
                                        SplitArgs{p.n_full, p.ks, part, cnt}, p.n_split);
}

}  // namespace

size_t gemm_workspace_bytes(int M, int K, int N) { return split_plan(M, K, N).bytes; }

hipError_t launch_lm_head_packed(const uint16_t *h, const uint16_t *wt, int M, int K, int N,
                                 uint16_t *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (wide_tiles(M, N) >= kWideTilesMin)
        return launch_pp_maybe_split<false>(h, K, nullptr, 0, wt, M, N, out, ws, ws_bytes, stream);
    return launch_packed(h, K, nullptr, 0, wt, M, N, out, stream);
}

hipError_t launch_lora_gemm(const uint16_t *x, const uint16_t *a, const uint16_t *wcat,
                            const int32_t *mask, int M, int K, int N, int r, uint16_t *t,
                            uint16_t *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    // the split-K shrink when the output buffer can hold its fp32 partials
    const int slices = (K + kSpSlice - 1) / kSpSlice;
    const bool split = r % kSpCh == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0 &&
                       (size_t)slices * M * r * sizeof(float) <= (size_t)M * N * sizeof(uint16_t);
    if (split) {
        float *part = reinterpret_cast<float *>(out);
        const dim3 pgrid((unsigned)((M + kSpRows - 1) / kSpRows), (unsigned)slices, (unsigned)(r / kSpCh));
        hipLaunchKernelGGL(lora_shrink_part_kernel, pgrid, dim3(256), 0, stream, x, a, M, K, r, part);
        const long long n = (long long)M * r;
        hipLaunchKernelGGL(lora_shrink_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           part, mask, M, r, slices, t);
    } else {
        const dim3 sgrid((unsigned)((M + kSRows - 1) / kSRows), (unsigned)(r / kSCols));
        hipLaunchKernelGGL(lora_shrink_kernel, sgrid, dim3(kSWaves * 64), 0, stream, x, a, mask, M, K,
                           r, t);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (wide_tiles(M, N) >= kWideTilesMin)
        return launch_pp_maybe_split<true>(x, K, t, r, wcat, M, N, out, ws, ws_bytes, stream);
    return launch_packed(x, K, t, r, wcat, M, N, out, stream);
}

hipError_t launch_pack_wt(const uint16_t *w, uint16_t *wt, int K, int N, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64));
    hipLaunchKernelGGL(pack_wt_kernel, grid, dim3(256), 0, stream, w, wt, K, N);
    return hipGetLastError();
}

hipError_t launch_lm_head_stats(const uint16_t *h, const uint16_t *wt, int M, int K, int N,
                                float k2, uint16_t *out, float *stats, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
    const SplitPlan p = split_plan(M, K, N);
    if (p.n_split == 0 || ws == nullptr || ws_bytes < p.bytes)
        return launch_pp<true, false>(h, K, nullptr, 0, wt, M, N, out, k2, stats, stream);
    uint32_t *cnt = static_cast<uint32_t *>(ws);
    float *part = reinterpret_cast<float *>(cnt + (size_t)p.n_split * kCounterStride);
    return launch_pp<true, false, true>(h, K, nullptr, 0, wt, M, N, out, k2, stats, stream,
                                        SplitArgs{p.n_full, p.ks, part, cnt}, p.n_split);
}

}  // namespace isd
