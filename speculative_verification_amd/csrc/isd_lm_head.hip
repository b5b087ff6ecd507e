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

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
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
// The workgroup owns a 256 x BN output tile (BN = 128 or 256) and keeps a
// single LDS buffer (55 or 74 KB): the next K step's tiles are held in
// registers while the current one is multiplied.  At BN = 128 two workgroups
// share a CU and their barrier phases interleave; at BN = 256 one workgroup
// of eight wavefronts fills it and moves a third less operand data per flop.

constexpr int kPBM = 256, kPBN = 128, kPBK = 64;
constexpr int kPLd = kPBK + 8;                              // LDS row length (bf16), padded
constexpr int kPVecRow = kPBK / 8;                          // 16-byte vectors per row per step

// The A operand may come in two K segments: columns [0, K1) from h [M, K1]
// and [K1, K1 + K2) from h2 [M, K2] (K2 = 0: none); wt is [N, K1 + K2].  Both
// K1 and K2 are multiples of 64, so a K step never straddles the two.
//
// With STATS the epilogue also emits, for every output row and every 128-column
// tile, the softmax partial of the bf16 logits it writes: an integer reference
// e = ceil(max * k2) and s = sum 2^(x * k2 - e) (k2 = log2(e) / T), stored as
// two floats at stats[(row * ceil(N / 128) + tile) * 2].  The ISD step can then
// take its row statistics from these instead of reading the logits back.
//
// BN is the tile width: 128 (256 threads, two workgroups per CU) or 256 (512
// threads, one workgroup per CU, a third less operand traffic per flop).
template <int BN, bool STATS>
__global__ __launch_bounds__(BN * 2, 256 / BN) void lm_head_packed_kernel(
    const uint16_t *__restrict__ h, int K1, const uint16_t *__restrict__ h2, int K2,
    const uint16_t *__restrict__ wt, int M, int N, uint16_t *__restrict__ out, int m_tiles,
    int total, int per_xcd, float k2, float *__restrict__ stats) {
    static_assert(BN % kPBN == 0, "statistics are per 128-column tile");
    constexpr int kThr = BN * 2;                       // 4 or 8 wavefronts
    constexpr int kWN = BN / 64;                       // wavefronts along N
    constexpr int kAPer = kPBM * kPVecRow / kThr;      // A vectors per thread per step
    constexpr int kBPer = BN * kPVecRow / kThr;        // B vectors per thread per step
    // operand tiles; with STATS the same memory later stages the whole output
    // tile ([256][BN + 8] bf16: 68 KB at BN = 128, 135 KB at BN = 256)
    constexpr int kStageLd = BN + 8;
    constexpr int kOperands = (kPBM + BN) * kPLd;
    constexpr int kSmem = STATS && kPBM * kStageLd > kOperands ? kPBM * kStageLd : kOperands;
    __shared__ __attribute__((aligned(16))) uint16_t smem[kSmem];
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

    if constexpr (!STATS) {
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
    } else {
        // The output tile is staged in LDS as bf16 (the K loop ended on a
        // barrier, so the operand tiles are free) and leaves as 16-byte row
        // chunks; thread t then reduces the 128 staged columns of row t in two
        // passes (max, then the sum of 2^(x k2 - e)).
        uint16_t *tileL = smem;   // [256][kStageLd]
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rl = wm * 128 + mi * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
                    const int cl = wn * 64 + ni * 32 + lane % 32;
                    tileL[rl * kStageLd + cl] = bf16_rne(acc[mi][ni][i]);
                }
        __syncthreads();
        // the logits leave the staged tile as 16-byte row chunks (a row's 16
        // chunks are consecutive threads), or element by element at a ragged
        // or unaligned edge
        const bool vec_out = (N % 8) == 0;
#pragma unroll 4
        for (int q = tid; q < kPBM * (BN / 8); q += kThr) {
            const int rl = q / (BN / 8), c8 = (q % (BN / 8)) * 8;
            const int grow = m0 + rl, gcol = n0 + c8;
            if (grow >= M) continue;
            const uint16_t *sp = &tileL[rl * kStageLd + c8];
            uint16_t *dp = out + (size_t)grow * N + gcol;
            if (vec_out && gcol + 8 <= N) {
                *reinterpret_cast<uint4 *>(dp) = *reinterpret_cast<const uint4 *>(sp);
            } else {
                for (int e = 0; e < 8 && gcol + e < N; ++e) dp[e] = sp[e];
            }
        }
    }
    if constexpr (STATS) {
        // thread tid reduces 128 columns of row tid % 256: 128-column tile
        // tid / 256 of the workgroup's BN columns
        static_assert(kThr == kPBM * (BN / kPBN), "one thread per row and 128-column tile");
        const uint16_t *tileL = smem;
        const int rl = tid % kPBM, sub = tid / kPBM;
        const int row = m0 + rl;
        const int c0 = n0 + sub * kPBN;
        const uint16_t *src = &tileL[rl * kStageLd + sub * kPBN];
        const float neg = -__builtin_inff();
        float m = neg;
#pragma unroll
        for (int q8 = 0; q8 < kPBN / 8; ++q8) {
            const uint4 w4 = *reinterpret_cast<const uint4 *>(src + q8 * 8);
            const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = c0 + q8 * 8 + 2 * e;
                if (c < N) m = fmaxf(m, __uint_as_float(w[e] << 16));
                if (c + 1 < N) m = fmaxf(m, __uint_as_float(w[e] & 0xFFFF0000u));
            }
        }
        const float ref = m == neg ? neg : ceilf(m * k2);
        float sum = 0.0f;
        if (ref != neg) {
#pragma unroll
            for (int q8 = 0; q8 < kPBN / 8; ++q8) {
                const uint4 w4 = *reinterpret_cast<const uint4 *>(src + q8 * 8);
                const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = c0 + q8 * 8 + 2 * e;
                    if (c < N) sum += __builtin_amdgcn_exp2f(fmaf(__uint_as_float(w[e] << 16), k2, -ref));
                    if (c + 1 < N)
                        sum += __builtin_amdgcn_exp2f(fmaf(__uint_as_float(w[e] & 0xFFFF0000u), k2, -ref));
                }
            }
        }
        if (row < M && c0 < N) {
            const size_t at = ((size_t)row * ((N + kPBN - 1) / kPBN) + c0 / kPBN) * 2;
            stats[at] = ref;
            stats[at + 1] = sum;
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

// Tile widths: the LM head (N = 151936) and its statistics variant run on
// 256-wide tiles, one workgroup per CU; the LoRA projection and other narrow
// projections (N = 24576) on 128-wide ones, two workgroups per CU.
constexpr int kHeadBN = 256;
constexpr int kLoraBN = 128;

template <int BN, bool STATS>
hipError_t launch_packed(const uint16_t *h, int K1, const uint16_t *h2, int K2, const uint16_t *wt,
                         int M, int N, uint16_t *out, float k2, float *stats, hipStream_t stream) {
    const int m_tiles = (M + kPBM - 1) / kPBM;
    const int n_tiles = (N + BN - 1) / BN;
    const long long total = (long long)m_tiles * n_tiles;
    if (total >= (1LL << 31) / kXcds) return hipErrorInvalidValue;
    const int per_xcd = (int)((total + kXcds - 1) / kXcds);
    hipLaunchKernelGGL((lm_head_packed_kernel<BN, STATS>), dim3((unsigned)(per_xcd * kXcds)),
                       dim3(BN * 2), 0, stream, h, K1, h2, K2, wt, M, N, out, m_tiles, (int)total,
                       per_xcd, k2, stats);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lm_head_packed(const uint16_t *h, const uint16_t *wt, int M, int K, int N,
                                 uint16_t *out, hipStream_t stream) {
    // 256-wide tiles when there are at least four per CU (the LM head: 1337 us
    // against 1434 us on 128-wide tiles); narrower projections balance better
    // on 128-wide ones (N = 24576: 230 us against 243 us)
    const long long wide_tiles = (long long)((M + kPBM - 1) / kPBM) * ((N + kHeadBN - 1) / kHeadBN);
    if (wide_tiles >= 4 * 256)
        return launch_packed<kHeadBN, false>(h, K, nullptr, 0, wt, M, N, out, 0.0f, nullptr, stream);
    return launch_packed<kLoraBN, false>(h, K, nullptr, 0, wt, M, N, out, 0.0f, nullptr, stream);
}

hipError_t launch_lora_gemm(const uint16_t *x, const uint16_t *a, const uint16_t *wcat,
                            const int32_t *mask, int M, int K, int N, int r, uint16_t *t,
                            uint16_t *out, hipStream_t stream) {
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
    return launch_packed<kLoraBN, false>(x, K, t, r, wcat, M, N, out, 0.0f, nullptr, stream);
}

hipError_t launch_pack_wt(const uint16_t *w, uint16_t *wt, int K, int N, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64));
    hipLaunchKernelGGL(pack_wt_kernel, grid, dim3(256), 0, stream, w, wt, K, N);
    return hipGetLastError();
}

hipError_t launch_lm_head_stats(const uint16_t *h, const uint16_t *wt, int M, int K, int N,
                                float k2, uint16_t *out, float *stats, hipStream_t stream) {
    return launch_packed<kHeadBN, true>(h, K, nullptr, 0, wt, M, N, out, k2, stats, stream);
}

}  // namespace isd
