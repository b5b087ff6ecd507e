// ISD step fed by the LM head's softmax partials, for gfx950.
//
// One extend forward produces the anchor rows p and the mask rows qn of a step
// ("Introspective Diffusion Language Models | Summary", section 3.3).  When the
// projection that produces them is isd_lm_head_stats, its epilogue already
// holds every logit in registers and writes, per row and 128-column tile, the
// softmax partial (e = ceil(max * k2), s = sum 2^(x * k2 - e)) of the bf16
// values it stores.  The step then needs the logits themselves only where a
// single entry or a short run matters:
//
//   decide  (one workgroup per sequence)  merge the partials of rows p_k and
//           q_k into their softmax denominators, read the logits at x_k, take
//           the ratios in fp64, the accept test, the first rejection j and
//           alpha, and publish the row-j constants for the residual draw;
//   residual items of the step kernel stream rows p_j and q_j as usual;
//   propose (one wavefront per mask row)  merge the partials of qn_k, find
//           the 128-column tile where the running mass crosses u * S, read
//           those 128 logits and finish the inverse-CDF draw there.
//
// Decide and propose read only the partials and the logits, never each
// other's results, so they share one launch ahead of the residual items when
// its workgroups fit on the CUs at once (fused_front_kernel); otherwise decide
// runs before the residual items and propose after them.  So the step reads
// the residual rows and a few kilobytes per row instead of all 3 * C * L rows
// of logits.

#include "isd_device.h"
#include "isd_internal.h"

#include <math.h>

namespace isd {

namespace {

constexpr float kNegInfF = -__builtin_inff();

// 2^n for an integer-valued float n, saturating far below the fp64 range.
__device__ __forceinline__ double pow2_i(float n) { return ldexp(1.0, (int)fmaxf(n, -2000.0f)); }

// A row's tile partials are (e, s) float pairs, 8 bytes per 128-column tile.
// A wavefront takes them kChunk tiles at a time with lane l holding tiles
// t0 + i * 64 + l, so each load instruction covers 512 consecutive bytes.
constexpr int kU = 24;
constexpr int kChunk = kU * kWave;   // 1536 tiles, 196,608 columns

struct Chunk {
    float e[kU];
    float s[kU];
};

__device__ __forceinline__ void load_chunk(const float *st, int n, int t0, int lane, Chunk &ch) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
        const int t = t0 + i * kWave + lane;
        if (t < n) {
            const uint64_t w = *reinterpret_cast<const uint64_t *>(st + 2 * t);
            ch.e[i] = __uint_as_float((uint32_t)w);
            ch.s[i] = __uint_as_float((uint32_t)(w >> 32));
        } else {
            ch.e[i] = kNegInfF;
            ch.s[i] = 0.0f;
        }
    }
}

// Fold a chunk into a lane's running (reference r, fp64 sum acc scaled to r).
__device__ __forceinline__ void fold_chunk(const Chunk &ch, float &r, double &acc) {
    float cm = kNegInfF;
#pragma unroll
    for (int i = 0; i < kU; ++i) cm = fmaxf(cm, ch.e[i]);
    if (cm > r) {
        if (r != kNegInfF) acc *= pow2_i(r - cm);
        r = cm;
    }
#pragma unroll
    for (int i = 0; i < kU; ++i)
        if (ch.e[i] != kNegInfF) acc += (double)ch.s[i] * pow2_i(ch.e[i] - r);
}

// Combine the lanes: ref = max e over the row, sum = sum s * 2^(e - ref).
__device__ __forceinline__ void finish_stats(float r, double acc, float &ref, double &sum) {
    const float R = wave_max(r);
    ref = R;
    sum = wave_sum_d(r == kNegInfF ? 0.0 : acc * pow2_i(r - R));
}

// Softmax denominator of one row from its n tile partials (one wavefront).
__device__ __forceinline__ void merge_row_stats(const float *st, int n, int lane, float &ref,
                                                double &sum) {
    float r = kNegInfF;
    double acc = 0.0;
    for (int t0 = 0; t0 < n; t0 += kChunk) {
        Chunk ch;
        load_chunk(st, n, t0, lane, ch);
        fold_chunk(ch, r, acc);
    }
    finish_stats(r, acc, ref, sum);
}

// Wavefront-scope ordering of the LDS staging area: writes before reads by
// other lanes of the same wavefront, and reads before the next overwrite.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ const float *row_stats(const float *base, const StepArgs &a, int c,
                                                  int k) {
    return base + 2 * ((long long)c * a.s_ldc + (long long)k * a.s_ld);
}

__device__ __forceinline__ long long fused_row_offset(const StepArgs &a, int c, int k) {
    return (long long)c * a.ldc + (long long)k * a.ld;
}

// ---------------------------------------------------------------------------
// Decision
// ---------------------------------------------------------------------------

constexpr int kDecideWaves = 16;

// Sequence c's decision, by a whole workgroup of NW wavefronts.
template <typename T, int NW>
__device__ __forceinline__ void decide_seq(const StepArgs &a, int c, int wave, int lane,
                                           float (&s_c)[2][kMaxL], double (&s_s)[2][kMaxL]) {
    const int L = a.L;
    // one wavefront per row: p rows (which = 0), then q rows (which = 1)
    const int rows = a.q_onehot ? L : 2 * L;
    for (int rr = wave; rr < rows; rr += NW) {
        const int which = rr / L, k = rr - which * L;
        float cr;
        double sr;
        merge_row_stats(row_stats(which ? a.q_stats : a.p_stats, a, c, k), a.n_stiles, lane, cr, sr);
        if (lane == 0) {
            s_c[which][k] = cr;
            s_s[which][k] = sr;
        }
    }
    __syncthreads();
    if (wave != 0) return;

    const bool valid = lane < L;
    const int kk = valid ? lane : 0;
    const int xk = valid ? a.x[c * L + kk] : 0;
    const bool bad = valid && (xk < 0 || xk >= a.V);
    if (bad) atomicOr(&a.ws.ctl->error, kErrBadToken);
    const float cp = s_c[0][kk], cq = a.q_onehot ? 0.0f : s_c[1][kk];
    const double sp = s_s[0][kk], sq = a.q_onehot ? 0.0 : s_s[1][kk];
    double px = 0.0, qx = 0.0;
    if (valid) {
        if (sp <= 0.0 || (!a.q_onehot && sq <= 0.0)) atomicOr(&a.ws.ctl->error, kErrEmptyRow);
        if (!bad) {
            const long long off = fused_row_offset(a, c, kk) + xk;
            const float lp = load_value<T>(static_cast<const T *>(a.p), off);
            const double k2 = (double)a.k2;
            if (sp > 0.0) px = exp2((double)lp * k2 - (double)cp) / sp;
            if (a.q_onehot) {
                qx = 1.0;
            } else {
                const float lq = load_value<T>(static_cast<const T *>(a.q), off);
                if (sq > 0.0) qx = exp2((double)lq * k2 - (double)cq) / sq;
            }
        }
    }
    // min(1, P(x)/Q(x)) with the Q(x) = 0 convention; the accept test may be relaxed
    const double r = qx > 0.0 ? fmin(1.0, px / qx) : (px > 0.0 ? 1.0 : 0.0);
    const double ra = a.relax1p == 1.0
                          ? r
                          : (qx > 0.0 ? fmin(1.0, (a.relax1p * px) / qx) : (px > 0.0 ? 1.0 : 0.0));
    const bool accepted = !valid || (double)a.ua[c * L + kk] < ra;
    const unsigned long long rej = __ballot(!accepted);
    const int j = rej ? wave_first(rej) : L;
    const float alpha = (float)(wave_sum_d(valid ? r : 0.0) / (double)L);
    if (valid) {
        if (a.p_x) a.p_x[c * L + kk] = (float)px;
        if (a.q_x) a.q_x[c * L + kk] = (float)qx;
        if (kk != j) a.out_tokens[c * L + kk] = kk < j ? xk : -1;   // j: the residual draw
    }
    // publish the row-j constants, then the flag the residual items read
    const int src = j < L ? j : 0;
    const float jcp = __shfl(cp, src), jcq = __shfl(cq, src);
    const double jsp = __shfl(sp, src), jsq = __shfl(sq, src);
    const int jx = __shfl(xk, src);
    publish_decision(a, c, j, j < L ? a.ur[c * L + j] : 0.0f, jcp, jcq, jsp, jsq, jx, lane);
    if (lane == 0) {
        if (a.alpha) a.alpha[c] = alpha;
        a.accept_len[c] = j;
        a.n_emitted[c] = j + (j < L ? 1 : 0);
    }
}

// ---------------------------------------------------------------------------
// Proposals
// ---------------------------------------------------------------------------

// The proposal of mask row rowid = c * L + k, by one wavefront; part: its
// chunk of LDS, where partials are re-laid out for contiguous runs.
template <typename T>
__device__ __forceinline__ void propose_row(const StepArgs &a, int rowid, uint64_t *part, int lane) {
    const int c = rowid / a.L, k = rowid - c * a.L;
    const float *st = row_stats(a.qn_stats, a, c, k);
    const int n = a.n_stiles;
    Chunk ch;
    load_chunk(st, n, 0, lane, ch);
    float cr;
    double S;
    {
        float r = kNegInfF;
        double acc = 0.0;
        fold_chunk(ch, r, acc);
        for (int t0 = kChunk; t0 < n; t0 += kChunk) {
            Chunk more;
            load_chunk(st, n, t0, lane, more);
            fold_chunk(more, r, acc);
        }
        finish_stats(r, acc, cr, S);
    }
    int token = 0;
    double pw = 0.0;
    if (!(S > 0.0)) {
        if (lane == 0) atomicOr(&a.ws.ctl->error, kErrEmptyRow);
    } else {
        const double target = (double)a.up[rowid] * S;
        // first tile whose running mass exceeds the target: each chunk goes
        // through LDS so that lane l owns a contiguous run of tiles, and one
        // scan of the lane sums finds the lane
        int tile = -1, last_pos = -1;
        double before = 0.0, base = 0.0;
        for (int t0 = 0; t0 < n && tile < 0; t0 += kChunk) {
            if (t0 > 0) load_chunk(st, n, t0, lane, ch);
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < kU; ++i)
                part[i * kWave + lane] =
                    (uint64_t)__float_as_uint(ch.e[i]) | ((uint64_t)__float_as_uint(ch.s[i]) << 32);
            wave_lds_sync();
            const int cn = min(kChunk, n - t0);
            const int per = (cn + kWave - 1) / kWave;
            double m[kU];
            double ls = 0.0;
            int mine_last = -1;
#pragma unroll
            for (int i = 0; i < kU; ++i) {
                const int t = lane * per + i;
                m[i] = 0.0;
                if (i < per && t < cn) {
                    const uint64_t w = part[t];
                    const float e = __uint_as_float((uint32_t)w);
                    if (e != kNegInfF)
                        m[i] = (double)__uint_as_float((uint32_t)(w >> 32)) * pow2_i(e - cr);
                }
                ls += m[i];
                if (m[i] > 0.0) mine_last = t0 + t;
            }
            const double inc = wave_incl_scan_d(ls, lane);
            double run = base + (inc - ls);
            int first = -1;
            double fb = 0.0;
#pragma unroll
            for (int i = 0; i < kU; ++i) {
                if (first < 0 && m[i] > 0.0 && run + m[i] > target) {
                    first = i;
                    fb = run;
                }
                run += m[i];
            }
            int lp = mine_last;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) lp = max(lp, __shfl_xor(lp, o));
            last_pos = max(last_pos, lp);
            const unsigned long long hit = __ballot(first >= 0);
            if (hit) {
                const int l = wave_first(hit);
                tile = t0 + l * per + __shfl(first, l);
                before = __shfl(fb, l);
            }
            base += __shfl(inc, kWave - 1);
        }
        double tile_target = target;
        if (tile < 0) {
            // rounding left the target unreached: the last tile with mass, its last positive entry
            tile = max(last_pos, 0);
            tile_target = __builtin_inf();
        }
        // the crossing tile: lane l holds columns 2l and 2l + 1
        const float tref = st[2 * tile];
        const double scale = pow2_i(tref - cr);
        const T *row = static_cast<const T *>(a.qn) + fused_row_offset(a, c, k);
        const long long col = (long long)tile * kStatsTile + 2 * lane;
        double w[2];
        float v[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            v[e] = col + e < a.V ? load_value<T>(row, col + e) : kNegInfF;
            w[e] = v[e] == kNegInfF ? 0.0 : (double)fast_exp2(fmaf(v[e], a.k2, -tref)) * scale;
        }
        const double ls = w[0] + w[1];
        const double inc = wave_incl_scan_d(ls, lane);
        const double c0 = before + (inc - ls) + w[0];
        const int first = c0 > tile_target ? 0 : (c0 + w[1] > tile_target ? 1 : -1);
        const unsigned long long hit = __ballot(first >= 0);
        long long tok;
        if (hit) {
            const int l = wave_first(hit);
            tok = (long long)tile * kStatsTile + 2 * l + __shfl(first, l);
        } else {
            const int mine = w[1] > 0.0 ? 2 * lane + 1 : (w[0] > 0.0 ? 2 * lane : -1);
            int best = mine;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) best = max(best, __shfl_xor(best, o));
            tok = (long long)tile * kStatsTile + max(best, 0);
        }
        token = (int)tok;
        const float lv = load_value<T>(row, tok);
        pw = exp2((double)lv * (double)a.k2 - (double)cr) / S;
    }
    if (lane == 0) {
        a.next_tokens[rowid] = token;
        if (a.qnext_x) a.qnext_x[rowid] = (float)pw;
    }
}

template <typename T>
__global__ __launch_bounds__(kDecideWaves * kWave) void fused_decide_kernel(StepArgs a) {
    __shared__ float s_c[2][kMaxL];
    __shared__ double s_s[2][kMaxL];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    decide_seq<T, kDecideWaves>(a, blockIdx.x, wave, lane, s_c, s_s);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void fused_propose_kernel(StepArgs a) {
    __shared__ uint64_t s_part[kWavesPerGroup][kChunk];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int rowid = blockIdx.x * kWavesPerGroup + wave;   // c * L + k
    if (rowid >= a.C * a.L) return;
    propose_row<T>(a, rowid, s_part[wave], lane);
}

// Decisions and proposals in one launch: they read only the LM head's partials
// and logits, never each other's results.  Workgroups of kFrontWaves
// wavefronts (two per SIMD, so the proposal code keeps its registers):
// workgroups 0 .. C - 1 decide a sequence each, the rest give each wavefront
// one mask row.  Their LDS (96 KB) keeps one workgroup per CU, so the launch
// is used when all its workgroups fit on the CUs at once.
constexpr int kFrontWaves = 8;
constexpr int kFrontMaxGroups = 256;

template <typename T>
__global__ __launch_bounds__(kFrontWaves * kWave) void fused_front_kernel(StepArgs a) {
    __shared__ float s_c[2][kMaxL];
    __shared__ double s_s[2][kMaxL];
    __shared__ uint64_t s_part[kFrontWaves][kChunk];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    if ((int)blockIdx.x < a.C) {
        decide_seq<T, kFrontWaves>(a, blockIdx.x, wave, lane, s_c, s_s);
        return;
    }
    const int rowid = ((int)blockIdx.x - a.C) * kFrontWaves + wave;
    if (rowid >= a.C * a.L) return;
    propose_row<T>(a, rowid, s_part[wave], lane);
}

int front_groups(const StepArgs &a) {
    return a.C + (a.C * a.L + kFrontWaves - 1) / kFrontWaves;
}

}  // namespace

bool fused_front_fits(const StepArgs &a) { return front_groups(a) <= kFrontMaxGroups; }

hipError_t launch_fused_front(const StepArgs &a, int dtype, hipStream_t stream) {
    const unsigned g = (unsigned)front_groups(a);
    if (dtype == kBf16)
        hipLaunchKernelGGL(fused_front_kernel<uint16_t>, dim3(g), dim3(kFrontWaves * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL(fused_front_kernel<float>, dim3(g), dim3(kFrontWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fused_decide(const StepArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kBf16)
        hipLaunchKernelGGL(fused_decide_kernel<uint16_t>, dim3((unsigned)a.C),
                           dim3(kDecideWaves * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL(fused_decide_kernel<float>, dim3((unsigned)a.C), dim3(kDecideWaves * kWave),
                           0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fused_propose(const StepArgs &a, int dtype, hipStream_t stream) {
    const unsigned blocks = (unsigned)((a.C * a.L + kWavesPerGroup - 1) / kWavesPerGroup);
    if (dtype == kBf16)
        hipLaunchKernelGGL(fused_propose_kernel<uint16_t>, dim3(blocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(fused_propose_kernel<float>, dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace isd
