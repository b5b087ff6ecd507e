// Internal declarations shared by the ISD step kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace isd {

// Work decomposition.  A "tile" is the contiguous span one wavefront streams
// per iteration: 4 groups of 64 lanes x 8 elements, group-major, so lane l
// holds elements g*512 + l*8 + e of the tile.  Each 8-element group is one
// 16-byte load per lane for bf16 (two for fp32): every wavefront load
// instruction covers 1 KiB (bf16) of consecutive bytes.
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kGroupElems = 8;
constexpr int kGroupsPerTile = 4;
constexpr int kLaneElems = kGroupElems * kGroupsPerTile;       // 32
constexpr int kTileElems = kWave * kLaneElems;                 // 2048
constexpr int kMaxL = 64;
constexpr int kMaxSegments = 32;
constexpr int kMaxResidSegments = 64;
constexpr int kMaxTopK = 64;           // largest top-k of the truncated path
constexpr int kMaxTruncSegments = 8;   // row segments of the truncated path
// Completion counters and flags each own a 128-byte line: atomics that share
// a line serialise at the memory side.
constexpr int kCounterStride = 32;   // uint32 words

// Device error word bits.
constexpr uint32_t kErrBadToken = 1u << 0;     // proposal id outside [0, V)
constexpr uint32_t kErrEmptyRow = 1u << 1;     // a row with no finite logit
constexpr uint32_t kErrWaitExpired = 1u << 2;  // a cross-workgroup wait gave up

// Workspace records.  Counters and flags return to zero at the end of the
// launch that uses them.
struct Control {               // 256 B at offset 0
    uint32_t ticket;           // step items taken past n_static (reset by the last taker)
    uint32_t reserved;
    uint32_t seq_done;         // sequences whose decision is done (alpha mean)
    uint32_t error;            // kErr* bits, cleared by isd_check_device_error
    uint32_t pad[60];
};

struct SegRec {                // softmax partial of one row segment
    float ref;                 // integer reference e: terms are 2^(x*k2 - e)
    float pad;
    double sum;                // sum of the segment's terms
};

struct ArgRec {                // argmax partial of one row segment
    float val;
    int32_t idx;
};

struct TileRec {               // mass of one 2048-element tile of a mask row
    float ref;
    float sum;                 // sum of 2^(x*k2 - ref) over the tile
};

struct ResTile {               // masses of one tile of a residual row pair, in units of 1/Sp
    float r;                   // sum of max(0, P - Q)
    float p;                   // sum of P (used only if the residual is empty)
};

struct SeqInfo {               // per-sequence decision, read by residual items
    int32_t j;                 // first rejected position (L if none)
    float u;                   // u_resid[c, j]
    float cp, cq;              // references of rows p[c, j], q[c, j]
    float inv_sp, inv_sq;      // 1 / softmax denominators of those rows
    float alpha;
    int32_t xj;                // x[c, j] (the argmax pick removed from the residual)
    float rho_hi, rho_lo;      // Sp / Sq of those rows as an unevaluated fp32 sum
};

struct Workspace {
    Control *ctl;
    uint32_t *seq_cnt;         // [C]     pq items finished per sequence      (strided)
    uint32_t *res_cnt;         // [C]     residual items finished per sequence (strided)
    uint32_t *flag;            // [C]     decision published for sequence c: the launch's epoch (strided)
    uint32_t *row_cnt;         // [C*L]   mask-row items finished per row      (strided)
    SegRec *seg;               // [2*C*L*Smax] sample: p rows then q rows
    ArgRec *arg;               // [2*C*L*Smax] greedy: p rows then mask rows (aliases seg)
    TileRec *tiles;            // [C*L*tiles_row] mask rows
    ResTile *rtiles;           // [C*tiles_row]  residual rows
    SeqInfo *info;             // [C]
    ArgRec *garg;              // [C*kMaxResidSegments*2] Gumbel-max partials (R, P) per residual segment
};

// Records of the truncated (top-k / top-p) path; all return to zero.
struct TruncWorkspace {
    uint32_t *row_cnt;         // [C*3L] segments finished per row (p, q, then mask rows; strided)
    uint32_t *seq_cnt;         // [C]    verify rows finished per sequence (strided)
    uint64_t *keys;            // [C*3L*St*64] top keys of each row segment
    uint64_t *lists;           // [C*2L*64*2] survivors of verify rows: (index, fp64 weight)
    uint64_t *pxq;             // [C*2L] fp64 P'(x_k), then Q'(x_k)
    uint32_t *alpha;           // [C] fp32 alpha (batch mean)
};

struct WorkspaceLayout {
    size_t off_seq_cnt, off_res_cnt, off_flag, off_row_cnt, off_seg, off_tiles,
        off_rtiles, off_info, off_garg, total;
    size_t off_trow_cnt, off_tseq_cnt, off_tkeys, off_tlists, off_tpxq, off_talpha;
    int smax;
    bool trunc;
};

// `trunc` adds the records of the truncated path.
WorkspaceLayout workspace_layout(int C, int L, int V, bool trunc);
Workspace workspace_at(void *base, const WorkspaceLayout &lay);
TruncWorkspace trunc_workspace_at(void *base, const WorkspaceLayout &lay);

// Everything one launch of the step kernel needs (passed by value).
struct StepArgs {
    int C, L, V;
    long long ld;              // elements between rows (c, k) and (c, k + 1)
    long long ldc;             // elements between rows (c, k) and (c + 1, k)
    float k2;                  // log2(e) / T
    // inputs
    const void *p, *q, *qn;
    const int32_t *x;
    const float *ua, *ur, *up;
    const int32_t *vmask, *pmask;   // per-sequence verify / propose masks (NULL: all)
    double relax1p;            // 1 + tau: the accept test uses min(1, (1 + tau) P/Q)
    int q_onehot;              // proposals are argmax picks: Q = onehot(x), q not read
    int sampler;               // correction draw: 0 inverse CDF, 1 Gumbel-max
    int top_k;                 // truncated path: keep the first top_k ranks (1..64)
    double top_p;              // truncated path: nucleus mass, or 1 (off)
    double temp;               // T
    // outputs (NULL when not requested)
    int32_t *accept_len, *out_tokens, *n_emitted;
    float *p_x, *q_x, *alpha, *alpha_mean;
    int32_t *next_tokens;
    float *qnext_x;
    Workspace ws;
    // decomposition
    int tiles_row;             // ceil(V / kTileElems)
    int smax;                  // segment records reserved per row in the workspace
    int S, tps;                // segments per verify row, tiles per segment
    int Sq, tpsq;              // segments per mask row, tiles per segment
    int Sr, tpsr;              // segments per residual row pair, tiles per segment
    int rows_pq;               // verify rows per sequence (2L sample, L greedy, 0 none)
    int n_pq;                  // C * rows_pq * S
    int q_blk;                 // mask-row items per sequence (L*Sq or 0)
    int r_blk;                 // residual items per sequence (Sr or 0)
    int n_items;
    int n_static;              // items taken by workgroup index; the rest by ticket
    int verify_outputs;        // write tokens / counts (0: alpha only)
    int order;                 // 0: per sequence [mask rows, residual]; 1: all mask rows first
    uint32_t spin_limit;
    uint32_t epoch;            // nonzero tag of this launch: the value a published decision carries
    // truncated path
    int St, tpst;              // segments per row, tiles per segment
    TruncWorkspace tws;
    // statistics path: per-(row, 128-column tile) softmax partials (ref, sum)
    const float *p_stats, *q_stats, *qn_stats;
    long long s_ld, s_ldc;     // entries between rows (c, k), (c, k + 1) and sequences
    int n_stiles;              // ceil(V / 128)
};

enum Dtype { kBf16 = 0, kF32 = 1 };
enum Mode { kSample = 0, kGreedy = 1 };

// Launches the step kernel for `a` (dtype/mode select the instantiation).
hipError_t launch_step(const StepArgs &a, int dtype, int mode, bool vec, hipStream_t stream);
// The statistics path: the decision from the LM head's partials (before the
// residual items of launch_step), and the proposals (after it).
hipError_t launch_fused_decide(const StepArgs &a, int dtype, hipStream_t stream);
hipError_t launch_fused_propose(const StepArgs &a, int dtype, hipStream_t stream);
// Both in one launch (before the residual items), when its workgroups fit on
// the CUs at once.
bool fused_front_fits(const StepArgs &a);
hipError_t launch_fused_front(const StepArgs &a, int dtype, hipStream_t stream);

// Launches the truncated (top-k / top-p) step kernel for `a` (sample mode).
hipError_t launch_trunc(const StepArgs &a, int dtype, bool vec, hipStream_t stream);

// Bookkeeping kernels of the multi-step decoding loop.
hipError_t launch_decode_masks(int C, int L, const int32_t *state, const int32_t *accept_len,
                               int32_t *bonus_mask, int32_t *anchor_mask, hipStream_t stream);
hipError_t launch_decode_commit(int C, int L, int32_t *state, const int32_t *accept_len,
                                const int32_t *out_tokens, const int32_t *bonus,
                                const int32_t *anchor, int32_t *history, int64_t hist_cap,
                                int64_t *tokens, int64_t *forwards, hipStream_t stream);

// LM-head GEMM on a pre-packed head wt = w^T [N, K], and the packing.  With a
// workspace of gemm_workspace_bytes(M, K, N) bytes (zero-filled once; each
// launch leaves its counters zero) the tiles of a last partial round are
// halved along K; 0 bytes: that split does not apply to the shape.
size_t gemm_workspace_bytes(int M, int K, int N);
hipError_t launch_lm_head_packed(const uint16_t *h, const uint16_t *wt, int M, int K, int N,
                                 uint16_t *out, void *ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_pack_wt(const uint16_t *w, uint16_t *wt, int K, int N, hipStream_t stream);

// The packed LM-head GEMM that also writes per-(row, 128-column tile) softmax
// partials (ref, sum) of its bf16 logits; k2 = log2(e) / T.
constexpr int kStatsTile = 128;
hipError_t launch_lm_head_stats(const uint16_t *h, const uint16_t *wt, int M, int K, int N,
                                float k2, uint16_t *out, float *stats, void *ws, size_t ws_bytes,
                                hipStream_t stream);

// Segment-gated LoRA projection: t = gate * (x a^T), then out = (x | t) wcat^T
// with wcat = (w | b) [N, K + r].
hipError_t launch_lora_gemm(const uint16_t *x, const uint16_t *a, const uint16_t *wcat,
                            const int32_t *mask, int M, int K, int N, int r, uint16_t *t,
                            uint16_t *out, void *ws, size_t ws_bytes, hipStream_t stream);

// Streaming-read probe over n_tiles 2048-element bf16 tiles (4 KiB each),
// tiles_per_group consecutive tiles per workgroup.
hipError_t launch_read_probe(const void *buf, long long n_tiles, int tiles_per_group,
                             uint32_t *sink, hipStream_t stream);

// LM-head GEMM (bf16 in, fp32 accumulate, bf16 out).
hipError_t launch_lm_head(const uint16_t *h, const uint16_t *w, int M, int K, int N,
                          uint16_t *out, hipStream_t stream);

}  // namespace isd
