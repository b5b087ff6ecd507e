// Bookkeeping of the multi-step decoding loop around the ISD step
// ("Introspective Diffusion Language Models | Summary", section 3.2).  A
// sequence in the verify state that keeps all L proposals (accept_len == L)
// also takes a bonus token from its anchor row L; one that rejects moves to
// the recovery state, whose next step draws no verification and only makes
// proposals.  One thread per sequence; the step, bonus and anchor draws
// themselves are the step kernel's.

#include "isd_internal.h"

namespace isd {
namespace {

constexpr int32_t kStateRecover = 0;
constexpr int32_t kStateVerify = 1;
constexpr int kLedgerThreads = 256;

__global__ __launch_bounds__(kLedgerThreads) void decode_masks_kernel(
    int C, int L, const int32_t *__restrict__ state, const int32_t *__restrict__ accept_len,
    int32_t *__restrict__ bonus_mask, int32_t *__restrict__ anchor_mask) {
    const int c = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (c >= C) return;
    const bool verifying = state[c] == kStateVerify;
    bonus_mask[c] = (verifying && accept_len[c] == L) ? 1 : 0;
    anchor_mask[c] = verifying ? 0 : 1;
}

__global__ __launch_bounds__(kLedgerThreads) void decode_commit_kernel(
    int C, int L, int32_t *__restrict__ state, const int32_t *__restrict__ accept_len,
    const int32_t *__restrict__ out_tokens, const int32_t *__restrict__ bonus,
    const int32_t *__restrict__ anchor, int32_t *__restrict__ history, long long cap,
    int64_t *__restrict__ tokens, int64_t *__restrict__ forwards) {
    const int c = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (c >= C) return;
    const bool verifying = state[c] == kStateVerify;
    const int j = verifying ? accept_len[c] : 0;
    const long long at = tokens[c];
    int n = 0;
    auto put = [&](int32_t tok) {
        if (history && at + n < cap) history[(long long)c * cap + at + n] = tok;
        ++n;
    };
    if (verifying) {
        // the accepted prefix, then the correction at j or, if all passed, the bonus
        const int m = j < L ? j + 1 : L;
        for (int k = 0; k < m; ++k) put(out_tokens[c * L + k]);
        if (j >= L) put(bonus[c]);
    } else {
        put(anchor[c]);
    }
    tokens[c] = at + n;
    forwards[c] += 1;
    state[c] = (verifying && j < L) ? kStateRecover : kStateVerify;
}

unsigned blocks_for(int C) { return (unsigned)((C + kLedgerThreads - 1) / kLedgerThreads); }

}  // namespace

hipError_t launch_decode_masks(int C, int L, const int32_t *state, const int32_t *accept_len,
                               int32_t *bonus_mask, int32_t *anchor_mask, hipStream_t stream) {
    hipLaunchKernelGGL(decode_masks_kernel, dim3(blocks_for(C)), dim3(kLedgerThreads), 0, stream,
                       C, L, state, accept_len, bonus_mask, anchor_mask);
    return hipGetLastError();
}

hipError_t launch_decode_commit(int C, int L, int32_t *state, const int32_t *accept_len,
                                const int32_t *out_tokens, const int32_t *bonus,
                                const int32_t *anchor, int32_t *history, int64_t hist_cap,
                                int64_t *tokens, int64_t *forwards, hipStream_t stream) {
    hipLaunchKernelGGL(decode_commit_kernel, dim3(blocks_for(C)), dim3(kLedgerThreads), 0, stream,
                       C, L, state, accept_len, out_tokens, bonus, anchor, history,
                       (long long)hist_cap, tokens, forwards);
    return hipGetLastError();
}

}  // namespace isd
