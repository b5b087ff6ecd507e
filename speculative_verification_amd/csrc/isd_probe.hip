// Streaming-read probe: the HBM read rate this part reaches with the access
// pattern of the step kernel.  Each workgroup streams one contiguous segment
// of 2048-element bf16 tiles with the step's own tile loader (one 16-byte
// non-temporal load per lane and group, the next tile in flight while the
// current one is folded), so the measured rate is the ceiling of that loop
// on the device, without any of the step's arithmetic.  The words are folded
// into a per-thread checksum that is stored only if it takes one particular
// value, which keeps every load live at no store traffic.

#include "isd_device.h"
#include "isd_internal.h"

namespace isd {
namespace {

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint16_t *__restrict__ buf,
                                                              int n_tiles, int tiles_per_group,
                                                              uint32_t *__restrict__ sink) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int t0 = (int)blockIdx.x * tiles_per_group;
    const int t1 = min(n_tiles, t0 + tiles_per_group);
    uint32_t acc = 0;
    stream_row<uint16_t, true>(buf, t0, t1, n_tiles * kTileElems, wave, lane,
                               [&](const TileRaw<uint16_t> &r, int) {
#pragma unroll
        for (int i = 0; i < TileRaw<uint16_t>::kWords; ++i) acc += r.w[i] ^ (acc >> 7);
    });
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, long long n_tiles, int tiles_per_group,
                             uint32_t *sink, hipStream_t stream) {
    const long long groups = (n_tiles + tiles_per_group - 1) / tiles_per_group;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)groups), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t *>(buf), (int)n_tiles, tiles_per_group, sink);
    return hipGetLastError();
}

}  // namespace isd
