// probe.hip -- a plain streaming-read kernel, the device analogue of a host
// memory-bandwidth probe: the achievable HBM read rate on this part, reported
// beside the 8 TB/s datasheet figure when the engines are measured.
//
// Each workgroup (4 waves) reads one contiguous range with coalesced 16-byte
// non-temporal buffer loads, 8 loads in flight per lane, and folds the data
// into one word so the loads cannot be dropped.
#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t *p, int64_t bytes,
                                                                   int64_t per_block, uint32_t *sink)
{
    const int64_t start = (int64_t)blockIdx.x * per_block;
    const int64_t end = min(start + per_block, bytes);
    if (start >= end) return;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p + start), 0, (int)(end - start), kBufferWord3);
    uint32_t acc = 0;
    const int len = (int)(end - start);
    for (int off = threadIdx.x * 16; off < len; off += kProbeThreads * 16 * kProbeUnroll) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off + u * kProbeThreads * 16, 0, kCacheNT);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // one word per workgroup (the sink has grid entries)
    acc ^= __shfl_xor(acc, 1);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

int launch_read_probe(const void *p, int64_t bytes, uint32_t *sink, int64_t sink_words,
                      hipStream_t stream)
{
    if (bytes <= 0) return 0;
    // 16 workgroups per CU, each range a multiple of 64 KB and below 2 GB
    const int64_t nblk_target = 256 * 16;
    int64_t per = (bytes + nblk_target - 1) / nblk_target;
    per = (per + 65535) / 65536 * 65536;
    if (per > 0x7fff0000LL) return -4;
    const int64_t grid = (bytes + per - 1) / per;
    if (grid > sink_words) return -5;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       (const uint8_t *)p, bytes, per, sink);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace q8
