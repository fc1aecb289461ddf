// ev_measure.hip -- streaming-read ceiling of the GPU, the reference the attention's K/V read rate
// is reported against (besides the 8 TB/s HBM peak).
//
// Every 16-byte chunk of the buffer is read exactly once with non-temporal loads and folded by
// XOR into a register; a store to the sink happens only when the fold equals a fixed constant, so
// the loads stay live without adding write traffic.  Each workgroup reads one contiguous part of
// the buffer, eight 16-byte loads per thread 4 KB apart in flight, two workgroups per CU: on
// MI355X this reads ~7.1 TB/s, where a grid-stride interleave of the same loads reads 5.6-6.5.
#include "ev_internal.h"

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadBlocksPerCu = 2;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4_t *src, size_t n16, uint32_t *sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = static_cast<size_t>(blockIdx.x) * per;
    const size_t b1 = b0 + per < n16 ? b0 + per : n16;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    size_t i = b0 + threadIdx.x;
    for (; i + 7 * kReadThreads < b1; i += 8 * kReadThreads) {
        u32x4_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = ev::ld16_stream(src + i + k * kReadThreads);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc ^= w[k];
    }
    for (; i < b1; i += kReadThreads) acc ^= ev::ld16_stream(src + i);
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u) *sink = x;
}

}  // namespace

extern "C" ev_status ev_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
    if (!src || !sink) return EV_ERR_NULL;
    if (bytes == 0 || bytes % 16) return EV_ERR_SHAPE;
    if (!ev::aligned16(src)) return EV_ERR_ALIGN;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    const int blocks = ev::device_cu_count() * kReadBlocksPerCu;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4_t *>(src), bytes / 16, sink);
    return ev::launch_status();
}
