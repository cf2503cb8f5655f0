// read_probe: a plain stream of reads, the practical read ceiling of the
// device, measured with the loads the decode kernels stream K/V rows with
// (16 bytes per lane, non-temporal).  Each workgroup instruction covers 4 KiB
// of consecutive bytes; eight loads per lane are in flight while the previous
// eight are folded.  On MI355X, 2 GiB: 6.56 TB/s at 8192 workgroups (best of
// 10), 6.19 at 4096, 5.95 at 2048; the same loop with plain loads 5.93.
#include "pkv.h"
#include "pkv_diag.h"
#include "pkv_device.h"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;  // a fold that (practically) never occurs

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n,
                                                                   u32x4* sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    auto load = [&](int64_t j) { return j < n ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u}; };
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    u32x4 cur[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) cur[k] = load(i + k * stride);
    for (; i < n; i += stride * kProbeUnroll) {
        u32x4 next[kProbeUnroll];  // the next batch is in flight while this one is folded
#pragma unroll
        for (int k = 0; k < kProbeUnroll; ++k) next[k] = load(i + (kProbeUnroll + k) * stride);
#pragma unroll
        for (int k = 0; k < kProbeUnroll; ++k) acc ^= cur[k];
#pragma unroll
        for (int k = 0; k < kProbeUnroll; ++k) cur[k] = next[k];
    }
    // keeps the loads live without a store per workgroup
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == kProbeMagic) sink[blockIdx.x] = acc;
}

}  // namespace
}  // namespace pkv

extern "C" int32_t pkv_read_probe(const void* data, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
    if (data == nullptr || sink == nullptr) return PKV_ERR_NULL_POINTER;
    if ((reinterpret_cast<uintptr_t>(data) | reinterpret_cast<uintptr_t>(sink)) & 15) return PKV_ERR_MISALIGNED;
    if (bytes == 0 || bytes % 16 != 0) return PKV_ERR_BAD_SHAPE;
    if (sink_bytes < (size_t)16 * PKV_READ_PROBE_WORKGROUPS) return PKV_ERR_WORKSPACE;
    hipLaunchKernelGGL(pkv::read_probe_kernel, dim3(PKV_READ_PROBE_WORKGROUPS), dim3(pkv::kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const pkv::u32x4*>(data),
                       (int64_t)(bytes / 16), static_cast<pkv::u32x4*>(sink));
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
