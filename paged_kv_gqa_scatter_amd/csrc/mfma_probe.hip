// mfma_probe: the practical rate of the bf16 matrix cores, measured with the
// instruction the prefill and the fused QKV projection run on
// (v_mfma_f32_32x32x16_bf16).  Every wave issues two independent accumulator
// chains on register operands; nothing else runs and nothing is read from
// memory.  Two workgroups of four waves per CU (two waves per SIMD).  The
// operands are hashed bit patterns (random sign and 7-bit mantissa, exponents
// spanning [2^-7, 2)): the clock this part holds under MFMA load depends on
// how many operand bits toggle, and operands with few mantissa bits would
// run it faster than attention's data does.  On MI355X: 1.85-1.87 PFLOP/s
// (about 0.75 of the 2.5 PFLOP/s figure, which assumes 2.4 GHz); operands
// that are multiples of 1/16 reach 2.22.
#include "pkv.h"
#include "pkv_diag.h"
#include "pkv_device.h"

namespace pkv {
namespace {

constexpr int kMfmaProbeThreads = 256;
// bf16 bits from a hash: random sign and mantissa, exponent 120..127
__device__ __forceinline__ uint16_t probe_bits(uint32_t h) {
    return (uint16_t)(((h >> 31) << 15) | ((120u + ((h >> 28) & 7u)) << 7) | (h & 0x7Fu));
}

// `never` is a NaN bit pattern from the host: a fold of finite values never
// has it, so the sink is never written, yet the compiler must keep the chains
__global__ __launch_bounds__(kMfmaProbeThreads) void mfma_probe_kernel(int32_t iters, uint32_t never, float* sink) {
    const uint32_t seed = threadIdx.x * 0x9E3779B1u + blockIdx.x * 0xC2B2AE3Du;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = __builtin_bit_cast(__bf16, probe_bits(seed + i * 0x85EBCA77u));
        b[i] = __builtin_bit_cast(__bf16, probe_bits((seed ^ 0x5BD1E995u) + i * 0x27D4EB2Fu));
    }
    f32x16 c0, c1;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        }
    }
    // |operands| < 2, so |c| < 4 x 16 x 8 x iters <= 2^29: the fold is finite
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] - c1[r] * 0.5f;
    if (__builtin_bit_cast(uint32_t, s) == never) sink[blockIdx.x * kMfmaProbeThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace pkv

extern "C" int32_t pkv_mfma_probe(int32_t iters, void* sink, size_t sink_bytes, void* stream) {
    if (sink == nullptr) return PKV_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(sink) & 3) return PKV_ERR_MISALIGNED;
    if (iters < 1 || iters > PKV_MFMA_PROBE_MAX_ITERS) return PKV_ERR_BAD_SHAPE;
    if (sink_bytes < (size_t)4 * pkv::kMfmaProbeThreads * PKV_MFMA_PROBE_WORKGROUPS) return PKV_ERR_WORKSPACE;
    hipLaunchKernelGGL(pkv::mfma_probe_kernel, dim3(PKV_MFMA_PROBE_WORKGROUPS), dim3(pkv::kMfmaProbeThreads), 0,
                       static_cast<hipStream_t>(stream), iters, 0x7FC00001u, static_cast<float*>(sink));
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
