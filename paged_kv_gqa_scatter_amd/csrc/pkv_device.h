// Device-side helpers shared by the libpkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 halves of a packed pair -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// <a, b> over one packed bf16 pair, accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// The same with the non-temporal hint (nt): for data read or written once,
// which the caches should not keep in place of data that is reused.
__device__ __forceinline__ u32x4 load16_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16_nt(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// 2^x (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max of v over lanes l and l ^ 32.  v_permlane32_swap exchanges the two
// halves of the wave in registers (no LDS round trip, unlike a shuffle);
// whichever result holds which half, the max of the pair is the same.
__device__ __forceinline__ float max_xor32(float v) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                     false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
}

// Symmetric INT8 quantisation of one row held by `kPieces` consecutive lanes
// (an aligned group), 8 bf16 values each ("从零搭建AI工程能力：手写KV Cache与
// 动态批处理实战" section 3.2 keeps the cache in INT8; the scheme is this
// library's): scale = max|x| / 127 and code = x / scale rounded to the
// nearest integer, ties to even, in fp32 with IEEE division (an all-zero row
// has scale 0 and codes 0).  Returns this lane's 8 codes; *scale gets the
// row's scale on every lane of the row.
template <int kPieces>
__device__ __forceinline__ u32x2 quantize_piece(u32x4 x, float* scale) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(x[i]);
        f[2 * i + 1] = bf16_hi(x[i]);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int off = kPieces / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    const float sc = amax / 127.f;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float c = sc > 0.f ? fminf(fmaxf(rintf(f[i] / sc), -127.f), 127.f) : 0.f;
        w[i / 4] |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * (i % 4));
    }
    *scale = sc;
    return u32x2{w[0], w[1]};
}

}  // namespace pkv
