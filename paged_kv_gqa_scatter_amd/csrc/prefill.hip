// paged_gqa_prefill: causal attention of chunks of query rows over a paged KV
// cache, on bf16 MFMA with fp32 accumulation.
//
// "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.1 tiles the queries in
// blocks of 128 and, for each, walks only the key blocks at or before it, so the
// full score matrix never exists.  Its per-tile softmax is not exact attention;
// here every query row keeps a running max and sum (online softmax) so the
// result is softmax(QK^T * scale) V exactly up to rounding.
//
// gfx950 design (one workgroup = 4 waves = 128 query rows of one query head):
//  * Each wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A
//    operand, the wave's Q rows stay in registers as the B operand.  In the
//    32x32 result a lane holds one query (column) and 16 keys, so the row max
//    and sum need only the lane and its partner lane 32 away.
//  * The probabilities are already laid out as the B operand of
//    O^T += V^T P^T (keys as the contraction index), so they are packed to bf16
//    in place.  V stays row-major in LDS and the V^T operand is read with
//    ds_read_b64_tr_b16, the gfx950 transposing LDS read.
//  * K/V tiles of 64 keys are gathered through the block table into LDS by the
//    whole workgroup; rows past the keys this tile may see are zero-filled so
//    that unwritten (NaN) slots never reach the MFMA.
//  * Causal tile skipping: a workgroup stops at its last query's position, and
//    a wave skips tiles that lie wholly after its own rows; the mask is applied
//    as a select.  Row r of a chunk of n rows on a sequence of length L is at
//    position L - n + r (chunked prefill on cached context).
//  * Launch order: the longest query tiles first, and the KV head in the low
//    bits of the workgroup index, so that workgroups reading the same K/V land
//    on the same XCD (workgroups are dealt round-robin over the 8 XCDs) and
//    share its L2.
#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kPrefillThreads = 256;
constexpr int kTileQ = 128;  // query rows per workgroup (32 per wave)
constexpr int kTileK = 64;   // keys per LDS tile
constexpr int kLdsPad = 8;   // bf16 elements of padding per LDS row
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // the bf16 pair (1.0, 1.0)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct PrefillKernelArgs {
    PrefillArgs a;
    int32_t log2_block;
    int32_t group;      // query heads per KV head
    int32_t q_tiles;    // tiles of the longest chunk
    float qk_scale_log2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing LDS read (see header comment): 4 bf16 of column d for 4 keys.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
    s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, t);
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillKernelArgs p) {
    constexpr int kRow = D + kLdsPad;  // LDS row stride in elements
    __shared__ __attribute__((aligned(16))) uint16_t sK[kTileK * kRow];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kTileK * kRow];
    const PrefillArgs& a = p.a;

    // workgroup -> (query tile, sequence, query head); KV head in the low bits
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, S = a.num_seqs;
    int idx = blockIdx.x;
    const int g = idx % Hkv;
    idx /= Hkv;
    const int hg = idx % p.group;
    idx /= p.group;
    const int s = idx % S;
    const int tile = p.q_tiles - 1 - idx / S;
    const int h = g * p.group + hg;

    // rows of this sequence, clamped so that bad offsets never leave q / out
    const int q0 = min(max(a.cu_q_lens[s], 0), a.total_q_tokens);
    const int n = min(min(max(a.cu_q_lens[s + 1], q0), a.total_q_tokens) - q0, a.max_q_len);
    if (tile * kTileQ >= n) return;
    const int cap = a.max_blocks_per_seq << p.log2_block;
    int L = a.seq_lens[s];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int ctx = L - n;  // cached keys before the chunk

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int qrow = tile * kTileQ + wave * 32 + (lane & 31);  // this lane's query row in the chunk
    const int qpos = ctx + qrow;                                // its absolute position
    const int wave_last = min(tile * kTileQ + wave * 32 + 31, n - 1);
    const int wave_qpos_max = ctx + wave_last;
    const int kend = min(L, ctx + min((tile + 1) * kTileQ, n));  // keys this workgroup may see: [0, kend)

    u32x4 qreg[D / 16];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const uint16_t* qp = a.q + ((int64_t)(q0 + qrow) * Hq + h) * D + half * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = qrow < n ? load16(qp + ks * 16) : zero;
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    const int32_t* table = a.block_table + (int64_t)s * a.max_blocks_per_seq;
    const int B = 1 << p.log2_block;
    const int64_t head_stride = (int64_t)B * D;

    for (int kt = 0; kt < kend; kt += kTileK) {
        __syncthreads();  // previous tile fully consumed
        constexpr int kPieces = D / 8;
#pragma unroll
        for (int pass = 0; pass < kTileK * kPieces / kPrefillThreads; ++pass) {
            const int e = pass * kPrefillThreads + tid;
            const int row = e / kPieces, piece = e % kPieces;
            const int key = kt + row;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (key < kend) {
                const int blk = table[key >> p.log2_block];
                if ((unsigned)blk < (unsigned)a.num_blocks) {
                    const int64_t off = ((int64_t)blk * Hkv + g) * head_stride + (int64_t)(key & (B - 1)) * D + piece * 8;
                    kv = load16(a.k_pool + off);
                    vv = load16(a.v_pool + off);
                }
            }
            *reinterpret_cast<u32x4*>(&sK[row * kRow + piece * 8]) = kv;
            *reinterpret_cast<u32x4*>(&sV[row * kRow + piece * 8]) = vv;
        }
        __syncthreads();
        if (kt > wave_qpos_max) continue;  // every key of this tile is after this wave's rows

        // S^T = K Q^T for two 32-key blocks
        f32x16 st[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
            const uint16_t* kp = &sK[(kb * 32 + (lane & 31)) * kRow + half * 8];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(kp + ks * 16);
                st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qreg[ks]), st[kb], 0, 0, 0);
            }
        }
        // scale, causal mask, tile max over this query's 32 keys (here and in lane ^ 32)
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kt + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                const float v = key <= qpos ? st[kb][r] * p.qk_scale_log2 : -INFINITY;
                st[kb][r] = v;
                mt = fmaxf(mt, v);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
        const float m_new = fmaxf(m, mt);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st[kb][r] = st[kb][r] == -INFINITY ? 0.f : fast_exp2(st[kb][r] - m_new);
        m = m_new;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;

        // O^T += V^T P^T, 16 keys per MFMA.  The row sum adds up exactly the
        // bf16-rounded weights the MFMA multiplies (dot with (1, 1)), so the
        // result stays a true weighted average of V rows.
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                u32x4 pb;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pb[i] = pack_bf16x2(st[kb][sub * 8 + 2 * i], st[kb][sub * 8 + 2 * i + 1]);
                    ps = dot2_bf16(pb[i], kOnesBf16x2, ps);
                }
                const int kbase = kb * 32 + sub * 16;
                const int row = kbase + half * 4 + ((lane & 15) >> 2);
                const int col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
                for (int i = 0; i < D / 32; ++i) {
                    const uint16_t* vp = &sV[row * kRow + i * 32 + col];
                    const u32x2 lo = lds_read_tr(vp);
                    const u32x2 hi = lds_read_tr(vp + 8 * kRow);
                    const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pb), acc[i], 0, 0, 0);
                }
            }
        lsum = lsum * alpha + ps;
    }

    lsum += __shfl_xor(lsum, 32, kWave);
    if (qrow >= n) return;
    const float inv = (qpos >= 0 && lsum > 0.f) ? 1.f / lsum : 0.f;  // a row with no key is zero
    uint16_t* op = a.out + ((int64_t)(q0 + qrow) * Hq + h) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = i * 32 + j * 8 + half * 4;
            u32x2 w = {pack_bf16x2(acc[i][4 * j] * inv, acc[i][4 * j + 1] * inv),
                       pack_bf16x2(acc[i][4 * j + 2] * inv, acc[i][4 * j + 3] * inv)};
            *reinterpret_cast<u32x2*>(op + d) = w;
        }
}

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0 || a.max_q_len == 0 || a.total_q_tokens == 0) return hipSuccess;
    PrefillKernelArgs kp;
    kp.a = a;
    kp.log2_block = ilog2(a.block_size);
    kp.group = a.num_q_heads / a.num_kv_heads;
    kp.q_tiles = (a.max_q_len + kTileQ - 1) / kTileQ;
    kp.qk_scale_log2 = a.scale * kLog2e;
    const int64_t blocks = (int64_t)kp.q_tiles * a.num_seqs * a.num_q_heads;
    if (a.head_dim == 128)
        hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)blocks), dim3(kPrefillThreads), 0, stream, kp);
    else
        hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)blocks), dim3(kPrefillThreads), 0, stream, kp);
    return hipGetLastError();
}

}  // namespace pkv
