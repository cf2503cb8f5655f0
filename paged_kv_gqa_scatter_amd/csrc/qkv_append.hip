// qkv_project_append: the fused QKV projection whose epilogue writes k and v
// straight into the paged cache.
//
// "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.3 computes q, k and v with
// one matmul against the merged weight W = [W_q; W_k; W_v] and cuts the output
// into the three parts; the k and v rows are then appended to the cache
// (section 4.3.1).  Here the two steps are one kernel: Y = X W^T in bf16 on
// the matrix cores with fp32 accumulation, and each output tile is rounded to
// bf16 and stored where it belongs -- q rows to q_out, k and v rows to the
// (block, KV head, slot) their token's position maps to -- so the k/v rows
// never make a round trip through HBM between a projection and an append.
//
// gfx950 design:
//  * Workgroup = 4 waves = a 128 x 128 tile of Y (tokens x output features);
//    each wave computes a 64 x 64 quarter as 2 x 2 v_mfma_f32_32x32x16_bf16
//    tiles.  Both X [T][d_model] and W [N][d_model] are row-major with d_model
//    contiguous, so both operands are read as rows.
//  * K steps of 64: the X and W slices of a step (2 x 16 KB) are copied into
//    LDS with global_load_lds_dwordx4, double-buffered, one barrier per step;
//    the copy of step k + 1 runs while step k is multiplied.  Each lane's
//    global offset is fixed for the workgroup (rows past the end repeat the
//    last row); the step moves the scalar base.  16-byte pieces are
//    XOR-swizzled per row so that the 16 rows an MFMA operand read touches
//    fall on distinct banks.
//  * Tiles are dealt so that each XCD (workgroups go round-robin over 8)
//    works through a contiguous run of tiles, ordered in groups of 8 token
//    tiles that sweep the feature tiles: the 64 workgroups an XCD holds at
//    once cover 8 x 8 tiles, so each X or W slice they read is fetched into
//    the XCD's L2 once for 8 tiles (at the prompt sizes: 15.5x the
//    algorithmic bytes of L2 misses with token tiles of one feature tile
//    together, 5.5x with the groups).
//  * Epilogue: a lane holds one feature column and 16 token rows of each
//    32 x 32 tile; the destination row of every token of the tile (its q_out
//    row and its cache slot) is computed once per workgroup into LDS.
//  * Calls with enough tokens to give every CU a 256 x 256 tile (prompt
//    sizes) use those, 8 waves each, with half the L2 bytes per flop.
//  * Calls with too few tokens to give every CU a 128 x 128 tile (decode
//    steps) use tiles of 32 tokens x tn features, tn the widest multiple of 8
//    up to 32 that still gives every CU a tile (24 at 6144 features: 256
//    tiles instead of 192 of 32), with d_model split over eight waves.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kQkvThreads = 256;
constexpr int kSkinnyThreads = 512;  // decode-step kernel: 8 waves split d_model
constexpr int kSkinnyWaves = kSkinnyThreads / kWave;
constexpr int kTileM = 128;  // tokens per workgroup
constexpr int kTileN = 128;  // output features per workgroup
constexpr int kTileK = 64;   // d_model per step
constexpr int kRowBytes = kTileK * 2;
constexpr int kStageBytes = kTileM * kRowBytes;  // one operand's slice of a step
constexpr int kXcds = 8;
constexpr int kGroupM = 8;   // token tiles per group of the tile order

struct QkvKernelArgs {
    QkvArgs a;
    int32_t n_out;    // (Hq + 2 Hkv) * D
    int32_t m_tiles;  // token tiles
    int32_t tiles;    // token tiles * feature tiles
    int32_t per_xcd;  // tiles dealt to each XCD
    int32_t tn;       // few-token kernel: output features per tile (8..32)
};

// global_load_lds_dwordx4 with a scalar base: lane l's 16 bytes at
// base + voff land at LDS byte address lds + 16 l.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Slot of 16-byte piece p of LDS row r (8 pieces per 128-byte row; an
// involution).  Two rows share a 256-byte bank sweep, so rows 2j and 2j + 1
// get key j: an operand read (16 consecutive rows, one piece) hits 16
// distinct bank groups.
__device__ __forceinline__ int swz(int r, int p) { return p ^ ((r >> 1) & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Element offset of (block, KV head 0, slot) of packed token t in the
// pools, where kv_append would write it; -1 if t has no valid slot.
__device__ __forceinline__ int64_t token_dst(const QkvArgs& a, int t) {
    if (t >= a.total_new_tokens) return -1;
    int lo = 0, hi = a.num_seqs - 1;  // the sequence owning row t: last s with cu[s] <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_new_lens[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int64_t pos = (int64_t)a.ctx_lens[lo] + (t - a.cu_new_lens[lo]);
    const int64_t lb = pos / a.block_size;
    if (pos < 0 || lb >= a.max_blocks_per_seq) return -1;
    const int blk = a.block_table[(int64_t)lo * a.max_blocks_per_seq + lb];
    if (blk < 0 || blk >= a.num_blocks) return -1;
    return ((int64_t)blk * a.num_kv_heads * a.block_size + (pos & (a.block_size - 1))) * a.head_dim;
}

// Store a 32 x 32 tile of Y as bf16: this lane's column n, rows
// r0 + 8 j + 4 (lane / 32) + i of the workgroup's tokens (token m0 + row).
// q columns go to q_out; k / v columns to the token's cache slot (dst[row]).
__device__ __forceinline__ void store_tile(const QkvArgs& a, int n_out, const f32x16& acc, int m0, int r0, int n,
                                           const int64_t* dst) {
    if (n >= n_out) return;
    const int lane = threadIdx.x & 63;
    const int nq = a.num_q_heads * a.head_dim, nkv = a.num_kv_heads * a.head_dim;
    uint16_t* base = a.q_out;
    int64_t col = n;
    const bool to_cache = n >= nq;
    if (to_cache) {
        const int f = n < nq + nkv ? n - nq : n - nq - nkv;
        base = n < nq + nkv ? a.k_pool : a.v_pool;
        col = (int64_t)(f / a.head_dim) * a.block_size * a.head_dim + f % a.head_dim;  // head's slab + dim
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int r = r0 + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
        const int t = m0 + r;
        if (t >= a.total_new_tokens) continue;
        const uint16_t v = __builtin_bit_cast(uint16_t, (__bf16)acc[e]);
        if (!to_cache) {
            base[(int64_t)t * nq + col] = v;
        } else if (dst[r] >= 0) {
            base[dst[r] + col] = v;
        }
    }
}

__global__ __launch_bounds__(kQkvThreads) void qkv_append_kernel(QkvKernelArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t sX[2][kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][kStageBytes];
    __shared__ int64_t s_dst[kTileM];  // per token of the tile: element offset of (block, head 0, slot), or -1

    const QkvArgs& a = p.a;
    // tile of this workgroup: a contiguous run of tiles per XCD; within it,
    // groups of kGroupM token tiles sweep the feature tiles, token tiles
    // fastest, so the workgroups resident on an XCD at once cover about
    // kGroupM x kGroupM tiles and share their X and W slices in its L2
    const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int tile = xcd * p.per_xcd + j;
    if (j >= p.per_xcd || tile >= p.tiles) return;
    const int n_tiles = p.tiles / p.m_tiles;
    const int group = tile / (kGroupM * n_tiles), first_m = group * kGroupM;
    const int group_m = min(p.m_tiles - first_m, kGroupM);
    const int within = tile - group * kGroupM * n_tiles;
    const int m0 = (first_m + within % group_m) * kTileM;
    const int n0 = (within / group_m) * kTileN;
    const int T = a.total_new_tokens, K = a.d_model;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // destination rows of the tile's tokens (where kv_append would write them)
    if (threadIdx.x < kTileM) s_dst[threadIdx.x] = token_dst(a, m0 + threadIdx.x);

    // copy lanes: wave w moves rows [32 w, 32 w + 32) of both slices, 8 rows per load
    uint32_t xoff[4], woff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * wave + 8 * i + lane / 8;
        const int piece = swz(r, lane % 8);
        xoff[i] = (uint32_t)((int64_t)min(m0 + r, T - 1) * K * 2 + piece * 16);
        woff[i] = (uint32_t)((int64_t)min(n0 + r, p.n_out - 1) * K * 2 + piece * 16);
    }
    auto issue = [&](int step, int stage) {
        const uint16_t* xb = a.x + (int64_t)step * kTileK;
        const uint16_t* wb = a.w + (int64_t)step * kTileK;
        const uint32_t lx = lds_addr(sX[stage]) + (uint32_t)(32 * wave * kRowBytes);
        const uint32_t lw = lds_addr(sW[stage]) + (uint32_t)(32 * wave * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(xb, xoff[i], lx + i * 1024);
            dma16(wb, woff[i], lw + i * 1024);
        }
    };

    // operand reads: lane -> row (lane % 32) of a 32-row block, piece 2 s + lane / 32 of step s
    const int wm = wave & 1, wn = wave >> 1;
    int aoff[2][4], boff[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ra = 64 * wm + 32 * t + (lane & 31), rb = 64 * wn + 32 * t + (lane & 31);
            aoff[t][s] = ra * kRowBytes + swz(ra, 2 * s + (lane >> 5)) * 16;
            boff[t][s] = rb * kRowBytes + swz(rb, 2 * s + (lane >> 5)) * 16;
        }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.f;

    const int steps = K / kTileK;
    issue(0, 0);
    for (int st = 0; st < steps; ++st) {
        const int cur = st & 1;
        wait_vm_all();     // this wave's copies of step st have landed
        __syncthreads();   // everyone's have, and nobody still reads the other stage
        if (st + 1 < steps) issue(st + 1, cur ^ 1);
        const uint8_t* xs = sX[cur];
        const uint8_t* ws = sW[cur];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 af[2], bfr[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[t] = *reinterpret_cast<const u32x4*>(xs + aoff[t][s]);
                bfr[t] = *reinterpret_cast<const u32x4*>(ws + boff[t][s]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[i]), as_bf16x8(bfr[jj]),
                                                                         acc[i][jj], 0, 0, 0);
        }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
            store_tile(a, p.n_out, acc[i][jj], m0, 64 * wm + 32 * i, n0 + 64 * wn + 32 * jj + (lane & 31), s_dst);
}

// Many tokens (prompt sizes): 256 x 256 tiles, 8 waves, one workgroup per CU.
// A 128 x 128 tile reads 32 KB from L2 per 64-deep step for 2 MFLOP, which
// at the matrix cores' full rate is as much as an XCD's L2 delivers to its
// CUs; a 256 x 256 tile reads 64 KB for 8 MFLOP, half the bytes per flop,
// and its step lasts twice as long, giving the next step's copies twice the
// time to land.  Wave w computes rows [128 (w % 2), +128) x columns
// [64 (w / 2), +64) of the tile as 4 x 2 MFMA tiles (6 LDS reads per 8
// MFMAs); wave w copies rows [32 w, 32 w + 32) of both slices.
//  * The fragments of substep s + 1 are read while substep s is multiplied,
//    one read after each of its first six MFMAs (fixed with scheduling-group
//    barriers), the W fragments first, so the first MFMAs of s + 1 wait for
//    reads issued five MFMAs earlier rather than for the last one issued.
//  * Epilogue through LDS: the tile is staged as bf16 rows in the (then
//    free) stage memory and leaves in 16-byte pieces, 32 lanes to a
//    512-byte row, instead of as 2-byte stores straight from the MFMA
//    layout.  A piece never straddles a head (D is a multiple of 8), so each
//    has one destination: its q_out row or its token's cache slot.
constexpr int kBigThreads = 512;
constexpr int kBigM = 256;
constexpr int kBigN = 256;
constexpr int kBigStageBytes = kBigM * kRowBytes;
constexpr int kBigGroupM = 4;  // token tiles per group: an XCD's 32 workgroups cover 4 x 8 tiles
constexpr int kOutPitch = kBigN + 8;  // bf16 per staged output row: +16 bytes puts rows 4 apart on other banks
constexpr int kBigLds = 4 * kBigStageBytes > kBigM * kOutPitch * 2 ? 4 * kBigStageBytes : kBigM * kOutPitch * 2;

__global__ __launch_bounds__(kBigThreads) void qkv_append_big_kernel(QkvKernelArgs p) {
    // two stages of the X and W slices; after the K loop, the staged output
    __shared__ __attribute__((aligned(16))) uint8_t sm[kBigLds];
    __shared__ int64_t s_dst[kBigM];
    uint8_t(*sX)[kBigStageBytes] = reinterpret_cast<uint8_t(*)[kBigStageBytes]>(sm);
    uint8_t(*sW)[kBigStageBytes] = reinterpret_cast<uint8_t(*)[kBigStageBytes]>(sm + 2 * kBigStageBytes);

    const QkvArgs& a = p.a;
    const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int tile = xcd * p.per_xcd + j;
    if (j >= p.per_xcd || tile >= p.tiles) return;
    const int n_tiles = p.tiles / p.m_tiles;
    const int group = tile / (kBigGroupM * n_tiles), first_m = group * kBigGroupM;
    const int group_m = min(p.m_tiles - first_m, kBigGroupM);
    const int within = tile - group * kBigGroupM * n_tiles;
    const int m0 = (first_m + within % group_m) * kBigM;
    const int n0 = (within / group_m) * kBigN;
    const int T = a.total_new_tokens, K = a.d_model;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    if (threadIdx.x < kBigM) s_dst[threadIdx.x] = token_dst(a, m0 + threadIdx.x);

    uint32_t xoff[4], woff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * wave + 8 * i + lane / 8;
        const int piece = swz(r, lane % 8);
        xoff[i] = (uint32_t)((int64_t)min(m0 + r, T - 1) * K * 2 + piece * 16);
        woff[i] = (uint32_t)((int64_t)min(n0 + r, p.n_out - 1) * K * 2 + piece * 16);
    }
    auto issue = [&](int step, int stage) {
        const uint16_t* xb = a.x + (int64_t)step * kTileK;
        const uint16_t* wb = a.w + (int64_t)step * kTileK;
        const uint32_t lx = lds_addr(sX[stage]) + (uint32_t)(32 * wave * kRowBytes);
        const uint32_t lw = lds_addr(sW[stage]) + (uint32_t)(32 * wave * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(xb, xoff[i], lx + i * 1024);
            dma16(wb, woff[i], lw + i * 1024);
        }
    };

    // operand reads: lane -> row (lane % 32) of a 32-row block, piece
    // 2 s + lane / 32 of substep s; the swizzle key depends on the row
    // modulo 16 only, so one offset per substep serves every 32-row block
    const int wm = wave & 1, wn = wave >> 1;
    int aoff[4], boff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int ra = 128 * wm + (lane & 31), rb = 64 * wn + (lane & 31);
        aoff[s] = ra * kRowBytes + swz(ra, 2 * s + (lane >> 5)) * 16;
        boff[s] = rb * kRowBytes + swz(rb, 2 * s + (lane >> 5)) * 16;
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.f;

    const int steps = K / kTileK;
    issue(0, 0);
    for (int st = 0; st < steps; ++st) {
        const int cur = st & 1;
        wait_vm_all();
        __syncthreads();
        if (st + 1 < steps) issue(st + 1, cur ^ 1);
        const uint8_t* xs = sX[cur];
        const uint8_t* ws = sW[cur];
        u32x4 af[2][4], bfr[2][2];  // fragments of substeps s (s % 2) and s + 1
        auto read = [&](int s) {
#pragma unroll
            for (int t = 0; t < 2; ++t) bfr[s & 1][t] = *reinterpret_cast<const u32x4*>(ws + boff[s] + t * 32 * kRowBytes);
#pragma unroll
            for (int t = 0; t < 4; ++t) af[s & 1][t] = *reinterpret_cast<const u32x4*>(xs + aoff[s] + t * 32 * kRowBytes);
        };
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s == 0) read(0);
            if (s + 1 < 4) read(s + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[s & 1][i]),
                                                                         as_bf16x8(bfr[s & 1][jj]), acc[i][jj], 0, 0, 0);
            if (s == 0) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // substep 0's own reads first
            if (s + 1 < 4) {
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read of substep s + 1
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
        }
    }

    __syncthreads();  // every wave is done with the stages
    uint16_t* so = reinterpret_cast<uint16_t*>(sm);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = 64 * wn + 32 * jj + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 128 * wm + 32 * i + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
                so[r * kOutPitch + c] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][jj][e]);
            }
        }
    __syncthreads();
    const int nq = a.num_q_heads * a.head_dim, nkv = a.num_kv_heads * a.head_dim;
#pragma unroll 4
    for (int it = 0; it < kBigM * (kBigN / 8) / kBigThreads; ++it) {
        const int q = it * kBigThreads + threadIdx.x;
        const int r = q / (kBigN / 8), n = n0 + 8 * (q % (kBigN / 8));  // row and first feature of the piece
        const int t = m0 + r;
        if (t >= T || n >= p.n_out) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(so + r * kOutPitch + (n - n0));
        if (n < nq) {
            store16(a.q_out + (int64_t)t * nq + n, v);
        } else if (s_dst[r] >= 0) {
            const int f = n < nq + nkv ? n - nq : n - nq - nkv;
            uint16_t* base = n < nq + nkv ? a.k_pool : a.v_pool;
            store16(base + s_dst[r] + (int64_t)(f / a.head_dim) * a.block_size * a.head_dim + f % a.head_dim, v);
        }
    }
}

// Few tokens (a decode step): the weight stream dominates and 128 x 128 tiles
// would leave most CUs idle, so a workgroup takes a 32 x tn tile (computed as
// 32 x 32, the columns past tn masked) and its
// eight waves split d_model (wave w: 64-wide steps w, w + 8, ..., three in
// flight), reducing through LDS at the end.  Operands come straight from
// global memory: lane (row i, half h) loads 64 contiguous bytes of its X row
// and of its W row per step
// (d_model k0 + 32 h .. k0 + 32 h + 31), and MFMA s of the step contracts
// bytes [16 s, 16 s + 16) of each -- the same order of d_model on both sides.
__global__ __launch_bounds__(kSkinnyThreads) void qkv_append_skinny_kernel(QkvKernelArgs p) {
    __shared__ float s_red[kSkinnyWaves - 1][16][kWave];
    __shared__ int64_t s_dst[32];

    const QkvArgs& a = p.a;
    const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int tile = xcd * p.per_xcd + j;
    if (j >= p.per_xcd || tile >= p.tiles) return;
    const int m0 = (tile % p.m_tiles) * 32;
    const int n0 = (tile / p.m_tiles) * p.tn;
    const int T = a.total_new_tokens, K = a.d_model;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (threadIdx.x < 32) s_dst[threadIdx.x] = token_dst(a, m0 + threadIdx.x);

    // columns past the tile's tn features repeat its last row (the same
    // cache lines) and are not stored
    const int h = lane >> 5, col = lane & 31;
    const uint16_t* xr = a.x + (int64_t)min(m0 + col, T - 1) * K + 32 * h;
    const uint16_t* wr = a.w + (int64_t)min(n0 + min(col, p.tn - 1), p.n_out - 1) * K + 32 * h;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    // this wave's steps w, w + 4, ..., three in flight (a ring of three
    // register sets); loads past the last step repeat it and are not used
    const int steps = K / 64;
    const int nsw = steps > wave ? (steps - wave + kSkinnyWaves - 1) / kSkinnyWaves : 0;
    u32x4 x0[4], w0[4], x1[4], w1[4], x2[4], w2[4];
    auto load = [&](u32x4* xv, u32x4* wv, int i) {
        const int64_t k = (int64_t)(wave + kSkinnyWaves * min(i, nsw - 1)) * 64;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            xv[c] = load16(xr + k + 8 * c);
            wv[c] = load16(wr + k + 8 * c);
        }
    };
    auto mma = [&](const u32x4* xv, const u32x4* wv) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xv[c]), as_bf16x8(wv[c]), acc, 0, 0, 0);
    };
    if (nsw > 0) {
        load(x0, w0, 0);
        load(x1, w1, 1);
        load(x2, w2, 2);
        for (int i = 0; i < nsw; i += 3) {
            mma(x0, w0);
            if (i + 3 < nsw) load(x0, w0, i + 3);
            if (i + 1 < nsw) {
                mma(x1, w1);
                if (i + 4 < nsw) load(x1, w1, i + 4);
            }
            if (i + 2 < nsw) {
                mma(x2, w2);
                if (i + 5 < nsw) load(x2, w2, i + 5);
            }
        }
    }
    if (wave > 0)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_red[wave - 1][e][lane] = acc[e];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += s_red[w][e][lane];
    store_tile(a, p.n_out, acc, m0, 0, col < p.tn ? n0 + col : p.n_out, s_dst);
}

}  // namespace

hipError_t launch_qkv_append(const QkvArgs& a, hipStream_t stream) {
    if (a.total_new_tokens == 0) return hipSuccess;
    QkvKernelArgs kp;
    kp.a = a;
    kp.n_out = (a.num_q_heads + 2 * a.num_kv_heads) * a.head_dim;
    kp.m_tiles = (a.total_new_tokens + kTileM - 1) / kTileM;
    kp.tiles = kp.m_tiles * ((kp.n_out + kTileN - 1) / kTileN);
    if (kp.tiles < device_cu_count()) {  // too few 128 x 128 tiles to fill the chip: 32 x 32 tiles
        // the widest tiles (a multiple of 8 features, at most 32) that still
        // give every CU one
        kp.m_tiles = (a.total_new_tokens + 31) / 32;
        kp.tn = 32;
        while (kp.tn > 8 && (int64_t)kp.m_tiles * ((kp.n_out + kp.tn - 1) / kp.tn) < device_cu_count()) kp.tn -= 8;
        kp.tiles = kp.m_tiles * ((kp.n_out + kp.tn - 1) / kp.tn);
        kp.per_xcd = (kp.tiles + kXcds - 1) / kXcds;
        hipLaunchKernelGGL(qkv_append_skinny_kernel, dim3((unsigned)(kp.per_xcd * kXcds)), dim3(kSkinnyThreads), 0,
                           stream, kp);
        return hipGetLastError();
    }
    const int big_m = (a.total_new_tokens + kBigM - 1) / kBigM;
    const int big_tiles = big_m * (int)((kp.n_out + kBigN - 1) / kBigN);
    if (big_tiles >= device_cu_count()) {  // enough 256 x 256 tiles to give every CU one
        kp.m_tiles = big_m;
        kp.tiles = big_tiles;
        kp.tn = kBigN;
        kp.per_xcd = (kp.tiles + kXcds - 1) / kXcds;
        hipLaunchKernelGGL(qkv_append_big_kernel, dim3((unsigned)(kp.per_xcd * kXcds)), dim3(kBigThreads), 0, stream,
                           kp);
        return hipGetLastError();
    }
    kp.tn = kTileN;
    kp.per_xcd = (kp.tiles + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(qkv_append_kernel, dim3((unsigned)(kp.per_xcd * kXcds)), dim3(kQkvThreads), 0, stream, kp);
    return hipGetLastError();
}

}  // namespace pkv
