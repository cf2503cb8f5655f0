// paged_gqa_decode: one query row per sequence over a paged KV cache, with the
// query heads of a GQA group sharing every K/V row they read.
//
// "扔掉 vLLM！从零构建 Qwen3-8B 推理引擎" section 4.4.2 reads a KV head once and
// uses it for all heads_per_group query heads of its group; that is the whole
// point here, because decode is bound by HBM bandwidth ("从零搭建AI工程能力"
// section 3.3).  The design on gfx950:
//
//  * Work items, grids and the merge of chunks are those of decode_common.h;
//    here a tile is 16 keys.
//  * Every wave streams its own tiles through a private ring of LDS stages
//    (4, or 2 when two workgroups share a CU): the K and V rows of a tile (16
//    rows of one contiguous (block, head) slab, as B >= 16) are copied by
//    global_load_lds_dwordx4, each wave load moving 1 KB of consecutive
//    bytes, and a stage is refilled as soon as its tile's LDS reads have
//    returned, so every stage is in flight while the wave waits.  The block
//    id is wave-uniform, so the slab address is scalar
//    arithmetic and every lane's offset is fixed for the item.  No barrier is
//    needed inside the loop: a wave only reads what it loaded itself.
//  * The G query heads of the group are the N side of the matrix cores,
//    padded to 16 columns: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K rows
//    from LDS, Q in registers, fp32 accumulate) leaves each lane the scores
//    of 4 keys for one head, which is already the operand layout of
//    O^T += V^T P^T (v_mfma_f32_16x16x16_bf16, keys as the contraction
//    index); V^T comes from LDS with ds_read_b64_tr_b16.  Counted per key,
//    the dot products on the vector ALUs alone cost more issue cycles than
//    HBM needs to deliver the row; on the matrix cores they are a few cycles.
//  * Online softmax in the exp2 domain (scale * log2 e folded in).  The
//    running max of a head moves only when a score outgrows it by more than
//    2^8 (checked per tile with one wave vote); the weights are rounded to
//    bf16 for the MFMA and the running sum adds exactly those values.  Rows
//    past the sequence end are masked to -inf, and their DMA reads a copy of
//    the last valid row, so no unwritten (NaN) slot reaches the MFMA.
//  * decode_append folds the step's kv_append into the same launch: the
//    workgroup of a sequence's last chunk writes the new K/V row (position
//    seq_len - 1) to the pools, and the wave that computes the tile holding
//    that position overwrites the row in its LDS stage with the new row once
//    the tile's copy has landed (and the rows past it, so that no unwritten
//    slot reaches the MFMA), so nothing waits for the store.
#include "decode_common.h"

namespace pkv {
namespace {

constexpr int kTileKeys = kDecodeTileKeys;  // keys per MFMA tile and per LDS stage of a wave
constexpr int kPlanCus = 256;        // compute units the split plan assumes (MI355X)
constexpr int kRoundTripTiles = 12;  // a load round trip, in tile compute times
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // the bf16 pair (1.0, 1.0)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ s16x4 as_s16x4(u32x2 v) { return __builtin_bit_cast(s16x4, v); }

// Transposing LDS read: within each 16-lane group, lane i receives element
// i % 4 of the 8 bytes addressed by lanes 4r + i / 4 (r = 0..3).
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
    s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, t);
}

// LDS slot of 16-byte piece `piece` of stage row `row` (an involution, so it
// also names the piece that lands in a slot).  The K reads (16 rows, one
// piece each) and the transposing V reads (4 rows, two adjacent pieces each)
// then never put two lanes of a group on one bank.
template <int D>
__device__ __forceinline__ int swz(int row, int piece) {
    return piece ^ ((((row & 3) << 1) | ((row >> 2) & 1)) & (D / 8 - 1));
}

// What a lane does with a 16-key tile, fixed for the whole item.
template <int D>
struct TileLanes {
    static constexpr int kPieces = D / 8;               // 16-byte pieces per row
    static constexpr int kRowsPerLoad = kWave / kPieces;
    static constexpr int kLoads = kTileKeys / kRowsPerLoad;  // wave loads per matrix and tile
    static constexpr int kDma = 2 * kLoads;                  // K and V
    int row[kLoads];     // DMA: row of the tile this lane's 16 bytes belong to
    int piece8[kLoads];  // DMA: element offset of the piece within the row
    int k_off[D / 32];   // QK: LDS element offset of this lane's K fragment, per 32 dims
    int v_off[D / 16];   // PV: LDS element offset of this lane's transposing read, per 16 dims
};

template <int D>
__device__ __forceinline__ TileLanes<D> tile_lanes(int lane) {
    using T = TileLanes<D>;
    TileLanes<D> tl;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        tl.row[i] = i * T::kRowsPerLoad + lane / T::kPieces;
        tl.piece8[i] = swz<D>(tl.row[i], lane % T::kPieces) * 8;
    }
    const int j = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) tl.k_off[c] = i16 * D + swz<D>(i16, c * 4 + j) * 8;
    const int vrow = 4 * j + (i16 >> 2), q = i16 & 3;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) tl.v_off[db] = vrow * D + swz<D>(vrow, 2 * db + (q >> 1)) * 8 + 4 * (q & 1);
    return tl;
}

// The four LDS stages of the block's waves (distinct objects, so the
// compiler never confuses the loads in flight into one with reads of another).
template <int D>
struct Stages {
    uint16_t* k[kStages];
    uint16_t* v[kStages];
};


// Copy tile rows [kt, kt + 16) of (block blk, KV head g) into a stage; rows at
// or past kend repeat row kend - 1.  kStream: load with the non-temporal hint.
template <int D, bool kStream>
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, int log2_block, int g, int blk, int kt, int kend,
                                           const TileLanes<D>& tl, uint32_t sk, uint32_t sv) {
    using T = TileLanes<D>;
    const int B = 1 << log2_block;
    const int64_t slab = ((int64_t)blk * a.num_kv_heads + g) * ((int64_t)B * D) + (int64_t)(kt & (B - 1)) * D;
    const uint16_t* kb = a.k_pool + slab;
    const uint16_t* vb = a.v_pool + slab;
    const int last = kend - 1 - kt;
    if (last >= kTileKeys - 1) {
#pragma unroll
        for (int i = 0; i < T::kLoads; ++i) {
            const uint32_t off = (uint32_t)(tl.row[i] * D + tl.piece8[i]) * 2u;
            dma16<kStream>(kb, off, sk + i * kWave * 16);
            dma16<kStream>(vb, off, sv + i * kWave * 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::kLoads; ++i) {
            const uint32_t off = (uint32_t)(min(tl.row[i], last) * D + tl.piece8[i]) * 2u;
            dma16<kStream>(kb, off, sk + i * kWave * 16);
            dma16<kStream>(vb, off, sv + i * kWave * 16);
        }
    }
}


// Per-wave view of the item.
template <int D>
struct WaveItem {
    const DecodeArgs* a;
    int log2_block, g, k0, kend, wave, lane, n_tiles;
    int ids0, ids1;  // block id of tile t in lane t % 64 of ids(t / 64)
    int L;           // keys of the sequence
    bool stream;     // not a shared pack: load the chunk's rows with the non-temporal hint
    bool append;     // decode_append: the new row (kn, vn: this lane's piece) is key L - 1
    u32x4 kn, vn;
    float c;         // scale * log2 e
    u32x4 qf[D / 32];
    TileLanes<D> tl;
    Stages<D> st;
};

template <int D>
__device__ __forceinline__ int tile_blk(const WaveItem<D>& w, int t) {
    const int v = t < kWave ? w.ids0 : w.ids1;
    return __builtin_amdgcn_readlane(v, t & (kWave - 1));
}

template <int D>
__device__ __forceinline__ int tile_key(const WaveItem<D>& w, int t) {
    return w.k0 + kTileKeys * (w.wave + kDecodeWaves * t);
}

template <int D>
__device__ __forceinline__ void issue(const WaveItem<D>& w, int t, int stage) {
    const int blk = tile_blk(w, t);
    const int b = (unsigned)blk < (unsigned)w.a->num_blocks ? blk : 0;  // a bad id reads block 0, masked below
    const uint32_t wave_bytes = (uint32_t)(w.wave * kTileKeys * D * 2);
    const uint32_t sk = lds_addr(w.st.k[stage]) + wave_bytes, sv = lds_addr(w.st.v[stage]) + wave_bytes;
    if (w.stream)
        issue_tile<D, true>(*w.a, w.log2_block, w.g, b, tile_key(w, t), w.kend, w.tl, sk, sv);
    else
        issue_tile<D, false>(*w.a, w.log2_block, w.g, b, tile_key(w, t), w.kend, w.tl, sk, sv);
}

// decode_append, on the tile holding key L - 1 (row r0 of the tile): the new
// K/V row replaces rows r0.. of the wave's stage (its copy may predate the
// store, or be a clamped copy of that row), and goes to the pools.
template <int D>
__device__ __forceinline__ void put_new_row(const WaveItem<D>& w, int t, int kS) {
    constexpr int kPieces = D / 8, kRowsPerLoad = kWave / kPieces;
    const int kt = tile_key(w, t);
    const int r0 = w.L - 1 - kt;
    uint16_t* sk = w.st.k[kS] + w.wave * kTileKeys * D;
    uint16_t* sv = w.st.v[kS] + w.wave * kTileKeys * D;
    const int piece = w.lane % kPieces;
#pragma unroll
    for (int j = 0; j < kTileKeys / kRowsPerLoad; ++j) {
        const int r = j * kRowsPerLoad + w.lane / kPieces;
        if (r >= r0) {
            store16(sk + r * D + swz<D>(r, piece) * 8, w.kn);
            store16(sv + r * D + swz<D>(r, piece) * 8, w.vn);
        }
    }
    const int blk = tile_blk(w, t);
    if ((unsigned)blk < (unsigned)w.a->num_blocks && w.lane < 2 * kPieces) {
        const int B = 1 << w.log2_block;
        const int64_t row = (((int64_t)blk * w.a->num_kv_heads + w.g) * B + ((w.L - 1) & (B - 1))) * D;
        if (w.lane < kPieces) store16(w.a->k_pool_w + row + piece * 8, w.kn);
        else store16(w.a->v_pool_w + row + piece * 8, w.vn);
    }
}

// Tile t from stage kS of a ring of R (all R stages in flight): wait for it,
// S^T, softmax, O^T, then refill its stage with tile t + R.
template <int D, int R, int kS>
__device__ __forceinline__ void tile_step(const WaveItem<D>& w, int t, WaveState<D>& ws) {
    constexpr int kDma = TileLanes<D>::kDma;
    static_assert(R == 2 || R == 4, "ring depth");
    const int after = min(R - 1, w.n_tiles - 1 - t);  // tiles issued after t
    if (after >= 3) wait_vmcnt<3 * kDma>();
    else if (after == 2) wait_vmcnt<2 * kDma>();
    else if (after == 1) wait_vmcnt<kDma>();
    else wait_vmcnt<0>();
    if (w.append && w.kend == w.L && tile_key(w, t) + kTileKeys >= w.kend) put_new_row<D>(w, t, kS);

    // every LDS read of the tile goes out before the first MFMA waits on one
    const uint16_t* sk = w.st.k[kS] + w.wave * kTileKeys * D;
    const uint16_t* sv = w.st.v[kS] + w.wave * kTileKeys * D;
    u32x4 kf[D / 32];
    u32x2 vf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) kf[c] = *reinterpret_cast<const u32x4*>(sk + w.tl.k_off[c]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) vf[db] = lds_read_tr(sv + w.tl.v_off[db]);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[c]), as_bf16x8(w.qf[c]), s, 0, 0, 0);

    // lane (j, h) holds the scores of keys kt + 4j + r (r = 0..3) for head h
    const int kt = tile_key(w, t);
    const bool ok_blk = (unsigned)tile_blk(w, t) < (unsigned)w.a->num_blocks;
    float z[4];
    if (ok_blk && kt + kTileKeys <= w.kend) {
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = s[r] * w.c;
    } else {
        const int key0 = kt + 4 * (w.lane >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = ok_blk && key0 + r < w.kend ? s[r] * w.c : -INFINITY;
    }
    const float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    if (__any(mx > ws.m + kRescaleSlack)) {
        float mh = fmaxf(mx, __shfl_xor(mx, 16, kWave));  // the head's max over the tile
        mh = fmaxf(mh, __shfl_xor(mh, 32, kWave));
        const float m_new = fmaxf(ws.m, mh);
        const float alpha = fast_exp2(ws.m - m_new);  // 0 while m is -inf
        ws.l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) ws.acc[db] *= alpha;
        ws.m = m_new;
    }
    // a head whose tile is all masked keeps m = -inf and gets zero weights
    const float mref = ws.m == -INFINITY ? 0.f : ws.m;
    const u32x2 pk = {pack_bf16x2(fast_exp2(z[0] - mref), fast_exp2(z[1] - mref)),
                      pack_bf16x2(fast_exp2(z[2] - mref), fast_exp2(z[3] - mref))};
    ws.l = dot2_bf16(pk[0], kOnesBf16x2, ws.l);
    ws.l = dot2_bf16(pk[1], kOnesBf16x2, ws.l);

#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        ws.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s16x4(vf[db]), as_s16x4(pk), ws.acc[db], 0, 0, 0);
    // the stage's reads have returned (the MFMAs hold them): refill it with tile t + R
    if (t + R < w.n_tiles) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
        issue(w, t + R, kS);
    }
}

template <int D, int R>
__device__ __forceinline__ void wave_tiles(const WaveItem<D>& w, WaveState<D>& ws) {
#pragma unroll
    for (int t = 0; t < R; ++t)
        if (t < w.n_tiles) issue(w, t, t);
    for (int t = 0; t < w.n_tiles; t += R) {
        tile_step<D, R, 0>(w, t, ws);
        if (t + 1 < w.n_tiles) tile_step<D, R, 1>(w, t + 1, ws);
        if constexpr (R == 4) {
            if (t + 2 < w.n_tiles) tile_step<D, R, 2>(w, t + 2, ws);
            if (t + 3 < w.n_tiles) tile_step<D, R, 3>(w, t + 3, ws);
        }
    }
}


// What a work item needs before its first K/V load, fetched in one round
// trip: the sequence length, this lane's query fragments and the block ids
// of this wave's tiles.
template <int D>
struct ItemInputs {
    int L_raw;
    int ids0, ids1;
    u32x4 qf[D / 32];
    u32x4 kn, vn;  // decode_append: this lane's piece of the new K/V row
    PackInputs pk;  // sequences sharing the chunk
};


template <int D, int G>
__device__ __forceinline__ ItemInputs<D> load_item_inputs(const DecodeKernelArgs& p, int s, int g, int c) {
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = wave_id();
    ItemInputs<D> in;
    in.L_raw = a.seq_lens[s];
    // Q^T fragment: column lane % 16, dims 32 c' + 8 (lane / 16) + [0, 8);
    // column h is head h of sequence s (zero past G), or, for the first
    // sequence of a run that may pack, head h % G of sequence s + h / G
    in.pk = load_pack_inputs<G>(p, s, c);
    const int h = lane & 15, j = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool lead = in.pk.on && s % pack_width<G>() == 0;
    const int qs = lead ? s + h / G : s;
    const bool qv = lead ? qs < a.num_seqs : h < G;
    const uint16_t* qp = a.q + ((int64_t)min(qs, a.num_seqs - 1) * a.num_q_heads + g * G + h % G) * D + 8 * j;
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) in.qf[cc] = qv ? load16(qp + 32 * cc) : zero;
    // block ids of tiles t = lane and lane + 64 (entries past the table row clamp to its end)
    const int32_t* table = a.block_table + (int64_t)s * a.max_blocks_per_seq;
    const int k0 = c * p.chunk;
    const int last = a.max_blocks_per_seq - 1;
    // (an empty table row, possible only when every sequence is empty, is not read)
    in.ids0 = last >= 0 ? table[min((k0 + kTileKeys * (wave + kDecodeWaves * lane)) >> p.log2_block, last)] : -1;
    in.ids1 = last >= 0 && p.chunk > kTileKeys * kDecodeWaves * kWave
                  ? table[min((k0 + kTileKeys * (wave + kDecodeWaves * (lane + kWave))) >> p.log2_block, last)]
                  : 0;
    in.kn = in.vn = zero;
    if (a.k_new) {
        const int64_t row = ((int64_t)s * a.num_kv_heads + g) * D + (lane % (D / 8)) * 8;
        in.kn = load16(a.k_new + row);
        in.vn = load16(a.v_new + row);
    }
    return in;
}


// One work item: chunk c of sequence s, KV head g; `slot` is its partial slot.
template <int D, int G, int R, typename Prefetch>
__device__ __forceinline__ void decode_item(const DecodeKernelArgs& p, DecodeShared<D, G>& sh, const Stages<D>& st,
                                            int s, int g, int c, int nchunks, int64_t slot,
                                            const ItemInputs<D>& in, Prefetch prefetch) {
    const DecodeArgs& a = p.a;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int Hq = a.num_q_heads;
    const int k0 = c * p.chunk;
    const int L = clamp_len(in.L_raw, a.max_blocks_per_seq << p.log2_block);
    const int k1 = min(k0 + p.chunk, L);
    const int tiles = (k1 - k0 + kTileKeys - 1) / kTileKeys;

    WaveItem<D> w;
    w.a = &a;
    w.log2_block = p.log2_block;
    w.g = g;
    w.k0 = k0;
    w.kend = k1;
    w.wave = wave;
    w.lane = lane;
    w.n_tiles = tiles > wave ? (tiles - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
    w.ids0 = in.ids0;
    w.ids1 = in.ids1;
    w.L = L;
    w.append = a.k_new != nullptr;
    w.kn = in.kn;
    w.vn = in.vn;
    w.c = p.qk_scale_log2;
    w.tl = tile_lanes<D>(lane);
    w.st = st;

    WaveState<D> ws;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) ws.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    ws.m = -INFINITY;
    ws.l = 0.f;
    wait_all_vm();  // the item's inputs (block ids, q, the pack's lengths and ids) are in
    // sequences sharing the chunk: a member's item exits (its run's first
    // item decodes it); the first item keeps the columns of its pack
    const int lead = s - s % pack_width<G>();
    const uint32_t pack = pack_of<G>(p, in.pk, c);
    // the next item's inputs go out before this item's tile copies: counted
    // in issue order, they retire with the first tile, so the next item
    // starts without a round trip of its own
    prefetch();
    if (s != lead && ((pack >> (s - lead)) & 1)) return;
    const bool packed = s == lead && pack != 0;
    w.stream = __builtin_amdgcn_readfirstlane(packed ? 0 : 1) != 0;  // a shared pack's rows are read by other packs
    const int h = lane & 15;
    const bool keep = h < G || (packed && ((pack >> (h / G)) & 1));
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) w.qf[cc] = keep ? in.qf[cc] : u32x4{0u, 0u, 0u, 0u};
    wave_tiles<D, R>(w, ws);

    if (packed)
        finish_pack<D, G>(p, reinterpret_cast<float*>(st.k[0]), reinterpret_cast<float*>(st.v[0]), ws, lead, g, c,
                          pack);
    else
        finish_item<D, G>(p, sh, ws, s, g, nchunks, slot);
}

// R: LDS ring depth per wave.  R = 4: 128 KB of stages at D = 128, one
// workgroup per CU; R = 2: 64 KB, two workgroups per CU, two waves per SIMD
// hiding each other's stalls, which pays when there is more work than one
// pass over the chip.
template <int D, int G, int R>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeKernelArgs p, int32_t* prefix_out) {
    __shared__ DecodeShared<D, G> sh;
    __shared__ __attribute__((aligned(16))) uint16_t sK[R][kDecodeWaves * kTileKeys * D];
    __shared__ __attribute__((aligned(16))) uint16_t sV[R][kDecodeWaves * kTileKeys * D];
    Stages<D> st;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        st.k[i] = sK[i];
        st.v[i] = sV[i];
    }

    run_items<D, G>(
        p, sh, prefix_out, [&](int s, int g, int c) { return load_item_inputs<D, G>(p, s, g, c); },
        [&](int s, int g, int c, int n, int64_t slot, const ItemInputs<D>& in, auto prefetch) {
            decode_item<D, G, R>(p, sh, st, s, g, c, n, slot, in, prefetch);
        });
}

}  // namespace

DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_seq_len, int64_t total_kv_tokens, int32_t tile_keys, int32_t wgs_per_cu,
                       int32_t max_chunk_keys) {
    DecodePlan pl{};
    const int64_t bound_tokens = (int64_t)num_seqs * max_seq_len;
    int64_t total = total_kv_tokens > 0 ? total_kv_tokens : bound_tokens;
    if (total > bound_tokens) total = bound_tokens;
    // chunk: the power of two in [16 tiles, 512 tiles] with the least
    // estimated time, counted in tile times (a tile of either cache format
    // moves about 8 KB per wave at D = 128): rounds of resident workgroups
    // (wgs_per_cu on each of a 256-CU part's CUs) times the round's length, a
    // load round trip (about 12 tiles) plus the tiles each wave streams.  The
    // item count is a bound (each sequence adds at most one partial chunk).
    // Finer steps (any multiple of one tile per wave, or 1.5x powers of two)
    // measured slower on multi-round launches (256 sequences on a shared
    // 4096-token prefix plus 16 of 32K tokens: a chunk that is not
    // a whole number of blocks also turns shared-chunk packing off).
    const int64_t slots = (int64_t)kPlanCus * wgs_per_cu;
    int max_chunk = kMaxTilesPerWave * tile_keys * kDecodeWaves;
    if (max_chunk_keys > 0 && max_chunk_keys < max_chunk) max_chunk = max_chunk_keys;
    int chunk = kDecodeWaves * 4 * tile_keys;
    int64_t best = -1;
    for (int c = chunk; c <= max_chunk; c *= 2) {
        const int64_t items = ((total + c - 1) / c + num_seqs) * num_kv_heads;
        const int64_t cost = (items + slots - 1) / slots * (kRoundTripTiles + c / (kDecodeWaves * tile_keys));
        if (best < 0 || cost < best) {
            best = cost;
            chunk = c;
        }
    }
    // a launch of one round: three quarters of that chunk, if the items
    // still fit the round, shorten its longest item (8 sequences of
    // 512..2048 keys, 8 KV heads: 512 -> 384 keys, 176 -> 216 items on 256
    // CUs; measured 15.0 -> 14.6 us)
    const int64_t items_at = ((total + chunk - 1) / chunk + num_seqs) * num_kv_heads;
    pl.last_first = items_at <= slots ? 1 : 0;
    if (items_at <= slots) {
        const int c34 = chunk / 4 * 3;
        if (c34 >= 4 * kDecodeWaves * tile_keys && ((total + c34 - 1) / c34 + num_seqs) * num_kv_heads <= slots)
            chunk = c34;
    }
    pl.ring = 4;
    pl.chunk = chunk;
    pl.items = ((total + chunk - 1) / chunk + num_seqs) * num_kv_heads;
    // at least one chunk: a launch whose sequences are all empty still runs
    // chunk 0 of each, which writes its zero rows
    pl.max_chunks = max_seq_len > 0 ? (max_seq_len + chunk - 1) / chunk : 1;
    const int64_t direct_items = (int64_t)num_seqs * pl.max_chunks;
    const int64_t real_items = (total + chunk - 1) / chunk + num_seqs;  // bound on chunks actually present
    // a direct grid when its empty workgroups are few (or the launch is small)
    pl.persistent = (num_seqs <= kMaxPersistentSeqs && direct_items > 2 * real_items &&
                     direct_items * num_kv_heads > 4096)
                        ? 1
                        : 0;
    pl.max_partials = pl.persistent ? (direct_items < real_items ? direct_items : real_items) : direct_items;
    pl.pack = pl.items > 2 * slots ? 1 : 0;
    pl.fused = can_fuse_merge(pl, num_seqs, num_kv_heads);
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    // the counters sit in a fixed region that no plan writes anything else
    // into, so a launch of any shape finds them as the last one left them
    pl.counter_offset = 0;
    pl.prefix_offset = kCounterBytes;
    pl.lse_offset = align(pl.prefix_offset + sizeof(int32_t) * (size_t)(num_seqs + 1));
    pl.o_offset = align(pl.lse_offset + sizeof(float) * (size_t)pl.max_partials * num_q_heads);
    pl.bytes = pl.o_offset + sizeof(float) * (size_t)pl.max_partials * num_q_heads * head_dim;
    return pl;
}

DecodePlan plan_decode_bf16(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_seq_len, int64_t total_kv_tokens) {
    // ring 4: one workgroup per CU at D = 128 (133..148 KB of LDS), two at
    // D = 64.  When the items outnumber one pass over the CUs, ring 2 at
    // D = 128 and G <= 4 (66..74 KB: two per CU) hides more stalls.
    DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, total_kv_tokens,
                                kTileKeys, head_dim == 64 ? 2 : 1);
    if (head_dim == 128 && num_q_heads <= 4 * num_kv_heads && pl.items > kPlanCus) {
        pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, total_kv_tokens, kTileKeys, 2);
        pl.ring = 2;
    }
    return pl;
}

namespace {

__global__ __launch_bounds__(256) void zero_counters_kernel(u32x4* p) {
    p[blockIdx.x * 256 + threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_workspace_reset(void* workspace, hipStream_t stream) {
    static_assert(kCounterBytes % (256 * 16) == 0, "whole workgroups of 16-byte stores");
    hipLaunchKernelGGL(zero_counters_kernel, dim3(kCounterBytes / (256 * 16)), dim3(256), 0, stream,
                       static_cast<u32x4*>(workspace));
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    DecodeKernelArgs kp;
    kp.a = a;
    kp.chunk = pl.chunk;
    kp.log2_block = ilog2(a.block_size);
    kp.max_chunks = pl.max_chunks;
    kp.persistent = pl.persistent;
    kp.pack = pl.pack;
    kp.last_first = pl.last_first;
    kp.max_partials = pl.max_partials;
    char* ws = static_cast<char*>(a.workspace);
    kp.counters = pl.fused ? reinterpret_cast<int32_t*>(ws + pl.counter_offset) : nullptr;
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + pl.prefix_offset);
    kp.lse = reinterpret_cast<float*>(ws + pl.lse_offset);
    kp.part = reinterpret_cast<float*>(ws + pl.o_offset);
    kp.qk_scale_log2 = a.scale * kLog2e;
    const int G = a.num_q_heads / a.num_kv_heads;
    if (a.head_dim == 128) {
        if (pl.ring == 2) {
            switch (G) {
                case 1: return launch_split<128, 1>(decode_kernel<128, 1, 2>, kp, prefix, stream);
                case 2: return launch_split<128, 2>(decode_kernel<128, 2, 2>, kp, prefix, stream);
                default: return launch_split<128, 4>(decode_kernel<128, 4, 2>, kp, prefix, stream);
            }
        }
        switch (G) {
            case 1: return launch_split<128, 1>(decode_kernel<128, 1, 4>, kp, prefix, stream);
            case 2: return launch_split<128, 2>(decode_kernel<128, 2, 4>, kp, prefix, stream);
            case 4: return launch_split<128, 4>(decode_kernel<128, 4, 4>, kp, prefix, stream);
            default: return launch_split<128, 8>(decode_kernel<128, 8, 4>, kp, prefix, stream);
        }
    }
    switch (G) {
        case 1: return launch_split<64, 1>(decode_kernel<64, 1, 4>, kp, prefix, stream);
        case 2: return launch_split<64, 2>(decode_kernel<64, 2, 4>, kp, prefix, stream);
        case 4: return launch_split<64, 4>(decode_kernel<64, 4, 4>, kp, prefix, stream);
        default: return launch_split<64, 8>(decode_kernel<64, 8, 4>, kp, prefix, stream);
    }
}

}  // namespace pkv
