"""Fused QKV projection + paged append on the GPU vs the CPU oracle (needs an
MI355X).

The oracle sums each output exactly (fp64) and rounds once to bf16; the
kernel accumulates in fp32 on the matrix cores and rounds its sum to bf16.
With e = d_model * 2^-24 * sum_k |x_k| |w_k| bounding the fp32 accumulation
error of an output, the two can differ by at most one bf16 step (of the
larger value) plus e, which is the bar here, element by element, on q and on
every k / v row written.  Slots no token maps to must keep their sentinel
(bit for bit).  The share of outputs equal to the oracle's bit for bit is
printed.
"""
import numpy as np
import pytest
import torch

import oracle
from case_oracle import bf16_ulp
from paged_kv_gqa_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _say(msg):
    print(msg, flush=True)


def _bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _inputs(rng, T, dm, n_out):
    x = W.bf16_normal(rng, (T, dm))
    w = W.bf16_normal(rng, (n_out, dm))
    # scale the weight by a power of two (exact) so that outputs are about N(0, 1)
    scale = 2.0 ** -round(np.log2(np.sqrt(dm)))
    w = torch.from_numpy(_f64(w).astype(np.float32) * np.float32(scale)).to(torch.bfloat16)
    return x, w.view(torch.int16).numpy().view(np.uint16)


def _run(x, w, hq, hkv, d, bs, nb, cu, ctx, table):
    import paged_kv_gqa_scatter_amd as pkv
    shape = (nb, hkv, bs, d)
    kp = torch.full(shape, W.NAN_SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vp = torch.full(shape, W.NAN_SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    q = pkv.qkv_project_append(_bits(x), _bits(w), kp, vp, torch.from_numpy(cu).cuda(), torch.from_numpy(ctx).cuda(),
                               torch.from_numpy(table).cuda(), hq)
    torch.cuda.synchronize()
    return _np(q), _np(kp), _np(vp)


def _check_values(gpu_bits, ref_bits, x_rows, w, what):
    """gpu vs oracle within one bf16 step plus the fp32 accumulation bound.
    x_rows [R][dm] are the inputs of the compared rows, gpu/ref [R][n] the
    outputs over w's rows [n][dm] (n = all output features or a slice)."""
    g, r = _f64(gpu_bits), _f64(ref_bits)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    e = x_rows.shape[1] * 2.0 ** -24 * (np.abs(_f64(x_rows)) @ np.abs(_f64(w)).T)
    tol = bf16_ulp(np.maximum(np.abs(g), np.abs(r))) + e
    bad = np.abs(g - r) > tol
    same = float(np.mean(gpu_bits == ref_bits))
    _say(f"  {what}: max|diff| {np.abs(g - r).max():.3e}, {same * 100:.2f}% bit-identical, {g.size} values")
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs off by more than one bf16 step + the fp32 bound"


def _compare(orc, x, w, hq, hkv, d, bs, nb, cu, ctx, table, tokens, what):
    """Run the GPU op on all tokens and the oracle on `tokens` (each as a
    one-token sequence at its own position), then compare q rows and the
    cache slots of those tokens; every slot no token maps to keeps the
    sentinel."""
    T = int(cu[-1])
    gq, gk, gv = _run(x, w, hq, hkv, d, bs, nb, cu, ctx, table)
    owner = np.searchsorted(cu, np.arange(T), side="right") - 1
    pos = ctx[owner] + (np.arange(T) - cu[owner])
    tok = np.asarray(tokens)
    kp = np.full(gk.shape, W.NAN_SENTINEL, np.uint16)
    vp = kp.copy()
    sub_table = np.ascontiguousarray(table[owner[tok]])
    rq = orc.qkv_project_append(kp, vp, np.ascontiguousarray(x[tok]), w, np.arange(tok.size + 1, dtype=np.int32),
                                pos[tok].astype(np.int32), sub_table, hq)
    _check_values(gq[tok].reshape(tok.size, -1), rq.reshape(tok.size, -1), x[tok], w[:hq * d], f"{what}: q")
    blk = table[owner[tok], pos[tok] // bs]
    slot = pos[tok] % bs
    nq, nkv = hq * d, hkv * d
    _check_values(gk[blk, :, slot, :].reshape(tok.size, -1), kp[blk, :, slot, :].reshape(tok.size, -1), x[tok],
                  w[nq:nq + nkv], f"{what}: k rows")
    _check_values(gv[blk, :, slot, :].reshape(tok.size, -1), vp[blk, :, slot, :].reshape(tok.size, -1), x[tok],
                  w[nq + nkv:], f"{what}: v rows")
    written = np.zeros((nb, bs), bool)
    written[table[owner, pos // bs], pos % bs] = True
    gk_s, gv_s = gk.transpose(0, 2, 1, 3), gv.transpose(0, 2, 1, 3)  # [block][slot][head][dim]
    assert (gk_s[~written] == W.NAN_SENTINEL).all() and (gv_s[~written] == W.NAN_SENTINEL).all(), "stray writes"
    assert (gk_s[written] != W.NAN_SENTINEL).all() and (gv_s[written] != W.NAN_SENTINEL).all(), "missing writes"


def _placement(rng, ctx_lens, new_lens, bs, spare=3):
    S = len(ctx_lens)
    ends = [c + n for c, n in zip(ctx_lens, new_lens)]
    nblk = [-(-e // bs) for e in ends]
    nb = sum(nblk) + spare
    perm = rng.permutation(nb).astype(np.int32)
    table = np.full((S, max(nblk)), -1, np.int32)
    o = 0
    for s in range(S):
        table[s, :nblk[s]] = perm[o:o + nblk[s]]
        o += nblk[s]
    cu = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int32)
    return table, cu, np.asarray(ctx_lens, np.int32), nb


@pytest.mark.parametrize("hq,hkv,d,bs,dm", [(4, 1, 64, 16, 256), (8, 2, 128, 32, 192), (2, 2, 64, 256, 64)])
def test_qkv_small_every_token(orc, hq, hkv, d, bs, dm):
    # ragged sequences starting mid-block, several token and feature tiles
    # with ragged tails (n_out 384 / 1536 / 384, T = 300)
    rng = np.random.default_rng(300 + hq + d + bs)
    table, cu, ctx, nb = _placement(rng, [5, 0, 17, 40], [130, 1, 120, 49], bs)
    n_out = (hq + 2 * hkv) * d
    x, w = _inputs(rng, int(cu[-1]), dm, n_out)
    _say(f"case qkv hq{hq} hkv{hkv} d{d} b{bs} dm{dm}: T {int(cu[-1])}, n_out {n_out}")
    _compare(orc, x, w, hq, hkv, d, bs, nb, cu, ctx, table, np.arange(int(cu[-1])), "every token")


def test_qkv_qwen3_decode_step(orc):
    # the decode step of the Qwen3-8B layer: 8 new tokens, d_model 4096,
    # 32 / 8 heads of 128, blocks of 256
    case = W.config2_decode()
    a = case.steps[0].append
    rng = np.random.default_rng(31)
    x, w = _inputs(rng, 8, 4096, (32 + 16) * 128)
    _say("case qkv qwen3-8b decode step: 8 tokens")
    _compare(orc, x, w, 32, 8, 128, 256, case.num_blocks, a.cu_new_lens, a.ctx_lens, a.block_table, np.arange(8),
             "8 tokens")


@pytest.mark.timeout(600)
def test_qkv_qwen3_prefill_sampled(orc):
    # the prompts of the Qwen3-8B prefill workload (4 x U[1024, 4096] tokens)
    # through the projection; the oracle checks sampled tokens, including
    # every sequence's first and last and the 128-token tile edges
    case = W.config3_prefill()
    a = case.steps[0].append
    T = int(a.cu_new_lens[-1])
    rng = np.random.default_rng(33)
    x, w = _inputs(rng, T, 4096, (32 + 16) * 128)
    cu = a.cu_new_lens
    pick = set(rng.choice(T, 24, replace=False).tolist()) | set(cu[:-1].tolist()) | set((cu[1:] - 1).tolist())
    pick |= {127, 128, 255, 256, 511, 512, T - 257, T - 256, T - 1}
    last = (T - 1) // 256 * 256  # first token of the last (ragged) 256-token tile
    pick |= {last - 1, last, last + 1}
    pick |= set(range(last + 64, last + 96))  # a whole 32-row block of an MFMA tile in the last tile
    _say(f"case qkv qwen3-8b prefill prompts: T {T}, {len(pick)} tokens sampled")
    _compare(orc, x, w, 32, 8, 128, 256, case.num_blocks, cu, a.ctx_lens, a.block_table, sorted(pick), "sampled")


def test_qkv_wide_tiles_ragged_tails(orc):
    # enough tokens for the 128 x 128 tile path (129 x 5 = 645 tiles), with a
    # ragged token tail (16400 = 128 * 128 + 16) and a ragged feature tail
    # (n_out 576 = 4.5 x 128)
    rng = np.random.default_rng(41)
    hq, hkv, d, bs, dm = 3, 3, 64, 16, 128
    table, cu, ctx, nb = _placement(rng, [3, 0, 9], [8000, 8000, 400], bs)
    x, w = _inputs(rng, int(cu[-1]), dm, (hq + 2 * hkv) * d)
    T = int(cu[-1])
    pick = set(rng.choice(T, 40, replace=False).tolist()) | {0, 127, 128, 255, 256, 511, 512, 7999, 8000, 16383,
                                                               16384, T - 1}
    _say(f"case qkv wide tiles: T {T}, n_out {(hq + 2 * hkv) * d}, {len(pick)} tokens sampled")
    _compare(orc, x, w, hq, hkv, d, bs, nb, cu, ctx, table, sorted(pick), "wide, ragged tails")


def test_qkv_big_tiles_ragged_tails(orc):
    # enough tokens for the 256 x 256 tile path (86 x 3 = 258 tiles), with a
    # ragged token tail (22000 = 85 * 256 + 240), a ragged feature tail
    # (n_out 576 = 2.25 x 256) and a d_model of three 64-deep steps
    rng = np.random.default_rng(43)
    hq, hkv, d, bs, dm = 3, 3, 64, 16, 192
    table, cu, ctx, nb = _placement(rng, [5, 0, 250], [9000, 12000, 1000], bs)
    x, w = _inputs(rng, int(cu[-1]), dm, (hq + 2 * hkv) * d)
    T = int(cu[-1])
    pick = set(rng.choice(T, 60, replace=False).tolist()) | {0, 1, 255, 256, 511, 512, 8999, 9000, 20999, 21000,
                                                               T - 241, T - 240, T - 239, T - 2, T - 1}
    pick |= set(range(21760, 21760 + 32))  # a whole 32-row block of the ragged last tile
    _say(f"case qkv big tiles: T {T}, n_out {(hq + 2 * hkv) * d}, dm {dm}, {len(pick)} tokens sampled")
    _compare(orc, x, w, hq, hkv, d, bs, nb, cu, ctx, table, sorted(pick), "big, ragged tails")


@pytest.mark.parametrize("dm", [256, 192])
def test_qkv_few_tokens(orc, dm):
    # 13 tokens over 3 sequences (a ragged token tile of the few-token path),
    # d_model a multiple of 128 or not
    rng = np.random.default_rng(50 + dm)
    hq, hkv, d, bs = 4, 2, 64, 32
    table, cu, ctx, nb = _placement(rng, [31, 0, 64], [2, 10, 1], bs)
    x, w = _inputs(rng, int(cu[-1]), dm, (hq + 2 * hkv) * d)
    _say(f"case qkv few tokens: T {int(cu[-1])}, dm {dm}")
    _compare(orc, x, w, hq, hkv, d, bs, nb, cu, ctx, table, np.arange(int(cu[-1])), "few tokens")


def test_qkv_few_tokens_narrow_ragged_tiles(orc):
    # 8 tokens and 6400 features (80 + 2 x 10 heads of 64): 32-feature tiles
    # would give 200 workgroups, so tiles of 24 features are used, the last
    # one holding 16
    rng = np.random.default_rng(61)
    hq, hkv, d, bs, dm = 80, 10, 64, 16, 256
    table, cu, ctx, nb = _placement(rng, [40, 7, 0], [3, 4, 1], bs)
    x, w = _inputs(rng, int(cu[-1]), dm, (hq + 2 * hkv) * d)
    _say(f"case qkv few tokens, narrow tiles: T {int(cu[-1])}, n_out {(hq + 2 * hkv) * d}")
    _compare(orc, x, w, hq, hkv, d, bs, nb, cu, ctx, table, np.arange(int(cu[-1])), "narrow ragged tiles")
