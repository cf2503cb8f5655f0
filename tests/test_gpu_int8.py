"""INT8 KV cache on the GPU vs the CPU oracle (needs an MI355X).

kv_append_int8 must match the oracle's quantiser bit for bit over the whole
cache (codes and fp32 scales; unwritten slots keep their sentinels).  Decode
over the INT8 cache is compared with the oracle's decode over the same INT8
cache at the attention bar of the bf16 path (max|err| <= 1e-2, rel-L2 <=
1e-2; at |ref| >= 4 a bf16 neighbour of the exact value): both read identical
codes and scales, so the remaining difference is the kernel's own rounding --
fp32 scores and weights, the weight times the value scale carried as a bf16
pair (16 significant bits), fp32 accumulation and one bf16 rounding of the
output, which is where nearly all of the difference comes from.  The quantisation error itself is checked
separately: the oracle's INT8 decode must stay within the closed-form bound
of the oracle's bf16 decode of the unquantised rows.
"""
import numpy as np
import pytest
import torch

import oracle
from case_oracle import compare, oracle_int8, oracle_pools
from oracle_pins import int8_decode_bound
from paged_kv_gqa_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _dev():
    from paged_kv_gqa_scatter_amd.runner import Int8DeviceCase
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return Int8DeviceCase


def _say(msg):
    print(msg, flush=True)


def _assert_cache_equal(gpu, ref, what):
    gk, gv, gks, gvs = gpu
    rk, rv, rks, rvs = ref
    assert np.array_equal(gk, rk), f"{what}: K codes differ"
    assert np.array_equal(gv, rv), f"{what}: V codes differ"
    assert np.array_equal(gks.view(np.uint32), rks.view(np.uint32)), f"{what}: K scales differ"
    assert np.array_equal(gvs.view(np.uint32), rvs.view(np.uint32)), f"{what}: V scales differ"


def _decode_only(case):
    """The case with its prefill calls dropped (their rows are still appended)."""
    for st in case.steps:
        st.prefill = None
    return case


# ---------------------------------------------------------------- kv_append_int8

@pytest.mark.parametrize("cfg", [2, 4])
def test_int8_append_bitexact(orc, cfg):
    case = _decode_only(W.CONFIGS[cfg]())
    _say(f"case {case.name}: kv_append_int8 bit-exact over codes and scales")
    dc = _dev()(case)
    dc.run_fills()
    for st in dc.steps:
        dc.append(st["append"])
    torch.cuda.synchronize()
    _, ref = oracle_int8(case, orc, decode=False)
    got = dc.pools_numpy()
    _assert_cache_equal(got, ref, case.name)
    assert (got[0] == W.INT8_CODE_SENTINEL).any() and np.isnan(got[2]).any(), "spare slots keep the sentinels"


def test_int8_append_mid_block_small_values(orc):
    # chunks starting mid-block, D 64, block 32, and rows of tiny, huge and
    # all-zero values (subnormal and zero scales; ties at the row maximum)
    rng = np.random.default_rng(78)
    case = W.build_case("int8_append_mid_block", rng, hq=8, hkv=2, d=64, bs=32, ctx_lens=[5, 33, 0, 63],
                        new_lens=[40, 1, 32, 3], kinds="pppp")
    case.steps[0].prefill = None
    a = case.steps[0].append
    f = lambda x: torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a.k_new[0] = f(np.full((2, 64), 1e-38))        # subnormal scales
    a.k_new[1] = 0                                 # zero rows
    a.v_new[2] = f(np.linspace(-3e4, 3e4, 128).reshape(2, 64))
    a.k_new[3, 0, ::2] = f(np.full(32, -7.0))     # the maximum repeated, both signs
    a.k_new[3, 0, 1::2] = f(np.full(32, 7.0))
    _say(f"case {case.name}")
    dc = _dev()(case)
    dc.run_fills()
    dc.append(dc.steps[0]["append"])
    torch.cuda.synchronize()
    _, ref = oracle_int8(case, orc, decode=False)
    _assert_cache_equal(dc.pools_numpy(), ref, case.name)


# ---------------------------------------------------------------- decode_int8

def test_int8_decode_config2(orc):
    case = W.config2_decode()
    _say(f"case {case.name}: INT8 cache")
    out = _dev()(case).run_all()[0]["decode"]
    ref, _ = oracle_int8(case, orc)
    compare(out, ref[0], "INT8 decode 8 seqs")


def test_int8_decode_config4_lengths(orc):
    case = _decode_only(W.config4_mixed())
    _say(f"case {case.name}: INT8 cache, the 64 decode sequences")
    out = _dev()(case).run_all()[0]["decode"]
    ref, _ = oracle_int8(case, orc)
    compare(out, ref[0], "INT8 decode 64 seqs (128..8192 keys)")


@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 256, 32, 8), (64, 32, 4, 1), (128, 32, 16, 2), (64, 256, 8, 8)])
def test_int8_decode_edge_lengths(orc, d, bs, hq, hkv):
    # lengths at tile and block edges, a single key, an empty sequence, and
    # one long enough for many splits
    lens = [1, 31, 32, 33, bs - 1, bs, bs + 1, 2 * bs, 512, 8192, 32769, 0]
    rng = np.random.default_rng(2000 + d + bs)
    ctx = [max(L - 1, 0) for L in lens]
    new = [1 if L > 0 else 0 for L in lens]
    case = W.build_case(f"int8_decode_edges_d{d}_b{bs}", rng, hq=hq, hkv=hkv, d=d, bs=bs, ctx_lens=ctx[:-1],
                        new_lens=new[:-1], kinds="d" * (len(lens) - 1))
    dec = case.steps[0].decode
    dec.seq_lens = np.append(dec.seq_lens, 0).astype(np.int32)
    dec.block_table = np.vstack([dec.block_table, np.full((1, dec.block_table.shape[1]), -1, np.int32)])
    dec.q = np.concatenate([dec.q, W.bf16_normal(rng, (1, hq, d))])
    _say(f"case {case.name}: lens {lens}")
    out = _dev()(case).run_all()[0]["decode"]
    ref, _ = oracle_int8(case, orc)
    compare(out, ref[0], "INT8 decode edge lengths")
    assert np.array_equal(out[-1], np.zeros_like(out[-1])), "empty sequence must give zeros"


@pytest.mark.timeout(900)
def test_int8_decode_config5_full(orc):
    # all 272 sequences, every head, and the whole INT8 cache bit for bit
    case = W.config5_prefix_long()
    _say(f"case {case.name}: INT8 cache, every sequence")
    dc = _dev()(case)
    out = dc.run_all()[0]["decode"]
    got = dc.pools_numpy()
    del dc
    torch.cuda.empty_cache()
    _, pools = oracle_int8(case, orc, decode=False)
    _assert_cache_equal(got, pools, case.name)
    del got
    d = case.steps[0].decode
    ref = orc.decode_int8(d.q, *pools, d.block_table, d.seq_lens, case.scale)
    compare(out, ref, f"INT8 decode {d.seq_lens.shape[0]} sequences x all heads")


def test_int8_quantisation_error_within_bound(orc):
    # how far the INT8 step lies from the bf16 one, at the decode step's full
    # size: the oracle's INT8 decode against its bf16 decode of the same rows
    # (the closed-form bound of the oracle pins), and the GPU INT8 decode
    # against the same bf16 reference within that bound plus the parity bar
    case = W.config2_decode()
    _say(f"case {case.name}: INT8 vs bf16 within the quantisation bound")
    out = _dev()(case).run_all()[0]["decode"]
    ref8, pools8 = oracle_int8(case, orc)
    K, V = oracle_pools(case, orc)
    d = case.steps[0].decode
    exact = orc.decode(d.q, K, V, d.block_table, d.seq_lens, case.scale)
    bound = int8_decode_bound(d.q, d.seq_lens, d.block_table, (K, V), pools8, case.scale)
    err_oracle = np.abs(ref8[0] - exact).max(axis=2)
    err_gpu = np.abs(out - exact).max(axis=2)
    _say(f"  quantisation error: oracle max {err_oracle.max():.3e}, GPU max {err_gpu.max():.3e}, "
         f"bound max {bound.max():.3e}")
    assert (err_oracle <= bound + 1e-12).all()
    assert (err_gpu <= bound + 1e-2).all()


# ---------------------------------------------------------------- decode_append_int8

def _decode_append_int8_check(orc, case, k_new, v_new, q, seq_lens, table, what):
    """decode_append_int8 on a case's fills (the step's rows not yet
    appended): the cache (codes and scales, bit for bit) against the oracle's
    kv_append_int8 of the new rows, the outputs against the oracle's INT8
    decode."""
    import paged_kv_gqa_scatter_amd as pkv
    dc = _dev()(case)
    dc.run_fills()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    bits = lambda x: dev(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    S = seq_lens.shape[0]
    ws = torch.zeros(pkv.decode_int8_workspace_bytes(S, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                                     int(seq_lens.max())), dtype=torch.uint8, device="cuda")
    out = pkv.paged_gqa_decode_append_int8(bits(q), bits(k_new), bits(v_new), *dc.pools[0],
                                           dev(table.astype(np.int32)), dev(seq_lens.astype(np.int32)),
                                           float(case.scale), max_seq_len=int(seq_lens.max()), workspace=ws)
    torch.cuda.synchronize()
    _, pools = oracle_int8(case, orc, upto_step=0, decode=False)
    live = np.nonzero(seq_lens > 0)[0]
    orc.kv_append_int8(*pools, k_new[live], v_new[live], np.arange(live.size + 1, dtype=np.int32),
                       (seq_lens[live] - 1).astype(np.int32), np.ascontiguousarray(table[live]))
    _assert_cache_equal(dc.pools_numpy(), pools, what)
    ref = orc.decode_int8(q, *pools, table, seq_lens, case.scale)
    got = out.float().cpu().numpy().astype(np.float64)
    compare(got, ref, what)
    return got


def test_int8_decode_append_config2(orc):
    case = W.config2_decode()
    a, d = case.steps[0].append, case.steps[0].decode
    _say(f"case {case.name}: decode_append_int8")
    _decode_append_int8_check(orc, case, a.k_new, a.v_new, d.q, d.seq_lens, d.block_table, "INT8 decode_append 8 seqs")


@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 256, 32, 8), (64, 32, 4, 1), (128, 32, 16, 2)])
def test_int8_decode_append_edge_lengths(orc, d, bs, hq, hkv):
    # the new row is key 0, the last key of a tile or a block, the first of a
    # new one, deep in a long many-chunk sequence, or absent (seq_len 0)
    lens = [1, 31, 32, 33, bs - 1, bs, bs + 1, 2 * bs, 700, 32769, 0]
    rng = np.random.default_rng(4000 + d + bs)
    ctx = [max(L - 1, 0) for L in lens]
    case = W.build_case(f"int8_decode_append_edges_d{d}_b{bs}", rng, hq=hq, hkv=hkv, d=d, bs=bs, ctx_lens=ctx[:-1],
                        new_lens=[1] * (len(lens) - 1), kinds="d" * (len(lens) - 1))
    a, dec = case.steps[0].append, case.steps[0].decode
    pad = W.bf16_normal(rng, (1, hkv, d))
    k_new = np.concatenate([a.k_new, pad])
    v_new = np.concatenate([a.v_new, pad])
    q = np.concatenate([dec.q, W.bf16_normal(rng, (1, hq, d))])
    seq_lens = np.append(dec.seq_lens, 0).astype(np.int32)
    table = np.vstack([dec.block_table, np.full((1, dec.block_table.shape[1]), -1, np.int32)])
    _say(f"case {case.name}: lens {lens}")
    out = _decode_append_int8_check(orc, case, k_new, v_new, q, seq_lens, table, "INT8 decode_append edge lengths")
    assert np.array_equal(out[-1], np.zeros_like(out[-1])), "empty sequence must give zeros"


# ---------------------------------------------------------------- HIP graphs

def test_int8_graph_replays_match_eager(orc):
    # append_int8 + decode_int8 of a decode step in one HIP graph: every replay
    # (eager work and synchronisations between them) equals the eager step
    case = W.config2_decode()
    _say(f"case {case.name}: INT8 step, graph replays vs eager")
    dc = _dev()(case)
    dc.run_fills()
    st = dc.steps[0]
    want = dc.run_step(0)["decode"].clone()
    torch.cuda.synchronize()
    ref, _ = oracle_int8(case, orc)
    compare(want.float().cpu().numpy().astype(np.float64), ref[0], "eager INT8 step")
    g = dc.capture_step(0)
    for rep in range(4):
        st["decode"].out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st["decode"].out.view(torch.int16), want.view(torch.int16)), f"replay {rep} differs"
        dc.decode(st["decode"])
        torch.cuda.synchronize()
        assert torch.equal(st["decode"].out.view(torch.int16), want.view(torch.int16))
    _say("  4 replays bit-identical to the eager step")


@pytest.mark.timeout(600)
def test_int8_decode_persistent_grid_2048_sequences(orc):
    # the largest batch of the persistent grid, over the INT8 cache
    rng = np.random.default_rng(4096)
    lens = rng.integers(1, 300, size=2048, endpoint=True)
    lens[7] = 32768
    case = W.build_case("int8_decode_2048_seqs", rng, hq=32, hkv=8, d=128, bs=256, ctx_lens=lens - 1,
                        new_lens=np.ones(2048, np.int64), kinds="d" * 2048)
    _say(f"case {case.name}: 2048 sequences, one of 32768 keys, INT8 cache")
    out = _dev()(case).run_all()[0]["decode"]
    _, pools = oracle_int8(case, orc, decode=False)
    d = case.steps[0].decode
    pick = sorted(set(rng.choice(2048, 24, replace=False).tolist()) | {0, 6, 7, 8, 2047})
    items = np.array([(s, 0, h) for s in pick for h in range(case.num_q_heads)], np.int32)
    cu = np.arange(2049, dtype=np.int32)
    ref = orc.attention_rows_int8(items, d.q, cu, *pools, d.block_table, d.seq_lens, case.num_q_heads, case.scale)
    compare(out[items[:, 0], items[:, 2]], ref, f"INT8 decode {len(pick)} of 2048 sequences x all heads")


@pytest.mark.parametrize("hq,hkv,d,bs,S,prefix,private,long_seq,cut", [
    # G 4 (packs of 4) with runs missing members and a private first sequence
    (32, 8, 128, 256, 64, 2048, (5, 17, 18, 20), None, {1: 1024, 2: 1500, 8: 1024, 13: 2048, 14: 1}),
    # G 8 (packs of 2) over blocks of 32, one long private sequence
    (64, 8, 128, 32, 65, 1024, (7,), 8191, {1: 1024, 2: 1000, 9: 32}),
])
def test_int8_decode_shared_prefix_packs(orc, hq, hkv, d, bs, S, prefix, private, long_seq, cut):
    # launches with enough work items decode sequences whose chunk is the
    # same physical blocks together (the chunk's codes converted once for
    # the pack); outputs against the oracle's INT8 decode, for the decode
    # step and then, on the same cache and workspace, for lengths cut at
    # block and chunk boundaries inside the prefix
    import paged_kv_gqa_scatter_amd as pkv
    from test_gpu_parity import _shared_case
    case = _shared_case(f"int8_shared_prefix_g{hq // hkv}_b{bs}", 8000 + hq + bs, hq, hkv, d, bs, S, prefix,
                        private, long_seq)
    _say(f"case {case.name}: {S} seqs, prefix {prefix}, private {private}, long {long_seq}, cut {cut}")
    dc = _dev()(case)
    out = dc.run_all()[0]["decode"]
    ref, pools = oracle_int8(case, orc)
    compare(out, ref[0], "INT8 decode step with shared chunks")
    dd = dc.steps[0]["decode"]
    lens = case.steps[0].decode.seq_lens.copy()
    for s, n in cut.items():
        lens[s] = n
    got = pkv.paged_gqa_decode_int8(dd.q, *dc.pools[0], dd.block_table, torch.from_numpy(lens).cuda(),
                                    float(case.scale), max_seq_len=dd.max_seq_len,
                                    total_kv_tokens=dd.total_kv_tokens, workspace=dd.workspace)
    torch.cuda.synchronize()
    d_ = case.steps[0].decode
    compare(got.float().cpu().numpy().astype(np.float64),
            orc.decode_int8(d_.q, *pools, d_.block_table, lens, case.scale), "INT8 decode, cut lengths")

