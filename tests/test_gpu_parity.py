"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

kv_append must match bit for bit over the whole pools (never-written slots
keep the NaN sentinel).  Attention outputs must satisfy max|err| <= 1e-2 and
relative L2 <= 1e-2 over each call's output (bf16 in/out, fp32 accumulation).
Full-size workloads are checked on every output where the oracle is cheap
enough, otherwise on sampled rows the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from case_oracle import compare, oracle_outputs, oracle_pools
from paged_kv_gqa_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _dev():
    from paged_kv_gqa_scatter_amd.runner import DeviceCase
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return DeviceCase


def _say(msg):
    print(msg, flush=True)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------- kv_append

@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_append_bitexact(orc, cfg):
    case = W.CONFIGS[cfg]()
    _say(f"case {case.name}: kv_append bit-exact over the pools")
    dc = _dev()(case)
    dc.run_fills()
    for i in range(len(dc.steps)):
        dc.append(dc.steps[i]["append"])
    torch.cuda.synchronize()
    gk, gv = dc.pools_numpy()
    K, V = oracle_pools(case, orc)
    assert np.array_equal(gk, K), "K pool differs"
    assert np.array_equal(gv, V), "V pool differs"
    assert (gk == W.NAN_SENTINEL).any(), "spare slots should keep the sentinel"


def test_append_mid_block_and_block16(orc):
    # chunks that start mid-block (ctx % B != 0), block size 16, D 64, several sequences
    rng = np.random.default_rng(77)
    case = W.build_case("append_mid_block", rng, hq=8, hkv=2, d=64, bs=16, ctx_lens=[5, 17, 0, 31],
                        new_lens=[40, 1, 16, 3], kinds="pppp")
    _say(f"case {case.name}")
    dc = _dev()(case)
    dc.run_fills()
    dc.append(dc.steps[0]["append"])
    torch.cuda.synchronize()
    gk, gv = dc.pools_numpy()
    K, V = oracle_pools(case, orc)
    assert np.array_equal(gk, K) and np.array_equal(gv, V)


# ---------------------------------------------------------------- whole workloads

def test_config1_tiny_prefill_then_decodes(orc):
    case = W.config1_tiny()
    _say(f"case {case.name}")
    outs = _dev()(case).run_all()
    ref, _ = oracle_outputs(case, orc)
    compare(outs[0]["prefill"], ref[0]["prefill"], "prefill 300 rows")
    for t in range(1, 9):
        compare(outs[t]["decode"], ref[t]["decode"], f"decode step {t}")


def test_config1_block_size_16_vs_256(orc):
    a = W.config1_tiny(block_size=16)
    b = W.config1_tiny(block_size=256)
    _say("case tiny: block size 16 vs 256")
    oa = _dev()(a).run_all()
    ob = _dev()(b).run_all()
    ref, _ = oracle_outputs(b, orc)
    for t in range(9):
        k = "prefill" if t == 0 else "decode"
        compare(ob[t][k], ref[t][k], f"B=256 step {t}")
        compare(oa[t][k], ob[t][k], f"B=16 vs B=256 step {t}")


def test_config2_decode(orc):
    case = W.config2_decode()
    _say(f"case {case.name}")
    outs = _dev()(case).run_all()
    ref, _ = oracle_outputs(case, orc)
    compare(outs[0]["decode"], ref[0]["decode"], "decode 8 seqs")


def test_config2_block_permutation_invariance(orc):
    a = W.config2_decode()
    rng = np.random.default_rng(2)  # same draws as config 2, then another placement
    ctx = rng.integers(512, 2048, size=8, endpoint=True)
    b = W.build_case("decode_replaced", rng, hq=32, hkv=8, d=128, bs=256, ctx_lens=ctx,
                     new_lens=np.ones(8, np.int64), kinds="d" * 8, placement_seed=1234)
    assert not np.array_equal(a.steps[0].decode.block_table, b.steps[0].decode.block_table)
    _say("case decode: same data, different block placement")
    oa = _dev()(a).run_all()[0]["decode"]
    ob = _dev()(b).run_all()[0]["decode"]
    compare(oa, ob, "placement A vs B")
    print(f"  bit-identical: {np.array_equal(oa, ob)}", flush=True)


def _prefill_sample_items(batch, rng, n_random=384):
    """(seq, row, head) items: tile edges, first/last rows, and random rows."""
    items = []
    S = batch.seq_lens.shape[0]
    Hq = batch.q.shape[1]
    for s in range(S):
        n = int(batch.cu_q_lens[s + 1] - batch.cu_q_lens[s])
        for r in sorted({0, 1, 127, 128, 129, n // 2, n - 129, n - 128, n - 2, n - 1}):
            if 0 <= r < n:
                for h in (0, 3, 4, Hq - 1):
                    items.append((s, r, h))
    for _ in range(n_random):
        s = int(rng.integers(S))
        n = int(batch.cu_q_lens[s + 1] - batch.cu_q_lens[s])
        items.append((s, int(rng.integers(n)), int(rng.integers(Hq))))
    return np.array(items, np.int32)


def test_config3_prefill_full(orc):
    # every (row, head) output of the four prompts against the oracle
    case = W.config3_prefill()
    _say(f"case {case.name}: every output")
    outs = _dev()(case).run_all()
    ref, _ = oracle_outputs(case, orc)
    p = case.steps[0].prefill
    compare(outs[0]["prefill"], ref[0]["prefill"], f"prefill {p.q.shape[0]} rows x {case.num_q_heads} heads")


def test_config3_prefill_sampled(orc):
    # tile edges and random rows: a quick look at the same launch
    case = W.config3_prefill()
    _say(f"case {case.name}: sampled rows")
    outs = _dev()(case).run_all()
    K, V = oracle_pools(case, orc)
    p = case.steps[0].prefill
    items = _prefill_sample_items(p, np.random.default_rng(33))
    ref = orc.attention_rows(items, p.q, p.cu_q_lens, K, V, p.block_table, p.seq_lens, case.num_q_heads, case.scale)
    rows = p.cu_q_lens[items[:, 0]] + items[:, 1]
    gpu = outs[0]["prefill"][rows, items[:, 2]]
    compare(gpu, ref, f"prefill {len(items)} sampled rows")


@pytest.mark.parametrize("d,new_lens", [(128, [300, 129, 517]), (128, [300, 129, 517, 200]),
                                        (64, [300, 129, 517, 200])])
def test_prefill_reduced_full(orc, d, new_lens):
    # several 128-row tiles with ragged tails, GQA 4, full comparison; 480
    # workgroups (under two per CU: the kernel that splits each workgroup's
    # keys between two halves) and 640 (the one-pass kernel), at head_dim
    # 128 and 64
    rng = np.random.default_rng(303)
    case = W.build_case(f"prefill_reduced_d{d}", rng, hq=32, hkv=8, d=d, bs=256, ctx_lens=[0] * len(new_lens),
                        new_lens=new_lens, kinds="p" * len(new_lens))
    _say(f"case {case.name}")
    outs = _dev()(case).run_all()
    ref, _ = oracle_outputs(case, orc)
    compare(outs[0]["prefill"], ref[0]["prefill"], f"prefill {len(new_lens)} prompts, d{d}")


def test_config4_mixed(orc):
    case = W.config4_mixed()
    _say(f"case {case.name}")
    outs = _dev()(case).run_all()
    ref, _ = oracle_outputs(case, orc)
    compare(outs[0]["decode"], ref[0]["decode"], "decode 64 seqs")
    compare(outs[0]["prefill"], ref[0]["prefill"], "2 chunks of 512 on 1024 cached")


@pytest.mark.timeout(900)
def test_config5_prefix_long_full(orc):
    # all 272 sequences (256 on the shared prefix, 16 of 32769 keys), every head
    case = W.config5_prefix_long()
    _say(f"case {case.name}: every sequence")
    dc = _dev()(case)
    out = dc.run_all()[0]["decode"]
    gk, gv = dc.pools_numpy()
    del dc
    torch.cuda.empty_cache()
    K, V = oracle_pools(case, orc)
    assert np.array_equal(gk, K) and np.array_equal(gv, V), "pools differ"
    del gk, gv
    d = case.steps[0].decode
    ref = orc.decode(d.q, K, V, d.block_table, d.seq_lens, case.scale)
    compare(out, ref, f"decode {d.seq_lens.shape[0]} sequences x all heads")


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 256, 32, 8), (64, 16, 4, 1), (128, 16, 16, 2), (64, 256, 8, 8)])
def test_decode_edge_lengths(orc, d, bs, hq, hkv):
    # lengths at block edges (the off-by-one lesson of exact multiples), a
    # single key, an empty sequence, and one long enough for many splits
    lens = [1, bs - 1, bs, bs + 1, 2 * bs, 512, 8192, 32769, 0]
    rng = np.random.default_rng(1000 + d + bs)
    ctx = [max(L - 1, 0) for L in lens]
    new = [1 if L > 0 else 0 for L in lens]
    # the empty sequence appends nothing: give it new_len 0 in the append and seq_len 0 in the decode
    case = W.build_case(f"decode_edges_d{d}_b{bs}", rng, hq=hq, hkv=hkv, d=d, bs=bs, ctx_lens=ctx[:-1],
                        new_lens=new[:-1], kinds="d" * (len(lens) - 1))
    dec = case.steps[0].decode
    dec.seq_lens = np.append(dec.seq_lens, 0).astype(np.int32)
    dec.block_table = np.vstack([dec.block_table, np.full((1, dec.block_table.shape[1]), -1, np.int32)])
    dec.q = np.concatenate([dec.q, W.bf16_normal(rng, (1, hq, d))])
    _say(f"case {case.name}: lens {lens}")
    out = _dev()(case).run_all()[0]["decode"]
    ref, _ = oracle_outputs(case, orc)
    compare(out, ref[0]["decode"], "decode edge lengths")
    assert np.array_equal(out[-1], np.zeros_like(out[-1])), "empty sequence must give zeros"


@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8)])
@pytest.mark.parametrize("ctx", [0, 1000])
def test_prefill_edge_qlens(orc, ctx, hq, hkv):
    # 8 / 2 heads: 168 workgroups (the split kernel); 32 / 8: 672 (one pass)
    qlens = [1, 127, 128, 129, 255, 256, 257]
    rng = np.random.default_rng(2000 + ctx)
    case = W.build_case(f"prefill_edges_ctx{ctx}_h{hq}", rng, hq=hq, hkv=hkv, d=128, bs=256,
                        ctx_lens=[ctx] * len(qlens), new_lens=qlens, kinds="p" * len(qlens))
    _say(f"case {case.name}: q_lens {qlens}")
    out = _dev()(case).run_all()[0]["prefill"]
    ref, _ = oracle_outputs(case, orc)
    compare(out, ref[0]["prefill"], "prefill edge q_lens")


def test_prefill_d64_block16_chunked(orc):
    rng = np.random.default_rng(404)
    case = W.build_case("prefill_d64_b16", rng, hq=4, hkv=1, d=64, bs=16, ctx_lens=[0, 37, 300],
                        new_lens=[300, 91, 8], kinds="ppp")
    _say(f"case {case.name}")
    out = _dev()(case).run_all()[0]["prefill"]
    ref, _ = oracle_outputs(case, orc)
    compare(out, ref[0]["prefill"], "prefill d64 b16")


def test_decode_equals_last_prefill_rows(orc):
    # prefill of all 308 tiny-case rows: rows 300..307 are the 8 decode steps' rows
    tiny = W.config1_tiny()
    outs = _dev()(tiny).run_all()
    dec = [outs[t]["decode"] for t in range(1, 9)]
    rng = np.random.default_rng(1)
    rng.permutation(32)
    k_all = W.bf16_normal(rng, (308, 1, 64))
    v_all = W.bf16_normal(rng, (308, 1, 64))
    q_all = W.bf16_normal(rng, (308, 4, 64))
    full = W.Case("tiny_full_prefill", 4, 1, 64, 16, 32, tiny.max_blocks_per_seq, tiny.scale, [], [W.Step(
        append=W.AppendBatch(k_all, v_all, np.array([0, 308], np.int32), np.zeros(1, np.int32),
                             tiny.steps[0].append.block_table),
        prefill=W.PrefillBatch(q_all, np.array([0, 308], np.int32), np.array([308], np.int32),
                               tiny.steps[0].append.block_table))])
    pf = _dev()(full).run_all()[0]["prefill"]
    for t in range(8):
        compare(dec[t][0], pf[300 + t], f"decode step {t + 1} vs prefill row {300 + t}")


def test_chunked_equals_unchunked(orc):
    # a 512-row chunk on 1024 cached tokens vs the same rows of a 1536-row prefill
    rng = np.random.default_rng(4)
    whole = W.build_case("whole_1536", rng, hq=32, hkv=8, d=128, bs=256, ctx_lens=[0], new_lens=[1536], kinds="p")
    st = whole.steps[0]
    chunk = W.Case("chunk_512_on_1024", 32, 8, 128, 256, whole.num_blocks, whole.max_blocks_per_seq, whole.scale,
                   [W.AppendBatch(st.append.k_new[:1024], st.append.v_new[:1024], np.array([0, 1024], np.int32),
                                  np.zeros(1, np.int32), st.append.block_table)],
                   [W.Step(append=W.AppendBatch(st.append.k_new[1024:], st.append.v_new[1024:],
                                                np.array([0, 512], np.int32), np.array([1024], np.int32),
                                                st.append.block_table),
                           prefill=W.PrefillBatch(st.prefill.q[1024:], np.array([0, 512], np.int32),
                                                  np.array([1536], np.int32), st.prefill.block_table))])
    _say("case chunked vs unchunked")
    a = _dev()(whole).run_all()[0]["prefill"][1024:]
    b = _dev()(chunk).run_all()[0]["prefill"]
    compare(b, a, "chunk vs whole rows 1024..1535")


# ---------------------------------------------------------------- HIP graphs

def test_graph_replays_match_eager(orc):
    # the mixed step (one append, a 64-sequence decode, two 512-row chunks)
    # captured in a HIP graph: every replay, with eager calls and
    # synchronisations between replays, equals the eager step bit for bit
    case = W.config4_mixed()
    _say(f"case {case.name}: graph replays vs eager")
    dc = _dev()(case)
    dc.run_fills()
    st = dc.steps[0]
    eager = dc.run_step(0)
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in eager.items()}
    ref, _ = oracle_outputs(case, orc)
    compare(_f64(want["decode"]), ref[0]["decode"], "eager decode")
    compare(_f64(want["prefill"]), ref[0]["prefill"], "eager prefill")
    g = dc.capture_step(0)
    for rep in range(4):
        st["decode"].out.zero_()
        st["prefill"].out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("decode", "prefill"):
            got = st[k].out
            assert torch.equal(got.view(torch.int16), want[k].view(torch.int16)), f"replay {rep}: {k} differs"
        dc.decode(st["decode"])  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(st["decode"].out.view(torch.int16), want["decode"].view(torch.int16))
    _say("  4 replays bit-identical to the eager step")


# ---------------------------------------------------------------- decode_append

def _decode_append_check(orc, case, k_new, v_new, q, seq_lens, table, what):
    """Run decode_append on a case's fills (the step's rows not yet appended)
    and compare pools (bit for bit) and outputs with kv_append + decode on
    the oracle."""
    import paged_kv_gqa_scatter_amd as pkv
    dc = _dev()(case)
    dc.run_fills()
    dev = lambda a, dt=torch.int32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    bits = lambda a: dev(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    S = seq_lens.shape[0]
    ws = torch.zeros(pkv.decode_workspace_bytes(S, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                                int(seq_lens.max())), dtype=torch.uint8, device="cuda")
    out = pkv.paged_gqa_decode_append(bits(q), bits(k_new), bits(v_new), dc.k_pool, dc.v_pool,
                                      dev(table.astype(np.int32)), dev(seq_lens.astype(np.int32)),
                                      float(case.scale), max_seq_len=int(seq_lens.max()), workspace=ws)
    torch.cuda.synchronize()
    K, V = case.empty_pool(), case.empty_pool()
    for f in case.fills:
        orc.kv_append(K, V, f.k_new, f.v_new, f.cu_new_lens, f.ctx_lens, f.block_table)
    live = np.nonzero(seq_lens > 0)[0]
    cu = np.arange(live.size + 1, dtype=np.int32)
    orc.kv_append(K, V, k_new[live], v_new[live], cu, (seq_lens[live] - 1).astype(np.int32),
                  np.ascontiguousarray(table[live]))
    gk, gv = dc.pools_numpy()
    assert np.array_equal(gk, K) and np.array_equal(gv, V), "pools differ from kv_append"
    ref = orc.decode(q, K, V, table, seq_lens, case.scale)
    compare(_f64(out), ref, what)
    return _f64(out)


def test_decode_append_config2(orc):
    case = W.config2_decode()
    _say(f"case {case.name}: decode_append")
    a, d = case.steps[0].append, case.steps[0].decode
    got = _decode_append_check(orc, case, a.k_new, a.v_new, d.q, d.seq_lens, d.block_table, "decode_append 8 seqs")
    plain = _dev()(case).run_all()[0]["decode"]  # kv_append + decode
    compare(got, plain, "decode_append vs kv_append + decode")


@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 256, 32, 8), (64, 16, 4, 1), (128, 16, 16, 2)])
def test_decode_append_edge_lengths(orc, d, bs, hq, hkv):
    # the new row is key 0 (seq_len 1), the last key of a block, the first of
    # a new block, deep in a long many-chunk sequence, or absent (seq_len 0)
    lens = [1, bs - 1, bs, bs + 1, 2 * bs, 700, 32769, 0]
    rng = np.random.default_rng(3000 + d + bs)
    ctx = [max(L - 1, 0) for L in lens]
    case = W.build_case(f"decode_append_edges_d{d}_b{bs}", rng, hq=hq, hkv=hkv, d=d, bs=bs, ctx_lens=ctx[:-1],
                        new_lens=[1] * (len(lens) - 1), kinds="d" * (len(lens) - 1))
    a, dec = case.steps[0].append, case.steps[0].decode
    S = len(lens)
    pad = W.bf16_normal(rng, (1, hkv, d))
    k_new = np.concatenate([a.k_new, pad])
    v_new = np.concatenate([a.v_new, pad])
    q = np.concatenate([dec.q, W.bf16_normal(rng, (1, hq, d))])
    seq_lens = np.append(dec.seq_lens, 0).astype(np.int32)
    table = np.vstack([dec.block_table, np.full((1, dec.block_table.shape[1]), -1, np.int32)])
    assert seq_lens.shape[0] == S
    _say(f"case {case.name}: lens {lens}")
    out = _decode_append_check(orc, case, k_new, v_new, q, seq_lens, table, "decode_append edge lengths")
    assert np.array_equal(out[-1], np.zeros_like(out[-1])), "empty sequence must give zeros"


# ---------------------------------------------------------------- block manager

def test_block_manager_prefix_sharing_end_to_end(orc):
    # one prompt cached, three forks that share it (its last block is
    # partial, so each fork's first append copies it), then a decode step
    # for all four with decode_append; pools bit-exact against the oracle's
    # kv_append and copies, outputs against the oracle through the same tables
    import paged_kv_gqa_scatter_amd as pkv
    from paged_kv_gqa_scatter_amd.blocks import BlockManager
    rng = np.random.default_rng(909)
    NB, Hq, Hkv, D, B, MBS = 96, 16, 4, 128, 16, 40
    scale = 1.0 / math.sqrt(D)
    bm = BlockManager(NB, B)
    kp = torch.full((NB, Hkv, B, D), W.NAN_SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vp = torch.full_like(kp, 0).view(torch.int16).fill_(W.NAN_SENTINEL).view(torch.bfloat16)
    K = np.full((NB, Hkv, B, D), W.NAN_SENTINEL, np.uint16)
    V = K.copy()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    bits = lambda a: dev(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    one = np.array([0, 0], np.int32)

    def write(seq, k_rows, v_rows):
        n = k_rows.shape[0]
        ctx = max(bm.seq_len(seq), 0)  # -1: a sequence the manager has not seen yet
        cow = bm.append(seq, n)
        if cow is not None:
            pkv.copy_blocks(kp, vp, [cow[0]], [cow[1]])
            K[cow[1]] = K[cow[0]]
            V[cow[1]] = V[cow[0]]
        table = bm.block_table([seq], MBS)
        cu = np.array([0, n], np.int32)
        cl = np.array([ctx], np.int32)
        pkv.kv_append(kp, vp, bits(k_rows), bits(v_rows), dev(cu), dev(cl), dev(table))
        orc.kv_append(K, V, k_rows, v_rows, cu, cl, table)

    prompt = [int(x) for x in rng.integers(50000, size=300)]
    kv = {}
    kv[0] = (W.bf16_normal(rng, (300, Hkv, D)), W.bf16_normal(rng, (300, Hkv, D)))
    write(0, *kv[0])
    bm.cache_prefix(0, prompt)
    for s in (1, 2, 3):
        extra = int(rng.integers(1, 70))
        toks = prompt + [int(x) for x in rng.integers(50000, size=extra)]
        assert bm.fork(s, toks) == 300
        kn, vn = W.bf16_normal(rng, (extra, Hkv, D)), W.bf16_normal(rng, (extra, Hkv, D))
        write(s, kn, vn)
    seqs = [0, 1, 2, 3]
    table = bm.block_table(seqs, MBS)
    assert len({int(table[s, 0]) for s in seqs}) == 1, "the prompt's first block is shared"
    # decode step: one new row per sequence, appended and attended in one launch
    lens, cows = [], 0
    for s in seqs:
        cow = bm.append(s, 1)
        if cow is not None:  # a sequence whose shared block another one wrote past its length
            pkv.copy_blocks(kp, vp, [cow[0]], [cow[1]])
            K[cow[1]] = K[cow[0]]
            V[cow[1]] = V[cow[0]]
            cows += 1
        lens.append(bm.seq_len(s))
    _say(f"  copy-on-write copies in the decode step: {cows}")
    table = bm.block_table(seqs, MBS)
    seq_lens = np.array(lens, np.int32)
    kn, vn = W.bf16_normal(rng, (4, Hkv, D)), W.bf16_normal(rng, (4, Hkv, D))
    q = W.bf16_normal(rng, (4, Hq, D))
    ws = torch.zeros(pkv.decode_workspace_bytes(4, Hq, Hkv, D, int(seq_lens.max())), dtype=torch.uint8,
                     device="cuda")
    out = pkv.paged_gqa_decode_append(bits(q), bits(kn), bits(vn), kp, vp, dev(table), dev(seq_lens), scale,
                                      max_seq_len=int(seq_lens.max()), workspace=ws)
    torch.cuda.synchronize()
    orc.kv_append(K, V, kn, vn, np.arange(5, dtype=np.int32), seq_lens - 1, table)
    gk = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    gv = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(gk, K) and np.array_equal(gv, V), "pools differ"
    ref = orc.decode(q, K, V, table, seq_lens, scale)
    compare(_f64(out), ref, "decode_append over shared prefix blocks")
    bm.close()


@pytest.mark.timeout(600)
def test_decode_persistent_grid_2048_sequences(orc):
    # the largest batch the persistent grid takes (its chunk prefix in LDS):
    # 2047 short sequences and one of 32768 keys, so that the direct grid would
    # be mostly empty; checked on sampled sequences
    rng = np.random.default_rng(2048)
    lens = rng.integers(1, 300, size=2048, endpoint=True)
    lens[1000] = 32768
    case = W.build_case("decode_2048_seqs", rng, hq=32, hkv=8, d=128, bs=256, ctx_lens=lens - 1,
                        new_lens=np.ones(2048, np.int64), kinds="d" * 2048)
    _say(f"case {case.name}: 2048 sequences, one of 32768 keys")
    out = _dev()(case).run_all()[0]["decode"]
    K, V = oracle_pools(case, orc)
    d = case.steps[0].decode
    pick = sorted(set(rng.choice(2048, 24, replace=False).tolist()) | {0, 999, 1000, 1001, 2047})
    items = np.array([(s, 0, h) for s in pick for h in range(case.num_q_heads)], np.int32)
    cu = np.arange(2049, dtype=np.int32)
    ref = orc.attention_rows(items, d.q, cu, K, V, d.block_table, d.seq_lens, case.num_q_heads, case.scale)
    compare(out[items[:, 0], items[:, 2]], ref, f"decode {len(pick)} of 2048 sequences x all heads")



def _shared_case(name, seed, hq, hkv, d, bs, S, prefix, private, long_seq=None):
    # S sequences of prefix + U[0, 600) cached keys sharing the prefix's
    # blocks, except `private` ones (U[1, 2800) keys of their own); an
    # optional last private sequence of `long_seq` keys
    rng = np.random.default_rng(seed)
    ctx = prefix + rng.integers(0, 600, S)
    for s in private:
        ctx[s] = rng.integers(1, 2800)
    if long_seq:
        ctx[S - 1] = long_seq
    shared = [s for s in range(S) if s not in private and not (long_seq and s == S - 1)]
    return W.build_case(name, rng, hq=hq, hkv=hkv, d=d, bs=bs, ctx_lens=ctx, new_lens=np.ones(S, np.int64),
                        kinds="d" * S, shared_prefix=prefix, shared_seqs=shared)


@pytest.mark.parametrize("hq,hkv,d,bs,S,prefix,private,long_seq,cut", [
    # G 4 (packs of 4): a full pack, packs missing a member (5; 17, 18), a run
    # whose first sequence is private (20); a direct grid
    (32, 8, 128, 256, 64, 2048, (5, 17, 18, 20), None, {1: 1024, 2: 1500, 8: 1024, 13: 2048, 14: 1}),
    # G 8 (packs of 2) over blocks of 32 with one long private sequence: the
    # persistent grid
    (64, 8, 128, 32, 65, 1024, (7,), 8191, {1: 1024, 2: 1000, 9: 32}),
    # G 1 (packs of 16) at D 64
    (8, 8, 64, 256, 64, 1024, (33,), None, {3: 512, 16: 512, 20: 1024, 34: 700}),
])
def test_decode_shared_prefix_packs(orc, hq, hkv, d, bs, S, prefix, private, long_seq, cut):
    # launches with many work items decode sequences whose chunk is the same
    # physical K/V in one item's spare MFMA columns; the outputs must be those
    # of separate decodes.  First the decode step, then a decode (no append)
    # over the same cache with some shared sequences cut to lengths at block
    # and 512-key boundaries inside the prefix (a member or a run's first
    # sequence then holds no keys past a shared chunk) or inside it
    import paged_kv_gqa_scatter_amd as pkv
    case = _shared_case(f"shared_prefix_g{hq // hkv}_d{d}_b{bs}", 7000 + hq + bs, hq, hkv, d, bs, S, prefix,
                        private, long_seq)
    _say(f"case {case.name}: {S} seqs, prefix {prefix}, private {private}, long {long_seq}, cut {cut}")
    dc = _dev()(case)
    out = dc.run_all()[0]["decode"]
    ref, _ = oracle_outputs(case, orc)
    compare(out, ref[0]["decode"], "decode step with shared chunks")
    dd = dc.steps[0]["decode"]
    lens = case.steps[0].decode.seq_lens.copy()
    for s, n in cut.items():
        lens[s] = n
    # the step's length bound and token count: the same split plan
    got = pkv.paged_gqa_decode(dd.q, dc.k_pool, dc.v_pool, dd.block_table, torch.from_numpy(lens).cuda(),
                               float(case.scale), max_seq_len=dd.max_seq_len, total_kv_tokens=dd.total_kv_tokens,
                               workspace=dd.workspace)
    torch.cuda.synchronize()
    K, V = oracle_pools(case, orc)
    d_ = case.steps[0].decode
    compare(_f64(got), orc.decode(d_.q, K, V, d_.block_table, lens, case.scale), "decode, cut lengths")


def test_decode_workspace_shared_across_shapes_and_formats():
    # one zero-filled workspace serving, in turn, a decode whose split kernel
    # merges (config 2), a persistent-grid decode of another shape, an INT8
    # decode that merges in its split kernel, and config 2 again: the chunk
    # counters (the first 16 KiB) are zero after every call, and the repeated
    # call gives the first one's outputs bit for bit
    import paged_kv_gqa_scatter_amd as pkv
    from paged_kv_gqa_scatter_amd.runner import Int8DeviceCase
    c2 = W.config2_decode()
    rng = np.random.default_rng(4096)
    lens = rng.integers(1, 300, size=300, endpoint=True)
    lens[7] = 20000
    cp = W.build_case("decode_300_seqs_one_long", rng, hq=32, hkv=8, d=128, bs=256, ctx_lens=lens - 1,
                      new_lens=np.ones(300, np.int64), kinds="d" * 300)
    d2, dp, d8 = _dev()(c2), _dev()(cp), Int8DeviceCase(c2)
    for dc in (d2, dp, d8):
        dc.run_fills()
        dc.append(dc.steps[0]["append"])
    steps = [("config 2", d2), ("persistent 300 seqs", dp), ("INT8 config 2", d8)]
    size = max(int(dc.steps[0]["decode"].workspace.numel()) for _, dc in steps)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    first = None
    for name, dc in steps + [steps[0]]:
        dd = dc.steps[0]["decode"]
        dd.workspace = ws
        out = dc.decode(dd).clone()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:16384])) == 0, f"{name}: chunk counters left non-zero"
        if first is None:
            first = out
        elif dc is d2:
            assert torch.equal(out.view(torch.int16), first.view(torch.int16)), "repeated call differs"
        _say(f"  {name}: counters zero after the call")
    # the persistent decode's outputs on the shared workspace, against the oracle
    orc = oracle.get()
    K, V = oracle_pools(cp, orc)
    d = cp.steps[0].decode
    pick = [0, 7, 150, 299]
    ref = orc.decode(d.q[pick], K, V, np.ascontiguousarray(d.block_table[pick]), d.seq_lens[pick], cp.scale)
    compare(_f64(dp.steps[0]["decode"].out)[pick], ref, "persistent decode on the shared workspace")


def test_decode_all_sequences_empty():
    # every sequence empty (max_seq_len 0): each output row must be zero, and
    # the _append variants must leave the caches alone (no sequence has a row
    # to append); with max_blocks_per_seq 0 the (empty) table row is not read
    import ctypes
    import paged_kv_gqa_scatter_amd as pkv
    S, Hq, Hkv, D, B, NB = 5, 8, 2, 128, 32, 3
    dev = "cuda"
    rng = np.random.default_rng(5)
    q = torch.from_numpy(W.bf16_normal(rng, (S, Hq, D)).view(np.int16)).to(dev)
    kn = torch.from_numpy(W.bf16_normal(rng, (S, Hkv, D)).view(np.int16)).to(dev)
    vn = torch.from_numpy(W.bf16_normal(rng, (S, Hkv, D)).view(np.int16)).to(dev)
    kp = torch.full((NB, Hkv, B, D), W.NAN_SENTINEL, dtype=torch.int32).to(torch.int16).to(dev)
    vp = kp.clone()
    codes = [torch.full((NB, Hkv, B, D), -128, dtype=torch.int8, device=dev) for _ in range(2)]
    scales = [torch.full((NB, Hkv, B), float("nan"), device=dev) for _ in range(2)]
    table = torch.full((S, 1), -1, dtype=torch.int32, device=dev)
    lens = torch.zeros(S, dtype=torch.int32, device=dev)
    nan_rows = lambda: torch.full((S, Hq, D), W.NAN_SENTINEL, dtype=torch.int32).to(torch.int16).to(dev)
    k0, v0 = kp.clone(), vp.clone()
    outs = {}
    outs["decode"] = pkv.paged_gqa_decode(q, kp, vp, table, lens, 0.088, max_seq_len=0, out=nan_rows())
    outs["decode_append"] = pkv.paged_gqa_decode_append(q, kn, vn, kp, vp, table, lens, 0.088, max_seq_len=0,
                                                        out=nan_rows())
    outs["decode_int8"] = pkv.paged_gqa_decode_int8(q, *codes, *scales, table, lens, 0.088, max_seq_len=0,
                                                    out=nan_rows())
    outs["decode_append_int8"] = pkv.paged_gqa_decode_append_int8(q, kn, vn, *codes, *scales, table, lens, 0.088,
                                                                  max_seq_len=0, out=nan_rows())
    # max_blocks_per_seq 0, straight through the C ABI (the table pointer is
    # valid but holds no row)
    out0 = nan_rows()
    ws = torch.zeros(pkv.decode_workspace_bytes(S, Hq, Hkv, D, 0), dtype=torch.uint8, device=dev)
    st = pkv.lib().pkv_paged_gqa_decode(out0.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                                        table.data_ptr(), 0, lens.data_ptr(), 0, 0, S, Hq, Hkv, D, B, NB,
                                        ctypes.c_float(0.088), ws.data_ptr(), ws.numel(),
                                        torch.cuda.current_stream().cuda_stream)
    assert st == 0, pkv.lib().pkv_status_string(st)
    outs["decode, max_blocks_per_seq 0"] = out0
    torch.cuda.synchronize()
    for name, o in outs.items():
        assert int(torch.count_nonzero(o.view(torch.int16))) == 0, f"{name}: rows of empty sequences not zero"
        _say(f"  {name}: all {S} rows zero")
    assert torch.equal(kp, k0) and torch.equal(vp, v0), "decode_append wrote a row for an empty sequence"
    assert bool((codes[0] == -128).all()) and bool(torch.isnan(scales[0]).all()), "INT8 append wrote a row"


def test_decode_workspace_reset():
    # a workspace whose chunk counters hold garbage (never zero-filled, or left
    # by an interrupted call) is made usable again by
    # pkv_decode_workspace_reset, a kernel (so it may be captured in a graph)
    import paged_kv_gqa_scatter_amd as pkv
    c2 = W.config2_decode()
    d2 = _dev()(c2)
    d2.run_fills()
    d2.append(d2.steps[0]["append"])
    dd = d2.steps[0]["decode"]
    good = d2.decode(dd).clone()
    ws = torch.randint(0, 255, (dd.workspace.numel(),), dtype=torch.uint8, device="cuda")
    pkv.decode_workspace_reset(ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:16384])) == 0, "counters not cleared"
    dd.workspace = ws
    out = d2.decode(dd).clone()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), good.view(torch.int16)), "decode on the reset workspace differs"
    assert int(torch.count_nonzero(ws[:16384])) == 0, "counters left non-zero"


@pytest.mark.parametrize("d,bs,hq,hkv,lens", [
    (128, 256, 32, 8, [1800, 0, 3, 16, 17, 255, 257, 4000]),            # an empty sequence mid-batch
    (64, 64, 8, 1, list(np.random.default_rng(71).integers(1, 600, 32))),  # 32 sequences, the most one round takes
    (128, 64, 16, 2, [20000]),                                         # one sequence cut into ~125 chunks
    (128, 128, 32, 4, list(np.random.default_rng(72).integers(1, 3000, 12))),
    (64, 32, 16, 2, [1, 2, 5, 33, 64, 65]),                            # shorter than a tile per wave
])
def test_decode_few_sequences(orc, d, bs, hq, hkv, lens):
    # few sequences of mixed lengths (an empty one among them, a single long
    # one, lengths shorter than a tile per wave): decode_append, pools bit
    # for bit and outputs against the oracle
    import paged_kv_gqa_scatter_amd as pkv
    lens = [int(x) for x in lens]
    live = [L for L in lens if L > 0]
    rng = np.random.default_rng(4000 + d + bs + len(lens))
    case = W.build_case(f"decode_few_d{d}_b{bs}_{len(lens)}seqs", rng, hq=hq, hkv=hkv, d=d, bs=bs,
                        ctx_lens=[L - 1 for L in live], new_lens=[1] * len(live), kinds="d" * len(live))
    a, dec = case.steps[0].append, case.steps[0].decode
    S = len(lens)
    q = W.bf16_normal(rng, (S, hq, d))
    k_new = W.bf16_normal(rng, (S, hkv, d))
    v_new = W.bf16_normal(rng, (S, hkv, d))
    table = np.full((S, dec.block_table.shape[1]), -1, np.int32)
    seq_lens = np.zeros(S, np.int32)
    j = 0
    for s, L in enumerate(lens):
        if L > 0:
            q[s], k_new[s], v_new[s] = dec.q[j], a.k_new[j], a.v_new[j]
            table[s], seq_lens[s] = dec.block_table[j], dec.seq_lens[j]
            j += 1
    _say(f"case {case.name}: lens {lens}")
    out = _decode_append_check(orc, case, k_new, v_new, q, seq_lens, table, "decode_append, few sequences")
    for s, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(out[s], np.zeros_like(out[s])), "empty sequence must give zeros"


def test_read_probe_reads_without_writing():
    """pkv_read_probe over zeros: the status is OK and the sink, whose slots
    are written only when a workgroup's XOR fold hits the probe's constant,
    keeps its contents (a fold of zeros is zero)."""
    import paged_kv_gqa_scatter_amd as pkv
    data = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((16 * pkv.READ_PROBE_WORKGROUPS,), 0x5A, dtype=torch.uint8, device="cuda")
    pkv.read_probe(data, sink)
    torch.cuda.synchronize()
    assert bool((sink == 0x5A).all())


def test_mfma_probe_runs_without_writing():
    """pkv_mfma_probe for 16 rounds: the status is OK and the sink keeps its
    contents (a slot is written only if a finite fold had a NaN's bits)."""
    import paged_kv_gqa_scatter_amd as pkv
    sink = torch.full((4 * 256 * pkv.MFMA_PROBE_WORKGROUPS,), 0x5A, dtype=torch.uint8, device="cuda")
    pkv.mfma_probe(16, sink)
    torch.cuda.synchronize()
    assert bool((sink == 0x5A).all())


def test_invalid_block_ids_stay_inside_their_sequence(orc):
    # table entries are preconditions; a bad one (negative, or past the pool)
    # is read as block 0 and its keys masked by the decode, and skipped by
    # the append: nothing outside the buffers is touched, and every other
    # sequence's output and every other pool slot come out as with valid
    # tables (the corrupted sequence's own output is unspecified)
    import paged_kv_gqa_scatter_amd as pkv
    case = W.config2_decode()
    ref, (K, V) = oracle_outputs(case, orc)
    K0, V0 = oracle_pools(case, orc, upto_step=0)  # after the fills, before the step's rows
    B = case.block_size
    lens = case.steps[0].decode.seq_lens
    table = case.steps[0].decode.block_table
    s_bad = 3
    assert lens[s_bad] > 2 * B + 1, "entries 0 and 1 must not hold the new row"
    keep = np.arange(len(lens)) != s_bad

    # decode over a table whose entries 0 and 1 of one sequence are invalid
    d2 = _dev()(case)
    d2.run_fills()
    st = d2.steps[0]
    d2.append(st["append"])
    dd = st["decode"]
    bad = dd.block_table.clone()
    bad[s_bad, 0] = -1
    bad[s_bad, 1] = case.num_blocks + 7
    _say(f"case {case.name}: sequence {s_bad}'s table entries 0 and 1 set to -1 and num_blocks + 7")
    out = pkv.paged_gqa_decode(dd.q, *d2.pools[0], bad, dd.seq_lens, case.scale, max_seq_len=dd.max_seq_len,
                               total_kv_tokens=dd.total_kv_tokens, workspace=dd.workspace)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    compare(got[keep], ref[0]["decode"][keep], "decode, the other sequences")
    Kg, Vg = d2.pools_numpy()
    assert np.array_equal(Kg, K) and np.array_equal(Vg, V), "pools changed by a decode"

    # decode_append whose new row's block entry is invalid: that row is skipped
    d3 = _dev()(case)
    d3.run_fills()
    st3 = d3.steps[0]
    dd3 = st3["decode"]
    last = (int(lens[s_bad]) - 1) // B
    bad3 = dd3.block_table.clone()
    bad3[s_bad, last] = -1
    a = st3["append"]
    _say(f"  decode_append with sequence {s_bad}'s last block entry set to -1")
    out3 = pkv.paged_gqa_decode_append(dd3.q, a.k_new, a.v_new, *d3.pools[0], bad3, dd3.seq_lens, case.scale,
                                       max_seq_len=dd3.max_seq_len, total_kv_tokens=dd3.total_kv_tokens,
                                       workspace=dd3.workspace)
    torch.cuda.synchronize()
    got3 = out3.float().cpu().numpy().astype(np.float64)
    compare(got3[keep], ref[0]["decode"][keep], "decode_append, the other sequences")
    want_k, want_v = K.copy(), V.copy()
    blk, slot = int(table[s_bad, last]), (int(lens[s_bad]) - 1) % B
    want_k[blk, :, slot] = K0[blk, :, slot]  # the skipped row's slot keeps what it held
    want_v[blk, :, slot] = V0[blk, :, slot]
    Kg3, Vg3 = d3.pools_numpy()
    assert np.array_equal(Kg3, want_k) and np.array_equal(Vg3, want_v), "decode_append wrote outside its rows"


def test_decode_concurrent_streams(orc):
    # the library keeps no state between calls: two decode steps with their
    # own workspaces (both merging split sequences inside the kernel through
    # their workspace's counters), issued alternately on two streams with
    # nothing ordering them, give exactly the outputs of the calls run alone
    a_case, b_case = W.config2_decode(), W.config2_decode(seed=12)
    da, db = _dev()(a_case), _dev()(b_case)
    for d in (da, db):
        d.run_fills()
        d.append(d.steps[0]["append"])
    sa_dec, sb_dec = da.steps[0]["decode"], db.steps[0]["decode"]
    ra = da.decode(sa_dec).clone()
    rb = db.decode(sb_dec).clone()
    torch.cuda.synchronize()
    ref_a, _ = oracle_outputs(a_case, orc)
    ref_b, _ = oracle_outputs(b_case, orc)
    compare(ra.float().cpu().numpy().astype(np.float64), ref_a[0]["decode"], "stream A alone")
    compare(rb.float().cpu().numpy().astype(np.float64), ref_b[0]["decode"], "stream B alone")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    main = torch.cuda.current_stream()
    sa.wait_stream(main)
    sb.wait_stream(main)
    _say("case: two decode steps, 40 calls each, alternating between two streams")
    for _ in range(40):
        with torch.cuda.stream(sa):
            oa = da.decode(sa_dec)
        with torch.cuda.stream(sb):
            ob = db.decode(sb_dec)
    main.wait_stream(sa)
    main.wait_stream(sb)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ra.view(torch.int16)), "stream A differs from its lone call"
    assert torch.equal(ob.view(torch.int16), rb.view(torch.int16)), "stream B differs from its lone call"
    assert int(torch.count_nonzero(sa_dec.workspace[:16384])) == 0 and \
        int(torch.count_nonzero(sb_dec.workspace[:16384])) == 0, "counters left non-zero"
