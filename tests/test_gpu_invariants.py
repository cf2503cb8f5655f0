"""Properties of attention the GPU path must keep, checked without the oracle
(needs an MI355X).

- Constant V: when every V row of KV head g is the same bf16 vector c_g, every
  output row of a query head of group g is c_g (a softmax-weighted average of
  equal rows), bit for bit after bf16 rounding, for decode (with split-K) and
  prefill alike; a sequence with no keys gives zeros.
- Scale 0: all weights are equal, so an output row is the plain mean of the V
  rows it sees (positions 0..p), computed here in fp64 from the pools.
- GQA mapping: permuting the query heads inside each group permutes the
  outputs the same way, bit for bit (a group's heads share one pass over K/V
  and nothing else).
- Prefix aliasing: sequences whose tables point at the same prefix blocks give
  the outputs of the same data copied into private blocks.  The two runs take
  different kernel paths (shared chunks are decoded together), so they are
  compared at the parity tolerance and the bit-identical share is printed.
"""
import numpy as np
import pytest
import torch

from case_oracle import compare
from paged_kv_gqa_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _dev(case, **kw):
    from paged_kv_gqa_scatter_amd.runner import DeviceCase
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return DeviceCase(case, **kw)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _steps(dc):
    """Fills, then each step's append followed by its attention calls; yields
    (step index, step inputs) after the append."""
    dc.run_fills()
    for i, st in enumerate(dc.steps):
        if st["append"] is not None:
            dc.append(st["append"])
        yield i, st


# ---------------------------------------------------------------- constant V

@pytest.mark.parametrize("cfg", [1, 4])
def test_constant_v_rows_give_that_row(cfg):
    case = W.CONFIGS[cfg]()
    rng = np.random.default_rng(900 + cfg)
    c = W.bf16_normal(rng, (case.num_kv_heads, case.head_dim))  # one row per KV head
    c_t = torch.from_numpy(c.view(np.int16)).cuda().view(torch.bfloat16)
    G = case.num_q_heads // case.num_kv_heads
    want = np.repeat(c, G, axis=0)  # [Hq][D]: query head h reads KV head h / G
    _say(f"case {case.name}: every V row of KV head g set to c_g")
    dc = _dev(case)
    checked = 0
    for i, st in _steps(dc):
        dc.v_pool.copy_(c_t[None, :, None, :].expand_as(dc.v_pool))  # all slots, written or not
        for kind in ("decode", "prefill"):
            if st[kind] is None:
                continue
            out = (dc.decode if kind == "decode" else dc.prefill)(st[kind])
            torch.cuda.synchronize()
            got = out.view(torch.int16).cpu().numpy().view(np.uint16)
            if kind == "decode":
                lens = case.steps[i].decode.seq_lens
                live = lens > 0
                assert (got[~live].view(np.int16) == 0).all(), "a sequence without keys must give zeros"
                got = got[live]
            assert (got == want[None]).all(), f"step {i} {kind}: {int((got != want[None]).sum())} values differ from c"
            checked += got.shape[0]
    _say(f"  {checked} output rows equal to c bit for bit")


# ---------------------------------------------------------------- scale 0

def _mean_rows(pool, table, B, n, g):
    """fp64 mean of rows 0..n-1 of KV head g of the sequence with this table row."""
    j = np.arange(n)
    rows = pool[table[j // B], g, j % B].astype(np.uint32) << 16
    return rows.view(np.float32).astype(np.float64).mean(axis=0)


@pytest.mark.parametrize("cfg", [1, 4])
def test_scale_zero_gives_the_mean(cfg):
    import paged_kv_gqa_scatter_amd as pkv
    case = W.CONFIGS[cfg]()
    B, G = case.block_size, case.num_q_heads // case.num_kv_heads
    _say(f"case {case.name}: softmax scale 0")
    dc = _dev(case)
    for i, st in _steps(dc):
        _, Vp = dc.pools_numpy()
        d, p = st["decode"], st["prefill"]
        if d is not None:
            out = pkv.paged_gqa_decode(d.q, dc.k_pool, dc.v_pool, d.block_table, d.seq_lens, 0.0,
                                       max_seq_len=d.max_seq_len, total_kv_tokens=d.total_kv_tokens,
                                       workspace=d.workspace)
            torch.cuda.synchronize()
            b = case.steps[i].decode
            ref = np.zeros(out.shape)
            for s, L in enumerate(b.seq_lens):
                for g in range(case.num_kv_heads):
                    if L > 0:
                        ref[s, g * G:(g + 1) * G] = _mean_rows(Vp, b.block_table[s], B, L, g)
            compare(_f64(out), ref, f"step {i} decode, scale 0")
        if p is not None:
            out = pkv.paged_gqa_prefill(p.q, p.cu_q_lens, dc.k_pool, dc.v_pool, p.block_table, p.seq_lens, 0.0,
                                        max_q_len=p.max_q_len, max_seq_len=p.max_seq_len)
            torch.cuda.synchronize()
            b = case.steps[i].prefill
            ref = np.zeros(out.shape)
            for s in range(b.seq_lens.shape[0]):
                L, r0, r1 = int(b.seq_lens[s]), int(b.cu_q_lens[s]), int(b.cu_q_lens[s + 1])
                n = r1 - r0
                # rows see positions 0..L-n+r: running means over one cumsum per KV head
                for g in range(case.num_kv_heads):
                    j = np.arange(L)
                    rows = (Vp[b.block_table[s][j // B], g, j % B].astype(np.uint32) << 16).view(np.float32)
                    cm = np.cumsum(rows.astype(np.float64), axis=0) / (j + 1)[:, None]
                    ref[r0:r1, g * G:(g + 1) * G] = cm[L - n:L][:, None, :]
            compare(_f64(out), ref, f"step {i} prefill, scale 0")


# ---------------------------------------------------------------- GQA mapping

@pytest.mark.parametrize("cfg", [1, 4])
def test_permuting_heads_in_a_group_permutes_outputs(cfg):
    import paged_kv_gqa_scatter_amd as pkv
    case = W.CONFIGS[cfg]()
    Hq, G = case.num_q_heads, case.num_q_heads // case.num_kv_heads
    rng = np.random.default_rng(1100 + cfg)
    perm = np.concatenate([g * G + rng.permutation(G) for g in range(case.num_kv_heads)])
    assert not (perm == np.arange(Hq)).all()
    _say(f"case {case.name}: query heads permuted inside their groups")
    dc = _dev(case)
    idx = torch.from_numpy(perm).cuda()
    for i, st in _steps(dc):
        d, p = st["decode"], st["prefill"]
        if d is not None:
            base = dc.decode(d).clone()
            out = pkv.paged_gqa_decode(d.q[:, idx].contiguous(), dc.k_pool, dc.v_pool, d.block_table, d.seq_lens,
                                       float(case.scale), max_seq_len=d.max_seq_len,
                                       total_kv_tokens=d.total_kv_tokens, workspace=d.workspace)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), base[:, idx].view(torch.int16)), f"step {i}: decode"
        if p is not None:
            base = dc.prefill(p).clone()
            out = pkv.paged_gqa_prefill(p.q[:, idx].contiguous(), p.cu_q_lens, dc.k_pool, dc.v_pool, p.block_table,
                                        p.seq_lens, float(case.scale), max_q_len=p.max_q_len,
                                        max_seq_len=p.max_seq_len)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), base[:, idx].view(torch.int16)), f"step {i}: prefill"
    _say("  decode and prefill outputs permuted bit for bit")


# ---------------------------------------------------------------- prefix aliasing

@pytest.mark.parametrize("hq,hkv,d,S,prefix", [(32, 8, 128, 64, 2048), (8, 8, 64, 64, 1024)])
def test_shared_prefix_equals_private_copies(hq, hkv, d, S, prefix):
    # many sequences on one prefix (enough work items that shared chunks are
    # decoded together), then the same data with every sequence's prefix
    # blocks copied to blocks of its own
    import paged_kv_gqa_scatter_amd as pkv
    rng = np.random.default_rng(1200 + hq + d)
    bs = 256
    ctx = prefix + rng.integers(0, 600, S)
    case = W.build_case(f"prefix_alias_h{hq}_d{d}", rng, hq=hq, hkv=hkv, d=d, bs=bs, ctx_lens=ctx,
                        new_lens=np.ones(S, np.int64), kinds="d" * S, shared_prefix=prefix, spare=8.0)
    _say(f"case {case.name}: {S} sequences on a {prefix}-token prefix, shared vs private copies")
    dc = _dev(case)
    shared = dc.run_all()[0]["decode"]
    table = case.steps[0].decode.block_table.copy()
    npb = prefix // bs
    used = set(table[table >= 0].tolist())
    free = [b for b in range(case.num_blocks) if b not in used]
    assert len(free) >= (S - 1) * npb, "spare blocks for the copies"
    src, dst = [], []
    for s in range(1, S):  # sequence 0 keeps the original blocks
        new = free[(s - 1) * npb:s * npb]
        src += table[s, :npb].tolist()
        dst += new
        table[s, :npb] = new
    pkv.copy_blocks(dc.k_pool, dc.v_pool, src, dst)
    dd = dc.steps[0]["decode"]
    out = pkv.paged_gqa_decode(dd.q, dc.k_pool, dc.v_pool, torch.from_numpy(table).cuda(), dd.seq_lens,
                               float(case.scale), max_seq_len=dd.max_seq_len, total_kv_tokens=dd.total_kv_tokens,
                               workspace=dd.workspace)
    torch.cuda.synchronize()
    private = _f64(out)
    same = float(np.mean(private == shared))
    _say(f"  {same * 100:.2f}% of outputs bit-identical")
    compare(private, shared, "private copies vs shared prefix")
