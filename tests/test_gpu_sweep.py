"""Seeded random workloads on the GPU against the CPU oracle (needs an MI355X).

Each seed draws a shape -- head_dim 64 or 128, 1..8 query heads per KV
head, block size 16..256 -- and one of four regimes, so that the launches
land in every path of the decode kernel and in the prefill kernel:
  - a few sequences of up to 3000 keys (direct grid; split sequences merged
    inside the split kernel),
  - many short sequences and one long one (persistent grid over the compact
    item list, merge kernel),
  - many sequences on a shared prefix with enough work items that chunks of
    shared blocks are decoded together,
  - decode sequences mixed with prefill chunks on cached context (the
    mixed step, with the decode and the prefill side by side).
Every output is compared with the oracle at the attention tolerance; the
decode-only cases with blocks of at least 32 run over the INT8 cache too,
against the INT8 oracle at the tolerance of its own tests.
"""
import numpy as np
import pytest
import torch

import oracle
from case_oracle import compare, oracle_int8, oracle_outputs
from paged_kv_gqa_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _say(msg):
    print(msg, flush=True)


def _draw(seed):
    rng = np.random.default_rng(90000 + seed)
    regime = seed % 4
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    kw = {}
    if regime == 0:
        S = int(rng.integers(2, 9))
        ctx = rng.integers(0, 3000, S)
        kinds = "d" * S
    elif regime == 1:
        hkv = int(rng.choice([4, 8]))
        S = int(rng.integers(20, 61))
        ctx = rng.integers(0, 300, S)
        ctx[int(rng.integers(0, S))] = int(rng.integers(8000, 20000))
        kinds = "d" * S
    elif regime == 2:
        hkv, g, bs = 8, int(rng.choice([1, 2, 4])), int(rng.choice([64, 128, 256]))
        S = int(rng.integers(40, 65))
        prefix = bs * int(rng.integers(1024 // bs, 2048 // bs + 1))
        ctx = prefix + rng.integers(0, 600, S)
        private = set(rng.choice(S, int(rng.integers(0, 4)), replace=False).tolist())
        kw = dict(shared_prefix=prefix, shared_seqs=[s for s in range(S) if s not in private])
        kinds = "d" * S
    else:
        nd, npf = int(rng.integers(1, 9)), int(rng.integers(1, 3))
        S = nd + npf
        ctx = np.concatenate([rng.integers(0, 3000, nd), rng.integers(0, 1500, npf)])
        kinds = "d" * nd + "p" * npf
    new = np.array([1 if k == "d" else int(rng.integers(1, 300)) for k in kinds], np.int64)
    case = W.build_case(f"sweep{seed}_r{regime}_d{d}_g{g}_hkv{hkv}_b{bs}", rng, hq=g * hkv, hkv=hkv, d=d, bs=bs,
                        ctx_lens=np.asarray(ctx, np.int64), new_lens=new, kinds=kinds, **kw)
    return regime, case


@pytest.mark.timeout(600)
@pytest.mark.parametrize("seed", range(12))
def test_random_workload(orc, seed):
    from paged_kv_gqa_scatter_amd.runner import DeviceCase, Int8DeviceCase
    regime, case = _draw(seed)
    st = case.steps[0]
    nd = 0 if st.decode is None else st.decode.seq_lens.shape[0]
    npf = 0 if st.prefill is None else st.prefill.seq_lens.shape[0]
    keys = int(st.decode.seq_lens.sum()) if nd else 0
    _say(f"case {case.name}: {nd} decode seqs ({keys} keys), {npf} prefill chunks")
    got = DeviceCase(case).run_all()[0]
    ref, _ = oracle_outputs(case, orc)
    for kind in ("decode", "prefill"):
        if kind in got:
            compare(got[kind], ref[0][kind], f"{kind}")
    if npf == 0 and case.block_size >= 32:
        out = Int8DeviceCase(case).run_all()[0]["decode"]
        ref8, _ = oracle_int8(case, orc)
        compare(out, ref8[0], "INT8 decode")
