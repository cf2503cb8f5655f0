"""pkv_paged_gqa_decode_append_static (the decode step on the library's own
static scratch, for callers that cannot allocate) against
pkv_paged_gqa_decode_append with a caller workspace, through the C ABI, on
two calls in a row (the second smaller), and against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from case_oracle import compare, oracle_outputs
from paged_kv_gqa_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run_static(dc, a, dd, out):
    """The step through the static entry point (ctypes, no workspace)."""
    import paged_kv_gqa_scatter_amd as pkv
    k, v = dc.pools[0]
    S, Hq, D = dd.q.shape
    NB, Hkv, B, _ = k.shape
    st = pkv.lib().pkv_paged_gqa_decode_append_static(
        out.data_ptr(), dd.q.data_ptr(), a.k_new.data_ptr(), a.v_new.data_ptr(), k.data_ptr(), v.data_ptr(),
        dd.block_table.data_ptr(), dd.block_table.shape[1], dd.seq_lens.data_ptr(), dd.max_seq_len,
        dd.total_kv_tokens, S, Hq, Hkv, D, B, NB, ctypes.c_float(dc.case.scale),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, pkv.lib().pkv_status_string(st)
    return out


def _case_small():
    rng = np.random.default_rng(911)
    return W.build_case("decode_3_seqs", rng, hq=32, hkv=8, d=128, bs=256, ctx_lens=[699, 32, 0],
                        new_lens=[1, 1, 1], kinds="ddd")


@pytest.mark.parametrize("order", ["large_then_small"])
def test_static_scratch_matches_workspace_entry(order):
    from paged_kv_gqa_scatter_amd.runner import DeviceCase
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    orc = oracle.get()
    for case in (W.config2_decode(), _case_small()):
        _say(f"case {case.name}: static scratch vs caller workspace")
        dw, ds = DeviceCase(case), DeviceCase(case)
        for dc in (dw, ds):
            dc.run_fills()
        a_w, d_w = dw.steps[0]["append"], dw.steps[0]["decode"]
        a_s, d_s = ds.steps[0]["append"], ds.steps[0]["decode"]
        ref_out = dw.decode_append(a_w, d_w).clone()
        out = torch.full_like(d_s.out.view(torch.int16), W.NAN_SENTINEL).view(torch.bfloat16)
        _run_static(ds, a_s, d_s, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "outputs differ from the workspace entry"
        gk, gv = ds.pools_numpy()
        wk, wv = dw.pools_numpy()
        assert np.array_equal(gk, wk) and np.array_equal(gv, wv), "appended pools differ"
        ref, _ = oracle_outputs(case, orc)
        compare(out.float().cpu().numpy().astype(np.float64), ref[0]["decode"], f"{case.name} static vs oracle")
