"""Run a seeded workload through the CPU oracle (host pools, fp64 outputs),
and compare GPU outputs against it with the acceptance tolerance."""
from __future__ import annotations

import numpy as np

# Acceptance bar for attention outputs with bf16 inputs/outputs, over the whole
# output of a call: relative L2 error <= 1e-2, and every element within 1e-2
# absolute -- except where bf16 itself cannot hold the exact value that
# closely.  bf16 keeps 8 significant bits, so from |o| = 4 on half the spacing
# of representable outputs (2^-6 in [4, 8)) exceeds 1e-2: the exact -4.11244
# lies between -4.125 and -4.09375, and even its correctly rounded output
# -4.125 is 0.0126 away.  Only there (|ref| >= 4) an element also passes if it
# is one of the two bf16 values bracketing the exact result (the kernel's fp32
# result before its one output rounding may sit on either side of the
# midpoint).  Below 4 half a bf16 step is at most 2^-7 = 0.0078, so a
# correctly rounded output always meets 1e-2 and no exception applies.
TOL_MAX_ABS = 1e-2
TOL_REL_L2 = 1e-2
BRACKET_FROM = 4.0


def bf16_ulp(x):
    """Spacing of bf16 numbers in the binade of |x| (normal range)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def bf16_bracket(ref):
    """The bf16 values just below and just above each exact value (equal when
    the value is representable)."""
    ref = np.asarray(ref, np.float64)
    u = bf16_ulp(ref)
    return np.floor(ref / u) * u, np.ceil(ref / u) * u


def oracle_pools(case, orc, upto_step=None):
    """Host pools after the fills and the appends of steps [0, upto_step)."""
    K = case.empty_pool()
    V = case.empty_pool()
    for f in case.fills:
        orc.kv_append(K, V, f.k_new, f.v_new, f.cu_new_lens, f.ctx_lens, f.block_table)
    n = len(case.steps) if upto_step is None else upto_step
    for st in case.steps[:n]:
        a = st.append
        orc.kv_append(K, V, a.k_new, a.v_new, a.cu_new_lens, a.ctx_lens, a.block_table)
    return K, V


def oracle_outputs(case, orc):
    """Every output row of every step, in order (appends applied first)."""
    K = case.empty_pool()
    V = case.empty_pool()
    for f in case.fills:
        orc.kv_append(K, V, f.k_new, f.v_new, f.cu_new_lens, f.ctx_lens, f.block_table)
    outs = []
    for st in case.steps:
        a = st.append
        orc.kv_append(K, V, a.k_new, a.v_new, a.cu_new_lens, a.ctx_lens, a.block_table)
        r = {}
        if st.decode is not None:
            d = st.decode
            r["decode"] = orc.decode(d.q, K, V, d.block_table, d.seq_lens, case.scale)
        if st.prefill is not None:
            p = st.prefill
            r["prefill"] = orc.attention(p.q, p.cu_q_lens, K, V, p.block_table, p.seq_lens, case.num_q_heads,
                                         case.scale)
        outs.append(r)
    return outs, (K, V)


def int8_empty_pools(case):
    """Host INT8 cache of a case: codes hold -128, scales NaN."""
    from paged_kv_gqa_scatter_amd.workloads import INT8_CODE_SENTINEL
    shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    codes = [np.full(shape, INT8_CODE_SENTINEL, np.int8) for _ in range(2)]
    scales = [np.full(shape[:3], np.nan, np.float32) for _ in range(2)]
    return codes[0], codes[1], scales[0], scales[1]


def oracle_int8(case, orc, upto_step=None, decode=True):
    """The case over an INT8 cache: the host cache after the fills and the
    appends of steps [0, upto_step), and (decode=True) every decode step's
    output, each computed after its step's append."""
    pools = int8_empty_pools(case)
    for f in case.fills:
        orc.kv_append_int8(*pools, f.k_new, f.v_new, f.cu_new_lens, f.ctx_lens, f.block_table)
    outs = []
    n = len(case.steps) if upto_step is None else upto_step
    for st in case.steps[:n]:
        a = st.append
        orc.kv_append_int8(*pools, a.k_new, a.v_new, a.cu_new_lens, a.ctx_lens, a.block_table)
        if decode and st.decode is not None:
            d = st.decode
            outs.append(orc.decode_int8(d.q, *pools, d.block_table, d.seq_lens, case.scale))
    return outs, pools


def compare(gpu: np.ndarray, ref: np.ndarray, what: str):
    """Max abs error and relative L2 error over the whole tensor."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    diff = gpu - ref
    mx = float(np.abs(diff).max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff))
    where = ""
    if diff.size:
        i = np.unravel_index(int(np.abs(diff).argmax()), diff.shape)
        where = f"  worst at {tuple(int(x) for x in i)}: gpu {gpu[i]:.6g} ref {ref[i]:.6g}"
    ad = np.abs(diff)
    within_abs = ad <= TOL_MAX_ABS
    lo, hi = bf16_bracket(ref)
    bracketed = (np.abs(ref) >= BRACKET_FROM) & ((gpu == lo) | (gpu == hi))
    n_br = int(np.count_nonzero(~within_abs & bracketed))
    print(f"  {what}: max|err| {mx:.3e}  rel-L2 {rel:.3e}  ({gpu.size} values){where}"
          + (f"  [{n_br} beyond 1e-2 at |ref| >= 4, each a bf16 neighbour of ref]" if n_br else ""), flush=True)
    bad = ~(within_abs | bracketed)
    if bad.any():
        j = np.unravel_index(int(np.argmax(np.where(bad, ad, -1))), ad.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements off by more than 1e-2 (and not a bf16 neighbour "
                             f"of a reference >= 4 in magnitude); e.g. at {tuple(int(x) for x in j)}: "
                             f"gpu {gpu[j]:.6g} ref {ref[j]:.6g}")
    assert rel <= TOL_REL_L2, f"{what}: rel-L2 {rel} > {TOL_REL_L2}"
    return mx, rel
