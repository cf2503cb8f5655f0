"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every ``pin_*`` function takes an oracle instance and raises AssertionError on
a mismatch, so the same pins run against the real oracle (``test_oracle.py``)
and against copies of it with a planted mistake (``test_oracle_mutations.py``),
which must fail at least one pin.

What pins what:
  * hand-worked cases in tests/golden (softmax weights, inclusive causal mask,
    GQA grouping, chunk alignment, max subtraction, append addressing);
  * a library routine on special cases: torch's CPU fp64
    scaled_dot_product_attention with an explicit mask, KV heads expanded with
    repeat_interleave;
  * brute force on tiny inputs: the dense definition over contiguous K/V that
    never went through a block table;
  * closed forms: constant V returns V, scale 0 returns the prefix mean, a
    single key returns its V row, an empty sequence returns zeros;
  * invariants: permuting physical block placement, block size 16 vs 256,
    decode = last prefill row, chunked = unchunked, GQA = MHA with expanded
    KV heads, permuting query heads inside a group.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from paged_kv_gqa_scatter_amd.workloads import INT8_CODE_SENTINEL, NAN_SENTINEL, bf16_normal

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# small helpers (bf16 bits <-> float, tiny paged cases built by plain indexing)
# ----------------------------------------------------------------------------

def to_bf16_exact(x) -> np.ndarray:
    """Exact decimals -> bf16 bits; refuses values bf16 cannot hold."""
    a = np.asarray(x, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)
    assert torch.equal(t.to(torch.float32), torch.from_numpy(np.ascontiguousarray(a))), "value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def place_rows(pool, table_row, rows, start=0):
    """Write rows [T][Hkv][D] at logical positions start.. of one sequence by
    plain numpy indexing (independent of any append routine)."""
    B = pool.shape[2]
    for t in range(rows.shape[0]):
        pos = start + t
        pool[table_row[pos // B], :, pos % B, :] = rows[t]


class Tiny:
    """A random paged case: contiguous K/V per sequence plus its paged copy."""

    def __init__(self, rng, S, hq, hkv, d, bs, seq_lens, q_lens, spare=3, scale=None, perm=None):
        self.S, self.hq, self.hkv, self.d, self.bs = S, hq, hkv, d, bs
        self.seq_lens = np.asarray(seq_lens, np.int32)
        self.q_lens = np.asarray(q_lens, np.int32)
        self.cu = np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)
        nblk = [-(-int(L) // bs) for L in self.seq_lens]
        self.mbs = max(1, max(nblk))
        self.nb = sum(nblk) + spare
        drawn = rng.permutation(self.nb).astype(np.int32)  # always drawn, so the samples below do not move
        perm = drawn if perm is None else np.asarray(perm, np.int32)
        self.table = np.full((S, self.mbs), -1, np.int32)
        o = 0
        for s in range(S):
            self.table[s, :nblk[s]] = perm[o:o + nblk[s]]
            o += nblk[s]
        self.k = [bf16_normal(rng, (int(L), hkv, d)) for L in self.seq_lens]
        self.v = [bf16_normal(rng, (int(L), hkv, d)) for L in self.seq_lens]
        self.q = bf16_normal(rng, (int(self.cu[-1]), hq, d))
        self.scale = np.float32(1.0 / math.sqrt(d) if scale is None else scale)
        self.build_pools()

    def build_pools(self):
        shape = (self.nb, self.hkv, self.bs, self.d)
        self.kp = np.full(shape, NAN_SENTINEL, np.uint16)
        self.vp = np.full(shape, NAN_SENTINEL, np.uint16)
        for s in range(self.S):
            place_rows(self.kp, self.table[s], self.k[s])
            place_rows(self.vp, self.table[s], self.v[s])

    def run(self, orc, **kw):
        return orc.attention(self.q, self.cu, self.kp, self.vp, self.table, self.seq_lens, self.hq, self.scale, **kw)


def dense_reference(t: Tiny) -> np.ndarray:
    """The dense definition over contiguous K/V (never paged): numpy fp64."""
    G = t.hq // t.hkv
    out = np.zeros((int(t.cu[-1]), t.hq, t.d))
    q = bf16_to_f64(t.q)
    for s in range(t.S):
        K = bf16_to_f64(t.k[s])
        V = bf16_to_f64(t.v[s])
        n, L = int(t.q_lens[s]), int(t.seq_lens[s])
        for r in range(n):
            p = L - n + r
            for h in range(t.hq):
                if p < 0:
                    continue
                z = float(t.scale) * (K[:p + 1, h // G, :] @ q[t.cu[s] + r, h])
                w = np.exp(z - z.max())
                out[t.cu[s] + r, h] = (w @ V[:p + 1, h // G, :]) / w.sum()
    return out


def sdpa_reference(t: Tiny) -> np.ndarray:
    """torch CPU fp64 scaled_dot_product_attention, KV heads expanded with
    repeat_interleave, explicit boolean mask aligned to the end of the keys."""
    G = t.hq // t.hkv
    out = np.zeros((int(t.cu[-1]), t.hq, t.d))
    for s in range(t.S):
        n, L = int(t.q_lens[s]), int(t.seq_lens[s])
        if n == 0 or L == 0:
            continue
        q = torch.from_numpy(bf16_to_f64(t.q[t.cu[s]:t.cu[s] + n])).permute(1, 0, 2)  # [Hq][n][D]
        k = torch.from_numpy(bf16_to_f64(t.k[s])).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = torch.from_numpy(bf16_to_f64(t.v[s])).permute(1, 0, 2).repeat_interleave(G, dim=0)
        pos = torch.arange(n) + (L - n)
        mask = torch.arange(L)[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(t.scale))
        out[t.cu[s]:t.cu[s] + n] = o.permute(1, 0, 2).numpy()
    return out


# ----------------------------------------------------------------------------
# golden (hand-worked) cases
# ----------------------------------------------------------------------------

def golden_files():
    return sorted(f for f in os.listdir(GOLDEN) if f.endswith(".json"))


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def golden_pools(g):
    shape = (g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"])
    kp = np.full(shape, NAN_SENTINEL, np.uint16)
    vp = np.full(shape, NAN_SENTINEL, np.uint16)
    table = np.asarray(g["block_table"], np.int32)
    place_rows(kp, table[0], to_bf16_exact(g["k_rows"]))
    place_rows(vp, table[0], to_bf16_exact(g["v_rows"]))
    return kp, vp, table


def int8_pools(shape):
    """Empty INT8 pools: codes hold the sentinel -128, scales NaN."""
    codes = np.full(shape, INT8_CODE_SENTINEL, np.int8)
    scales = np.full(shape[:3], np.nan, np.float32)
    return codes, codes.copy(), scales, scales.copy()


def pin_golden_int8(orc, g, name):
    if g["kind"] == "quantize_int8":
        codes, scales = orc.quantize_int8(to_bf16_exact(g["rows"]))
        assert np.array_equal(codes, np.asarray(g["expected_codes"], np.int8)), name
        assert np.array_equal(scales, np.asarray(g["expected_scales"], np.float32)), name
        return
    shape = (g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"])
    kc, vc, ks, vs = int8_pools(shape)
    table = np.asarray(g["block_table"], np.int32)
    orc.kv_append_int8(kc, vc, ks, vs, to_bf16_exact(g["k_new"]), to_bf16_exact(g["v_new"]), g["cu_new_lens"],
                       g["ctx_lens"], table)
    ekc, evc, eks, evs = int8_pools(shape)
    for w in g["expected_writes"]:
        at = (w["block"], w["kv_head"], w["slot"])
        ekc[at], evc[at], eks[at], evs[at] = w["k_codes"], w["v_codes"], w["k_scale"], w["v_scale"]
    assert np.array_equal(kc, ekc) and np.array_equal(vc, evc), name
    assert np.array_equal(ks, eks, equal_nan=True) and np.array_equal(vs, evs, equal_nan=True), name
    out = orc.decode_int8(to_bf16_exact(g["q"]), kc, vc, ks, vs, table, g["seq_lens"], np.float32(g["scale"]))
    err = np.abs(out - np.asarray(g["expected"], np.float64)).max()
    assert err <= g["tol"], f"{name}: max err {err}"


def pin_golden_qkv(orc, g, name):
    shape = (g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"])
    kp = np.full(shape, NAN_SENTINEL, np.uint16)
    vp = np.full(shape, NAN_SENTINEL, np.uint16)
    q = orc.qkv_project_append(kp, vp, to_bf16_exact(g["x"]), to_bf16_exact(g["w"]), g["cu_new_lens"],
                               g["ctx_lens"], np.asarray(g["block_table"], np.int32), g["num_q_heads"])
    assert np.array_equal(q, to_bf16_exact(g["expected_q"])), f"{name}: q {bf16_to_f64(q).ravel()}"
    ek = np.full(shape, NAN_SENTINEL, np.uint16)
    ev = np.full(shape, NAN_SENTINEL, np.uint16)
    for w in g["expected_writes"]:
        ek[w["block"], w["kv_head"], w["slot"]] = to_bf16_exact(w["k"])
        ev[w["block"], w["kv_head"], w["slot"]] = to_bf16_exact(w["v"])
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev), name


def pin_golden(orc, name):
    g = load_golden(name)
    if g["kind"] == "qkv_project_append":
        pin_golden_qkv(orc, g, name)
        return
    if g["kind"] in ("quantize_int8", "int8_append_decode"):
        pin_golden_int8(orc, g, name)
        return
    if g["kind"] == "append":
        shape = (g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"])
        kp = np.full(shape, NAN_SENTINEL, np.uint16)
        vp = np.full(shape, NAN_SENTINEL, np.uint16)
        orc.kv_append(kp, vp, to_bf16_exact(g["k_new"]), to_bf16_exact(g["v_new"]), g["cu_new_lens"],
                      g["ctx_lens"], np.asarray(g["block_table"], np.int32))
        ek = np.full(shape, NAN_SENTINEL, np.uint16)
        ev = np.full(shape, NAN_SENTINEL, np.uint16)
        for w in g["expected_writes"]:
            ek[w["block"], w["kv_head"], w["slot"]] = to_bf16_exact(w["k"])
            ev[w["block"], w["kv_head"], w["slot"]] = to_bf16_exact(w["v"])
        assert np.array_equal(kp, ek) and np.array_equal(vp, ev), name
        return
    kp, vp, table = golden_pools(g)
    q = to_bf16_exact(g["q"])
    if g["kind"] == "decode":
        out = orc.decode(q, kp, vp, table, g["seq_lens"], np.float32(g["scale"]))
    else:
        out = orc.attention(q, g["cu_q_lens"], kp, vp, table, g["seq_lens"], g["num_q_heads"],
                            np.float32(g["scale"]))
    exp = np.asarray(g["expected"], np.float64)
    assert out.shape == exp.shape, name
    err = np.abs(out - exp).max()
    assert err <= g["tol"], f"{name}: max err {err}"


def pin_all_golden(orc):
    for name in golden_files():
        pin_golden(orc, name)


# ----------------------------------------------------------------------------
# library routine, brute force
# ----------------------------------------------------------------------------

def _tiny_mix(seed):
    """A few tiny shapes: several sequences, ragged lengths, chunks on cached
    context, G in {1, 2, 4}, D in {8, 64}, blocks 4 and 16."""
    rng = np.random.default_rng(seed)
    cases = []
    cases.append(Tiny(rng, 3, 4, 1, 8, 4, [7, 13, 40], [7, 5, 1]))
    cases.append(Tiny(rng, 2, 8, 2, 64, 16, [33, 17], [9, 17]))
    cases.append(Tiny(rng, 3, 2, 2, 8, 4, [1, 4, 5], [1, 1, 2]))
    return cases


def pin_vs_sdpa(orc):
    for i, t in enumerate(_tiny_mix(11)):
        err = np.abs(t.run(orc) - sdpa_reference(t)).max()
        assert err <= 1e-12, f"case {i}: |oracle - sdpa| = {err}"


def pin_vs_dense(orc):
    for i, t in enumerate(_tiny_mix(12)):
        err = np.abs(t.run(orc) - dense_reference(t)).max()
        assert err <= 1e-12, f"case {i}: |oracle - dense| = {err}"


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def pin_constant_v(orc):
    rng = np.random.default_rng(21)
    t = Tiny(rng, 2, 4, 2, 64, 16, [37, 5], [3, 1])
    c = bf16_normal(rng, (t.hkv, t.d))
    t.v = [np.broadcast_to(c, v.shape).copy() for v in t.v]
    t.build_pools()
    out = t.run(orc)
    G = t.hq // t.hkv
    want = bf16_to_f64(c)[np.arange(t.hq) // G]
    # fp64 sums of <= 37 terms: relative error <= 2 * 37 * 2^-53, |c| < 8
    assert np.abs(out - want[None]).max() <= 2 * 37 * 2.0 ** -53 * 8


def pin_scale_zero_mean(orc):
    rng = np.random.default_rng(22)
    t = Tiny(rng, 2, 4, 1, 8, 4, [9, 14], [9, 2], scale=0.0)
    out = t.run(orc)
    for s in range(t.S):
        V = bf16_to_f64(t.v[s])
        n, L = int(t.q_lens[s]), int(t.seq_lens[s])
        for r in range(n):
            p = L - n + r
            want = V[:p + 1, 0, :].mean(axis=0)
            assert np.abs(out[t.cu[s] + r] - want[None]).max() <= 1e-13


def pin_single_key(orc):
    rng = np.random.default_rng(23)
    t = Tiny(rng, 2, 4, 2, 64, 16, [1, 20], [1, 20])
    out = t.run(orc)
    G = t.hq // t.hkv
    for s in range(t.S):  # the first row of each sequence sees key 0 alone
        want = bf16_to_f64(t.v[s][0])[np.arange(t.hq) // G]
        assert np.array_equal(out[t.cu[s]], want)


def pin_empty_sequence(orc):
    rng = np.random.default_rng(24)
    t = Tiny(rng, 2, 4, 1, 8, 4, [0, 6], [1, 1])
    out = t.run(orc)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.isfinite(out).all()


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def pin_block_permutation(orc):
    rng = np.random.default_rng(31)
    t = Tiny(rng, 3, 4, 2, 8, 4, [11, 23, 6], [11, 3, 1])
    a = t.run(orc)
    t2 = Tiny(np.random.default_rng(31), 3, 4, 2, 8, 4, [11, 23, 6], [11, 3, 1],
              perm=np.random.default_rng(99).permutation(t.nb))
    assert not np.array_equal(t.table, t2.table)
    assert np.array_equal(a, t2.run(orc))


def pin_block_size_16_vs_256(orc):
    a = Tiny(np.random.default_rng(32), 1, 4, 1, 64, 16, [308], [300])
    b = Tiny(np.random.default_rng(32), 1, 4, 1, 64, 256, [308], [300], perm=np.arange(200)[::-1] % 3)
    b.k, b.v, b.q = a.k, a.v, a.q
    b.build_pools()
    assert b.table.shape[1] == 2 and a.table.shape[1] == 20
    assert np.array_equal(a.run(orc), b.run(orc))


def pin_decode_is_last_prefill_row(orc):
    rng = np.random.default_rng(33)
    t = Tiny(rng, 1, 4, 1, 64, 16, [45], [45])
    full = t.run(orc)
    for L in (1, 16, 17, 45):
        q = t.q[L - 1:L].reshape(1, t.hq, t.d)
        dec = orc.decode(q, t.kp, t.vp, t.table, [L], t.scale)
        assert np.array_equal(dec[0], full[L - 1])


def pin_chunked_equals_unchunked(orc):
    rng = np.random.default_rng(34)
    t = Tiny(rng, 1, 4, 1, 8, 4, [30], [30])
    full = t.run(orc)
    # the last 12 rows as a chunk on 18 cached tokens
    q = t.q[18:30]
    out = orc.attention(q, [0, 12], t.kp, t.vp, t.table, [30], t.hq, t.scale)
    assert np.array_equal(out, full[18:30])


def pin_gqa_is_expanded_mha(orc):
    rng = np.random.default_rng(35)
    t = Tiny(rng, 2, 8, 2, 8, 4, [13, 7], [5, 7])
    a = t.run(orc)
    G = t.hq // t.hkv
    m = Tiny(np.random.default_rng(35), 2, 8, 8, 8, 4, [13, 7], [5, 7])
    m.table = t.table
    m.nb = t.nb
    m.k = [np.repeat(k, G, axis=1) for k in t.k]
    m.v = [np.repeat(v, G, axis=1) for v in t.v]
    m.q = t.q
    m.scale = t.scale
    m.build_pools()
    assert np.array_equal(a, m.run(orc))


def pin_head_permutation_in_group(orc):
    rng = np.random.default_rng(36)
    t = Tiny(rng, 1, 8, 2, 8, 4, [10], [3])
    a = t.run(orc)
    perm = np.array([2, 0, 3, 1, 7, 5, 4, 6])  # stays inside each group of 4
    t.q = np.ascontiguousarray(t.q[:, perm])
    b = t.run(orc)
    assert np.array_equal(b, a[:, perm])


# ----------------------------------------------------------------------------
# kv_append
# ----------------------------------------------------------------------------

def pin_append_matches_indexing(orc):
    rng = np.random.default_rng(41)
    t = Tiny(rng, 3, 4, 2, 8, 4, [9, 14, 3], [1, 1, 1])
    shape = t.kp.shape
    kp = np.full(shape, NAN_SENTINEL, np.uint16)
    vp = np.full(shape, NAN_SENTINEL, np.uint16)
    ctx = np.array([2, 5, 0], np.int32)  # some rows start mid-block
    new = t.seq_lens - ctx
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    k_new = np.concatenate([t.k[s][ctx[s]:] for s in range(3)])
    v_new = np.concatenate([t.v[s][ctx[s]:] for s in range(3)])
    orc.kv_append(kp, vp, k_new, v_new, cu, ctx, t.table)
    ek = np.full(shape, NAN_SENTINEL, np.uint16)
    ev = np.full(shape, NAN_SENTINEL, np.uint16)
    for s in range(3):
        place_rows(ek, t.table[s], t.k[s][ctx[s]:], start=int(ctx[s]))
        place_rows(ev, t.table[s], t.v[s][ctx[s]:], start=int(ctx[s]))
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev)


def pin_append_rejects_duplicate_slot(orc):
    import oracle as _o
    kp = np.full((2, 1, 4, 2), NAN_SENTINEL, np.uint16)
    vp = kp.copy()
    rows = to_bf16_exact(np.ones((2, 1, 2)))
    table = np.array([[1], [1]], np.int32)  # both sequences point at block 1
    try:
        orc.kv_append(kp, vp, rows, rows, [0, 1, 2], [0, 0], table)
    except _o.OracleError:
        return
    raise AssertionError("duplicate slot not reported")


# ----------------------------------------------------------------------------
# INT8 KV cache
# ----------------------------------------------------------------------------

def _int8_rows(rng):
    """bf16 rows of several magnitudes, with ties for the maximum, an all-zero
    row and rows whose entries are all equal."""
    rows = [bf16_normal(rng, (40, 64))]
    for mag in (1e-3, 1e3, 3.0):
        x = rng.standard_normal((20, 64)).astype(np.float32) * np.float32(mag)
        rows.append(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    special = np.zeros((4, 64), np.float32)
    special[1, :] = -2.5            # every entry is the maximum
    special[2, ::7] = 6.0           # the maximum appears several times, both signs
    special[2, 3::7] = -6.0
    special[3, 5] = 1e-37           # a single tiny value (its scale is a subnormal fp32)
    rows.append(torch.from_numpy(special).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    return np.concatenate(rows)


def pin_int8_quantizer_bounds(orc):
    """Closed-form properties of symmetric absmax quantisation: codes in
    [-127, 127]; the largest |x| of a row maps to +-127 exactly; every value
    is recovered within half a step (|x - code * scale| <= scale / 2, plus the
    fp32 rounding of the quotient); a zero row has scale 0 and codes 0."""
    rows = _int8_rows(np.random.default_rng(81))
    x = bf16_to_f64(rows)
    codes, scales = orc.quantize_int8(rows)
    c = codes.astype(np.float64)
    s = scales.astype(np.float64)
    amax = np.abs(x).max(axis=1)
    assert (np.abs(c) <= 127).all()
    nz = amax > 0
    assert (s[~nz] == 0).all() and (c[~nz] == 0).all()
    at_max = np.abs(x) == amax[:, None]
    assert (np.abs(c)[at_max & nz[:, None]] == 127).all(), "the row maximum does not map to 127"
    assert (np.sign(c) == np.sign(np.round(x / np.where(s > 0, s, 1)[:, None]))).all()
    err = np.abs(x - c * s[:, None])
    assert (err <= s[:, None] * (0.5 + 1e-6) + 1e-45).all(), f"max step error {np.max(err / np.where(s > 0, s, 1)[:, None])}"
    assert np.allclose(s[nz], amax[nz] / 127, rtol=1e-6, atol=0)


def pin_int8_quantizer_symmetries(orc):
    """Negating a row negates its codes; scaling it by a power of two scales
    the scale and keeps the codes (both exact in fp32)."""
    rows = _int8_rows(np.random.default_rng(82))[:60]
    codes, scales = orc.quantize_int8(rows)
    neg = rows ^ np.uint16(0x8000)
    nc, ns = orc.quantize_int8(neg)
    assert np.array_equal(nc, -codes) and np.array_equal(ns, scales)
    x = bf16_to_f64(rows) * 8.0  # exact in bf16 for these magnitudes
    big = to_bf16_exact(x.astype(np.float32))
    bc, bs = orc.quantize_int8(big)
    assert np.array_equal(bc, codes) and np.array_equal(bs, scales * np.float32(8))


def _int8_tiny(seed, S, hq, hkv, d, bs, seq_lens, q_lens):
    """A paged INT8 case with codes and scales drawn directly (not by the
    quantiser), and its dequantised contiguous K/V as fp64."""
    rng = np.random.default_rng(seed)
    t = Tiny(rng, S, hq, hkv, d, bs, seq_lens, q_lens)
    kc, vc, ks, vs = int8_pools(t.kp.shape)
    dense = []
    for s in range(S):
        L = int(t.seq_lens[s])
        rows = {}
        for name, codes, scales in (("k", kc, ks), ("v", vc, vs)):
            c = rng.integers(-127, 128, size=(L, hkv, d)).astype(np.int8)
            sc = (rng.uniform(0.001, 0.05, size=(L, hkv)) * rng.choice([1.0, 8.0], size=(L, hkv))).astype(np.float32)
            for p in range(L):
                blk, slot = t.table[s][p // bs], p % bs
                codes[blk, :, slot, :] = c[p]
                scales[blk, :, slot] = sc[p]
            rows[name] = c.astype(np.float64) * sc.astype(np.float64)[:, :, None]
        dense.append(rows)
    return t, kc, vc, ks, vs, dense


def pin_int8_attention_vs_sdpa(orc):
    """Attention over an INT8 cache equals torch's fp64
    scaled_dot_product_attention over the dequantised K/V (codes times their
    row's scale, computed here by plain numpy), for decode rows and chunked
    prefill rows, GQA groups 1, 2 and 4."""
    for seed, args in ((91, (3, 4, 2, 16, 4, [7, 12, 1], [1, 3, 1])),
                       (92, (2, 4, 1, 8, 16, [40, 19], [5, 19])),
                       (93, (2, 2, 2, 8, 4, [9, 6], [9, 1]))):
        t, kc, vc, ks, vs, dense = _int8_tiny(seed, *args)
        G = t.hq // t.hkv
        items = [(s, r, h) for s in range(t.S) for r in range(int(t.q_lens[s])) for h in range(t.hq)]
        out = orc.attention_rows_int8(items, t.q, t.cu, kc, vc, ks, vs, t.table, t.seq_lens, t.hq, t.scale)
        i = 0
        for s in range(t.S):
            n, L = int(t.q_lens[s]), int(t.seq_lens[s])
            q = torch.from_numpy(bf16_to_f64(t.q[t.cu[s]:t.cu[s] + n])).permute(1, 0, 2)
            k = torch.from_numpy(dense[s]["k"]).permute(1, 0, 2).repeat_interleave(G, dim=0)
            v = torch.from_numpy(dense[s]["v"]).permute(1, 0, 2).repeat_interleave(G, dim=0)
            pos = torch.arange(n) + (L - n)
            mask = torch.arange(L)[None, :] <= pos[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(t.scale))
            ref = ref.permute(1, 0, 2).reshape(n * t.hq, t.d).numpy()
            got = out[i:i + n * t.hq]
            i += n * t.hq
            assert np.abs(got - ref).max() <= 1e-9, f"seed {seed} seq {s}: {np.abs(got - ref).max()}"


def pin_int8_append_matches_indexing(orc):
    """kv_append into INT8 pools writes, at each new row's slot, exactly the
    quantiser's codes and scale of that row (placed by plain numpy indexing)
    and touches no other slot."""
    rng = np.random.default_rng(94)
    t = Tiny(rng, 3, 4, 2, 8, 4, [9, 14, 3], [1, 1, 1])
    kc, vc, ks, vs = int8_pools(t.kp.shape)
    ctx = np.array([2, 5, 0], np.int32)
    cu = np.concatenate([[0], np.cumsum(t.seq_lens - ctx)]).astype(np.int32)
    k_new = np.concatenate([t.k[s][ctx[s]:] for s in range(3)])
    v_new = np.concatenate([t.v[s][ctx[s]:] for s in range(3)])
    orc.kv_append_int8(kc, vc, ks, vs, k_new, v_new, cu, ctx, t.table)
    ekc, evc, eks, evs = int8_pools(t.kp.shape)
    for s in range(3):
        for name, rows, codes, scales in (("k", t.k[s], ekc, eks), ("v", t.v[s], evc, evs)):
            c, sc = orc.quantize_int8(rows[ctx[s]:])
            for i in range(c.shape[0]):
                p = int(ctx[s]) + i
                codes[t.table[s][p // t.bs], :, p % t.bs, :] = c[i]
                scales[t.table[s][p // t.bs], :, p % t.bs] = sc[i]
    assert np.array_equal(kc, ekc) and np.array_equal(vc, evc)
    assert np.array_equal(ks, eks, equal_nan=True) and np.array_equal(vs, evs, equal_nan=True)


def int8_decode_bound(q, seq_lens, block_table, bf16_pools, int8_pools, scale):
    """How far decode over the INT8 cache may lie from decode over the bf16
    cache it was quantised from, per output row (s, h): with every score
    moved by at most Delta = scale * max_k sum_d |q_d| |k_d - k^_d| and every
    value by at most eps_v = max |v - v^|, the softmax weights change by a
    factor within exp(+-2 Delta), so |O^ - O| <= eps_v + (exp(2 Delta) - 1) max|v|.
    Returns fp64 [S][Hq]."""
    K, V = bf16_pools
    kc, vc, ks, vs = int8_pools
    S, Hq, D = q.shape
    Hkv, B = K.shape[1], K.shape[2]
    G = Hq // Hkv
    qf = bf16_to_f64(q)
    out = np.zeros((S, Hq))
    for s in range(S):
        L = int(seq_lens[s])
        if L == 0:
            continue
        pos = np.arange(L)
        blk, slot = block_table[s][pos // B], pos % B
        Kb, Vb = bf16_to_f64(K[blk, :, slot, :]), bf16_to_f64(V[blk, :, slot, :])  # [L][Hkv][D]
        Kq = kc[blk, :, slot, :].astype(np.float64) * ks[blk, :, slot].astype(np.float64)[..., None]
        Vq = vc[blk, :, slot, :].astype(np.float64) * vs[blk, :, slot].astype(np.float64)[..., None]
        for g in range(Hkv):
            delta = float(scale) * (np.abs(Kb[:, g] - Kq[:, g]) @ np.abs(qf[s, g * G:(g + 1) * G]).T).max(axis=0)
            eps_v = np.abs(Vb[:, g] - Vq[:, g]).max()
            out[s, g * G:(g + 1) * G] = eps_v + np.expm1(2 * delta) * np.abs(Vb[:, g]).max()
    return out


def pin_int8_error_within_bound(orc):
    """Decode over the INT8 cache (rows quantised by the oracle's append)
    stays within the quantisation bound of decode over the bf16 cache, and
    the bound is not vacuous."""
    rng = np.random.default_rng(95)
    t = Tiny(rng, 3, 8, 2, 64, 32, [70, 1, 33], [1, 1, 1])
    kc, vc, ks, vs = int8_pools(t.kp.shape)
    cu = np.concatenate([[0], np.cumsum(t.seq_lens)]).astype(np.int32)
    orc.kv_append_int8(kc, vc, ks, vs, np.concatenate(t.k), np.concatenate(t.v), cu, np.zeros(3, np.int32), t.table)
    q = t.q.reshape(3, t.hq, t.d)
    exact = orc.decode(q, t.kp, t.vp, t.table, t.seq_lens, t.scale)
    quant = orc.decode_int8(q, kc, vc, ks, vs, t.table, t.seq_lens, t.scale)
    bound = int8_decode_bound(q, t.seq_lens, t.table, (t.kp, t.vp), (kc, vc, ks, vs), t.scale)
    with np.errstate(invalid="ignore"):  # a planted mistake may make either side non-finite
        err = np.abs(quant - exact).max(axis=2)
    assert (err <= bound + 1e-12).all(), f"worst ratio {np.max(err / bound)}"
    assert 0 < err.max() and bound.max() < 1.0, (err.max(), bound.max())  # well below max|v| (about 3)


# ----------------------------------------------------------------------------
# fused QKV projection + paged append
# ----------------------------------------------------------------------------

def _qkv_case(rng, hq, hkv, d, bs, ctx_lens, new_lens):
    """Placement of a few sequences' new rows: table, cu_new_lens, and each
    packed row's (sequence, position)."""
    S = len(ctx_lens)
    ends = [c + n for c, n in zip(ctx_lens, new_lens)]
    nblk = [-(-e // bs) for e in ends]
    mbs = max(nblk)
    nb = sum(nblk) + 2
    perm = rng.permutation(nb).astype(np.int32)
    table = np.full((S, mbs), -1, np.int32)
    o = 0
    for s in range(S):
        table[s, :nblk[s]] = perm[o:o + nblk[s]]
        o += nblk[s]
    cu = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int32)
    where = [(s, ctx_lens[s] + i) for s in range(S) for i in range(new_lens[s])]
    return table, cu, np.asarray(ctx_lens, np.int32), nb, where


def pin_qkv_selection_weights(orc):
    """With a merged weight whose rows each pick one input feature (scaled by
    a power of two), the projection is exact: q, k and v are those features,
    and k / v land at each row's slot (placed here by plain indexing)."""
    rng = np.random.default_rng(101)
    hq, hkv, d, bs, dm = 4, 2, 8, 4, 64
    n_out = (hq + 2 * hkv) * d
    table, cu, ctx, nb, where = _qkv_case(rng, hq, hkv, d, bs, [3, 0, 6], [2, 5, 1])
    T = int(cu[-1])
    x = bf16_normal(rng, (T, dm))
    pick = rng.permutation(dm)[:n_out] if n_out <= dm else rng.integers(dm, size=n_out)
    mult = 2.0 ** (np.arange(n_out) % 3)
    wf = np.zeros((n_out, dm), np.float32)
    wf[np.arange(n_out), pick] = mult
    kp = np.full((nb, hkv, bs, d), NAN_SENTINEL, np.uint16)
    vp = kp.copy()
    q = orc.qkv_project_append(kp, vp, x, to_bf16_exact(wf), cu, ctx, table, hq)
    y = to_bf16_exact(bf16_to_f64(x)[:, pick] * mult)  # exact: a power-of-two multiple of a bf16 value
    assert np.array_equal(q.reshape(T, -1), y[:, :hq * d])
    ek = np.full_like(kp, NAN_SENTINEL)
    ev = np.full_like(vp, NAN_SENTINEL)
    for t, (s, pos) in enumerate(where):
        ek[table[s][pos // bs], :, pos % bs, :] = y[t, hq * d:(hq + hkv) * d].reshape(hkv, d)
        ev[table[s][pos // bs], :, pos % bs, :] = y[t, (hq + hkv) * d:].reshape(hkv, d)
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev)


def _assert_nearest_bf16(got_bits, y):
    """Each got value is the bf16 number nearest to the exact y (ties to the
    even last bit), checked through the floor of y on the bf16 grid of its
    binade (a formulation of its own, independent of the oracle's)."""
    g = bf16_to_f64(got_bits)
    for a, b in zip(g.ravel(), np.asarray(y, np.float64).ravel()):
        if b == 0:
            assert a == 0
            continue
        e = math.floor(math.log2(abs(b)))
        if 2.0 ** e > abs(b):
            e -= 1
        sp = 2.0 ** (max(e, -126) - 7)
        lo = math.floor(b / sp) * sp
        hi = lo + sp
        if b - lo < hi - b:
            want = lo
        elif hi - b < b - lo:
            want = hi
        else:
            want = lo if int(round(lo / sp)) % 2 == 0 else hi
        assert a == want, f"got {a}, exact {b}, nearest {want}"


def pin_qkv_rounds_the_exact_product_to_nearest(orc):
    """Random inputs and weights: every output is the bf16 number nearest to
    the exact dot product (numpy fp64: exact for these few bf16 terms), and
    k / v sit where kv_append would put those rows."""
    rng = np.random.default_rng(102)
    hq, hkv, d, bs, dm = 2, 1, 16, 16, 96
    table, cu, ctx, nb, where = _qkv_case(rng, hq, hkv, d, bs, [15, 1], [3, 2])
    T = int(cu[-1])
    x = bf16_normal(rng, (T, dm))
    w = bf16_normal(rng, ((hq + 2 * hkv) * d, dm))
    kp = np.full((nb, hkv, bs, d), NAN_SENTINEL, np.uint16)
    vp = kp.copy()
    q = orc.qkv_project_append(kp, vp, x, w, cu, ctx, table, hq)
    y = bf16_to_f64(x) @ bf16_to_f64(w).T
    got = np.zeros((T, (hq + 2 * hkv) * d), np.uint16)
    got[:, :hq * d] = q.reshape(T, -1)
    for t, (s, pos) in enumerate(where):
        got[t, hq * d:(hq + hkv) * d] = kp[table[s][pos // bs], :, pos % bs, :].ravel()
        got[t, (hq + hkv) * d:] = vp[table[s][pos // bs], :, pos % bs, :].ravel()
    _assert_nearest_bf16(got, y)


ALL_PINS = [pin_all_golden, pin_vs_sdpa, pin_vs_dense, pin_constant_v, pin_scale_zero_mean, pin_single_key,
            pin_empty_sequence, pin_block_permutation, pin_block_size_16_vs_256, pin_decode_is_last_prefill_row,
            pin_chunked_equals_unchunked, pin_gqa_is_expanded_mha, pin_head_permutation_in_group,
            pin_append_matches_indexing, pin_append_rejects_duplicate_slot, pin_int8_quantizer_bounds,
            pin_int8_quantizer_symmetries, pin_int8_attention_vs_sdpa, pin_int8_append_matches_indexing,
            pin_int8_error_within_bound, pin_qkv_selection_weights, pin_qkv_rounds_the_exact_product_to_nearest]
