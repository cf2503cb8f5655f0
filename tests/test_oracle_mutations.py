"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies the oracle's C source, plants one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand), compiles the copy
into a temporary library and runs every pin against it; at least one pin must
fail.  The real oracle is never modified.
"""
import os

import pytest

import oracle
import oracle_pins as P

MUTATIONS = {
    "gqa_interleaved_heads": ("p, h / group, num_kv_heads", "p, h % num_kv_heads, num_kv_heads"),
    "mask_excludes_diagonal": ("const int nkeys = p + 1;", "const int nkeys = p;"),
    "mask_top_left_aligned": ("int p = seq_lens[s] - n + r;", "int p = r;"),
    "no_max_subtraction": ("z[j] = exp(z[j] - zmax);", "z[j] = exp(z[j]);"),
    "scale_dropped": ("z[j] = scale * dot;", "z[j] = dot;"),
    "block_index_modulo": ("int blk = table_row[j / block_size];\n        if (blk < 0",
                           "int blk = table_row[j % block_size];\n        if (blk < 0"),
    "no_normalisation": ("out_row[d] /= denom;", "out_row[d] /= 1.0;"),
    "pool_head_major": ("size_t krow = ((size_t)blk * num_kv_heads + kv_head) * block_size",
                        "size_t krow = ((size_t)kv_head * num_blocks + blk) * block_size"),
    "v_wrong_head": ("size_t vrow = ((size_t)blk * num_kv_heads + kv_head)",
                     "size_t vrow = ((size_t)blk * num_kv_heads + 0)"),
    "q_row_ignores_offset": ("(size_t)(cu_q_lens[s] + r) * num_q_heads + h", "(size_t)r * num_q_heads + h"),
    "append_ignores_ctx": ("long pos = (long)ctx_lens[s] + (t - cu_new_lens[s]);",
                           "long pos = (long)(t - cu_new_lens[s]);"),
    "append_v_from_k": ("memcpy(v_pool + dst, v_new + src", "memcpy(v_pool + dst, k_new + src"),
    "append_slot_off_by_one": ("long slot = pos % block_size;", "long slot = (pos + 1) % block_size;"),
    "int8_scale_over_128": ("float scale = amax / 127.0f;", "float scale = amax / 128.0f;"),
    "int8_round_half_away": ("rintf(bf16_to_float(row[d]) / scale)", "roundf(bf16_to_float(row[d]) / scale)"),
    "int8_truncate": ("rintf(bf16_to_float(row[d]) / scale)", "truncf(bf16_to_float(row[d]) / scale)"),
    "int8_dequant_drops_scale": ("(double)pool->codes[row * head_dim + d] * (double)pool->scales[row]",
                                 "(double)pool->codes[row * head_dim + d]"),
    "int8_scale_of_wrong_row": ("(double)pool->scales[row]", "(double)pool->scales[row ^ 1]"),
    "int8_append_v_from_k": ("v_scales + row, v_new + src", "v_scales + row, k_new + src"),
    "qkv_weight_transposed": ("acc += bf16_to_double(xt[k]) * bf16_to_double(wn[k]);",
                              "acc += bf16_to_double(xt[k]) * bf16_to_double(w[(size_t)k * n_out + n]);"),
    "qkv_k_from_q_slice": ("memcpy(k_pool + dst, y + nq + (size_t)g * head_dim",
                           "memcpy(k_pool + dst, y + (size_t)g * head_dim"),
    "qkv_v_from_k_slice": ("memcpy(v_pool + dst, y + nq + nkv + (size_t)g * head_dim",
                           "memcpy(v_pool + dst, y + nq + (size_t)g * head_dim"),
    "qkv_round_truncates": ("ldexp(nearbyint(ldexp(a, -q)), q)", "ldexp(trunc(ldexp(a, -q)), q)"),
    "qkv_round_half_away": ("ldexp(nearbyint(ldexp(a, -q)), q)", "ldexp(round(ldexp(a, -q)), q)"),
    "softmax_sum_skips_last": ("for (int j = 0; j < nkeys; ++j) {\n        z[j] = exp",
                               "for (int j = 0; j < nkeys - 1; ++j) {\n        z[j] = exp"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant_src), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, oracle.OracleError) as e:  # a pin failed: the mistake is visible
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
    os.remove(lib)
