"""Plant one mistake at a time in a copy of the oracle's C source and check that
the pins catch every one. This guards the pins themselves: a pin set that lets a
dropped term, a wrong sign or a transposed index through is not a pin set."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

# (name, text in pa_oracle.c, replacement, occurrences expected)
MUTANTS = [
    ("copy_direction", "memcpy(key_cache + dst * block_bytes, key_cache + src * block_bytes,",
     "memcpy(key_cache + src * block_bytes, key_cache + dst * block_bytes,", 1),
    ("copy_v_from_k", "memcpy(value_cache + dst * block_bytes, value_cache + src * block_bytes,",
     "memcpy(value_cache + dst * block_bytes, key_cache + src * block_bytes,", 1),
    ("swap_half_block", "memcpy(dst_key + dst * block_bytes, src_key + src * block_bytes, (size_t)block_bytes);",
     "memcpy(dst_key + dst * block_bytes, src_key + src * block_bytes, (size_t)block_bytes / 2);", 1),
    ("swap_v_from_k", "memcpy(dst_value + dst * block_bytes, src_value + src * block_bytes,",
     "memcpy(dst_value + dst * block_bytes, src_key + src * block_bytes,", 1),
    ("swap_skips_first_pair", "for (int64_t i = 0; i < num_pairs; ++i) {\n        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];\n        if (src < 0 || dst < 0)\n            continue;\n        memcpy(dst_key",
     "for (int64_t i = 1; i < num_pairs; ++i) {\n        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];\n        if (src < 0 || dst < 0)\n            continue;\n        memcpy(dst_key", 1),
    ("gqa_interleaved", "const int h = kv * group + g;", "const int h = g * num_kv_heads + kv;", 2),
    ("scale_dropped", "l[t] = scale * dot;", "l[t] = dot;", 1),
    ("exp_sign", "l[t] = exp(l[t] - m);", "l[t] = exp(m - l[t]);", 1),
    ("no_normalise", "const double w = l[t] / z;", "const double w = l[t];", 1),
    ("row_from_block_index", "+ t % block_size;", "+ t / block_size;", 1),
    ("layout_token_major", "int64_t row = (block * num_kv_heads + kv) * block_size + t % block_size;",
     "int64_t row = (block * block_size + t % block_size) * num_kv_heads + kv;", 1),
    ("table_ignored", "int64_t block = table_row[t / block_size];",
     "int64_t block = t / block_size;", 1),
    ("max_skips_first", "for (int t = 0; t < L; ++t)\n                if (l[t] > m)",
     "for (int t = 1; t < L; ++t)\n                if (l[t] > m)", 1),
    ("last_token_dropped", "for (int t = 0; t < L; ++t) {\n                const double w = l[t] / z;",
     "for (int t = 0; t < L - 1; ++t) {\n                const double w = l[t] / z;", 1),
    ("dot_term_dropped", "for (int d = 0; d < head_size; ++d)\n            dot +=",
     "for (int d = 1; d < head_size; ++d)\n            dot +=", 1),
    ("v_from_k_pool", "gather_head(V, value_cache,", "gather_head(V, key_cache,", 3),
    ("lse_sign", "const double w = sp[p] * exp(mp[p] - M);", "const double w = sp[p] * exp(M - mp[p]);", 1),
    ("partition_skips_token", "const int t0 = p * partition_size;",
     "const int t0 = p * partition_size + (p > 0);", 1),
    ("partition_unnormalised", "const double w = l[t] / sp[p];", "const double w = l[t];", 1),
    ("prefill_pos_off_by_one", "const int pos = L - nq + i;", "const int pos = L - nq + i - 1;", 1),
    ("prefill_pos_origin", "const int pos = L - nq + i;", "const int pos = i;", 1),
    ("prefill_no_causal_mask", "const int pos = L - nq + i;", "const int pos = L - 1;", 1),
    ("prefill_rows_reversed", "const int64_t row = (int64_t)query_start[s] + i;",
     "const int64_t row = (int64_t)query_start[s] + (nq - 1 - i);", 1),
    ("prefill_head_map", "const int head = kv * group + hh;",
     "const int head = hh * num_kv_heads + kv;", 1),
    ("scatter_offset", "int64_t offset = slot % block_size;", "int64_t offset = slot / block_size;", 1),
    ("scatter_kv_swap", "memcpy(value_cache + dst, value + src, row);",
     "memcpy(value_cache + dst, key + src, row);", 1),
    ("scatter_head_stride", "size_t src = (size_t)(i * num_kv_heads + h) * row;",
     "size_t src = (size_t)(i * num_kv_heads) * row;", 1),
]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, count, tmp_path):
    text = open(SRC).read()
    assert text.count(old) == count, f"mutation site for {name} not found as expected"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / f"lib{name}.so")))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError) as e:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
