"""Plant plausible mistakes in a copy of the oracle source; the pins must catch each.

Every mutant is compiled from a textual edit of ``oracle/mla_oracle.c`` into a
temporary library and checked by ``oracle_pins.py`` in a child process (so a
mutant that crashes cannot take the test run down). A mutant passes every pin
only if the pins are blind to that mistake, which fails this test.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

# (name, text in mla_oracle.c, replacement)
MUTANTS = [
    ("slot_index_swapped", "* block_size +\n                    t % block_size;\n      load_token(kv_cache, kv_fp8, kvs, row, k);\n      double dot",
     "* block_size +\n                    (t + 1) % block_size;\n      load_token(kv_cache, kv_fp8, kvs, row, k);\n      double dot"),
    ("page_index_off_by_one", "block_table[b * max_blocks + t / block_size] * block_size +\n                    t % block_size;\n      load_token(kv_cache, kv_fp8, kvs, row, k);\n      double wt",
     "block_table[b * max_blocks + (t + 1) / block_size] * block_size +\n                    t % block_size;\n      load_token(kv_cache, kv_fp8, kvs, row, k);\n      double wt"),
    ("rope_dropped", "for (int d = 0; d < ORACLE_D; ++d) dot += qv[d] * k[d];",
     "for (int d = 0; d < ORACLE_DV; ++d) dot += qv[d] * k[d];"),
    ("values_from_rope_side", "o[d] += wt * k[d];", "o[d] += wt * k[d + 64];"),
    ("scale_dropped", "x[t - t0] = s * dot;", "x[t - t0] = dot;"),
    ("weight_sign", "exp(x[t - t0] - m)", "exp(m - x[t - t0])"),
    ("lse_log2", "lse[row_out] = m + log(l);", "lse[row_out] = m + log2(l);"),
    ("lse_missing_max", "lse[row_out] = m + log(l);", "lse[row_out] = log(l);"),
    ("no_normalise", "for (int d = 0; d < ORACLE_DV; ++d) o[d] /= l;", ""),
    ("q_head_batch_transposed", "q[((b * q_len + qi) * num_heads + h) * ORACLE_D + d]",
     "q[(((h % batch) * q_len + qi) * num_heads + (b % num_heads)) * ORACLE_D + d]"),
    ("q_token_head_transposed", "q[((b * q_len + qi) * num_heads + h) * ORACLE_D + d]",
     "q[((b * num_heads + h) * q_len + qi) * ORACLE_D + d]"),
    ("causal_off_by_one", "int64_t visible = n - (q_len - 1 - qi);",
     "int64_t visible = n - (q_len - qi);"),
    ("causal_reversed", "int64_t visible = n - (q_len - 1 - qi);",
     "int64_t visible = n - qi;"),
    ("causal_ignored", "if (t1 > visible) t1 = visible;", ""),
    ("sparse_skip_bound", "if (t < 0 || t >= n) continue;\n      int64_t row",
     "if (t < 0 || t > n) continue;\n      int64_t row"),
    ("sparse_weight_index", "double wt = exp(x[j] - m);", "double wt = exp(x[0] - m);"),
    ("sparse_q_row", "qv[d] = bf16_bits_to_double(q[(b * num_heads + h) * ORACLE_D + d]);",
     "qv[d] = bf16_bits_to_double(q[((h % batch) * num_heads + (b % num_heads)) * ORACLE_D + d]);"),
    ("sparse_scale_dropped", "x[j] = s * dot;", "x[j] = dot;"),
    ("gemm_neighbour_element", "e4m3[a[i * k + t]]", "e4m3[a[i * k + (t ^ 1)]]"),
    ("gemm_weight_scale_group0", "(double)b_scale[(j / 128) * kg + t / 128]",
     "(double)b_scale[(j / 128) * kg]"),
    ("gemm_act_scale_group0", "(double)a_scale[i * kg + t / 128]", "(double)a_scale[i * kg]"),
    ("absorb_weight_transposed", "bf16_bits_to_double(w[(h * k_in + i) * n_out + j])",
     "bf16_bits_to_double(w[(h * k_in + (i + j) % k_in) * n_out + j])"),
    ("absorb_head_zero", "int64_t h = bh % heads;", "int64_t h = 0;"),
    ("out_row_token_head_transposed", "int64_t row_out = (i * q_len + qi) * num_heads + h;",
     "int64_t row_out = (i * num_heads + h) * q_len + qi;"),
    ("e4m3_bias", "exponent - 7);", "exponent - 8);"),
    ("e4m3_subnormal", "ldexp((double)mantissa / 8.0, -6)", "ldexp((double)mantissa / 8.0, -7)"),
    ("kv_scale_dropped", "k[d] = e4m3[p[d]] * kv_scale;", "k[d] = e4m3[p[d]];"),
    ("merge_weight_sign", "double w = exp(ls - M);", "double w = exp(M - ls);"),
    ("merge_unnormalised", "for (int d = 0; d < ORACLE_DV; ++d) o[d] /= wsum;", ""),
    ("tail_overread", "if (t1 > visible) t1 = visible;\n    int64_t row_out",
     "if (t1 > visible) t1 = visible;\n    if (t1 == n && t1 % block_size) t1 = (t1 / block_size + 1) * block_size;\n    int64_t row_out"),
]


def test_mutant_list_applies():
    src = open(oracle.SOURCE).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) >= 1, f"mutant {name} no longer matches the oracle source"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert old in src
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / f"{name}.c"
    c_path.write_text(mutated)
    lib = tmp_path / f"lib{name}.so"
    oracle.build(str(c_path), str(lib))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), "--lib", str(lib)],
                       capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode != 0, f"no pin caught mutant {name}:\n{r.stdout}\n{r.stderr}"
