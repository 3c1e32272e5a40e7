"""The oracle's pins catch plausible mistakes (no GPU).

Each case plants one mistake in a copy of oracle/oracle.c (a dropped term, a
wrong sign, index or layout, a transposed operand), builds it on the CPU into
a temporary library and runs tests/test_oracle_pins.py,
tests/test_oracle_fp8.py, tests/test_oracle_blocks.py and
tests/test_oracle_prefill.py against that library in a subprocess.  The pin suite must fail for every mutant and pass for the
unmodified copy.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_oracle_fp8.py"),
        os.path.join(ROOT, "tests", "test_oracle_blocks.py"),
        os.path.join(ROOT, "tests", "test_oracle_prefill.py"),
        os.path.join(ROOT, "tests", "test_oracle_prefill_fp8.py")]

# (name, original text, planted text) -- the first occurrence is replaced
MUTANTS = [
    ("scale_dropped", "x[t] = scale * dot;", "x[t] = dot;"),
    ("gqa_modulo", "int kv_head = h / group;", "int kv_head = h % num_kv_heads;"),
    ("block_index_mod", "int64_t block = table[t / block_size];",
     "int64_t block = table[(t / block_size) % 2];"),
    ("max_not_subtracted", "x[t] = exp(x[t] - m);", "x[t] = exp(x[t]);"),
    ("softmax_sign", "x[t] = exp(x[t] - m);", "x[t] = exp(m - x[t]);"),
    ("not_normalised", "for (int d = 0; d < head_dim; ++d) out_row[d] /= z;", ""),
    ("first_token_dropped",
     "for (int64_t t = 0; t < len; ++t) {\n    int64_t block = table[t / block_size];\n    int offset",
     "for (int64_t t = 1; t < len; ++t) {\n    int64_t block = table[t / block_size];\n    int offset"),
    ("v_read_token_major",
     "int64_t vi = v_index(block, kv_head, offset, d, num_kv_heads, block_size, head_dim);",
     "int64_t vi = ((block * num_kv_heads + kv_head) * (int64_t)block_size + offset) *\n"
     "                       head_dim + d;"),
    # a consistent but different V layout (writes and reads move together)
    ("v_both_token_major",
     "return slice + ((int64_t)(offset / 4) * head_dim + dim) * 4 + offset % 4;",
     "return slice + (int64_t)offset * head_dim + dim;"),
    ("v_both_dim_major",
     "return slice + ((int64_t)(offset / 4) * head_dim + dim) * 4 + offset % 4;",
     "return slice + (int64_t)dim * block_size + offset;"),
    ("k_offset_shift", "(int)(t % block_size)) * head_dim;",
     "(int)((t + 1) % block_size)) * head_dim;"),
    # E4M3 coding and the FP8 append
    ("e4m3_bias", "expo - 10); /* 1.frac", "expo - 9); /* 1.frac"),
    ("e4m3_ties_up", "(above == below && fmod(n, 2.0) != 0.0)", "(above == below)"),
    ("e4m3_no_saturation", "if (a >= 448.0) return (uint8_t)((sign << 7) | 0x7e);",
     "if (a >= 448.0) return (uint8_t)((sign << 7) | 0x7f);"),
    ("e4m3_subnormal_step", "u = ldexp(1.0, -9);\n", "u = ldexp(1.0, -8);\n"),
    ("fp8_scale_multiplied", "float kx = (float)decode(k[src], dtype) * k_inv;",
     "float kx = (float)decode(k[src], dtype) * k_scale;"),
    ("fp8_v_scale_for_k",
     "return oracle_e4m3_to_f64(((const uint8_t *)cache)[index]) * scale;",
     "return oracle_e4m3_to_f64(((const uint8_t *)cache)[index]);"),
    ("f16_bias", "expo - 25); /* 1.frac", "expo - 24); /* 1.frac"),
    ("bf16_bias", "expo - 134); /* 1.frac", "expo - 133); /* 1.frac"),
    ("f16_sign_dropped", "return sign ? -mag : mag;", "return mag;"),
    ("merge_not_rescaled", "double c = pl[p] * exp(pm[p] - big);", "double c = pl[p];"),
    ("q_index_transposed", "const uint16_t *qrow = q + ((int64_t)s * num_heads + h) * head_dim;",
     "const uint16_t *qrow = q + ((int64_t)h * num_seqs + s) * head_dim;"),
    ("write_offset_shift", "int offset = (int)(slot % block_size);",
     "int offset = (int)((slot + 1) % block_size);"),
    ("copy_first_head_only", "for (int j = 0; j < num_kv_heads; ++j)\n      for (int o = 0; o < block_size; ++o)",
     "for (int j = 0; j < 1; ++j)\n      for (int o = 0; o < block_size; ++o)"),
    ("copy_v_token_major",
     "int64_t vd = v_index(dst, j, o, d, num_kv_heads, block_size, head_dim);",
     "int64_t vd = (((dst * num_kv_heads + j) * (int64_t)block_size + o) * head_dim + d);"),
    ("copy_reversed", "memcpy(kc + kd * elem_bytes, kc + ks * elem_bytes, (size_t)elem_bytes);",
     "memcpy(kc + ks * elem_bytes, kc + kd * elem_bytes, (size_t)elem_bytes);"),
    ("copy_accepts_dst_as_src", "    if (role[b] == 3) {", "    if (role[b] == 7) {"),
    ("swap_reads_destination", "memcpy(dk + kd * elem_bytes, sk + ks * elem_bytes, (size_t)elem_bytes);",
     "memcpy(dk + kd * elem_bytes, sk + kd * elem_bytes, (size_t)elem_bytes);"),
    ("swap_v_skipped", "memcpy(dv + vd * elem_bytes, sv + vs * elem_bytes, (size_t)elem_bytes);", ""),
    ("prefill_sees_own_position_not", "int64_t p = len - n + i; /* the row's own position",
     "int64_t p = len - n + i - (i > 0); /* the row's own position"),
    ("prefill_position_from_chunk_start", "int64_t p = len - n + i; /* the row's own position",
     "int64_t p = (len - n + i) % (n + 1); /* the row's own position"),
    ("prefill_gqa_modulo", "int kv_head = h / group;\n        const uint16_t *qrow = q + ((row0",
     "int kv_head = h % num_kv_heads;\n        const uint16_t *qrow = q + ((row0"),
    ("prefill_sees_next_token", "int64_t p = len - n + i; /* the row's own position",
     "int64_t p = len - n + i + (i + 1 < n); /* the row's own position"),
    ("prefill_fp8_v_takes_k_scale",
     "orow[d] += x[t] * cache_value(v_cache, vi, cache_dtype, v_scale);",
     "orow[d] += x[t] * cache_value(v_cache, vi, cache_dtype, k_scale);"),
    ("prefill_fp8_k_scale_dropped",
     "dot += decode(qrow[d], dtype) * cache_value(k_cache, krow + d, cache_dtype, k_scale);",
     "dot += decode(qrow[d], dtype) * cache_value(k_cache, krow + d, cache_dtype, 1.0);"),
]
# planted edits that need a second, matching one elsewhere
EXTRA = {}


def _build_variant(tmp, name, old, new):
    src = open(oracle.SRC).read()
    if old is not None:
        assert old in src, name
        src = src.replace(old, new, 1)
        if name in EXTRA:
            o2, n2 = EXTRA[name]
            assert o2 in src
            src = src.replace(o2, n2, 1)
    c = os.path.join(tmp, f"{name}.c")
    open(c, "w").write(src)
    return oracle.build(c, os.path.join(tmp, f"lib{name}.so"))


def _run_pins(lib):
    env = dict(os.environ, PAGED_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p",
                        "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_pins_catch_every_mutant(tmp_path):
    tmp = str(tmp_path)
    jobs = [("control", None, None)] + MUTANTS
    libs = {name: _build_variant(tmp, name, old, new) for name, old, new in jobs}
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip(libs, ex.map(_run_pins, libs.values())))
    rc, out = results.pop("control")
    assert rc == 0, out
    survivors = [n for n, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"mutants not caught by the pins: {survivors}"
