"""Plant plausible mistakes in copies of the oracle's C source and check that at
least one pin fails for each: the pins are strong enough to catch a dropped
term, a wrong sign or index, a transposed operand or a bad rounding.

Each mutant is a textual substitution applied to oracle/pagedkv_ref.c, compiled
with gcc into a temporary library and loaded through ``oracle.ref.Oracle`` in a
child process (a mutant that reads out of bounds may crash; that counts as
caught).  Everything runs on the CPU.
"""
import json
import os
import subprocess
import sys
import warnings

import numpy as np
import pytest

import oracle_pins
from oracle import build_oracle, ref

MUTANTS = [
    ("slot: offset uses i / B", "+ (i % block_size);", "+ (i / block_size);"),
    ("slot: table indexed by i mod B", "table_row[i / block_size]", "table_row[i % block_size]"),
    ("slot: block not scaled by B", "(int64_t)table_row[i / block_size] * block_size",
     "(int64_t)table_row[i / block_size]"),
    ("row offset drops the head", "return (slot * n_kv_heads + g) * (int64_t)head_dim;",
     "return (slot * n_kv_heads) * (int64_t)head_dim;"),
    ("row offset transposes slot and head", "return (slot * n_kv_heads + g) * (int64_t)head_dim;",
     "return (g * n_kv_heads + slot) * (int64_t)head_dim;"),
    ("GQA: interleaved head mapping",
     "const int32_t g = h / (P->n_q_heads / P->n_kv_heads);\n    const int32_t* row = P->block_tables + (int64_t)s * P->max_blocks_per_seq;\n    const int64_t qoff",
     "const int32_t g = h % P->n_kv_heads;\n    const int32_t* row = P->block_tables + (int64_t)s * P->max_blocks_per_seq;\n    const int64_t qoff"),
    ("scale dropped", "z[i] = P->scale * dot;", "z[i] = dot;"),
    ("softmax sign flipped", "double w = exp(z[i] - m);", "double w = exp(m - z[i]);"),
    ("no normalisation", "for (int32_t d = 0; d < D; ++d) out_row[d] /= sum_w;",
     "for (int32_t d = 0; d < D; ++d) out_row[d] /= 1.0;"),
    ("last token dropped", "ref_weighted_values(P, s, h, z, 0, L, m, out_row);",
     "ref_weighted_values(P, s, h, z, 0, L - 1, m, out_row);"),
    ("q row of the wrong sequence", "const int64_t qoff = ((int64_t)s * P->n_q_heads + h) * D;",
     "const int64_t qoff = ((int64_t)h) * D;"),
    ("value read from the key cache",
     "out_row[d] += w * ref_load(P->v_cache, voff + d, P->dtype);",
     "out_row[d] += w * ref_load(P->k_cache, voff + d, P->dtype);"),
    ("merge drops l_j", "double w = l[j] * exp(m[j] - M);", "double w = exp(m[j] - M);"),
    ("merge sign flipped", "double w = l[j] * exp(m[j] - M);", "double w = l[j] * exp(M - m[j]);"),
    ("partition end off by one", "int32_t hi = lo + part_tokens < L ? lo + part_tokens : L;",
     "int32_t hi = lo + part_tokens < L ? lo + part_tokens - 1 : L;"),
    ("f16 subnormal scale", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("f16 exponent bias", "v = ldexp((double)(1024 + m), e - 25);",
     "v = ldexp((double)(1024 + m), e - 24);"),
    ("bf16 bits misplaced", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("encode truncates", "double r = nearbyint(q);", "double r = floor(q);"),
    ("encode rounds half away from zero", "double r = nearbyint(q);", "double r = round(q);"),
    ("encode misses the binade carry", "if (r >= 2.0 * one) {", "if (r > 2.0 * one) {"),
    ("append copies row 0 for everyone", "(const char*)k_new + s * row_bytes", "(const char*)k_new"),
    ("append writes one slot late", "const int64_t slot = ref_physical_slot(row, block_size, p);",
     "const int64_t slot = ref_physical_slot(row, block_size, p) + 1;"),
    ("L = 0 not handled", "    if (L <= 0) {\n        for (int32_t d = 0; d < D; ++d) out_row[d] = 0.0;\n        return;\n    }\n    ref_scores",
     "    ref_scores"),
    ("copy drops the last filled row", "for (int32_t r = 0; r < n_rows[i]; ++r) {",
     "for (int32_t r = 0; r < n_rows[i] - 1; ++r) {"),
    ("copy runs backwards (destination into source)",
     "memcpy((char*)k_cache + to * row_bytes, (const char*)k_cache + from * row_bytes, row_bytes);",
     "memcpy((char*)k_cache + from * row_bytes, (const char*)k_cache + to * row_bytes, row_bytes);"),
    ("copy forgets the value cache",
     "            memcpy((char*)v_cache + to * row_bytes, (const char*)v_cache + from * row_bytes, row_bytes);\n",
     ""),
    ("copy target not scaled by B", "const int64_t to = (int64_t)dst[i] * block_size + r;",
     "const int64_t to = (int64_t)dst[i] + r;"),
    ("copy moves whole blocks whatever n_rows", "for (int32_t r = 0; r < n_rows[i]; ++r) {",
     "for (int32_t r = 0; r < (n_rows[i] ? block_size : 0); ++r) {"),
    ("prefill query misses its own key", "h / group, pos + 1, z,", "h / group, pos, z,"),
    ("prefill query sees the whole chunk (no causal mask)", "h / group, pos + 1, z,",
     "h / group, context_lens[s], z,"),
    ("prefill position ignores the earlier context",
     "const int32_t pos = context_lens[s] - n + (int32_t)(t - cu_q[s]);",
     "const int32_t pos = (int32_t)(t - cu_q[s]);"),
    ("prefill GQA: interleaved head mapping", "h / group, pos + 1, z,", "h % n_kv_heads, pos + 1, z,"),
    ("n-token append ignores the start position",
     "ref_physical_slot(row, block_size, (int64_t)start_pos[s] + (j - cu_new[s]));",
     "ref_physical_slot(row, block_size, (int64_t)(j - cu_new[s]));"),
    ("swap moves one row too few", "        for (int32_t r = 0; r < block_size; ++r) {\n            const int64_t slot = (int64_t)blocks[i] * block_size + r; /* row r of the block */",
     "        for (int32_t r = 0; r < block_size - 1; ++r) {\n            const int64_t slot = (int64_t)blocks[i] * block_size + r; /* row r of the block */"),
    ("swap ignores the block list", "const int64_t slot = (int64_t)blocks[i] * block_size + r; /* row r of the block */",
     "const int64_t slot = (int64_t)i * block_size + r; /* row r of the block */"),
    ("swap in writes the host slot into every row's first slot",
     "const int64_t h = (int64_t)i * block_size + r;            /* row r of host slot i */",
     "const int64_t h = (int64_t)i * block_size;            /* row r of host slot i */"),
    ("n-token append repeats the chunk's first row",
     "memcpy((char*)k_cache + slot * row_bytes, (const char*)k_new + j * row_bytes, row_bytes);",
     "memcpy((char*)k_cache + slot * row_bytes, (const char*)k_new + cu_new[s] * row_bytes, row_bytes);"),
]


def _failing_pins(orc):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                with np.errstate(all="ignore"):
                    pin(orc)
        except Exception as e:  # an assertion, or the mutant rejecting inputs
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.fixture(scope="module")
def source():
    with open(build_oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new, tmp_path):
    assert source.count(old) >= 1, "mutation site not found: %r" % old
    mutated = source.replace(old, new, 1)
    src = os.path.join(tmp_path, "mutant.c")
    lib = os.path.join(tmp_path, "libmutant.so")
    with open(src, "w") as f:
        f.write(mutated)
    build_oracle.build(src=src, lib=lib)
    here = os.path.dirname(os.path.abspath(__file__))
    script = ("import sys, json; sys.path[:0] = [%r, %r]; import test_oracle_mutants as t; "
              "from oracle import ref; print(json.dumps(t._failing_pins(ref.Oracle(%r))))"
              % (here, os.path.dirname(here), lib))
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, OMP_NUM_THREADS="1"))
    if r.returncode < 0:
        return  # the mutant crashed the process (a signal): caught
    assert r.returncode == 0, r.stderr[-2000:]
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, "no pin caught the mutant %r" % name


def test_unmutated_passes_all():
    assert _failing_pins(ref.default()) == []
