"""Each plausible mistake planted in a copy of the oracle must fail at least one pin.

The mistakes are planted by text substitution in a temporary copy of
``oracle/oracle.c``, compiled with gcc, and the pins of ``oracle_pins.py`` run
against that build in a child process (a crash counts as detected).  The real
oracle source is never modified.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "oracle_pins.py")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("gqa-modulo-mapping", "const int g = h / group;", "const int g = h % num_kv_heads;"),
    ("gqa-wrong-group-size", "const int g = h / group;", "const int g = h / (group * 2);"),
    ("scale-dropped", "score[t] = scale * dot;", "score[t] = dot;"),
    ("scale-squared", "score[t] = scale * dot;", "score[t] = scale * scale * dot;"),
    ("context-one-short", "g, context_lens[s], num_kv_heads,",
     "g, context_lens[s] - (context_lens[s] > 1), num_kv_heads,"),
    ("context-one-long", "g, context_lens[s], num_kv_heads,",
     "g, context_lens[s] + (context_lens[s] % 16 != 0), num_kv_heads,"),
    ("v-read-row-major", "vtile[(long)d * block_size + off]", "vtile[off * head_dim + d]"),
    ("k-offset-dropped", "((long)(d / KCHUNK) * block_size + off) * KCHUNK",
     "((long)(d / KCHUNK) * block_size) * KCHUNK"),
    ("k-token-major-layout", "((long)(d / KCHUNK) * block_size + off) * KCHUNK + d % KCHUNK",
     "(off * (head_dim / KCHUNK) + d / KCHUNK) * KCHUNK + d % KCHUNK"),
    ("k-chunk-dims-reversed", "* KCHUNK + d % KCHUNK;", "* KCHUNK + (KCHUNK - 1 - d % KCHUNK);"),
    ("k-read-other-head", "dot += qv[d] * bf16_value(k_cache[k_index(blk, g, off, d,",
     "dot += qv[d] * bf16_value(k_cache[k_index(blk, (g + 1) % num_kv_heads, off, d,"),
    ("softmax-sign", "score[t] = exp(score[t] - m);", "score[t] = exp(m - score[t]);"),
    ("max-not-subtracted", "score[t] = exp(score[t] - m);", "score[t] = exp(score[t]);"),
    ("not-normalised", "double p = score[t] / l;", "double p = score[t];"),
    ("table-index-by-offset", "long blk = table_row[t / block_size];",
     "long blk = table_row[t % block_size];"),
    ("table-ignored", "long blk = table_row[t / block_size];", "long blk = t / block_size;"),
    ("query-of-group-leader", "qv[d] = bf16_value(q[pair * head_dim + d]);",
     "qv[d] = bf16_value(q[(pair - h + (h / group) * group) * head_dim + d]);"),
    ("dot-drops-last-dim", "for (int d = 0; d < head_dim; ++d)\n            dot +=",
     "for (int d = 0; d < head_dim - 1; ++d)\n            dot +="),
    ("max-is-first-score", "if (score[t] > m)\n            m = score[t];",
     "if (0)\n            m = score[t];"),
    ("write-v-row-major",
     "long vdst = ((blk * num_kv_heads + h) * head_dim + d) * block_size + off;",
     "long vdst = ((blk * num_kv_heads + h) * block_size + off) * head_dim + d;"),
    ("write-offset-zero", "long off = (long)(slot % block_size);", "long off = 0;"),
    ("write-head-swap",
     "long kdst = k_index(blk, h, off, d, num_kv_heads, head_dim, block_size);",
     "long kdst = k_index(blk, num_kv_heads - 1 - h, off, d, num_kv_heads, head_dim, block_size);"),
    ("write-keeps-padding", "if (slot < 0 || slot >= num_slots)\n            continue;\n        long blk",
     "if (slot >= num_slots)\n            continue;\n        if (slot < 0) slot = 0;\n        long blk"),
    ("copy-k-only", "v_cache[dst * block_elems + e] = v_cache[src * block_elems + e];", ";"),
    ("copy-direction-swapped", "k_cache[dst * block_elems + e] = k_cache[src * block_elems + e];",
     "k_cache[src * block_elems + e] = k_cache[dst * block_elems + e];"),
    ("copy-skips-nothing", "|| src == dst)\n            continue;\n        for (long e",
     ")\n            continue;\n        for (long e"),
    ("copy-half-block", "for (long e = 0; e < block_elems; ++e)", "for (long e = 0; e < block_elems / 2; ++e)"),
    ("prefill-top-left-causal",
     "const int p = context_lens[s] - m + (int)(row - query_start[s]);",
     "const int p = (int)(row - query_start[s]);"),
    ("prefill-mask-excludes-self", "p >= 0 ? p + 1 : 0,", "p >= 0 ? p : 0,"),
    ("prefill-mask-sees-next", "p >= 0 ? p + 1 : 0,", "p >= 0 ? p + 2 : 0,"),
    ("prefill-negative-rows-clamped", "p >= 0 ? p + 1 : 0,", "p >= 0 ? p + 1 : 1,"),
    ("prefill-rows-of-first-sequence", "seq_of_row[r] = s;", "seq_of_row[r] = 0;"),
    ("prefill-kv-head-of-query", "block_tables + (long)s * max_blocks, h / group, p",
     "block_tables + (long)s * max_blocks, h % num_kv_heads, p"),
    ("rope-sin-sign", "const double ra = a * c - b * sn;", "const double ra = a * c + b * sn;"),
    ("rope-half-split-off-by-one", "const int ib = style == 0 ? 2 * k + 1 : k + half;",
     "const int ib = style == 0 ? 2 * k + 1 : (k + half + 1) % head_dim;"),
    ("rope-one-frequency", "(double)positions[t] * (double)inv_freq[k];",
     "(double)positions[t] * (double)inv_freq[0];"),
    ("rope-first-position-only", "(double)positions[t] * (double)inv_freq[k];",
     "(double)positions[0] * (double)inv_freq[k];"),
    ("rope-pairs-swapped", "const int ia = style == 0 ? 2 * k : k;",
     "const int ia = style == 0 ? 2 * k + 1 : k;\n            const int ib_ = 0; (void)ib_;"),
    ("bf16-round-truncates", "double r = rint(m * 256.0);", "double r = trunc(m * 256.0);"),
    ("bf16-round-ties-away", "double r = rint(m * 256.0);", "double r = round(m * 256.0);"),
    ("pv-uses-first-token", "o[d] += p * bf16_value(vtile[(long)d * block_size + off]);",
     "o[d] += p * bf16_value(v_cache[(long)d * block_size]);"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert old in source, f"mutation site for {name} not found in oracle.c"
    mutated = source.replace(old, new)
    src = tmp_path / "oracle_mutant.c"
    src.write_text(mutated)
    lib = tmp_path / "liboracle_mutant.so"
    cc = shutil.which("gcc") or "cc"
    subprocess.run([cc, "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(src), "-o",
                    str(lib), "-lm"], check=True, capture_output=True)
    r = subprocess.run([sys.executable, PINS, str(lib)], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}"
    assert "FAIL" in r.stdout or r.returncode < 0 or r.returncode > 1, r.stdout + r.stderr
