"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source, plants one mistake (a dropped term, a
wrong sign, index or operand, a changed comparison), builds the copy into a
temporary directory and runs the pin suite against it in a subprocess.  The
suite must fail for every mutant.  Nothing here touches the real oracle build.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "s2o_oracle.c")

MUTANTS = {
    "pool drops the last row": ("for (int r = 0; r < p->tile_m; ++r) sum = sum",
                                "for (int r = 0; r < p->tile_m - 1; ++r) sum = sum"),
    "score reads the wrong KV head": (
        "int g = h / (p->Hq / p->Hkv);\n    int64_t n = oracle_list_len(p, t);",
        "int g = h % p->Hkv;\n    int64_t n = oracle_list_len(p, t);"),
    "ties go to the higher index": ("return (a->j > c->j) - (a->j < c->j);",
                                    "return (a->j < c->j) - (a->j > c->j);"),
    "list sorted ascending": ("if (a->s > c->s) return -1;\n    if (a->s < c->s) return 1;",
                              "if (a->s > c->s) return 1;\n    if (a->s < c->s) return -1;"),
    "accumulator not rescaled": ("for (int k = 0; k < p->d; ++k) st->acc[k] *= rescale;", ""),
    "rescale with the wrong sign": ("double rescale = exp(st->m - m_new);",
                                    "double rescale = exp(m_new - st->m);"),
    "gain against l before the chunk": ("double gain = mass / st[r].l;",
                                        "double gain = mass / (st[r].l - mass);"),
    "non-strict stop comparison": ("if (force_n <= 0 && worst < tau) break;",
                                   "if (force_n <= 0 && worst <= tau) break;"),
    "mean gain over rows decides": ("if (gain > worst) worst = gain;",
                                    "worst += gain / p->tile_m;"),
    "triggering chunk dropped": ("executed = c + 1;\n        if (force_n <= 0 && worst < tau) break;",
                                 "if (force_n <= 0 && worst < tau) break;\n        executed = c + 1;"),
    "diagonal masked out": ("if (k0 + e <= i) keys[n++] = k0 + e;", "if (k0 + e < i) keys[n++] = k0 + e;"),
    "transposed Q/K rows in the logit": (
        "dot += (double)widen(Q, p->dtype, q_index(p, b, h, i, k)) *\n"
        "               (double)widen(K, p->dtype, kv_index(p, b, g, j, k));",
        "dot += (double)widen(Q, p->dtype, q_index(p, b, h, j, k)) *\n"
        "               (double)widen(K, p->dtype, kv_index(p, b, g, i, k));"),
    "pass 2 skips its first chunk": ("for (int32_t c = 0; c < limit; ++c) {", "for (int32_t c = 1; c < limit; ++c) {"),
    "segment mean drops its last tile": ("for (int u = first; u < last; ++u) {", "for (int u = first; u < last - 1; ++u) {"),
    "segment lists keyed by tile": ("int seg = (int)(oracle_seg_start(p, t) / p->seg_len);", "int seg = t % num_segments(p);"),
    "block mean drops a row": ("for (int r = 0; r < p->tile_n; ++r)", "for (int r = 1; r < p->tile_n; ++r)"),
    "block chunk ignores the list": ("keys[e] = p->block_lists ? (int64_t)list[c] * BN + e",
                                     "keys[e] = p->block_lists ? (int64_t)c * BN + e"),
    "guide drops the last key row": ("for (int64_t j = 0; j < n; ++j) sum = sum", "for (int64_t j = 0; j < n - 1; ++j) sum = sum"),
    "query order ignored by the tiles": ("for (int r = 0; r < p->tile_m; ++r) rows[r] = a + order[row0 - a + r];",
                                         "for (int r = 0; r < p->tile_m; ++r) rows[r] = row0 + r;"),
    "pass 1 stops at the tile's first row": ("        if (rows[r] > last) last = rows[r];", "        if (rows[r] < last) last = rows[r];"),
    "query score with the wrong head": ("acc = fmaf(widen(Q, p->dtype, q_index(p, b, h, a + i, k)), guide[k], acc);",
                                        "acc = fmaf(widen(Q, p->dtype, q_index(p, b, (h + 1) % p->Hq, a + i, k)), guide[k], acc);"),
    "shared representative drops a head": ("for (int j = 0; j < G; ++j) {\n        rep_query_head",
                                           "for (int j = 1; j < G; ++j) {\n        rep_query_head"),
    "shared lists laid out per query head": (
        "static int32_t list_head(const oracle_problem *p, int h) { return p->share_gqa ? h / (p->Hq / p->Hkv) : h; }",
        "static int32_t list_head(const oracle_problem *p, int h) { return p->share_gqa ? h % p->Hkv : h; }"),
    "block scored by its first key": ("            oracle_pool_block(p, K, b, g, j, kbar);",
                                      "            for (int k = 0; k < p->d; ++k) kbar[k] = widen(K, p->dtype, kv_index(p, b, g, j * p->tile_n, k));"),
}


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique"
    path = os.path.join(tmp, "m_%d.c" % abs(hash(name)))
    open(path, "w").write(src.replace(old, new))
    lib = path[:-2] + ".so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    path, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, S2O_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            futs = {n: ex.submit(_run_mutant, n, o, w, tmp) for n, (o, w) in MUTANTS.items()}
            survivors = [n for n, f in futs.items() if f.result() == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
