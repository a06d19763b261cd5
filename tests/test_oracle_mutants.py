"""Planted mistakes in the oracle's source must each fail at least one pin.

Each mutant is ``oracle.c`` with one plausible mistake edited in (a dropped
term, a wrong sign, a wrong index or bound).  It is compiled into a temporary
directory and the whole pin suite runs against it in a child process, so a
mutant that reads out of bounds and crashes also counts as caught.  The
unedited source run through the same harness must pass every pin.
"""
import concurrent.futures
import json
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

# (name, [(text to replace, replacement, expected occurrences)])
MUTANTS = [
    # one key past the causal bound, kept inside the cache so the mutant cannot crash
    ("causal_bound_plus_one", [("j <= pos;", "j <= pos + (pos + 1 < P->start_pos + P->T);", 2),
                               ("const int n = pos - lo + 1;",
                                "const int n = pos - lo + 1 + (pos + 1 < P->start_pos + P->T);", 1)]),
    ("window_lo_minus_one", [("if (window > 0 && pos - window + 1 > 0) return pos - window + 1;",
                              "if (window > 0 && pos - window > 0) return pos - window;", 1)]),
    ("kv_head_modulo", [("const int kv_h = h / num_kv_groups;",
                         "const int kv_h = h % P->num_kv_heads;", 1)]),
    ("missing_scale", [("scores[j - lo] = dot * scale;", "scores[j - lo] = dot;", 1)]),
    ("negated_scores", [("scores[j - lo] = dot * scale;", "scores[j - lo] = -dot * scale;", 1)]),
    ("zero_output", [("out_row[d] += p * (double)v_row[d];", "out_row[d] += 0.0 * p * (double)v_row[d];", 1)]),
    ("no_max_subtraction", [("scores[i] = exp(scores[i] - row_max);", "scores[i] = exp(scores[i]);", 1)]),
    ("dot_drops_first_dim", [("for (int d = 0; d < D; ++d)\n            dot +=",
                              "for (int d = 1; d < D; ++d)\n            dot +=", 1)]),
    ("q_stride_ignored", [("(int64_t)t * P->q_row_stride", "(int64_t)t * P->num_heads * D", 1)]),
    ("v_head_stride_packed", [("const float *v_row = P->v + key_offset(P, kv_h, j);",
                               "const float *v_row = P->v + key_offset(P, kv_h, j) - (int64_t)kv_h * "
                               "P->kv_head_stride + (P->page_table ? 0 : (int64_t)kv_h * (P->start_pos + P->T) * D);", 1)]),
    ("softmax_denominator_off", [("scores[i] = scores[i] / total;",
                                  "scores[i] = scores[i] / (total + 1e-3);", 1)]),
    ("value_row_relative_to_lo", [("P->v + key_offset(P, kv_h, j);", "P->v + key_offset(P, kv_h, j - lo);", 1)]),
    ("ring_slot_off_by_one", [("return P->ring > 0 ? j % P->ring : j;",
                               "return P->ring > 0 ? (j + 1) % P->ring : j;", 1)]),
    ("kv_write_slot_off_by_one", [("const int64_t row = ring_slots > 0 ? pos % ring_slots : pos;",
                                   "const int64_t row = ring_slots > 0 ? (pos + 1) % ring_slots : pos;", 1)]),
    ("kv_write_first_token_wins", [("for (int i = 0; i < T; ++i) {\n        const int64_t pos",
                                    "for (int i = T - 1; i >= 0; --i) {\n        const int64_t pos", 1)]),
    ("kv_write_v_from_k", [("v_cache[dst + d] = v_src[src + d];", "v_cache[dst + d] = k_src[src + d];", 1)]),
    ("ring_keys_of_value_slots", [("const float *k_row = P->k + key_offset(P, kv_h, j);",
                                   "const float *k_row = P->k + key_offset(P, kv_h, P->ring > 0 ? j + P->ring - 1 : j);", 1)]),
    ("paged_row_off_by_one", [("+ j % P->page_size) * P->head_dim;", "+ (j + 1) % P->page_size) * P->head_dim;", 1)]),
    ("paged_pool_head_major", [("((page * P->num_kv_heads + kv_h) * P->page_size",
                                "(((int64_t)kv_h * P->num_pages + page) * P->page_size", 1)]),
    ("query_row_of_first_token", [("const int pos = P->start_pos + t;", "const int pos = P->start_pos;", 1)]),
]

CHILD = r"""
import json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins
orc = oracle.Oracle({lib!r})
res = {{}}
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc); res[pin.__name__] = "pass"
    except AssertionError as e:
        res[pin.__name__] = "fail"
    except Exception as e:
        res[pin.__name__] = "error: " + type(e).__name__
print("RESULT " + json.dumps(res))
"""


def _run(name, edits, workdir):
    src = open(oracle.SOURCE).read()
    for old, new, count in edits:
        assert src.count(old) == count, (name, old, src.count(old))
        src = src.replace(old, new)
    c_path = os.path.join(workdir, name + ".c")
    so_path = os.path.join(workdir, name + ".so")
    with open(c_path, "w") as f:
        f.write(src)
    oracle.build(c_path, so_path)
    root = os.path.dirname(oracle.HERE)
    tests = os.path.dirname(os.path.abspath(__file__))
    code = CHILD.format(root=root, tests=tests, lib=so_path)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600, env=env)
    for line in p.stdout.splitlines():
        if line.startswith("RESULT "):
            return p.returncode, json.loads(line[7:])
    return p.returncode, None


@pytest.fixture(scope="module")
def outcomes():
    with tempfile.TemporaryDirectory() as d:
        jobs = [("unmutated", [])] + MUTANTS
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            futs = {name: ex.submit(_run, name, edits, d) for name, edits in jobs}
            return {name: f.result() for name, f in futs.items()}


def test_harness_passes_unmutated_source(outcomes):
    rc, res = outcomes["unmutated"]
    assert rc == 0 and res is not None
    assert all(v == "pass" for v in res.values()), res


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_mutant_is_caught(outcomes, name):
    rc, res = outcomes[name]
    if res is None:
        return  # the mutant crashed the child: caught
    caught = [k for k, v in res.items() if v != "pass"]
    assert caught, f"planted mistake {name} passed every pin"
