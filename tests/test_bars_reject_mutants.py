"""The GPU parity bars can fail: planted mistakes are rejected (CPU only).

The outputs of oracle mutants (the oracle's source with one plausible mistake
edited in, built by test_oracle_mutants' recipe) on sampled rows of the
full-size bf16 workloads are handed to gpu_util.assert_parity as if a GPU had
produced them, against the true oracle on the same rows.  Each mistake that
changes the rows must be rejected; at these input scales softmax rows are
near-uniform, so this shows that the relative-RMS bar, not the max-abs bar,
does most of the work.

Two mistakes are below the bf16 noise floor on the head_dim-512 global layer
(63488 keys per row, so one key more or one dimension less moves a row by
about 4e-3 relative, under the 5e-3 bar; a correct bf16 kernel sits near
1.6e-3): the causal bound one key late and a dot product missing one
dimension.  Both are rejected on the other workloads, and the same kernels'
band and dot products are checked at small shapes, where they are visible,
by the GPU tests (small shapes of every head_dim, planted keys just past the
band, the closed-form band).  They are listed as known blind spots below, so
that a change of bar or workload that alters this shows up here.
"""
from __future__ import annotations

import os
import tempfile

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_parity
from test_oracle_mutants import MUTANTS

EDITS = dict(MUTANTS)
# the softmax of constant scores: every valid key weighted equally (a kernel
# that ignores Q.K^T)
EDITS["uniform_softmax"] = [("scores[j - lo] = dot * scale;", "scores[j - lo] = 0.0 * dot * scale;", 1)]

CHECKED = ["causal_bound_plus_one", "window_lo_minus_one", "kv_head_modulo", "missing_scale",
           "uniform_softmax", "negated_scores", "zero_output", "dot_drops_first_dim",
           "value_row_relative_to_lo"]
WORKLOADS = ["mistral_bf16_chunked", "gemma_global_bf16", "gemma_swa_bf16"]
# (mutant, workload) pairs whose rows equal the true ones (the mistake only
# matters with a window)
NO_EFFECT = {(m, w) for m in ("window_lo_minus_one", "value_row_relative_to_lo")
             for w in ("mistral_bf16_chunked", "gemma_global_bf16")}
KNOWN_BLIND = {("causal_bound_plus_one", "gemma_global_bf16"), ("dot_drops_first_dim", "gemma_global_bf16")}
ROWS_PER_CHUNK = 48


@pytest.fixture(scope="module")
def mutant_oracles():
    with tempfile.TemporaryDirectory() as d:
        libs = {}
        for name in CHECKED:
            src = open(oracle.SOURCE).read()
            for old, new, count in EDITS[name]:
                assert src.count(old) == count, (name, old)
                src = src.replace(old, new)
            c_path = os.path.join(d, name + ".c")
            with open(c_path, "w") as f:
                f.write(src)
            libs[name] = oracle.Oracle(oracle.build(c_path, os.path.join(d, name + ".so")))
        yield libs


@pytest.fixture(scope="module")
def sampled_rows():
    """Per workload: [(chunk args, row_t, row_h, true oracle rows)]."""
    orc = oracle.default()
    out = {}
    rng = np.random.default_rng(20261203)
    for name in WORKLOADS:
        wl = workloads.WORKLOADS[name]
        x = workloads.make_inputs(wl)
        H, KVH, D, W = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.window
        cases = []
        for ci, (T, sp) in enumerate(wl.chunks):
            _, q = x.q_rows(ci)
            rt = rng.integers(0, T, ROWS_PER_CHUNK)
            rh = rng.integers(0, H, ROWS_PER_CHUNK)
            args = (q, x.k_f32, x.v_f32, T, sp, H, KVH, D)
            kw = dict(window=W, kv_head_stride=wl.capacity * D)
            cases.append((args, kw, rt, rh, orc.rows(*args, rt, rh, **kw)))
        out[name] = (wl, cases)
    return out


def _rejected(got, ref, dtype):
    try:
        assert_parity(got, ref, dtype, "planted mistake", record=False)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("workload", WORKLOADS)
@pytest.mark.parametrize("mutant", CHECKED)
def test_bars_reject_planted_mistake(mutant_oracles, sampled_rows, mutant, workload):
    wl, cases = sampled_rows[workload]
    got = np.concatenate([mutant_oracles[mutant].rows(*args, rt, rh, **kw)
                          for args, kw, rt, rh, _ in cases])
    ref = np.concatenate([c[4] for c in cases])
    if (mutant, workload) in NO_EFFECT:
        assert np.array_equal(got, ref)
        return
    rejected = _rejected(got, ref, wl.dtype)
    if (mutant, workload) in KNOWN_BLIND:
        assert not rejected, "now rejected: remove it from KNOWN_BLIND and the docstring"
    else:
        assert rejected, f"{mutant} on {workload} passes the parity bars"
