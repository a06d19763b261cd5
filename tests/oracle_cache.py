"""Full fp64 oracle outputs of the workloads, cached on disk.

Every row of every chunk of a workload, computed by ``oracle`` (and nothing
else: the inputs come from ``workloads``, the arithmetic from the oracle's C
source) and kept as ``.npy`` files keyed by (workload, seed, chunk, digest of
the oracle source), so that the GPU parity tests can compare all T*H rows at
full size and a rerun on the same machine reads them back.  The cache lives
in $PA_ORACLE_CACHE (default: pa_oracle_cache under the system temporary
directory); nothing here is committed.

Run as a script to fill the cache for the named workloads (all by default):
    python tests/oracle_cache.py [workload ...]
"""
from __future__ import annotations

import hashlib
import os
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def cache_dir() -> str:
    d = os.environ.get("PA_ORACLE_CACHE") or os.path.join(tempfile.gettempdir(), "pa_oracle_cache")
    os.makedirs(d, exist_ok=True)
    return d


def _digest() -> str:
    return hashlib.sha256(open(oracle.SOURCE, "rb").read()).hexdigest()[:12]


def reference(name: str, chunk: int, x: workloads.Inputs | None = None) -> np.ndarray:
    """fp64 [T, H, D] oracle output of chunk `chunk` of workload `name`."""
    wl = workloads.WORKLOADS[name]
    T, sp = wl.chunks[chunk]
    path = os.path.join(cache_dir(), f"{name}_s{wl.seed}_c{chunk}_{_digest()}.npy")
    if os.path.exists(path):
        try:
            ref = np.load(path)
            if ref.shape == (T, wl.num_heads, wl.head_dim) and ref.dtype == np.float64:
                return ref
        except (OSError, ValueError):
            pass
    x = x or workloads.make_inputs(wl)
    _, q_f32 = x.q_rows(chunk)
    ref = oracle.default().attention(q_f32, x.k_f32, x.v_f32, T, sp, wl.num_heads, wl.num_kv_heads,
                                     wl.head_dim, window=wl.window, kv_head_stride=wl.capacity * wl.head_dim)
    tmp = f"{path}.{os.getpid()}.tmp.npy"
    np.save(tmp, ref)
    os.replace(tmp, path)
    return ref


def main(names):
    for name in names or sorted(workloads.WORKLOADS):
        wl = workloads.WORKLOADS[name]
        x = workloads.make_inputs(wl)
        for ci in range(len(wl.chunks)):
            t0 = time.perf_counter()
            reference(name, ci, x)
            print(f"{name} chunk {ci}: {time.perf_counter() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
