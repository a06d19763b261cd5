"""Helpers shared by the GPU tests: device copies of seeded inputs, calls
through the C ABI, and the error measures the parity bars use."""
from __future__ import annotations

import numpy as np

TOL_MAX_ABS = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
# relative RMS error ||gpu - ref|| / ||ref||: a secondary bar that a kernel
# ignoring Q.K^T, reading the wrong kv head or shifting the band by one key
# cannot meet (the max-abs bar alone can, on near-uniform softmax rows)
TOL_REL_RMS = {"f32": 1e-5, "bf16": 5e-3, "f16": 5e-3}


def device():
    import torch
    return torch.device("cuda:0")


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device())
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = gpu - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.sqrt((ref ** 2).sum()))
    rel = float(np.sqrt((diff ** 2).sum()) / denom) if denom > 0 else float(np.sqrt((diff ** 2).sum()))
    return max_abs, rel


# every comparison made in this process: (group, dtype, what, rows, max_abs, rel_rms);
# the test session prints the worst per group and dtype at its end
RECORD = []


def assert_parity(gpu, ref, dtype, what="", group=None, record=True):
    """Fail unless gpu (any shape, last axis head_dim) meets both bars against
    the oracle's ref.  group names the case family in the end-of-session
    summary (default: the first word of what)."""
    gpu = np.asarray(gpu)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    max_abs, rel = errors(gpu, ref)
    rows = int(np.prod(gpu.shape[:-1])) if gpu.ndim > 1 else 1
    if record:
        RECORD.append((group or (what.split() or ["?"])[0], dtype, what, rows, max_abs, rel))
    print(f"  {what}: max|gpu-oracle| {max_abs:.3e} (bar {TOL_MAX_ABS[dtype]:.0e}), "
          f"rel-RMS {rel:.3e} (bar {TOL_REL_RMS[dtype]:.0e}) over {rows} rows", flush=True)
    assert max_abs <= TOL_MAX_ABS[dtype], (what, max_abs)
    assert rel <= TOL_REL_RMS[dtype], (what, rel)
    return max_abs, rel


def summary_lines():
    """Worst max-abs and rel-RMS per (group, dtype) over the comparisons made."""
    worst = {}
    for group, dtype, what, rows, max_abs, rel in RECORD:
        w = worst.setdefault((group, dtype), [0, 0, 0.0, "", 0.0, ""])
        w[0] += 1
        w[1] += rows
        if max_abs >= w[2]:
            w[2], w[3] = max_abs, what
        if rel >= w[4]:
            w[4], w[5] = rel, what
    out = []
    for (group, dtype), (n, rows, ma, mwhat, rr, rwhat) in sorted(worst.items()):
        out.append(f"{group:<28} {dtype:<5} {n:4d} cmp {rows:9d} rows  max-abs {ma:.3e} "
                   f"(bar {TOL_MAX_ABS[dtype]:.0e})  rel-RMS {rr:.3e} (bar {TOL_REL_RMS[dtype]:.0e})"
                   f"  worst: {mwhat}")
    return out


def run_packed(x, T, sp, H, KVH, D, W, q_rows=None):
    """Packed call on the first T rows of x.q_store (or q_rows) with caches
    holding exactly L = sp + T rows per kv head; returns fp32 [T, H, D]."""
    import torch

    import causal_gqa_attention_prefill_amd as pa
    dt = x.wl.dtype
    L = sp + T
    q = to_device(x.q_store[:T] if q_rows is None else q_rows, dt)
    k = to_device(np.ascontiguousarray(x.k_store[:, :L]), dt)
    v = to_device(np.ascontiguousarray(x.v_store[:, :L]), dt)
    out = torch.empty(T, H * D, dtype=torch.float32, device=device())
    pa.prefill_attn(q, k, v, out, T, sp, H, KVH, D, W)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(T, H, D)
