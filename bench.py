"""Benchmark of chunked causal GQA prefill attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the Mistral-7B-shaped bf16 prefill of an 8192-token prompt as four T=2048
chunks (start_pos 0, 2048, 4096, 6144) into a cache allocated for 8192
positions (32 query / 8 kv heads, head_dim 128), i.e. four calls of the C
ABI.  Inputs are resident in HBM before the timed region starts.

Output: one JSON line.  ``value`` is attention TFLOP/s over the timed steps
(wall clock), FLOPs = 4 * heads * head_dim * (valid (query, key) pairs) per
call.  The ``roofline`` object prices the fused kernel against the dense bf16
MFMA peak, with the average launch time taken from HIP events on the launch
stream around the timed steps; ``cpu_baseline`` times the fp64 oracle on a
bounded sample of the same workload on the host cores, and compares the GPU
output of those rows with the oracle's (``parity``).  ``determinism`` reruns
the step five times after the timed region and compares the outputs bit for
bit.  After the timed region: ``per_call`` gives each call's own time
(repeated back to back, and alone between its own events); with the default
workload, ``other_workloads`` times the head_dim 512 global layer (with and
without the V mirror) and the sliding-window layer the same way, each with
its own roofline entry.  Diagnostics go to stderr.

Warm-up: the --warmup steps (default 10), then more of the same untimed steps
until at least WARMUP_S seconds of them have run, so that the GPU has left its
idle clocks before the timed region (from idle it needs some tens of
milliseconds of load).  The JSON line reports the requested warm-up steps
(``warmup``) and what actually ran (``warmup_steps_run``, ``warmup_s``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "prefill attention TFLOP/s and % of MI355X bf16 MFMA peak (T=2048 chunk)"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # dense MFMA, MI355X
HBM_GBS = 8000.0
WARMUP_S = 0.5
KERNEL_SOURCE = os.path.join(ROOT, "causal_gqa_attention_prefill_amd", "csrc", "prefill_attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def valid_pairs(T: int, start_pos: int, window: int) -> int:
    """Valid (query, key) pairs of one chunk: row t keeps keys lo..pos."""
    pos = np.arange(start_pos, start_pos + T, dtype=np.int64)
    lo = np.maximum(0, pos - window + 1) if window > 0 else np.zeros_like(pos)
    return int((pos - lo + 1).sum())


def attention_flops(T: int, start_pos: int, num_heads: int, head_dim: int, window: int) -> int:
    """One multiply-add (2 flops) per element for q.k and again for p.v."""
    return 4 * num_heads * head_dim * valid_pairs(T, start_pos, window)


def algorithmic_bytes(wl, T: int, start_pos: int) -> int:
    """Each input element read once, each output element written once: Q rows
    of the chunk, K and V rows the chunk's bands touch, fp32 output."""
    eb = 4 if wl.dtype == "f32" else 2
    lo_first = max(0, start_pos - wl.window + 1) if wl.window > 0 else 0
    keys = start_pos + T - lo_first
    return (T * wl.num_heads * wl.head_dim * eb + 2 * wl.num_kv_heads * keys * wl.head_dim * eb
            + T * wl.num_heads * wl.head_dim * 4)


def source_digest() -> str:
    """Digest of the kernel source's code: comments and blank space removed,
    so that an edit of the comments alone keeps the measurements taken on it."""
    import re
    text = open(KERNEL_SOURCE, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters, kept
    with the digest of the kernel source they were taken on; None once the
    source has changed."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_sha256_16") != source_digest():
        return None
    return entry.get("bytes_per_launch")


# parity bars of the gnosis page (fp32: max |gpu - cpu| <= 1e-4) and of the
# bf16 / fp16 path, plus relative RMS error bars that a kernel ignoring Q.K^T
# or shifting the band by one key cannot meet on near-uniform softmax rows
BAR_MAX_ABS = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
BAR_REL_RMS = {"f32": 1e-5, "bf16": 5e-3, "f16": 5e-3}


def cpu_model() -> str | None:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, x, target_s: float, threads: int | None = None, gpu_out=None):
    """The fp64 oracle on the host cores (all of them unless threads is given),
    on sampled rows of the same chunks.  gpu_out: each chunk's GPU output
    ([T, H, D] host arrays); the rows the oracle computes are compared with
    it and the errors returned as a second value."""
    import oracle
    orc = oracle.default()
    threads = threads or oracle.default_threads()
    H, KVH, D, W = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.window
    rng = np.random.default_rng(12345)
    diffs, refs = [], []

    def run(rows_per_chunk, keep):
        flops, t_total, n = 0, 0.0, 0
        for ci, (T, sp) in enumerate(wl.chunks):
            _, q_f32 = x.q_rows(ci)
            rt = rng.integers(0, T, rows_per_chunk)
            rh = rng.integers(0, H, rows_per_chunk)
            t0 = time.perf_counter()
            ref = orc.rows(q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, rt, rh, window=W,
                           kv_head_stride=wl.capacity * D, nthreads=threads)
            t_total += time.perf_counter() - t0
            if keep and gpu_out is not None:
                diffs.append(gpu_out[ci][rt, rh].astype(np.float64) - ref)
                refs.append(ref)
            pos = sp + rt
            lo = np.maximum(0, pos - W + 1) if W > 0 else np.zeros_like(pos)
            flops += int(4 * D * (pos - lo + 1).sum())
            n += rows_per_chunk
        return flops, t_total, n

    f, t, _ = run(threads * 4, False)                # pilot
    rate = f / max(t, 1e-9)
    per_row = f / (threads * 4 * len(wl.chunks))
    rows = max(threads, int(target_s * rate / per_row / len(wl.chunks)))
    f, t, n = run(rows, True)
    base = {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} (token, head) rows drawn uniformly from the {len(wl.chunks)} chunks "
                      f"({rows} per chunk), fp64 oracle, {t:.1f} s wall, {f / 1e9:.1f} GFLOP",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    parity = None
    if diffs:
        d = np.concatenate(diffs)
        r = np.concatenate(refs)
        max_abs = float(np.abs(d).max())
        rel = float(np.sqrt((d ** 2).sum() / (r ** 2).sum()))
        finite = bool(all(np.isfinite(o).all() for o in gpu_out))
        parity = {"rows": n, "of": "the rows the CPU baseline computed, GPU output of the last step",
                  "max_abs": max_abs, "rel_rms": rel, "all_outputs_finite": finite,
                  "bar_max_abs": BAR_MAX_ABS[wl.dtype], "bar_rel_rms": BAR_REL_RMS[wl.dtype],
                  "ok": finite and max_abs <= BAR_MAX_ABS[wl.dtype] and rel <= BAR_REL_RMS[wl.dtype]}
    return base, parity


def prepare_calls(wl, x, dev, vmirror=False):
    """Each chunk's C-ABI call of a workload with its arguments checked and
    marshalled once (PreparedCall), over device copies of the inputs x, so
    that a timed loop issues only the calls (µs-scale kernels would otherwise
    wait on the host).  vmirror: through prefill_attn_vmirror_ex with a V
    mirror of the cache's capacity, filled up to each chunk's start by one
    untimed call, so that each timed call rewrites only its own keys' tiles
    (the steady state of a chunked prefill; linear caches without a window)."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    H, KVH, D, W = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.window

    def dev_tensor(a):
        if wl.dtype == "f32":
            return torch.from_numpy(a).to(dev)
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        return t.view(torch.bfloat16 if wl.dtype == "bf16" else torch.float16)

    page_kw = {}
    if wl.ring:
        # the cache as a ring of wl.ring slots per kv head (key j in slot j % ring),
        # as left by writing the keys up to the chunk's last one
        assert len(wl.chunks) == 1
        L = wl.chunks[0][1] + wl.chunks[0][0]
        k = dev_tensor(workloads.ring_cache(x.k_store, wl.ring, L, 0))
        v = dev_tensor(workloads.ring_cache(x.v_store, wl.ring, L, 0))
        kv_stride, ring_slots = wl.ring * D, wl.ring
    elif wl.page_size:
        # the cache as a pool of pages in scrambled order plus the sequence's page table
        assert len(wl.chunks) == 1
        L = wl.chunks[0][1] + wl.chunks[0][0]
        npages = -(-L // wl.page_size) + 16
        kp, table = workloads.paged_cache(x.k_store, wl.page_size, L, npages, wl.seed, 0)
        vp, _ = workloads.paged_cache(x.v_store, wl.page_size, L, npages, wl.seed, 0)
        k, v = dev_tensor(kp), dev_tensor(vp)
        kv_stride, ring_slots = 0, None
        page_kw = {"page_table": torch.from_numpy(table).to(dev), "page_size": wl.page_size}
    else:
        k = dev_tensor(x.k_store)
        v = dev_tensor(x.v_store)
        kv_stride, ring_slots = wl.capacity * D, None
    mirror = None
    if vmirror:
        if wl.ring or wl.page_size or W:
            raise ValueError("the V mirror serves linear caches without a window")
        mb = pa.vmirror_bytes(wl.dtype, KVH, D, wl.capacity)
        if mb == 0:
            raise ValueError(f"{wl.name}: no kernel of this dtype and head_dim reads a V mirror")
        mirror = torch.empty(mb, dtype=torch.uint8, device=dev)
    calls = []
    for ci, (T, sp) in enumerate(wl.chunks):
        q = dev_tensor(x.q_rows(ci)[0])
        out = torch.empty(T, H * D, dtype=torch.float32, device=dev)
        nb = pa.workspace_bytes(wl.dtype, T, sp, H, KVH, D, W)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        if mirror is not None:
            mkw = {"v_mirror": mirror, "mirror_capacity": wl.capacity}
            # the keys before the chunk, as earlier chunks would have left them
            pa.PreparedCall(q, H * D, k, v, kv_stride, out, H * D, T, sp, H, KVH, D, W, workspace=ws,
                            mirror_keys=0, **mkw)()
            calls.append(pa.PreparedCall(q, H * D, k, v, kv_stride, out, H * D, T, sp, H, KVH, D, W,
                                         workspace=ws, mirror_keys=sp, **mkw))
        else:
            calls.append(pa.PreparedCall(q, H * D, k, v, kv_stride, out, H * D, T, sp, H, KVH, D, W,
                                         workspace=ws, ring_slots=ring_slots, **page_kw))
    return calls


def warm_and_time(step, sync, steps: int, warmup: int, warmup_s: float):
    """The requested warm-up steps, then more until warmup_s seconds have
    passed (from idle the GPU needs some tens of ms of load to reach its
    working clock: the first 25 steps of the default workload run ~15% slower
    than steady state); then `steps` steps back to back, timed by the wall
    clock (job throughput) and by one pair of HIP events on the launch stream
    (average launch time).  Returns (warm-up steps run, warm-up seconds,
    wall seconds, stream milliseconds)."""
    import torch
    n_warm, t_w = 0, time.perf_counter()
    for _ in range(warmup):
        step()
        n_warm += 1
    sync()
    while time.perf_counter() - t_w < warmup_s:
        for _ in range(10):
            step()
        n_warm += 10
        sync()
    warm_s = time.perf_counter() - t_w
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sync()
    t_start = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    sync()
    return n_warm, warm_s, time.perf_counter() - t_start, e0.elapsed_time(e1)


def other_workload(name: str, steps: int, warmup_s: float, vmirror: bool = False):
    """A compact measurement of another workload in the same process (same
    protocol, no CPU baseline): throughput, stream time per call and the
    roofline fraction of its dtype's peak."""
    import torch
    wl = workloads.WORKLOADS[name]
    x = workloads.make_inputs(wl)
    calls = prepare_calls(wl, x, torch.device("cuda:0"), vmirror)
    torch.cuda.synchronize()

    def step():
        for call in calls:
            call()

    n_warm, warm_s, elapsed, gpu_ms = warm_and_time(step, torch.cuda.synchronize, steps, 10, warmup_s)
    flops = sum(attention_flops(T, sp, wl.num_heads, wl.head_dim, wl.window) for T, sp in wl.chunks)
    nbytes = sum(algorithmic_bytes(wl, T, sp) for T, sp in wl.chunks)
    per_call_ms = gpu_ms / (steps * len(calls))
    roof = roofline(wl, flops, nbytes, len(calls), per_call_ms,
                    read_traffic(wl.name + ("+vmirror" if vmirror else "")))
    del calls, x
    torch.cuda.empty_cache()
    return {"value": round(flops / (elapsed / steps) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(elapsed * 1e3 / steps, 4), "stream_us_per_call": round(per_call_ms * 1e3, 2),
            "steps": steps, "warmup_steps_run": n_warm, "description": wl.summary, "roofline": roof}


def roofline(wl, flops_step: int, bytes_step: int, n_calls: int, mean_launch_ms: float, traffic):
    """The dominant kernel's roofline entry: algorithmic flops per launch over
    the average launch time on the stream, against the dtype's dense matrix
    peak; below the ridge of that peak over HBM bandwidth (short chunks over
    long caches) algorithmic bytes per launch against HBM instead."""
    peak = PEAK_TFLOPS[wl.dtype]
    if flops_step / bytes_step < peak * 1e12 / (HBM_GBS * 1e9):
        gbs = bytes_step / n_calls / (mean_launch_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_GBS, 4), "traffic": traffic}
    achieved = flops_step / n_calls / (mean_launch_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic}


def sample_device(step, sync, samples: int = 3, load_s: float = 1.0, timeout_s: float = 30.0):
    """GPU clocks and socket power read by amd-smi while the workload runs.

    The workload first runs for load_s seconds; then amd-smi runs as a child
    process `samples` times in a row while steps keep being launched, so every
    reading is taken under load.  Returns the readings (None when the tool is
    missing or its output cannot be read).
    """
    import shutil
    import subprocess
    # under a profiler the child would inherit its tool library: no sample
    if any(k.startswith("ROCPROF") for k in os.environ):
        return None
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None

    def run_for(cond):
        n = 0
        while cond():
            for _ in range(10):
                step()
            sync()
            n += 10
        return n

    t0 = time.perf_counter()
    n = run_for(lambda: time.perf_counter() - t0 < load_s)
    readings = []
    for _ in range(samples):
        try:
            proc = subprocess.Popen([exe, "metric", "-g", "0", "-p", "-c", "--json"],
                                    stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError:
            return None
        t1 = time.perf_counter()
        n += run_for(lambda: proc.poll() is None and time.perf_counter() - t1 < timeout_s)
        if proc.poll() is None:
            proc.kill()
        try:
            out, _ = proc.communicate(timeout=5)
        except subprocess.TimeoutExpired:
            return None
        rec = parse_amd_smi(out)
        if rec is None:
            return None
        readings.append(rec)
    clocks = [r["gfx_clock_mhz_mean"] for r in readings]
    return {"gfx_clock_mhz_mean": clocks, "socket_power_w": [r["socket_power_w"] for r in readings],
            "gfx_clock_mhz_last": readings[-1]["gfx_clock_mhz"],
            "sampled_by": f"amd-smi metric -p -c, {samples} readings under load ({n} steps in "
                          f"{time.perf_counter() - t0:.1f} s)"}


def parse_amd_smi(text: str):
    """Per-die gfx clocks (MHz) and socket power (W) from `amd-smi metric -p -c
    --json` output, or None."""
    try:
        starts = [i for i in (text.find("{"), text.find("[")) if i >= 0]
        rec = json.loads(text[min(starts):])
        gpu = rec["gpu_data"][0] if isinstance(rec, dict) else rec[0]
        clocks = [gpu["clock"][k]["clk"]["value"] for k in sorted(gpu["clock"]) if k.startswith("gfx_")]
        power = gpu["power"]["socket_power"]["value"]
        return {"gfx_clock_mhz": clocks,
                "gfx_clock_mhz_mean": round(sum(clocks) / len(clocks), 1) if clocks else None,
                "socket_power_w": power}
    except (ValueError, KeyError, IndexError, TypeError):
        return None


def calibrate_copy(nbytes: int):
    """A copy kernel of known size: FETCH_SIZE / WRITE_SIZE per dispatch of this
    kernel, divided by nbytes, is the factor that turns the counters into bytes."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "dispatches": 5}), flush=True)


def kv_write_bench(args):
    """The step before the attention: each chunk's K and V rows (one [T x KVH*D]
    source each) stored in the workload's cache (rows start_pos+i, or ring slots).
    Bytes = the rows read once and written once.  The kernels take a few
    microseconds, less than a host launch, so the K timed steps are recorded
    into one HIP graph on a side stream and replayed between two events."""
    import torch
    import causal_gqa_attention_prefill_amd as pa
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU.", file=sys.stderr)
        sys.exit(2)
    lib = pa.load()
    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS[args.workload]
    KVH, D = wl.num_kv_heads, wl.head_dim
    eb = 4 if wl.dtype == "f32" else 2
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    rows = wl.ring or wl.capacity
    k_cache = torch.zeros(KVH, rows, D, dtype=tdt, device=dev)
    v_cache = torch.zeros_like(k_cache)
    gen = torch.Generator(device=dev).manual_seed(wl.seed)
    side = torch.cuda.Stream()
    calls, keep, bytes_step = [], [], 0
    for T, sp in wl.chunks:
        ks = torch.randn(T, KVH * D, generator=gen, device=dev).to(tdt)
        vs = torch.randn(T, KVH * D, generator=gen, device=dev).to(tdt)
        calls.append((pa.binding.DTYPE_CODES[wl.dtype], ks.data_ptr(), vs.data_ptr(), KVH * D,
                      k_cache.data_ptr(), v_cache.data_ptr(), rows * D, wl.ring, T, sp, KVH, D,
                      side.cuda_stream))
        keep.append((ks, vs))
        bytes_step += 2 * 2 * min(T, wl.ring or T) * KVH * D * eb
    fn = lib.prefill_kv_write
    torch.cuda.synchronize()

    def step():
        for a in calls:
            st = fn(*a)
            if st != pa.PA_OK:
                raise pa.PrefillAttnError(st, "prefill_kv_write")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    n_warm, t_w = 0, time.perf_counter()
    with torch.cuda.stream(side):
        # replays of the K-step graph: at least one, then until --warmup-s has passed
        while n_warm < 1 or time.perf_counter() - t_w < args.warmup_s:
            g.replay()
            side.synchronize()
            n_warm += 1
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(side)
        g.replay()
        e1.record(side)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    print(f"kv write: {len(calls)} calls per step, {ms_step * 1e3:.2f} us per step on the stream "
          f"({ms_step * 1e3 / len(calls):.2f} us per call)", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "KV cache write GB/s (K and V rows read once and written once)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": n_warm * args.steps, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "num_kv_heads": KVH, "head_dim": D,
                   "chunks": [list(c) for c in wl.chunks], "ring_slots": wl.ring or None,
                   "bytes_per_step": bytes_step, "wall_ms_per_step": round(elapsed * 1e3 / args.steps, 4),
                   "timing": "K steps replayed from one HIP graph between two events"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_GBS, 4), "traffic": None},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed steps before the timed ones; more of them run until at least "
                         f"{WARMUP_S} s of work has passed, so that the GPU has left its idle clocks")
    ap.add_argument("--warmup-s", type=float, default=WARMUP_S,
                    help="least seconds of untimed steps before the timed ones (0 for counter "
                         "collection runs, which profile every dispatch)")
    ap.add_argument("--workload", default="mistral_bf16_chunked", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="oracle threads for the CPU baseline (default: every visible core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--vmirror", action="store_true",
                    help="call prefill_attn_vmirror_ex with a V mirror filled up to each chunk's start "
                         "(head_dim 512 bf16/fp16 workloads without a window)")
    ap.add_argument("--no-others", dest="others", action="store_false",
                    help="with the default workload, skip the compact measurement of the head_dim 512 "
                         "global layer and the sliding-window layer after the timed region")
    ap.add_argument("--no-device-sample", action="store_true",
                    help="skip reading GPU clocks and power with amd-smi after the timed steps")
    ap.add_argument("--kv-write", action="store_true",
                    help="time the KV cache write of the workload's chunks (prefill_kv_write) "
                         "instead of the attention; HBM-bound, priced against 8 TB/s")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times "
                         "(reference for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    if args.kv_write:
        kv_write_bench(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(each GPU would run its own shard of kv heads; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import causal_gqa_attention_prefill_amd as pa
    pa.load()
    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS[args.workload]
    H, KVH, D, W = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.window

    t0 = time.perf_counter()
    x = workloads.make_inputs(wl)

    calls = prepare_calls(wl, x, dev, args.vmirror)
    torch.cuda.synchronize()
    print(f"inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    flops_step = sum(attention_flops(T, sp, H, D, W) for T, sp in wl.chunks)
    bytes_step = sum(algorithmic_bytes(wl, T, sp) for T, sp in wl.chunks)

    def step():
        for call in calls:
            call()

    # warm-up, then the timed region: K steps back to back
    n_warm, warmup_s, elapsed, gpu_ms = warm_and_time(step, torch.cuda.synchronize, args.steps,
                                                      args.warmup, args.warmup_s)

    # the outputs of the last timed step (every call writes its own buffer)
    outs = [c.out.clone() for c in calls]
    # determinism (not timed): five more steps give the same bits
    identical = True
    for _ in range(5):
        step()
        identical &= all(bool(torch.equal(c.out, o)) for c, o in zip(calls, outs))
    torch.cuda.synchronize()

    # diagnostics (not timed): each call's own time, from that call repeated
    # back to back between one pair of HIP events after as many untimed
    # repeats, about 10 ms each (events around every call of a step would add
    # a gap to each launch)
    per_call_ms = np.zeros(len(calls))
    est_ms = gpu_ms / (args.steps * len(calls))
    reps = int(min(500, max(10, 10.0 / max(est_ms, 1e-3))))
    for i, call in enumerate(calls):
        for _ in range(reps):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        per_call_ms[i] = a.elapsed_time(b) / reps
    # and each call alone between its own pair of events, 20 times after 3
    # untimed calls: median and minimum (this includes the gap that the
    # events put before each launch)
    single_ms = np.zeros((len(calls), 2))
    for i, call in enumerate(calls):
        for _ in range(3):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in evs:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        t_ = np.array([a.elapsed_time(b) for a, b in evs])
        single_ms[i] = np.median(t_), t_.min()
    ms_per_step = elapsed * 1e3 / args.steps
    value = flops_step / (elapsed / args.steps) / 1e12
    # the fused kernel (with the merge kernel when a call splits its keys):
    # algorithmic flops per launch over the average launch time on the stream
    mean_launch_ms = gpu_ms / (args.steps * len(calls))
    peak = PEAK_TFLOPS[wl.dtype]
    traffic = read_traffic(wl.name + ("+vmirror" if args.vmirror else ""))
    for i, (T, sp) in enumerate(wl.chunks):
        f = attention_flops(T, sp, H, D, W)
        b = algorithmic_bytes(wl, T, sp)
        print(f"call {i}: T={T} start_pos={sp} {per_call_ms[i] * 1e3:8.1f} us  "
              f"{f / per_call_ms[i] / 1e9:7.1f} TFLOP/s  {100 * f / per_call_ms[i] / 1e9 / peak:5.1f}% of peak  "
              f"{b / per_call_ms[i] / 1e6:7.1f} GB/s algorithmic  plan={pa.plan(wl.dtype, T, sp, H, KVH, D, W)}",
              file=sys.stderr, flush=True)
    print(f"timed: {args.steps} steps, {gpu_ms * 1e3 / args.steps:.1f} us per step on the stream "
          f"({mean_launch_ms * 1e3:.1f} us per call), {ms_per_step * 1e3:.1f} us per step wall clock",
          file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "warmup_s": round(warmup_s, 3),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.summary, "num_heads": H,
                   "num_kv_heads": KVH, "head_dim": D, "window": W,
                   "chunks": [list(c) for c in wl.chunks], "cache_capacity": wl.capacity,
                   "flops_per_step": flops_step, "algorithmic_bytes_per_step": bytes_step,
                   "peak_fraction": round(value / peak, 4), "parallelism": "single GPU",
                   "stream_ms_per_step": round(gpu_ms / args.steps, 4)},
        "roofline": roofline(wl, flops_step, bytes_step, len(calls), mean_launch_ms, traffic),
    }
    # clocks and power under the same load (after the timed region, outside it)
    result["device"] = None if args.no_device_sample else sample_device(step, torch.cuda.synchronize)
    # the other bf16 workloads the metric's bar covers, measured the same way
    # in the same process (after the headline's timed region, outside it)
    if args.others and wl.name == "mistral_bf16_chunked":
        result["other_workloads"] = {}
        for name, vm in (("gemma_global_bf16", False), ("gemma_swa_bf16", False),
                         ("gemma_global_bf16", True)):
            key = name + ("+vmirror" if vm else "")
            result["other_workloads"][key] = other_workload(name, args.steps, args.warmup_s, vm)
            print(f"{key}: {result['other_workloads'][key]}", file=sys.stderr, flush=True)
    # each call's own time (diagnostics above, outside the timed region)
    result["per_call"] = [{"T": T, "start_pos": sp, "us": round(ms * 1e3, 2),
                           "mfma_frac": round(attention_flops(T, sp, H, D, W) / (ms * 1e-3) / 1e12 / peak, 4),
                           "us_alone_median": round(sm[0] * 1e3, 2), "us_alone_min": round(sm[1] * 1e3, 2)}
                          for (T, sp), ms, sm in zip(wl.chunks, per_call_ms, single_ms)]
    result["per_call_how"] = (f"us: each call repeated {reps} times back to back between one pair of HIP events, "
                              f"after {reps} untimed repeats; us_alone_*: 20 calls each between its own pair "
                              f"of events, after 3 untimed calls")
    if args.vmirror:
        result["config"]["entry_point"] = "prefill_attn_vmirror_ex (V mirror filled up to the chunk's start)"
    if wl.ring:
        result["config"]["ring_slots"] = wl.ring
    if wl.page_size:
        result["config"]["page_size"] = wl.page_size
    result["determinism"] = {"runs": 6, "identical": identical,
                             "of": "the outputs of the last timed step and of five more steps, bit for bit"}
    result["parity"] = None
    if not args.no_cpu_baseline:
        gpu_out = [o.float().cpu().numpy().reshape(T, H, D) for o, (T, _) in zip(outs, wl.chunks)]
        result["cpu_baseline"], result["parity"] = cpu_baseline(wl, x, args.cpu_seconds,
                                                                args.cpu_threads, gpu_out)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
