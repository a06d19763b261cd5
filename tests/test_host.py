"""Host-side logic pinned to figures the pages print (CPU only)."""
import json
import os
import subprocess
import sys

import bench
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_flop_count_matches_gnosis_figure():
    g = json.load(open(os.path.join(GOLDEN, "gnosis_mistral_prefill_work.json")))
    assert g["num_heads"] // g["num_kv_heads"] == g["num_kv_groups"]
    # bench counts both products (4 flops per valid pair and dim); the page
    # counts the score product only (2), over all layers
    per_layer = bench.attention_flops(g["prompt_tokens"], 0, g["num_heads"], g["head_dim"], 0) / 2
    total_gflop = per_layer * g["layers"] / 1e9
    assert abs(total_gflop - g["attention_gflop_page"]) <= g["attention_gflop_tolerance"], total_gflop


def test_valid_pairs_closed_forms():
    # causal from 0: T (T + 1) / 2; late chunk: T * start_pos + T (T + 1) / 2
    assert bench.valid_pairs(2048, 0, 0) == 2048 * 2049 // 2
    assert bench.valid_pairs(2048, 6144, 0) == 2048 * 6144 + 2048 * 2049 // 2
    # a window shorter than start_pos keeps exactly `window` keys per row
    assert bench.valid_pairs(2048, 129024, 1024) == 2048 * 1024
    # window 1 keeps one key per row
    assert bench.valid_pairs(77, 5, 1) == 77


def test_workloads_follow_the_pages():
    pad = json.load(open(os.path.join(GOLDEN, "tensorsharp_gemma_padding.json")))
    g = workloads.WORKLOADS["gemma_global_bf16"]
    T, sp = g.chunks[0]
    assert g.head_dim == pad["head_dim"] and T == pad["chunk_tokens"]
    assert (sp + T) % pad["kv_pad_multiple"] == 0
    assert abs(sp - pad["late_chunk_start_pos_approx"]) < 2048
    m = workloads.WORKLOADS["mistral_f32"]
    gn = json.load(open(os.path.join(GOLDEN, "gnosis_mistral_prefill_work.json")))
    assert (m.num_heads, m.num_kv_heads, m.head_dim, m.chunks[0][0]) == (
        gn["num_heads"], gn["num_kv_heads"], gn["head_dim"], gn["prompt_tokens"])
    c = workloads.WORKLOADS["mistral_bf16_chunked"]
    assert [sp for _, sp in c.chunks] == [0, 2048, 4096, 6144] and c.capacity == 8192


def test_inputs_are_seeded_and_rounded():
    wl = workloads.WORKLOADS["tiny_f32"]
    a, b = workloads.make_inputs(wl), workloads.make_inputs(wl)
    assert (a.q_f32 == b.q_f32).all() and (a.k_f32 == b.k_f32).all()
    x = workloads.make_random(2, 1, 32, 5, 3, dtype="bf16", seed=4)
    # the fp32 image is exactly the bf16 value
    assert (workloads.round_to_bf16_bits(x.k_f32) == x.k_store).all()
    y = workloads.make_random(2, 1, 32, 5, 3, dtype="f16", seed=4)
    import numpy as np
    assert (y.k_store.view(np.float16).astype(np.float32) == y.k_f32).all()


def test_bench_refuses_several_gpus():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_parse_amd_smi():
    gpu = {"gpu": 0,
           "power": {"socket_power": {"value": 1012, "unit": "W"}, "gfx_voltage": "N/A"},
           "clock": {**{f"gfx_{i}": {"clk": {"value": 2000 + 10 * i, "unit": "MHz"},
                                     "max_clk": {"value": 2400, "unit": "MHz"}} for i in range(8)},
                     "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}}}
    text = "warning line\n" + json.dumps({"gpu_data": [gpu]})
    rec = bench.parse_amd_smi(text)
    assert rec["gfx_clock_mhz"] == [2000 + 10 * i for i in range(8)]
    assert rec["gfx_clock_mhz_mean"] == 2035.0 and rec["socket_power_w"] == 1012
    assert bench.parse_amd_smi(json.dumps([gpu]))["socket_power_w"] == 1012
    assert bench.parse_amd_smi("no output") is None
    assert bench.parse_amd_smi(json.dumps({"gpu_data": [{"gpu": 0}]})) is None


def test_cpu_baseline_reports_parity_of_its_rows():
    """The bench line's parity comes from the rows the CPU baseline computes:
    the oracle's own output passes, a 1% scaled one fails the fp32 bars."""
    import numpy as np

    import oracle
    wl = workloads.WORKLOADS["tiny_f32"]
    x = workloads.make_inputs(wl)
    T, sp = wl.chunks[0]
    ref = oracle.default().attention(x.q_f32, x.k_f32, x.v_f32, T, sp, wl.num_heads,
                                     wl.num_kv_heads, wl.head_dim)
    base, par = bench.cpu_baseline(wl, x, 0.05, threads=2, gpu_out=[ref.astype(np.float32)])
    assert base["kind"] == "oracle" and base["cores"] == 2 and base["value"] > 0
    assert par["ok"] and par["max_abs"] < 1e-6 and par["rows"] > 0
    _, bad = bench.cpu_baseline(wl, x, 0.05, threads=2, gpu_out=[(ref * 1.01).astype(np.float32)])
    assert not bad["ok"] and bad["rel_rms"] > 5e-3


def test_source_digest_keys_traffic_records_to_code(tmp_path, monkeypatch):
    """The traffic counters stay attached to the kernel code they were taken
    on: an edit of comments or blank space keeps the digest, a code edit
    changes it, and a record with another digest is not reported."""
    src = tmp_path / "k.hip"
    base = "// header\nint f(int x) {\n    return x + 1;   // one\n}\n/* block\n comment */\n"
    src.write_text(base)
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    d0 = bench.source_digest()
    src.write_text("// other header\n\nint f(int x) {\n  return x + 1;\n}\n/* changed */\n")
    assert bench.source_digest() == d0
    src.write_text(base.replace("x + 1", "x + 2"))
    d1 = bench.source_digest()
    assert d1 != d0
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"w": {"kernel_source_sha256_16": d1, "bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.read_traffic("w") == 123
    src.write_text(base)
    assert bench.read_traffic("w") is None
    assert bench.read_traffic("missing") is None
