"""prefill_attn_noalloc_ex against prefill_attn_ex, through the C ABI.

Two calls in a row per case, the second with a smaller input, so that the
second runs over what the first left in the shared scratch array.  Where
prefill_attn_ex's plan fits the array the two entry points run the same
kernels and must agree bit for bit; where it does not (V read in place,
fewer key splits) they must agree within the parity bars, and both with the
oracle."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, device, to_device

pytestmark = pytest.mark.gpu

LIMIT = 32 << 20

# (dtype, H, KVH, D, window, [(T, start_pos) of the two calls, larger first])
CASES = [
    ("bf16", 8, 8, 128, 0, [(64, 6000), (20, 3000)]),          # split keys, partials fit
    ("f32", 32, 8, 128, 0, [(300, 200), (90, 100)]),           # fp32, split keys
    ("bf16", 8, 2, 512, 0, [(512, 3000), (100, 2000)]),        # V copy + splits: too big, reduced
    ("f16", 8, 4, 256, 700, [(512, 3000), (64, 900)]),         # window, split keys
    ("bf16", 32, 8, 128, 0, [(2048, 300), (700, 100)]),        # paired tiles / no scratch
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-D{c[3]}-W{c[4]}" for c in CASES])
def test_noalloc_matches_ex(orc, case):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    pa.load()
    assert pa.header_define("PA_NOALLOC_SCRATCH_BYTES") == LIMIT
    dtype, H, KVH, D, W, calls = case
    for i, (T, sp) in enumerate(calls):
        L = sp + T
        x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=1000 + i + D + T, dtype=dtype)
        q, k, v = (to_device(a, dtype) for a in (x.q_store, x.k_store, x.v_store))
        ws_b = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
        ws = torch.empty(ws_b, dtype=torch.uint8, device=device()) if ws_b else None
        out_ex = torch.empty(T, H * D, device=device())
        pa.prefill_attn_ex(q, H * D, k, v, L * D, out_ex, H * D, T, sp, H, KVH, D, W, workspace=ws)
        out_na = torch.full((T, H * D), float("nan"), device=device())
        print(f"  noalloc {dtype} D{D} W{W} T{T} sp{sp}: ex workspace {ws_b} bytes", flush=True)
        pa.prefill_attn_noalloc_ex(q, H * D, k, v, L * D, out_na, H * D, T, sp, H, KVH, D, W)
        torch.cuda.synchronize()
        a = out_na.cpu().numpy().reshape(T, H, D)
        b = out_ex.cpu().numpy().reshape(T, H, D)
        if ws_b <= LIMIT:
            assert a.tobytes() == b.tobytes(), f"call {i}: same plan, different bits"
        else:
            assert_parity(a, b.astype(np.float64), dtype, f"noalloc vs ex {dtype} D{D} T{T}",
                          group="noalloc")
        ref = orc.attention(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, window=W)
        assert_parity(a, ref, dtype, f"noalloc vs oracle {dtype} D{D} T{T}", group="noalloc")
