"""bf16 and fp16 outputs of the strided entry points (out_dtype).

The kernels compute the same fp32 rows whatever the output type and round
them to the nearest even 16-bit value at the store, so a call with a bf16
(fp16) output must give, bit for bit, the fp32 output of the same call
rounded by torch on the CPU.  Every path that writes outputs is covered: the
32-row kernel, the 16-row kernels (key halves, V in operand order), the fp32
kernel, both split merges, and the ring and paged forms.  Output rows have a
padded stride whose padding must stay untouched, and sampled rows of the
16-bit output are also held to the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, device, to_device

pytestmark = pytest.mark.gpu

NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import causal_gqa_attention_prefill_amd as pa
    assert torch.cuda.is_available(), "no GPU"
    pa.load()


CASES = [
    # dtype, D, H, KVH, T, start_pos, window, form, expected key splits ("1", "few", "many")
    ("bf16", 128, 32, 8, 2048, 0, 0, "linear", "1"),        # 32-row kernel, one pass
    ("bf16", 128, 8, 2, 16, 6000, 0, "linear", "many"),     # merge_splits_wide
    ("bf16", 128, 8, 2, 200, 300, 0, "linear", "few"),      # merge_splits
    ("bf16", 256, 8, 4, 2048, 5000, 300, "linear", "1"),    # 16-row kernel, key halves
    ("bf16", 512, 16, 4, 2048, 0, 0, "linear", "1"),        # 16-row kernel, V operand-order copy
    ("f16", 64, 16, 4, 1024, 100, 0, "linear", None),
    ("f32", 128, 32, 8, 1024, 0, 0, "linear", None),        # fp32 kernel
    ("bf16", 256, 8, 4, 64, 3000, 100, "ring", None),
    ("bf16", 128, 16, 4, 4, 3000, 0, "paged", "many"),
]

PAD = 4   # extra elements per output row


def _call(x, dtype, form, T, sp, H, KVH, D, W, out):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    L = sp + T
    q = to_device(x.q_store, dtype)
    nb = pa.workspace_bytes(dtype, T, sp, H, KVH, D, W)
    ws = torch.empty(nb, dtype=torch.uint8, device=device()) if nb else None
    if form == "linear":
        k, v = to_device(x.k_store, dtype), to_device(x.v_store, dtype)
        pa.prefill_attn_ex(q, H * D, k, v, L * D, out, H * D + PAD, T, sp, H, KVH, D, W,
                           workspace=ws)
    elif form == "ring":
        R = W + T - 1
        k = to_device(workloads.ring_cache(x.k_store, R, L, NAN_BITS[dtype]), dtype)
        v = to_device(workloads.ring_cache(x.v_store, R, L, NAN_BITS[dtype]), dtype)
        pa.prefill_attn_ring_ex(q, H * D, k, v, R * D, R, out, H * D + PAD, T, sp, H, KVH, D, W,
                                workspace=ws)
    else:
        P = 64
        npages = -(-L // P) + 3
        kp, table = workloads.paged_cache(x.k_store, P, L, npages, seed=L, fill=NAN_BITS[dtype])
        vp, _ = workloads.paged_cache(x.v_store, P, L, npages, seed=L, fill=NAN_BITS[dtype])
        pa.prefill_attn_paged_ex(q, H * D, to_device(kp, dtype), to_device(vp, dtype), P,
                                 torch.from_numpy(table).to(device()), out, H * D + PAD, T, sp, H,
                                 KVH, D, W, workspace=ws)


@pytest.mark.parametrize("dtype,D,H,KVH,T,sp,W,form,splits", CASES,
                         ids=[f"{c[0]}-D{c[1]}-T{c[4]}-sp{c[5]}-W{c[6]}-{c[7]}" for c in CASES])
def test_out_dtype(orc, dtype, D, H, KVH, T, sp, W, form, splits):
    import torch
    import causal_gqa_attention_prefill_amd as pa
    S = pa.plan(dtype, T, sp, H, KVH, D, W)["kv_splits"]
    if splits == "1":
        assert S == 1
    elif splits == "few":
        assert 1 < S <= 8
    elif splits == "many":
        assert S > 8
    x = workloads.make_random(H, KVH, D, T, sp, std=0.5, seed=T + sp + D + 7, dtype=dtype)
    stride = H * D + PAD
    outs = {}
    for od, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)):
        out = torch.full((T, stride), -7.0, dtype=tdt, device=device())
        _call(x, dtype, form, T, sp, H, KVH, D, W, out)
        torch.cuda.synchronize()
        outs[od] = out.cpu()
        # the padding of every row is left as it was
        assert bool((outs[od][:, H * D:] == -7.0).all()), od
    o32 = outs["f32"][:, :H * D]
    for od, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        got = outs[od][:, :H * D]
        want = o32.to(tdt)
        same = got.view(torch.int16) == want.view(torch.int16)
        assert bool(same.all()), f"{od}: {int((~same).sum())} elements differ from the rounded fp32 output"
    # sampled rows of the bf16 output against the oracle
    rng = np.random.default_rng(T + sp)
    n = min(64, T * H)
    rt = rng.integers(0, T, n)
    rh = rng.integers(0, H, n)
    ref = orc.rows(x.q_f32, x.k_f32, x.v_f32, T, sp, H, KVH, D, rt, rh, window=W)
    got = outs["bf16"][:, :H * D].float().numpy().reshape(T, H, D)[rt, rh]
    assert_parity(got, ref, "bf16" if dtype == "f32" else dtype, f"bf16 out of {dtype} D{D} {form}")
