"""Pins of the oracle to things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when that build disagrees with what the pages or the mathematics fix:

  brute force   a dense fp64 score matrix, a 0/1 mask built from the band
                definition, softmax without max subtraction (another path)
  library       torch.nn.functional.scaled_dot_product_attention in fp64 on
                the CPU with an explicit bottom-right band mask and torch's
                own grouped-query mapping (enable_gqa)
  closed forms  q = 0 or identical keys give the plain mean of the valid value
                rows; V[kh, j, :] = j + 1000*kh pins the causal bound, the
                window bound and the kv-head map at once; V constant per kv
                head pins the map alone; L = 1 and window = 1 give one value
                row; a hand-derived three-key example
  invariants    rows sum to one; chunked prefill equals one-shot prefill and
                T=1 decode equals a row of it (the gnosis page's
                chunked-vs-token-by-token parity test, "What already
                shipped"); keys just outside [lo, pos] cannot change a row,
                keys on its edges do; a per-kv-head shift of every key leaves
                the output unchanged even when the raw scores would overflow
                exp
  ring cache    keys written in order into slot pos % R (the TensorSharp
                page, section 4, requirement R4): the closed form above still
                holds, and a chunk loop through the ring gives the rows of the
                one-shot prefill over the linear cache, bit for bit
  cache write   appended rows equal the source rows and nothing else moves;
                a ring slot holds the last token written to it; writing each
                chunk into a ring and then attending equals the one-shot
                prefill
  paged cache   pages in scrambled pool order give the linear result bit for
                bit; the closed form above holds through pages

The module is shared by ``test_oracle_pins.py`` (the real oracle must pass
every pin) and ``test_oracle_mutants.py`` (each planted mistake must fail at
least one).
"""
from __future__ import annotations

import math

import numpy as np

RNG_SEED = 20260629


def _rand(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def _case(rng, H, KVH, D, T, sp, std=1.0, capacity=None):
    L = sp + T
    cap = capacity or L
    q = _rand(rng, (T, H * D), std)
    k = _rand(rng, (KVH, cap, D), std)
    v = _rand(rng, (KVH, cap, D), std)
    return q, k, v


def _band(T, sp, W, L):
    """0/1 mask [T, L]: row t keeps keys j with pos-W < j <= pos (W > 0) or j <= pos."""
    pos = sp + np.arange(T)[:, None]
    j = np.arange(L)[None, :]
    keep = j <= pos
    if W > 0:
        keep &= j > pos - W
    return keep


def brute_force(q, k, v, T, sp, H, KVH, D, W):
    """Dense fp64 attention: kv head of query head h from an explicit repeat,
    softmax as exp(S) / sum(exp(S)) with masked entries removed (no max shift)."""
    L = sp + T
    G = H // KVH
    kv_of_head = np.repeat(np.arange(KVH), G)
    keep = _band(T, sp, W, L)
    out = np.zeros((T, H, D))
    q64 = q.astype(np.float64).reshape(T, -1)
    for h in range(H):
        kh = kv_of_head[h]
        Qh = q64[:, h * D:(h + 1) * D]
        Kh = k[kh, :L].astype(np.float64)
        Vh = v[kh, :L].astype(np.float64)
        S = (Qh @ Kh.T) / math.sqrt(D)
        E = np.where(keep, np.exp(S), 0.0)
        P = E / E.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ Vh
    return out


# ---------------------------------------------------------------- pins ----

def pin_brute_force(orc):
    rng = np.random.default_rng(RNG_SEED)
    for H, KVH in ((1, 1), (2, 1), (2, 2), (4, 2), (4, 1)):
        for D in (1, 2, 4, 8):
            for T, sp in ((1, 0), (3, 0), (5, 2), (8, 8), (4, 7)):
                L = sp + T
                for W in (0, 1, 2, 3, L, L + 5):
                    q, k, v = _case(rng, H, KVH, D, T, sp)
                    got = orc.attention(q, k, v, T, sp, H, KVH, D, window=W)
                    ref = brute_force(q, k, v, T, sp, H, KVH, D, W)
                    err = np.abs(got - ref).max()
                    assert err <= 1e-12, (H, KVH, D, T, sp, W, err)


def pin_torch_sdpa(orc):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(RNG_SEED + 1)
    for H, KVH, D, T, sp, W in ((8, 2, 16, 37, 50, 0), (8, 2, 16, 37, 50, 20), (4, 4, 32, 16, 0, 0),
                                (6, 3, 8, 21, 5, 7), (4, 1, 64, 9, 100, 0), (2, 2, 4, 40, 0, 1)):
        L = sp + T
        q, k, v = _case(rng, H, KVH, D, T, sp, std=1.5)
        got = orc.attention(q, k, v, T, sp, H, KVH, D, window=W)
        tq = torch.from_numpy(q.astype(np.float64)).reshape(T, H, D).permute(1, 0, 2)[None]
        tk = torch.from_numpy(k.astype(np.float64))[None]
        tv = torch.from_numpy(v.astype(np.float64))[None]
        mask = torch.from_numpy(_band(T, sp, W, L))
        ref = F.scaled_dot_product_attention(tq.contiguous(), tk.contiguous(), tv.contiguous(),
                                             attn_mask=mask, enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        err = np.abs(got - ref).max()
        assert err <= 1e-10, (H, KVH, D, T, sp, W, err)


def pin_rows_sum_to_one(orc):
    rng = np.random.default_rng(RNG_SEED + 2)
    H, KVH, D, T, sp = 4, 2, 16, 12, 20
    q, k, v = _case(rng, H, KVH, D, T, sp, std=2.0)
    for W in (0, 5):
        for t in (0, 5, 11):
            for h in (0, 3):
                lo, p = orc.row_probabilities(q, k, v, T, sp, H, KVH, D, t, h, window=W)
                pos = sp + t
                assert lo == (max(0, pos - W + 1) if W else 0)
                assert p.size == pos - lo + 1
                assert (p >= 0).all() and abs(p.sum() - 1.0) <= 1e-12
    # observable form: V == 1 gives out == 1
    ones = np.ones_like(v)
    for W in (0, 3):
        out = orc.attention(q, k, ones, T, sp, H, KVH, D, window=W)
        assert np.abs(out - 1.0).max() <= 1e-14


def pin_single_key(orc):
    """L = 1: the only key gets probability exactly one."""
    rng = np.random.default_rng(RNG_SEED + 3)
    H, KVH, D = 4, 2, 8
    q, k, v = _case(rng, H, KVH, D, 1, 0)
    out = orc.attention(q, k, v, 1, 0, H, KVH, D)
    for h in range(H):
        assert np.array_equal(out[0, h], v[h // (H // KVH), 0].astype(np.float64)), h


def pin_closed_form_band(orc):
    """q = 0 makes every valid key equally likely; with V[kh, j, d] = j + 1000*kh
    the output is (lo + pos)/2 + 1000*kv_head(h) for every d."""
    for H, KVH, D, T, sp, W in ((4, 2, 8, 10, 0, 0), (4, 2, 8, 10, 30, 0), (8, 2, 4, 13, 5, 4),
                                (6, 3, 2, 9, 40, 1), (4, 4, 4, 7, 3, 2), (4, 1, 4, 6, 0, 100)):
        L = sp + T
        G = H // KVH
        q = np.zeros((T, H * D), np.float32)
        rng = np.random.default_rng(RNG_SEED + 4)
        k = _rand(rng, (KVH, L, D))
        v = np.empty((KVH, L, D), np.float32)
        for kh in range(KVH):
            v[kh] = (np.arange(L)[:, None] + 1000.0 * kh).astype(np.float32)
        out = orc.attention(q, k, v, T, sp, H, KVH, D, window=W)
        for t in range(T):
            pos = sp + t
            lo = max(0, pos - W + 1) if W > 0 else 0
            for h in range(H):
                want = (lo + pos) / 2.0 + 1000.0 * (h // G)
                assert np.abs(out[t, h] - want).max() <= 1e-9, (t, h, W, out[t, h, 0], want)


def pin_identical_keys_mean(orc):
    """All keys of a kv head equal: output = mean of the valid value rows."""
    rng = np.random.default_rng(RNG_SEED + 5)
    H, KVH, D, T, sp = 4, 2, 8, 9, 6
    L = sp + T
    q = _rand(rng, (T, H * D), 3.0)
    k = np.repeat(_rand(rng, (KVH, 1, D)), L, axis=1)
    v = _rand(rng, (KVH, L, D))
    for W in (0, 3):
        out = orc.attention(q, k, v, T, sp, H, KVH, D, window=W)
        for t in range(T):
            pos = sp + t
            lo = max(0, pos - W + 1) if W > 0 else 0
            for h in range(H):
                want = v[h // (H // KVH), lo:pos + 1].astype(np.float64).mean(axis=0)
                assert np.abs(out[t, h] - want).max() <= 1e-12


def pin_gqa_map(orc):
    """V constant per kv head (kh + 1): output = kv_head(h) + 1; MHA and MQA included."""
    rng = np.random.default_rng(RNG_SEED + 6)
    for H, KVH in ((8, 2), (8, 4), (6, 2), (4, 4), (4, 1)):
        D, T, sp = 4, 5, 3
        L = sp + T
        q, k, _ = _case(rng, H, KVH, D, T, sp)
        v = np.empty((KVH, L, D), np.float32)
        for kh in range(KVH):
            v[kh] = kh + 1.0
        out = orc.attention(q, k, v, T, sp, H, KVH, D)
        for h in range(H):
            assert np.abs(out[:, h] - (h // (H // KVH) + 1.0)).max() <= 1e-12, (H, KVH, h)


def pin_window_edges(orc):
    """window = 1 keeps only the query's own key; window >= L is no window."""
    rng = np.random.default_rng(RNG_SEED + 7)
    H, KVH, D, T, sp = 4, 2, 8, 6, 9
    L = sp + T
    q, k, v = _case(rng, H, KVH, D, T, sp)
    out1 = orc.attention(q, k, v, T, sp, H, KVH, D, window=1)
    for t in range(T):
        for h in range(H):
            assert np.array_equal(out1[t, h], v[h // 2, sp + t].astype(np.float64))
    full = orc.attention(q, k, v, T, sp, H, KVH, D, window=0)
    for W in (L, L + 1, 10 * L):
        assert np.array_equal(orc.attention(q, k, v, T, sp, H, KVH, D, window=W), full)


def pin_chunked_equals_one_shot(orc):
    """Prefill in chunks over a growing cache gives the one-shot rows bit for bit;
    T = 1 at start_pos = p gives row p (decode)."""
    rng = np.random.default_rng(RNG_SEED + 8)
    H, KVH, D, N = 4, 2, 16, 24
    q, k, v = _case(rng, H, KVH, D, N, 0)
    for W in (0, 5):
        whole = orc.attention(q, k, v, N, 0, H, KVH, D, window=W)
        start = 0
        for T in (7, 9, 8):
            part = orc.attention(q[start:start + T], k, v, T, start, H, KVH, D, window=W,
                                 kv_head_stride=N * D)
            assert np.array_equal(part, whole[start:start + T]), (W, start)
            start += T
        for p in (0, 1, 13, N - 1):
            one = orc.attention(q[p:p + 1], k, v, 1, p, H, KVH, D, window=W, kv_head_stride=N * D)
            assert np.array_equal(one[0], whole[p]), (W, p)


def pin_mask_edges(orc):
    """Keys just outside a row's band [lo, pos] cannot change that row (planted
    huge keys at pos+1 and lo-1); keys on the band's edges do change it."""
    rng = np.random.default_rng(RNG_SEED + 9)
    H, KVH, D, T, sp = 4, 2, 8, 8, 12
    L = sp + T
    q, k, v = _case(rng, H, KVH, D, T, sp)
    for W in (0, 4):
        base = orc.attention(q, k, v, T, sp, H, KVH, D, window=W)
        for t in (0, 3, 7):
            pos = sp + t
            lo = max(0, pos - W + 1) if W > 0 else 0
            outside = [j for j in (pos + 1, lo - 1) if 0 <= j < L]
            inside = [pos, lo]
            for j in outside:
                k2, v2 = k.copy(), v.copy()
                k2[:, j] = 50.0 * np.sign(q[t].reshape(H, D)[0])  # huge score for head 0
                v2[:, j] = 1e6
                got = orc.attention(q, k2, v2, T, sp, H, KVH, D, window=W)
                assert np.array_equal(got[t], base[t]), ("outside key leaked", W, t, j)
            for j in inside:
                v2 = v.copy()
                v2[:, j] += 1.0
                got = orc.attention(q, k, v2, T, sp, H, KVH, D, window=W)
                assert np.abs(got[t] - base[t]).min() > 0, ("edge key ignored", W, t, j)


def pin_shift_invariance(orc):
    """K' = K + u (u fixed per kv head) adds a per-row constant to the scores:
    the output cannot change, even when the shifted scores (~800) would overflow exp."""
    rng = np.random.default_rng(RNG_SEED + 10)
    H, KVH, D, T, sp = 4, 2, 16, 6, 10
    L = sp + T
    # values on a 1/8 grid so that K + 256 is exact in fp32
    q = np.abs(np.round(rng.standard_normal((T, H * D)) * 8) / 8).astype(np.float32) + 0.5
    k = (np.round(rng.standard_normal((KVH, L, D)) * 8) / 8).astype(np.float32)
    v = _rand(rng, (KVH, L, D))
    base = orc.attention(q, k, v, T, sp, H, KVH, D)
    shifted = orc.attention(q, k + np.float32(256.0), v, T, sp, H, KVH, D)
    assert np.isfinite(shifted).all()
    assert np.abs(shifted - base).max() <= 1e-9


def pin_hand_example(orc):
    """Worked by hand.  D = 2, one head, T = 2 at start_pos = 1 (L = 3).
    q = (1, 0) for both rows; k_j = (sqrt(2) * a_j, 0) with a = (0, ln 2, ln 3), so
    the scaled scores q.k_j / sqrt(2) are exactly a_j and exp gives 1, 2, 3.
    Row 0 (pos 1) weighs keys 0, 1 by 1/3, 2/3; row 1 (pos 2) weighs keys 0..2 by
    1/6, 2/6, 3/6.  With v = (6, 0), (0, 6), (6, 6): row 0 = (2, 4), row 1 = (4, 5).
    With window 2, row 1 keeps keys 1, 2 with weights 2/5, 3/5: (3.6, 6)."""
    s2 = math.sqrt(2.0)
    q = np.array([[1.0, 0.0], [1.0, 0.0]], np.float32)
    k = np.array([[[0.0, 0.0], [s2 * math.log(2.0), 0.0], [s2 * math.log(3.0), 0.0]]], np.float32)
    v = np.array([[[6.0, 0.0], [0.0, 6.0], [6.0, 6.0]]], np.float32)
    out = orc.attention(q, k, v, 2, 1, 1, 1, 2)
    # fp32 storage of sqrt(2)*ln(x) perturbs the exact scores by ~1e-7 relative
    assert np.abs(out[:, 0] - np.array([[2.0, 4.0], [4.0, 5.0]])).max() <= 1e-6, out
    outw = orc.attention(q, k, v, 2, 1, 1, 1, 2, window=2)
    assert np.abs(outw[1, 0] - np.array([3.6, 6.0])).max() <= 1e-6, outw
    assert np.abs(outw[0, 0] - np.array([2.0, 4.0])).max() <= 1e-6, outw


def pin_strided_layouts(orc):
    """A padded query row stride and a cache allocated beyond L (NaN past L) give
    the packed result: rows past L are never read."""
    rng = np.random.default_rng(RNG_SEED + 11)
    H, KVH, D, T, sp = 4, 2, 8, 5, 7
    L = sp + T
    q, k, v = _case(rng, H, KVH, D, T, sp)
    packed = orc.attention(q, k, v, T, sp, H, KVH, D, window=3)
    qs = H * D + 24
    qp = np.full((T, qs), np.nan, np.float32)
    qp[:, :H * D] = q
    cap = L + 9
    kp = np.full((KVH, cap, D), np.nan, np.float32)
    vp = np.full((KVH, cap, D), np.nan, np.float32)
    kp[:, :L], vp[:, :L] = k, v
    got = orc.attention(qp, kp, vp, T, sp, H, KVH, D, window=3, q_row_stride=qs, kv_head_stride=cap * D)
    assert np.array_equal(got, packed)
    rows_t = np.array([0, 4, 2, 4])
    rows_h = np.array([3, 0, 1, 2])
    sub = orc.rows(qp, kp, vp, T, sp, H, KVH, D, rows_t, rows_h, window=3, q_row_stride=qs,
                   kv_head_stride=cap * D)
    assert np.array_equal(sub, packed[rows_t, rows_h])


def _ring_writes(rows, ring_slots, upto, ring=None):
    """Write keys 0 .. upto-1 of rows [KVH, positions, D] one by one into slot
    pos % ring_slots of a ring (NaN where nothing was written), as the cache
    writes of a sliding-window layer do."""
    if ring is None:
        ring = np.full((rows.shape[0], ring_slots, rows.shape[2]), np.nan, np.float32)
    for j in range(upto):
        ring[:, j % ring_slots] = rows[:, j]
    return ring


def pin_ring_closed_form(orc):
    """Ring cache (key j in slot j % R, written in order): with q = 0 and
    V[kh, j] = j + 1000*kh the output is still (lo + pos)/2 + 1000*kv_head(h)."""
    for H, KVH, D, T, sp, W, R in ((4, 2, 4, 6, 20, 5, 10), (4, 1, 8, 9, 31, 3, 11),
                                   (2, 2, 2, 5, 0, 4, 8), (4, 2, 4, 1, 57, 7, 7)):
        L = sp + T
        G = H // KVH
        q = np.zeros((T, H * D), np.float32)
        rng = np.random.default_rng(RNG_SEED + 12)
        k = _rand(rng, (KVH, L, D))
        v = np.empty((KVH, L, D), np.float32)
        for kh in range(KVH):
            v[kh] = (np.arange(L)[:, None] + 1000.0 * kh).astype(np.float32)
        out = orc.attention(q, _ring_writes(k, R, L), _ring_writes(v, R, L), T, sp, H, KVH, D,
                            window=W, ring_slots=R)
        for t in range(T):
            pos = sp + t
            lo = max(0, pos - W + 1)
            for h in range(H):
                want = (lo + pos) / 2.0 + 1000.0 * (h // G)
                assert np.abs(out[t, h] - want).max() <= 1e-9, (t, h, R, out[t, h, 0], want)


def pin_ring_chunked_equals_linear(orc):
    """A prompt prefilled chunk by chunk through a ring of window + T - 1 slots
    (each chunk's keys written before its call, older ones overwritten, unwritten
    slots NaN) gives the rows of the one-shot prefill over the linear cache."""
    rng = np.random.default_rng(RNG_SEED + 13)
    H, KVH, D, N, W = 4, 2, 8, 40, 6
    q, k, v = _case(rng, H, KVH, D, N, 0)
    full = orc.attention(q, k, v, N, 0, H, KVH, D, window=W)
    for chunks, extra in (((7, 7, 1, 12, 13), 0), ((9, 9, 9, 9, 4), 3)):
        R = W + max(chunks) - 1 + extra
        kr = vr = None
        start = 0
        for T in chunks:
            kr = _ring_writes(k, R, start + T, kr)
            vr = _ring_writes(v, R, start + T, vr)
            got = orc.attention(q[start:start + T], kr, vr, T, start, H, KVH, D, window=W,
                                ring_slots=R)
            assert np.array_equal(got, full[start:start + T]), (chunks, start)
            rows_t = np.array([0, T - 1])
            rows_h = np.array([H - 1, 0])
            sub = orc.rows(q[start:start + T], kr, vr, T, start, H, KVH, D, rows_t, rows_h,
                           window=W, ring_slots=R)
            assert np.array_equal(sub, full[start + rows_t, rows_h])
            start += T
    # a ring one slot short of what a chunk reads at once is refused
    try:
        orc.attention(q[:8], k[:, :8], v[:, :8], 8, 0, H, KVH, D, window=W, ring_slots=W + 8 - 2)
    except ValueError:
        pass
    else:
        raise AssertionError("short ring accepted")


def pin_kv_write_linear(orc):
    """Appending a chunk writes rows start_pos .. start_pos+T-1 of every kv head
    from the (strided) source and touches nothing else."""
    rng = np.random.default_rng(RNG_SEED + 14)
    KVH, D, T, sp, cap, srs = 3, 8, 6, 5, 20, 3 * 8 + 8
    ks, vs = _rand(rng, (T, srs)), _rand(rng, (T, srs))
    kc = np.full((KVH, cap, D), np.nan, np.float32)
    vc = np.full((KVH, cap, D), np.nan, np.float32)
    orc.kv_write(ks, vs, srs, kc, vc, cap * D, T, sp, KVH, D)
    for kh in range(KVH):
        assert np.array_equal(kc[kh, sp:sp + T], ks[:, kh * D:(kh + 1) * D])
        assert np.array_equal(vc[kh, sp:sp + T], vs[:, kh * D:(kh + 1) * D])
    assert np.isnan(kc[:, :sp]).all() and np.isnan(kc[:, sp + T:]).all()
    assert np.isnan(vc[:, :sp]).all() and np.isnan(vc[:, sp + T:]).all()


def pin_kv_write_ring(orc):
    """In a ring of R slots each slot ends up holding the chunk's last token
    whose position falls on it (in-order writes), or what it held before."""
    rng = np.random.default_rng(RNG_SEED + 15)
    KVH, D = 2, 4
    for T, sp, R in ((11, 3, 4), (3, 9, 8), (8, 0, 8), (1, 29, 5)):
        ks, vs = _rand(rng, (T, KVH * D)), _rand(rng, (T, KVH * D))
        old = _rand(rng, (KVH, R, D))
        kc, vc = old.copy(), old.copy()
        orc.kv_write(ks, vs, KVH * D, kc, vc, R * D, T, sp, KVH, D, ring_slots=R)
        for slot in range(R):
            hits = [i for i in range(T) if (sp + i) % R == slot]
            for kh in range(KVH):
                want_k = ks[hits[-1], kh * D:(kh + 1) * D] if hits else old[kh, slot]
                want_v = vs[hits[-1], kh * D:(kh + 1) * D] if hits else old[kh, slot]
                assert np.array_equal(kc[kh, slot], want_k), (T, sp, R, slot)
                assert np.array_equal(vc[kh, slot], want_v), (T, sp, R, slot)


def pin_kv_write_then_attend(orc):
    """Prefill as the pages run it, chunk by chunk: write the chunk's K/V into a
    ring (then attend over it) equals the one-shot prefill over the whole
    prompt's K/V, bit for bit."""
    rng = np.random.default_rng(RNG_SEED + 16)
    H, KVH, D, N, W = 4, 2, 8, 30, 5
    q = _rand(rng, (N, H * D))
    ksrc, vsrc = _rand(rng, (N, KVH * D)), _rand(rng, (N, KVH * D))
    k_lin = np.ascontiguousarray(ksrc.reshape(N, KVH, D).transpose(1, 0, 2))
    v_lin = np.ascontiguousarray(vsrc.reshape(N, KVH, D).transpose(1, 0, 2))
    full = orc.attention(q, k_lin, v_lin, N, 0, H, KVH, D, window=W)
    R = W + 9 - 1
    kr = np.full((KVH, R, D), np.nan, np.float32)
    vr = np.full((KVH, R, D), np.nan, np.float32)
    start = 0
    for T in (9, 1, 9, 4, 7):
        orc.kv_write(ksrc[start:start + T], vsrc[start:start + T], KVH * D, kr, vr, R * D, T,
                     start, KVH, D, ring_slots=R)
        got = orc.attention(q[start:start + T], kr, vr, T, start, H, KVH, D, window=W,
                            ring_slots=R)
        assert np.array_equal(got, full[start:start + T]), start
        start += T


def _pages(rows, page_size, L, num_pages, order):
    """Pool [num_pages, KVH, page_size, D] (NaN where no key sits) and table:
    block b of keys goes to page order[b]."""
    kvh, _, d = rows.shape
    pool = np.full((num_pages, kvh, page_size, d), np.nan, np.float32)
    n = -(-L // page_size)
    for b in range(n):
        for r in range(page_size):
            j = b * page_size + r
            if j < L:
                pool[order[b], :, r] = rows[:, j]
    return pool, np.array(order[:n], np.int32)


def pin_paged_equals_linear(orc):
    """A paged cache (pages in scrambled pool order, NaN in unused pool rows)
    gives the linear cache's result bit for bit, with and without a window;
    blocks below every row's window may point anywhere, even off the pool."""
    rng = np.random.default_rng(RNG_SEED + 17)
    H, KVH, D = 4, 2, 8
    for T, sp, W, P in ((5, 40, 0, 8), (9, 30, 7, 4), (1, 63, 16, 16), (12, 0, 0, 4)):
        L = sp + T
        q, k, v = _case(rng, H, KVH, D, T, sp)
        want = orc.attention(q, k, v, T, sp, H, KVH, D, window=W)
        npages = -(-L // P) + 3
        order = list(rng.permutation(npages))
        kp, table = _pages(k, P, L, npages, order)
        vp, _ = _pages(v, P, L, npages, order)
        if W:
            lo_min = max(0, sp - W + 1)
            table = table.copy()
            table[:lo_min // P] = -5            # blocks no row reads
        got = orc.attention_paged(q, kp, vp, table, P, T, sp, H, KVH, D, window=W)
        assert np.array_equal(got, want), (T, sp, W, P)
        rt, rh = np.array([T - 1, 0]), np.array([0, H - 1])
        sub = orc.rows_paged(q, kp, vp, table, P, T, sp, H, KVH, D, rt, rh, window=W)
        assert np.array_equal(sub, want[rt, rh])
    # a key some row reads whose page is off the pool is refused
    q, k, v = _case(rng, H, KVH, D, 3, 5)
    kp, table = _pages(k, 4, 8, 2, [1, 0])
    vp, _ = _pages(v, 4, 8, 2, [1, 0])
    bad = table.copy()
    bad[1] = 7
    try:
        orc.attention_paged(q, kp, vp, bad, 4, 3, 5, H, KVH, D)
    except ValueError:
        pass
    else:
        raise AssertionError("page off the pool accepted")


def pin_paged_closed_form(orc):
    """q = 0 over a paged cache with V[kh, j] = j + 1000*kh: (lo + pos)/2 + 1000*kv_head(h)."""
    H, KVH, D, T, sp, W, P = 4, 2, 4, 6, 37, 9, 8
    L, G = sp + T, H // KVH
    rng = np.random.default_rng(RNG_SEED + 18)
    k = _rand(rng, (KVH, L, D))
    v = np.empty((KVH, L, D), np.float32)
    for kh in range(KVH):
        v[kh] = (np.arange(L)[:, None] + 1000.0 * kh).astype(np.float32)
    order = [3, 0, 5, 1, 4, 2, 6]
    kp, table = _pages(k, P, L, 7, order)
    vp, _ = _pages(v, P, L, 7, order)
    out = orc.attention_paged(np.zeros((T, H * D), np.float32), kp, vp, table, P, T, sp, H, KVH, D,
                              window=W)
    for t in range(T):
        pos = sp + t
        lo = max(0, pos - W + 1)
        for h in range(H):
            assert np.abs(out[t, h] - ((lo + pos) / 2.0 + 1000.0 * (h // G))).max() <= 1e-9


ALL_PINS = [
    pin_brute_force,
    pin_torch_sdpa,
    pin_rows_sum_to_one,
    pin_single_key,
    pin_closed_form_band,
    pin_identical_keys_mean,
    pin_gqa_map,
    pin_window_edges,
    pin_chunked_equals_one_shot,
    pin_mask_edges,
    pin_shift_invariance,
    pin_hand_example,
    pin_strided_layouts,
    pin_ring_closed_form,
    pin_ring_chunked_equals_linear,
    pin_kv_write_linear,
    pin_kv_write_ring,
    pin_kv_write_then_attend,
    pin_paged_equals_linear,
    pin_paged_closed_form,
]
