"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees.  None of them re-calls the oracle's own formula as its expectation:
they use brute force with a different evaluation order (no max subtraction,
exact summation), closed forms, invariants, a library routine
(torch's scaled_dot_product_attention in float64), and a hand-worked example.

The semantics pinned (TensorRT-LLM PR #17062 "Support Inkling-NVFP4 model",
Description, Architecture list; PR #17062 review comment on _build_rel_logits;
PR #17860 "Inkling attn backend cleanup fake registry", the commit asserting
num_heads % num_kv_heads and the commit testing the window_left hand-off):
  * bias indexed by (query token, head, distance t - s), added before softmax;
  * distances at or past rel_extent - 1 share the last bucket;
  * local layers see keys t-W+1 .. t, global layers keys 0 .. t;
  * query head h reads KV head h // (Hq / Hkv).
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# small helpers

def _gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _rand(shape, g, dtype, std=1.0):
    return (torch.randn(shape, generator=g) * std).to(dtype)


def _cu(lens):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    return cu


def _f64(x):
    return x.detach().to(torch.float64).numpy()


def _round_to(x, dt):
    """x rounded to the nearest value of dtype dt, ties to even: fp32 through
    the C float conversion (struct), bf16 (8 significant bits) directly."""
    if dt == torch.float32:
        return struct.unpack("f", struct.pack("f", x))[0]
    if x == 0.0 or not math.isfinite(x):
        return x
    _, e = math.frexp(x)
    e = max(e, -125)
    return math.ldexp(round(math.ldexp(x, 8 - e)), e - 8)   # round(): ties to even


def _brute_row(qv, keys, vals, brow, t, W, R, scale):
    """Pure-Python row: weights exp(score) without max subtraction, fsum."""
    weights = []
    for s in range(len(keys)):
        if s > t or (W > 0 and t - s >= W):
            continue
        dot = math.fsum(a * b for a, b in zip(qv, keys[s]))
        bucket = t - s if t - s < R else R - 1
        weights.append((s, math.exp(scale * dot + brow[bucket])))
    l = math.fsum(w for _, w in weights)
    D = len(qv)
    out = [math.fsum(w * vals[s][i] for s, w in weights) / l for i in range(D)]
    return out, math.log(l)


def _tiny_prefill(seed, lens, Hq, Hkv, D, R, dtype, bias_std=1.0):
    g = _gen(seed)
    T = sum(lens)
    q = _rand((T, Hq, D), g, dtype)
    k = _rand((T, Hkv, D), g, dtype)
    v = _rand((T, Hkv, D), g, dtype)
    b = _rand((T, Hq, R), g, dtype, bias_std)
    return q, k, v, b


# --------------------------------------------------------------------------
# pins

def pin_brute_force_prefill(orc):
    """All rows and LSEs of tiny prefill problems against pure-Python brute force."""
    cases = [
        # lens, Hq, Hkv, D, W, R, dtype
        ([7, 13], 4, 2, 5, 0, 3, torch.float32),
        ([24], 4, 1, 3, 5, 30, torch.bfloat16),
        ([1, 24], 4, 4, 4, 2, 6, torch.float32),
        ([9, 4], 2, 2, 8, 1, 2, torch.bfloat16),
        ([17], 4, 2, 6, 5, 4, torch.float32),
    ]
    for ci, (lens, Hq, Hkv, D, W, R, dt) in enumerate(cases):
        q, k, v, b = _tiny_prefill(100 + ci, lens, Hq, Hkv, D, R, dt)
        scale = 0.37
        out, lse = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=R,
                               sm_scale=scale, want_lse=True)
        qd, kd, vd, bd = _f64(q), _f64(k), _f64(v), _f64(b)
        G = Hq // Hkv
        start = 0
        for n in lens:
            for t in range(n):
                tok = start + t
                for h in range(Hq):
                    g = h // G
                    keys = [list(kd[start + s, g]) for s in range(n)]
                    vals = [list(vd[start + s, g]) for s in range(n)]
                    ref, ref_lse = _brute_row(list(qd[tok, h]), keys, vals,
                                              list(bd[tok, h]), t, W, R, scale)
                    err = np.max(np.abs(out[tok, h] - np.array(ref)))
                    assert err < 1e-12, f"case {ci} tok {tok} h {h}: {err}"
                    assert abs(lse[tok, h] - ref_lse) < 1e-12, f"lse case {ci}"
            start += n


def pin_brute_force_decode(orc):
    """Decode rows (query at n-1) against pure-Python brute force."""
    for ci, (lens, Hq, Hkv, D, W, R, dt) in enumerate([
            ([1, 5, 19], 4, 2, 4, 0, 6, torch.float32),
            ([12, 20], 4, 1, 5, 7, 7, torch.bfloat16),
            ([3, 16], 2, 2, 3, 3, 2, torch.float32)]):
        g = _gen(200 + ci)
        B = len(lens)
        q = _rand((B, Hq, D), g, dt)
        k = _rand((sum(lens), Hkv, D), g, dt)
        v = _rand((sum(lens), Hkv, D), g, dt)
        b = _rand((B, Hq, R), g, dt)
        out, lse = orc.decode(q, k, v, b, _cu(lens), window=W, rel_extent=R,
                              sm_scale=0.5, want_lse=True)
        qd, kd, vd, bd = _f64(q), _f64(k), _f64(v), _f64(b)
        G = Hq // Hkv
        start = 0
        for bi, n in enumerate(lens):
            for h in range(Hq):
                g_ = h // G
                keys = [list(kd[start + s, g_]) for s in range(n)]
                vals = [list(vd[start + s, g_]) for s in range(n)]
                ref, ref_lse = _brute_row(list(qd[bi, h]), keys, vals, list(bd[bi, h]),
                                          n - 1, W, R, 0.5)
                assert np.max(np.abs(out[bi, h] - np.array(ref))) < 1e-12, (ci, bi, h)
                assert abs(lse[bi, h] - ref_lse) < 1e-12, (ci, bi, h)
            start += n


def _sdpa_reference(q, k, v, b, lens, W, R, scale, with_bias=True):
    """torch SDPA (float64, CPU) with the bias written as an additive mask."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    outs = []
    start = 0
    for n in lens:
        qs = q[start:start + n].to(torch.float64).permute(1, 0, 2)           # [Hq,n,D]
        ks = k[start:start + n].to(torch.float64).permute(1, 0, 2)
        vs = v[start:start + n].to(torch.float64).permute(1, 0, 2)
        ks = ks.repeat_interleave(G, dim=0)
        vs = vs.repeat_interleave(G, dim=0)
        pos = torch.arange(n)
        dist = pos[:, None] - pos[None, :]                                     # t - s
        allowed = dist >= 0
        if W > 0:
            allowed &= dist < W
        if with_bias:
            bucket = dist.clamp(0, R - 1)
            bias_rows = b[start:start + n].to(torch.float64).permute(1, 0, 2)  # [Hq,n,R]
            mask = torch.gather(bias_rows, 2, bucket.expand(Hq, n, n))
            mask = mask.masked_fill(~allowed, float("-inf"))
            o = torch.nn.functional.scaled_dot_product_attention(
                qs, ks, vs, attn_mask=mask, scale=scale)
        else:
            o = torch.nn.functional.scaled_dot_product_attention(
                qs, ks, vs, attn_mask=allowed.expand(Hq, n, n), scale=scale)
        outs.append(o.permute(1, 0, 2))
        start += n
    return torch.cat(outs, 0).numpy()


def pin_sdpa_additive_mask(orc):
    """The method is SDPA with mask[t,s] = bias[t,h,min(t-s,R-1)] on visible pairs."""
    lens = [40, 23]
    for W, R in ((9, 12), (0, 16), (30, 64)):
        q, k, v, b = _tiny_prefill(300 + W, lens, 4, 2, 16, R, torch.float32)
        out = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=R, sm_scale=0.21)
        ref = _sdpa_reference(q, k, v, b, lens, W, R, 0.21)
        assert np.max(np.abs(out - ref)) < 1e-12, (W, R)


def pin_zero_bias_is_plain_attention(orc):
    """Zero bias reproduces plain windowed/causal attention (SDPA, boolean mask)."""
    lens = [33, 10]
    for W in (0, 7):
        q, k, v, _ = _tiny_prefill(400 + W, lens, 4, 1, 8, 5, torch.bfloat16)
        b = torch.zeros((sum(lens), 4, 5), dtype=torch.bfloat16)
        out = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=5,
                          sm_scale=1 / math.sqrt(8))
        ref = _sdpa_reference(q, k, v, b, lens, W, 5, 1 / math.sqrt(8), with_bias=False)
        assert np.max(np.abs(out - ref)) < 1e-12, W


def pin_window_one_returns_own_value(orc):
    """W = 1: every query sees only itself, so O[t,h] = V[t, h // G] exactly."""
    lens = [11, 6]
    q, k, v, b = _tiny_prefill(500, lens, 4, 2, 6, 3, torch.bfloat16)
    out = orc.prefill(q, k, v, b, _cu(lens), window=1, rel_extent=3, sm_scale=0.7)
    ref = _f64(v).repeat(2, axis=1)
    assert np.array_equal(out, ref)


def pin_first_row_returns_first_value(orc):
    """Row t = 0 of every sequence sees only key 0: O = V[0, h // G] exactly."""
    lens = [5, 9, 1]
    q, k, v, b = _tiny_prefill(510, lens, 4, 2, 6, 4, torch.float32)
    for W in (0, 3):
        out = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=4, sm_scale=1.3)
        for st in _cu(lens)[:-1]:
            assert np.array_equal(out[st], _f64(v[st]).repeat(2, axis=0))


def pin_uniform_scores_average_window(orc):
    """K = 0 and bias = 0: O[t] is the plain mean of the visible values."""
    lens = [20]
    _, _, v, _ = _tiny_prefill(520, lens, 2, 1, 4, 4, torch.float32)
    q = torch.randn((20, 2, 4))
    k = torch.zeros((20, 1, 4))
    b = torch.zeros((20, 2, 4))
    for W in (0, 1, 6):
        out = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=4, sm_scale=1.0)
        vd = _f64(v)[:, 0]
        for t in range(20):
            lo = 0 if W <= 0 else max(0, t - W + 1)
            ref = vd[lo:t + 1].mean(axis=0)
            assert np.max(np.abs(out[t, 0] - ref)) < 1e-13 and np.max(
                np.abs(out[t, 1] - ref)) < 1e-13, (W, t)


def pin_bias_at_distance_selects_key(orc):
    """K = 0, bias 50 at distance d0 only: query t attends key t - d0."""
    n, R, d0 = 16, 8, 3
    v = torch.randn((n, 1, 4))
    q = torch.randn((n, 1, 4))
    k = torch.zeros((n, 1, 4))
    b = torch.zeros((n, 1, R))
    b[:, :, d0] = 50.0
    for W in (0, 6):
        out = orc.prefill(q, k, v, b, [0, n], window=W, rel_extent=R, sm_scale=1.0)
        for t in range(d0, n):
            assert np.max(np.abs(out[t, 0] - _f64(v[t - d0, 0]))) < 1e-12, (W, t)


def pin_clamped_bucket(orc):
    """Global layer, bias 50 only in the last bucket: query t attends keys 0..t-R+1."""
    n, R = 18, 4
    v = torch.randn((n, 1, 3))
    q = torch.randn((n, 1, 3))
    k = torch.zeros((n, 1, 3))
    b = torch.zeros((n, 1, R))
    b[:, :, R - 1] = 50.0
    out = orc.prefill(q, k, v, b, [0, n], window=0, rel_extent=R, sm_scale=1.0)
    vd = _f64(v)[:, 0]
    for t in range(n):
        far = t - (R - 1)
        ref = vd[:far + 1].mean(axis=0) if far >= 0 else vd[:t + 1].mean(axis=0)
        assert np.max(np.abs(out[t, 0] - ref)) < 1e-12, t


def pin_gqa_head_mapping(orc):
    """K = 0, V[s, g] = g + 1: query head h must return h // (Hq/Hkv) + 1."""
    n, Hq, Hkv = 7, 8, 2
    q = torch.randn((n, Hq, 4))
    k = torch.zeros((n, Hkv, 4))
    v = torch.zeros((n, Hkv, 4))
    for g in range(Hkv):
        v[:, g] = g + 1.0
    b = torch.randn((n, Hq, 3))
    out = orc.prefill(q, k, v, b, [0, n], window=0, rel_extent=3, sm_scale=1.0)
    G = Hq // Hkv
    for h in range(Hq):
        assert np.all(out[:, h] == h // G + 1.0), h


def pin_row_constant_bias_shift(orc):
    """Adding c[t,h] to a whole bias row leaves the output unchanged."""
    lens = [15, 30]
    q, k, v, b = _tiny_prefill(600, lens, 4, 2, 8, 10, torch.float32)
    c = torch.randn((sum(lens), 4, 1)) * 3.0
    b2 = (b.double() + c.double()).float()
    for W in (0, 4):
        o1 = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=10, sm_scale=0.4)
        o2 = orc.prefill(q, k, v, b2, _cu(lens), window=W, rel_extent=10, sm_scale=0.4)
        assert np.max(np.abs(o1 - o2)) < 1e-6, W   # b2 is rounded to fp32


def pin_masked_positions_have_no_effect(orc):
    """Changing anything a row cannot see leaves that row bit-identical."""
    lens = [26, 12]
    for W, R in ((0, 6), (5, 5), (9, 30)):
        q, k, v, b = _tiny_prefill(700 + W, lens, 4, 2, 6, R, torch.float32)
        base = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=R, sm_scale=0.6)
        g = _gen(800 + W)
        for t in (0, 4, 13, 25):
            k2, v2, b2 = k.clone(), v.clone(), b.clone()
            # future keys, keys before the window, and the other sequence
            k2[t + 1:26] = torch.randn(k2[t + 1:26].shape, generator=g)
            v2[t + 1:26] = torch.randn(v2[t + 1:26].shape, generator=g)
            if W > 0 and t - W + 1 > 0:
                k2[:t - W + 1] = torch.randn(k2[:t - W + 1].shape, generator=g)
                v2[:t - W + 1] = torch.randn(v2[:t - W + 1].shape, generator=g)
            k2[26:] = 1e3
            v2[26:] = -1e3
            # bias buckets the row cannot reach: d > t, and d >= W on local layers
            if t + 1 < R:
                b2[t, :, t + 1:] = torch.randn(b2[t, :, t + 1:].shape, generator=g)
            if W > 0 and W < R:
                b2[t, :, W:] = torch.randn(b2[t, :, W:].shape, generator=g)
            o2 = orc.prefill(q, k2, v2, b2, _cu(lens), window=W, rel_extent=R, sm_scale=0.6)
            assert np.array_equal(base[t], o2[t]), (W, R, t)


def pin_decode_is_last_prefill_row(orc):
    """Decode at n keys equals prefill row n-1 on the same keys and bias row."""
    lens = [9, 21, 1]
    for W, R in ((0, 8), (6, 6)):
        q, k, v, b = _tiny_prefill(900 + W, lens, 4, 2, 5, R, torch.bfloat16)
        pre = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=R, sm_scale=0.45)
        last = [c - 1 for c in _cu(lens)[1:]]
        dec = orc.decode(q[last], k, v, b[last], _cu(lens), window=W, rel_extent=R,
                         sm_scale=0.45)
        assert np.array_equal(dec, pre[last]), (W, R)


def _tiny_history(seed, n_keys, n_new, Hq, Hkv, D, R, dtype):
    """Keys of len n_keys[b] per sequence; queries and bias rows for the last
    n_new[b] positions."""
    g = _gen(seed)
    q = _rand((sum(n_new), Hq, D), g, dtype)
    k = _rand((sum(n_keys), Hkv, D), g, dtype)
    v = _rand((sum(n_keys), Hkv, D), g, dtype)
    b = _rand((sum(n_new), Hq, R), g, dtype)
    return q, k, v, b


def pin_brute_force_prefill_history(orc):
    """Prefill over a cached history: each new token's row at its absolute
    position n - L + i against pure-Python brute force."""
    cases = [
        # n_keys, n_new, Hq, Hkv, D, W, R, dtype
        ([9, 20], [3, 20], 4, 2, 4, 0, 6, torch.float32),
        ([16, 5], [1, 2], 2, 1, 5, 4, 9, torch.bfloat16),
        ([23], [7], 4, 4, 3, 6, 5, torch.float32),
    ]
    for ci, (nk, nq, Hq, Hkv, D, W, R, dt) in enumerate(cases):
        q, k, v, b = _tiny_history(1300 + ci, nk, nq, Hq, Hkv, D, R, dt)
        out, lse = orc.prefill_history(q, k, v, b, _cu(nq), _cu(nk), window=W, rel_extent=R,
                                       sm_scale=0.4, want_lse=True)
        qd, kd, vd, bd = _f64(q), _f64(k), _f64(v), _f64(b)
        G = Hq // Hkv
        cq, ck = _cu(nq), _cu(nk)
        for bi, (n, L) in enumerate(zip(nk, nq)):
            for i in range(L):
                tok = cq[bi] + i
                for h in range(Hq):
                    keys = [list(kd[ck[bi] + s, h // G]) for s in range(n)]
                    vals = [list(vd[ck[bi] + s, h // G]) for s in range(n)]
                    ref, ref_lse = _brute_row(list(qd[tok, h]), keys, vals, list(bd[tok, h]),
                                              n - L + i, W, R, 0.4)
                    assert np.max(np.abs(out[tok, h] - np.array(ref))) < 1e-12, (ci, tok, h)
                    assert abs(lse[tok, h] - ref_lse) < 1e-12, (ci, tok, h)


def pin_history_rows_of_full_prefill(orc):
    """A prefill of the last L tokens over the first n - L as history returns
    the last L rows of a plain prefill of all n tokens (chunked prefill
    changes nothing)."""
    lens, new = [30, 12, 7], [11, 12, 1]
    for W, R in ((0, 9), (5, 5), (13, 40)):
        q, k, v, b = _tiny_prefill(1400 + W, lens, 4, 2, 5, R, torch.bfloat16)
        full = orc.prefill(q, k, v, b, _cu(lens), window=W, rel_extent=R, sm_scale=0.35)
        sel = [c - m + i for c, m in zip(_cu(lens)[1:], new) for i in range(m)]
        part = orc.prefill_history(q[sel], k, v, b[sel], _cu(new), _cu(lens), window=W,
                                   rel_extent=R, sm_scale=0.35)
        assert np.array_equal(part, full[sel]), (W, R)


def pin_history_single_query_is_decode(orc):
    """One new token per sequence over its history equals single-token decode."""
    lens = [6, 17, 1]
    g = _gen(1500)
    q = _rand((3, 4, 4), g, torch.float32)
    k = _rand((sum(lens), 2, 4), g, torch.float32)
    v = _rand((sum(lens), 2, 4), g, torch.float32)
    b = _rand((3, 4, 8), g, torch.float32)
    for W in (0, 4):
        dec = orc.decode(q, k, v, b, _cu(lens), window=W, rel_extent=8, sm_scale=0.6)
        hist = orc.prefill_history(q, k, v, b, _cu([1, 1, 1]), _cu(lens), window=W,
                                   rel_extent=8, sm_scale=0.6)
        assert np.array_equal(dec, hist), W


def pin_history_rejects_more_queries_than_keys(orc):
    """A sequence with more new tokens than keys is rejected."""
    q = torch.randn((3, 2, 2))
    k = torch.randn((2, 1, 2))
    b = torch.randn((3, 2, 3))
    try:
        orc.prefill_history(q, k, k, b, [0, 3], [0, 2], window=0, rel_extent=3, sm_scale=1.0)
    except ValueError:
        return
    raise AssertionError("more queries than keys accepted")


def pin_gqa_equals_repeated_mha(orc):
    """GQA equals MHA with every KV head repeated for its query heads."""
    lens = [14, 5]
    q, k, v, b = _tiny_prefill(1000, lens, 6, 2, 4, 7, torch.float32)
    o1 = orc.prefill(q, k, v, b, _cu(lens), window=4, rel_extent=7, sm_scale=0.5)
    o2 = orc.prefill(q, k.repeat_interleave(3, 1), v.repeat_interleave(3, 1), b,
                     _cu(lens), window=4, rel_extent=7, sm_scale=0.5)
    assert np.array_equal(o1, o2)


def pin_global_equals_wide_window(orc):
    """Full causal equals a sliding window at least as long as the sequence."""
    lens = [19]
    q, k, v, b = _tiny_prefill(1100, lens, 2, 1, 4, 25, torch.float32)
    o1 = orc.prefill(q, k, v, b, _cu(lens), window=0, rel_extent=25, sm_scale=0.5)
    o2 = orc.prefill(q, k, v, b, _cu(lens), window=19, rel_extent=25, sm_scale=0.5)
    assert np.array_equal(o1, o2)


def pin_row_subset_matches(orc):
    """Asking for a subset of rows returns exactly those rows of the full result."""
    lens = [10, 17]
    q, k, v, b = _tiny_prefill(1200, lens, 4, 2, 4, 5, torch.bfloat16)
    full = orc.prefill(q, k, v, b, _cu(lens), window=3, rel_extent=5, sm_scale=0.3)
    rows = [(26, 3), (0, 0), (11, 2), (10, 1)]
    sub = orc.prefill(q, k, v, b, _cu(lens), window=3, rel_extent=5, sm_scale=0.3, rows=rows)
    for i, (tok, h) in enumerate(rows):
        assert np.array_equal(sub[i], full[tok, h])


def pin_worked_example(orc):
    """Hand-worked two-token example (tests/golden/two_token_worked_example.json)."""
    with open(os.path.join(GOLDEN, "two_token_worked_example.json")) as f:
        ex = json.load(f)
    q = torch.tensor(ex["q"], dtype=torch.float32)
    k = torch.tensor(ex["k"], dtype=torch.float32)
    v = torch.tensor(ex["v"], dtype=torch.float32)
    b = torch.tensor(ex["bias"], dtype=torch.float32)
    out, lse = orc.prefill(q, k, v, b, [0, 2], window=ex["window"],
                           rel_extent=ex["rel_extent"], sm_scale=ex["sm_scale"],
                           want_lse=True)
    cf = ex["closed_form"]
    s = 1.0 / (1.0 + math.exp(-cf["row1_weight_on_key0_logit_gap"]))
    exp_out = np.array([[[1.0, 0.0]], [[s, 1.0 - s]]])
    exp_lse = np.array([[cf["row0_lse"]],
                        [cf["row1_lse_base"] + math.log1p(math.exp(-cf["row1_weight_on_key0_logit_gap"]))]])
    assert np.max(np.abs(out - exp_out)) < 1e-15
    assert np.max(np.abs(lse - exp_lse)) < 1e-15
    # the same example through decode: the query of a 2-key sequence is row 1
    dec = orc.decode(q[1:2], k, v, b[1:2], [0, 2], window=ex["window"],
                     rel_extent=ex["rel_extent"], sm_scale=ex["sm_scale"])
    assert np.max(np.abs(dec[0] - exp_out[1])) < 1e-15


def pin_rejects_indivisible_heads(orc):
    """Hq not divisible by Hkv is rejected, never silently mapped."""
    q = torch.randn((4, 3, 2))
    k = torch.randn((4, 2, 2))
    b = torch.randn((4, 3, 2))
    try:
        orc.prefill(q, k, k, b, [0, 4], window=0, rel_extent=2, sm_scale=1.0)
    except ValueError:
        return
    raise AssertionError("indivisible head counts accepted")


# --------------------------------------------------------------------------
# the bias given by its projection, bias[t,h,d] = sum_k r[t,h,k] w[k,d]

def _tiny_projected(seed, n_keys, n_new, Hq, Hkv, D, R, d_rel, dtype):
    g = _gen(seed)
    q = _rand((sum(n_new), Hq, D), g, dtype)
    k = _rand((sum(n_keys), Hkv, D), g, dtype)
    v = _rand((sum(n_keys), Hkv, D), g, dtype)
    r = _rand((sum(n_new), Hq, d_rel), g, dtype, 0.7)
    w = _rand((d_rel, R), g, dtype, 0.7)
    return q, k, v, r, w


def pin_brute_force_prefill_projected(orc):
    """Rows and LSEs against pure-Python brute force whose bias row is the
    fsum over k of r[t,h,k] w[k,d] rounded once to the inputs' dtype, with and
    without a cached history."""
    cases = [
        # n_keys, n_new (None: no history), Hq, Hkv, D, W, R, d_rel, dtype
        ([6, 11], None, 4, 2, 3, 0, 4, 3, torch.float32),
        ([9, 20], [3, 20], 2, 1, 4, 5, 7, 2, torch.bfloat16),
        ([13], [13], 2, 2, 2, 0, 16, 5, torch.float32),
    ]
    for ci, (n_keys, n_new, Hq, Hkv, D, W, R, d_rel, dt) in enumerate(cases):
        new = n_new if n_new is not None else n_keys
        q, k, v, r, w = _tiny_projected(300 + ci, n_keys, new, Hq, Hkv, D, R, d_rel, dt)
        scale = 0.41
        out, lse = orc.prefill_projected(q, k, v, r, w, _cu(new),
                                         _cu(n_keys) if n_new is not None else None,
                                         window=W, sm_scale=scale, want_lse=True)
        qd, kd, vd, rd, wd = _f64(q), _f64(k), _f64(v), _f64(r), _f64(w)
        G = Hq // Hkv
        tok, k0 = 0, 0
        for n, L in zip(n_keys, new):
            for i in range(L):
                t = n - L + i
                for h in range(Hq):
                    g = h // G
                    brow = [_round_to(math.fsum(rd[tok, h, kk] * wd[kk, d] for kk in range(d_rel)), dt)
                            for d in range(R)]
                    keys = [list(kd[k0 + s, g]) for s in range(n)]
                    vals = [list(vd[k0 + s, g]) for s in range(n)]
                    ref, ref_lse = _brute_row(list(qd[tok, h]), keys, vals, brow, t, W, R, scale)
                    err = np.max(np.abs(out[tok, h] - np.array(ref)))
                    assert err < 1e-12, f"case {ci} tok {tok} h {h}: {err}"
                    assert abs(lse[tok, h] - ref_lse) < 1e-12, f"lse case {ci}"
                tok += 1
            k0 += n


def pin_projection_rounds_like_torch(orc):
    """r = (1, 1): the bias entry is w[0,d] + w[1,d] rounded to the dtype.
    That sum is exact in fp32 (bf16 inputs) and in fp64 (fp32 inputs), so
    torch's own conversion of it (round to nearest, ties to even) gives the
    entry, and the result equals the prefill given that tensor exactly.  The
    first columns hold exact bf16 ties: 1 + 2^-8 must round down to 1 and
    1 + 3*2^-8 up to 1 + 2^-6."""
    n, Hq, D, R = 10, 2, 4, 40
    g = _gen(47)
    for dt, wide in ((torch.bfloat16, torch.float32), (torch.float32, torch.float64)):
        q, k, v = (_rand((n, Hq, D), g, dt), _rand((n, 1, D), g, dt), _rand((n, 1, D), g, dt))
        r = torch.ones((n, Hq, 2), dtype=dt)
        w = _rand((2, R), g, dt, 3.0)
        w[0, 0], w[1, 0] = 1.0, 2.0 ** -8
        w[0, 1], w[1, 1] = 1.0 + 2.0 ** -7, 2.0 ** -8
        w[0, 2], w[1, 2] = -1.0, -(2.0 ** -8)
        s = w[0].to(wide) + w[1].to(wide)
        assert torch.equal(s.double(), w[0].double() + w[1].double())   # the sum is exact
        b = s.to(dt)
        if dt == torch.bfloat16:
            assert b[0].item() == 1.0 and b[1].item() == 1.0 + 2.0 ** -6 and b[2].item() == -1.0
        bias = b.expand(n, Hq, R).contiguous()
        got = orc.prefill_projected(q, k, v, r, w, [0, n], window=0, sm_scale=0.5)
        ref = orc.prefill(q, k, v, bias, [0, n], window=0, rel_extent=R, sm_scale=0.5)
        assert np.array_equal(got, ref), str(dt)


def pin_projection_by_permutation(orc):
    """w a permutation matrix (w[k, perm[k]] = 1): the bias row is r with its
    columns permuted, bias[t,h,perm[k]] = r[t,h,k], so the result equals the
    prefill given that tensor exactly.  perm is not an involution, so reading
    w transposed gives a different row."""
    n, Hq, D, R = 14, 2, 4, 6
    perm = [2, 0, 5, 1, 3, 4]
    g = _gen(41)
    q, k, v = (_rand((n, Hq, D), g, torch.float32), _rand((n, 1, D), g, torch.float32),
               _rand((n, 1, D), g, torch.float32))
    r = _rand((n, Hq, R), g, torch.float32, 2.0)
    w = torch.zeros((R, R))
    for kk, d in enumerate(perm):
        w[kk, d] = 1.0
    b = torch.empty_like(r)
    for kk, d in enumerate(perm):
        b[:, :, d] = r[:, :, kk]
    for W in (0, 5):
        got = orc.prefill_projected(q, k, v, r, w, [0, 6, n], window=W, sm_scale=0.8)
        ref = orc.prefill(q, k, v, b, [0, 6, n], window=W, rel_extent=R, sm_scale=0.8)
        assert np.array_equal(got, ref), W


def pin_projection_equal_columns_is_unbiased(orc):
    """All columns of w equal: every bias row is one constant, which the
    softmax cancels, so the result is attention without a bias."""
    n, Hq, D, R, d_rel = 12, 2, 4, 5, 3
    g = _gen(43)
    q, k, v = (_rand((n, Hq, D), g, torch.float32), _rand((n, 2, D), g, torch.float32),
               _rand((n, 2, D), g, torch.float32))
    r = _rand((n, Hq, d_rel), g, torch.float32, 3.0)
    w = _rand((d_rel, 1), g, torch.float32).expand(d_rel, R).contiguous()
    got = orc.prefill_projected(q, k, v, r, w, [0, n], window=0, sm_scale=0.6)
    ref = orc.prefill(q, k, v, torch.zeros((n, Hq, R)), [0, n], window=0, rel_extent=R,
                      sm_scale=0.6)
    assert np.max(np.abs(got - ref)) < 1e-12


def pin_projection_last_column_is_clamped_bucket(orc):
    """r[t,h] = e_0 and w[0] = 50 in the last column only: every distance at
    or beyond R-1 carries the bias, so query t averages keys 0 .. t-R+1."""
    n, R, d_rel = 18, 4, 2
    v = torch.randn((n, 1, 3))
    q = torch.randn((n, 1, 3))
    k = torch.zeros((n, 1, 3))
    r = torch.zeros((n, 1, d_rel))
    r[:, :, 0] = 1.0
    w = torch.zeros((d_rel, R))
    w[0, R - 1] = 50.0
    w[1, 0] = 50.0          # never used: r[..., 1] = 0
    out = orc.prefill_projected(q, k, v, r, w, [0, n], window=0, sm_scale=1.0)
    vd = _f64(v)[:, 0]
    for t in range(n):
        far = t - (R - 1)
        ref = vd[:far + 1].mean(axis=0) if far >= 0 else vd[:t + 1].mean(axis=0)
        assert np.max(np.abs(out[t, 0] - ref)) < 1e-12, t


ALL_PINS = [
    pin_brute_force_prefill,
    pin_brute_force_decode,
    pin_sdpa_additive_mask,
    pin_zero_bias_is_plain_attention,
    pin_window_one_returns_own_value,
    pin_first_row_returns_first_value,
    pin_uniform_scores_average_window,
    pin_bias_at_distance_selects_key,
    pin_clamped_bucket,
    pin_gqa_head_mapping,
    pin_row_constant_bias_shift,
    pin_masked_positions_have_no_effect,
    pin_decode_is_last_prefill_row,
    pin_gqa_equals_repeated_mha,
    pin_global_equals_wide_window,
    pin_row_subset_matches,
    pin_worked_example,
    pin_rejects_indivisible_heads,
    pin_brute_force_prefill_history,
    pin_history_rows_of_full_prefill,
    pin_history_single_query_is_decode,
    pin_history_rejects_more_queries_than_keys,
    pin_brute_force_prefill_projected,
    pin_projection_rounds_like_torch,
    pin_projection_by_permutation,
    pin_projection_equal_columns_is_unbiased,
    pin_projection_last_column_is_clamped_bucket,
]


def failing_pins(orc):
    """Names of the pins the given oracle fails (any exception counts)."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:  # noqa: BLE001 - a crash of the oracle is a failure too
            failed.append(pin.__name__)
    return failed
