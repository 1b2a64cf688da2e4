"""GPU parity of rba_prefill against the CPU oracle (same seeded inputs).

Sizes span several 128-query and 64-key tiles with ragged tails, windows and
bias extents that are not tile multiples, page sizes below, at and above the
64-key tile, the clamped-bucket region of global layers, GQA 1..4, and the
degenerate cases (one-token sequences, an empty sequence, rel_extent 1,
window 1).
"""
import math
import zlib

import numpy as np
import pytest
import torch

import rba_inputs as ri
from gpu_helpers import (LSE_MAX_ABS, assert_parity, device, errors, gpu_prefill,
                         oracle_prefill, oracle_prefill_history, sample_positions)

pytestmark = pytest.mark.gpu


def spec(hq, hkv, d, W, R, P, dtype=torch.bfloat16, **kw):
    return ri.LayerSpec(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, window=W, rel_extent=R,
                        page_size=P, dtype=dtype, **kw)


CASES = [
    # id, spec, lens, pool pages (None = exact)
    ("local-w100-r100-p64", spec(8, 4, 128, 100, 100, 64), [1, 130, 700], None),
    ("local-w256-p16", spec(4, 2, 128, 256, 256, 16), [300, 1000], 200),
    ("local-w512-gqa2", spec(4, 2, 128, 512, 512, 64), [1500, 640], 64),
    ("global-r128-clamp", spec(8, 2, 128, 0, 128, 64), [517, 1100], 40),
    ("global-r1024-gqa4", spec(8, 2, 128, 0, 1024, 64), [2100], 40),
    ("global-p128", spec(4, 1, 128, 0, 200, 128), [77, 900], 12),
    ("global-p256-r64", spec(4, 4, 128, 0, 64, 256), [1024, 3], 8),
    ("global-p32-mha", spec(2, 2, 128, 0, 256, 32), [333], 20),
    ("d64-local", spec(4, 2, 64, 192, 192, 64), [400, 129], 16),
    ("d64-global", spec(4, 1, 64, 0, 96, 16), [260], 20),
    ("r1-degenerate", spec(4, 2, 128, 0, 1, 64), [200], 4),
    ("r-odd-clamp", spec(4, 2, 128, 0, 37, 64), [300], 5),
    ("window1", spec(4, 2, 128, 1, 8, 64), [150], 3),
    ("empty-and-single", spec(4, 2, 128, 0, 64, 64), [0, 1, 65, 0, 2], 8),
    # head groupings of the work-group: 4 and 8 query heads per KV head share
    # one work-group (32 queries per head), 3 query heads share none
    ("local-gqa4", spec(16, 4, 128, 512, 512, 64), [700, 129], None),
    ("global-gqa8", spec(16, 2, 128, 0, 1024, 64), [1300], None),
    ("local-gqa3", spec(6, 2, 128, 300, 300, 64), [500], None),
    ("global-gqa3", spec(6, 2, 128, 0, 256, 64), [400], None),
    # sequence ends just below, at and just above the 64-key tile and the
    # query tile of either layer kind
    ("tile-edges-local", spec(4, 2, 128, 512, 512, 64), [63, 64, 65, 127, 128, 129], None),
    ("tile-edges-global", spec(8, 2, 128, 0, 1024, 64), [63, 64, 65, 127, 128, 129], None),
    # windows wider and narrower than the bias extent
    ("local-w300-r64", spec(4, 2, 128, 300, 64, 64), [700], None),
    ("local-w64-r512", spec(4, 2, 128, 64, 512, 64), [400], None),
]


@pytest.mark.parametrize("cid,sp,lens,pages", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity(cid, sp, lens, pages):
    dev = device()
    case = ri.make_prefill(sp, lens, seed=zlib.crc32(cid.encode()) % 100000, device=dev, num_pages=pages)
    out, lse = gpu_prefill(case, want_lse=True)
    torch.cuda.synchronize()
    if case.total_tokens == 0:
        return
    ref, ref_lse = oracle_prefill(case, want_lse=True)
    assert_parity(out, ref, sp.dtype, cid)
    g_lse = lse.cpu().double().numpy()
    assert np.max(np.abs(g_lse - ref_lse)) <= LSE_MAX_ABS, cid


def test_prefill_fp32_tiny_workload():
    """The tiny fp32 local layer: 256 tokens, 4/2 heads, head_dim 64, window 64."""
    dev = device()
    case = ri.build_workload("tiny-local-prefill-fp32", dev)["prefill"]
    out, lse = gpu_prefill(case, want_lse=True)
    ref, ref_lse = oracle_prefill(case, want_lse=True)
    assert_parity(out, ref, torch.float32, "tiny fp32")
    assert np.max(np.abs(lse.cpu().double().numpy() - ref_lse)) <= 1e-5


@pytest.mark.parametrize("W", [0, 50])
def test_prefill_fp32_ragged(W):
    dev = device()
    sp = spec(4, 2, 128, W, 40, 16, dtype=torch.float32)
    case = ri.make_prefill(sp, [70, 1, 33], seed=77, device=dev, num_pages=12)
    out = gpu_prefill(case)
    assert_parity(out, oracle_prefill(case), torch.float32, f"fp32 W={W}")


def test_page_table_bit_exact():
    """Identity and shuffled page tables over the same logical K/V give the
    bitwise-identical output: the arithmetic depends only on key positions."""
    dev = device()
    sp = spec(8, 2, 128, 0, 256, 64)
    lens = [700, 300]
    a = ri.make_prefill(sp, lens, seed=5, device=dev, num_pages=20, shuffle=False)
    b = ri.make_prefill(sp, lens, seed=5, device=dev, num_pages=20, shuffle=True)
    assert not torch.equal(a.block_table, b.block_table)
    assert torch.equal(a.q, b.q) and torch.equal(a.bias, b.bias)
    oa = gpu_prefill(a)
    ob = gpu_prefill(b)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_masked_positions_cannot_leak():
    """NaN in every pool slot no key reaches, and in bias buckets no row uses,
    leaves the output bit-identical (masks select, never multiply)."""
    dev = device()
    sp = spec(4, 2, 128, 96, 96, 64)
    case = ri.make_prefill(sp, [150, 77], seed=11, device=dev, num_pages=10)
    # the generator already NaN-fills unowned pages and tail slots; build a
    # twin whose unreachable slots hold zeros instead
    k0 = torch.nan_to_num(case.k_pool, nan=0.0)
    v0 = torch.nan_to_num(case.v_pool, nan=0.0)
    assert torch.isnan(case.k_pool).any()
    o_nan = gpu_prefill(case)
    o_zero = gpu_prefill(case, k_pool=k0, v_pool=v0)
    # bias buckets a row never reads: d > t (none for W = R here except the
    # first rows), set them to NaN
    bias2 = case.bias.clone()
    for tok, t in ((0, 0), (1, 1), (150, 0), (151, 1)):
        bias2[tok, :, t + 1:] = float("nan")
    case2 = ri.PrefillCase(**{**case.__dict__, "bias": bias2})
    o_bias = gpu_prefill(case2)
    torch.cuda.synchronize()
    assert torch.equal(o_nan.view(torch.int16), o_zero.view(torch.int16))
    assert torch.equal(o_nan.view(torch.int16), o_bias.view(torch.int16))


@pytest.mark.parametrize("W,R", [(0, 256), (200, 200)])
def test_gqa_equals_repeated_mha(W, R):
    """GQA with 4 query heads per KV head against MHA over a pool whose K/V
    heads are repeated per query head (h -> h // G).  On a global layer every
    head grouping visits the key tiles in the same order with the same score
    path per tile, so the rows are bit-identical.  A windowed layer's tile
    order rotates with the work-group's query range, which the grouping
    changes, so there the two meet within the bf16 bar.  Both meet the
    oracle."""
    dev = device()
    sp = spec(8, 2, 128, W, R, 64)
    case = ri.make_prefill(sp, [300, 777], seed=91, device=dev, num_pages=24)
    G = sp.num_q_heads // sp.num_kv_heads
    k_mha = case.k_pool.repeat_interleave(G, dim=1).contiguous()
    v_mha = case.v_pool.repeat_interleave(G, dim=1).contiguous()
    o_gqa = gpu_prefill(case)
    o_mha = gpu_prefill(case, k_pool=k_mha, v_pool=v_mha)
    torch.cuda.synchronize()
    if W <= 0:
        assert torch.equal(o_gqa.view(torch.int16), o_mha.view(torch.int16))
    else:
        max_abs, mean_rel = errors(o_mha, o_gqa.double().cpu().numpy())
        assert max_abs <= 2e-2 and mean_rel <= 5e-3
    assert_parity(o_mha, oracle_prefill(case), sp.dtype, "MHA twin")


# Global layers: lengths and extents give each work-group shape a different
# count of leading clamp-only tiles (odd and even), page sizes below, at and
# above the 64-key tile, head_dim 64 and 128, GQA 2..8, and a cached history.
CLAMP_ONLY_CASES = [
    ("r64-p64", spec(8, 2, 128, 0, 64, 64), [1000, 65, 700, 129], None),
    ("r100-p16", spec(8, 2, 128, 0, 100, 16), [513, 300, 64], None),
    ("d64-r32-p32", spec(4, 1, 64, 0, 32, 32), [900, 257], None),
    ("gqa8-r128-p128", spec(16, 2, 128, 0, 128, 128), [2000], None),
    ("history-r64", spec(8, 2, 128, 0, 64, 64), [1500, 700], [333, 64]),
]


@pytest.mark.parametrize("cid,sp,lens,new", CLAMP_ONLY_CASES, ids=[c[0] for c in CLAMP_ONLY_CASES])
def test_clamp_only_tiles_bit_exact_across_groupings(cid, sp, lens, new):
    """On a global layer the leading tiles that are clamp-only for the whole
    work-group run in a phase of their own, whose length depends on the
    work-group's first query and so on the head grouping; the tiles after it
    run the general step.  GQA against MHA over a repeated pool moves tiles
    between the two, and the rows stay bit-identical (each wave's arithmetic
    is the same in both); both meet the oracle."""
    dev = device()
    seed = zlib.crc32(cid.encode()) % 100000
    if new is None:
        case = ri.make_prefill(sp, lens, seed=seed, device=dev,
                               num_pages=sum(-(-n // sp.page_size) for n in lens) + 3)
    else:
        case = ri.make_prefill_history(sp, lens, new, seed=seed, device=dev)
    G = sp.num_q_heads // sp.num_kv_heads
    k_mha = case.k_pool.repeat_interleave(G, dim=1).contiguous()
    v_mha = case.v_pool.repeat_interleave(G, dim=1).contiguous()
    o_gqa = gpu_prefill(case)
    o_mha = gpu_prefill(case, k_pool=k_mha, v_pool=v_mha)
    torch.cuda.synchronize()
    assert torch.equal(o_gqa.view(torch.int16), o_mha.view(torch.int16))
    ref = oracle_prefill(case) if new is None else oracle_prefill_history(case)
    assert_parity(o_gqa, ref, sp.dtype, cid)


SHORT_LAST_CASES = [
    # id, spec, key lens, new lens (None: no history).  The batch's last
    # sequence is shorter than one work-group's queries, so whole waves of its
    # work-group lie past it while their band still reaches its bias tiles.
    ("global-mha", spec(8, 8, 128, 0, 64, 64), [900, 70], None),
    ("global-mha-history", spec(8, 8, 128, 0, 64, 64), [900, 400], [300, 40]),
    ("global-gqa2", spec(8, 4, 128, 0, 128, 64), [600, 33], None),
    ("local-gqa2", spec(8, 4, 128, 256, 256, 64), [700, 20], None),
    ("global-d64-p32", spec(4, 4, 64, 0, 96, 32), [500, 50], None),
]


@pytest.mark.parametrize("cid,sp,lens,new", SHORT_LAST_CASES, ids=[c[0] for c in SHORT_LAST_CASES])
def test_short_last_sequence(cid, sp, lens, new):
    """Waves wholly past the batch's last sequence: their query rows are not
    stored, and their bias stage reads nothing (such rows sit past the
    resource's record count).  The host model of the stage addressing checks
    that no read leaves the tensor; here the outputs meet the oracle."""
    dev = device()
    seed = zlib.crc32(cid.encode()) % 100000
    if new is None:
        case = ri.make_prefill(sp, lens, seed=seed, device=dev)
    else:
        case = ri.make_prefill_history(sp, lens, new, seed=seed, device=dev)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    ref = oracle_prefill(case) if new is None else oracle_prefill_history(case)
    assert_parity(out, ref, sp.dtype, cid)


@pytest.mark.parametrize("R", [64, 1024])
def test_global_equals_window_wider_than_sequence(R):
    """A global layer and a windowed layer whose window exceeds every
    sequence see the same keys: equal within the bf16 bar (the two run
    different work-group shapes), and both meet the oracle."""
    dev = device()
    lens = [1000, 65, 700]
    glob = ri.make_prefill(spec(8, 2, 128, 0, R, 64), lens, seed=93, device=dev)
    wide = ri.PrefillCase(**{**glob.__dict__, "spec": spec(8, 2, 128, 4096, R, 64)})
    o_g = gpu_prefill(glob)
    o_w = gpu_prefill(wide)
    torch.cuda.synchronize()
    max_abs, mean_rel = errors(o_w, o_g.double().cpu().numpy())
    assert max_abs <= 2e-2 and mean_rel <= 5e-3
    ref = oracle_prefill(glob)
    assert_parity(o_g, ref, torch.bfloat16, "global")
    assert_parity(o_w, ref, torch.bfloat16, "wide window")


def test_window_one_returns_value_exactly():
    """window 1: each query sees only itself, so out[t,h] = v[t, h // G] bitwise."""
    dev = device()
    sp = spec(8, 2, 128, 1, 16, 64)
    case = ri.make_prefill(sp, [200, 3], seed=13, device=dev, num_pages=6)
    out = gpu_prefill(case)
    ref = case.v_log.repeat_interleave(4, dim=1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_row_constant_bias_shift():
    """Adding a constant to a whole bias row leaves the output unchanged.

    The bias is drawn on a 1/16 grid in [-2, 2] and shifted by integers in
    [-4, 4], so both the original and the shifted rows are exact in bf16 and
    the two problems have the same exact answer."""
    dev = device()
    sp = spec(4, 2, 128, 0, 128, 64)
    case = ri.make_prefill(sp, [300], seed=17, device=dev, num_pages=5)
    grid = (case.bias.float() * 16).round().clamp(-32, 32) / 16
    case1 = ri.PrefillCase(**{**case.__dict__, "bias": grid.to(torch.bfloat16)})
    c = torch.randint(-4, 5, (300, 4, 1), device=dev).float()
    shifted = (grid + c).to(torch.bfloat16)
    assert torch.equal(shifted.float(), grid + c)
    case2 = ri.PrefillCase(**{**case.__dict__, "bias": shifted})
    o1 = gpu_prefill(case1)
    o2 = gpu_prefill(case2)
    assert_parity(o1, oracle_prefill(case1), torch.bfloat16, "grid bias")
    assert_parity(o2, oracle_prefill(case2), torch.bfloat16, "shifted")
    max_abs, _ = errors(o1, o2.double().cpu().numpy())
    assert max_abs <= 2e-2


def test_zero_bias_is_plain_attention():
    """Zero bias: the kernel reproduces plain causal attention (torch SDPA in fp32)."""
    dev = device()
    sp = spec(4, 2, 128, 0, 64, 64)
    case = ri.make_prefill(sp, [257], seed=19, device=dev, num_pages=5)
    case.bias.zero_()
    out = gpu_prefill(case)
    q = case.q.float().permute(1, 0, 2).contiguous()
    k = case.k_log.float().repeat_interleave(2, 1).permute(1, 0, 2).contiguous()
    v = case.v_log.float().repeat_interleave(2, 1).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.cpu(), k.cpu(), v.cpu(), is_causal=True, scale=1 / math.sqrt(128))
    assert_parity(out, ref.permute(1, 0, 2).double().numpy(), torch.bfloat16, "zero bias")


@pytest.mark.parametrize("W,R,lens", [(96, 128, [300, 70]), (0, 64, [333])])
def test_zero_keys_bias_only_softmax(W, R, lens):
    """All keys zero: every score is its bias alone, so each output row is the
    softmax of the row's visible bias buckets applied to V, computed here
    directly in float64 (no oracle)."""
    dev = device()
    sp = spec(4, 2, 128, W, R, 64)
    case = ri.make_prefill(sp, lens, seed=23, device=dev, num_pages=None)
    out = gpu_prefill(case, k_pool=torch.zeros_like(case.k_pool))
    torch.cuda.synchronize()
    bias = case.bias.double().cpu()
    v = case.v_log.double().cpu().repeat_interleave(2, dim=1)      # [T, Hq, D]
    ref = torch.empty_like(v)
    cu = case.cu_list()
    for b, L in enumerate(case.seq_lens):
        t = torch.arange(L).view(L, 1)
        s_ = torch.arange(L).view(1, L)
        d = t - s_
        vis = (d >= 0) & ((d < W) if W > 0 else torch.ones_like(d, dtype=torch.bool))
        bucket = d.clamp(0, R - 1)
        rows = bias[cu[b]:cu[b] + L]                                # [L, Hq, R]
        logits = torch.gather(rows, 2, bucket.view(L, 1, L).expand(L, 4, L))
        logits = logits.masked_fill(~vis.view(L, 1, L), float("-inf"))
        p = torch.softmax(logits, dim=2)
        ref[cu[b]:cu[b] + L] = torch.einsum("ths,shd->thd", p, v[cu[b]:cu[b] + L])
    assert_parity(out, ref.numpy(), torch.bfloat16, f"zero keys W={W} R={R}")


@pytest.mark.parametrize("name", ["local-prefill-4x4096", "global-prefill-2x16384"])
def test_full_size_workload_sampled(name):
    """The full-size prefill workloads, in the launch configuration the
    benchmark times, checked on sampled rows: every head of at least 128
    tokens per sequence -- its first and last tokens, the 32/64-query and
    64-key tile edges, the window edge and the clamp border t - s = R - 1,
    and random positions."""
    dev = device()
    case = ri.build_workload(name, dev)["prefill"]
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    sp = case.spec
    g = torch.Generator().manual_seed(3)
    cu = case.cu_list()
    rows = []
    for b, L in enumerate(case.seq_lens):
        for t in sample_positions(L, 128, g, window=sp.window, rel_extent=sp.rel_extent):
            rows += [(cu[b] + t, h) for h in range(sp.num_q_heads)]
    assert len(rows) >= 128 * sp.num_q_heads * len(case.seq_lens)
    ref = oracle_prefill(case, rows=rows)
    tok = torch.tensor([r[0] for r in rows], device=dev)
    hd = torch.tensor([r[1] for r in rows], device=dev)
    sel = out[tok, hd]
    assert_parity(sel, ref, torch.bfloat16, name)


def _perturbed_pool(case, positions, seed):
    """Copies of the case's K and V pools in which the keys at the given
    logical positions (per sequence) hold other finite values: large ones
    (|x| up to ~40) of either sign, so a leak would show."""
    g = torch.Generator().manual_seed(seed)
    k_pool, v_pool = case.k_pool.clone(), case.v_pool.clone()
    table = case.block_table.cpu()
    P = case.spec.page_size
    for b, pos in enumerate(positions):
        for s in pos:
            page, slot = int(table[b, s // P]), s % P
            shape = k_pool[page, :, slot, :].shape
            k_pool[page, :, slot, :] = (torch.randn(shape, generator=g) * 13).to(k_pool.dtype).to(k_pool.device)
            v_pool[page, :, slot, :] = (torch.randn(shape, generator=g) * 13).to(v_pool.dtype).to(v_pool.device)
    return k_pool, v_pool


@pytest.mark.parametrize("W,R", [(100, 100), (0, 256)])
def test_masked_keys_inside_visible_tiles_have_no_effect(W, R):
    """Finite changes to keys a row cannot see, inside tiles it partly sees,
    leave that row bit-identical: future keys (after a cut position t0
    that is not on a tile edge) for rows up to t0, and keys before a row's
    window for rows whose window starts after them."""
    dev = device()
    sp = spec(8, 2, 128, W, R, 64)
    lens = [700, 450]
    case = ri.make_prefill(sp, lens, seed=29, device=dev, num_pages=20)
    base = gpu_prefill(case)
    cu = case.cu_list()
    # future keys: positions after t0 in each sequence
    t0 = [333, 161]
    kf, vf = _perturbed_pool(case, [range(t + 1, n) for t, n in zip(t0, lens)], seed=1)
    o_future = gpu_prefill(case, k_pool=kf, v_pool=vf)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        a = base[cu[b]:cu[b] + t0[b] + 1].view(torch.int16)
        c = o_future[cu[b]:cu[b] + t0[b] + 1].view(torch.int16)
        assert torch.equal(a, c), f"future keys changed rows of sequence {b}"
        # rows after t0 see the changed keys, so they must differ somewhere
        assert not torch.equal(base[cu[b] + t0[b] + 1:cu[b + 1]], o_future[cu[b] + t0[b] + 1:cu[b + 1]])
    if W > 0:
        # keys before the window of rows t >= t1
        t1 = [450, 321]
        ko, vo = _perturbed_pool(case, [range(0, t - W + 1) for t in t1], seed=2)
        o_old = gpu_prefill(case, k_pool=ko, v_pool=vo)
        torch.cuda.synchronize()
        for b in range(len(lens)):
            a = base[cu[b] + t1[b]:cu[b + 1]].view(torch.int16)
            c = o_old[cu[b] + t1[b]:cu[b + 1]].view(torch.int16)
            assert torch.equal(a, c), f"keys before the window changed rows of sequence {b}"
