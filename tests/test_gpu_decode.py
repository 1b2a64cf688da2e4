"""GPU parity of rba_decode (split-K partials + LSE merge) against the oracle.

Context lengths straddle page boundaries (63, 64, 65, 127, 128, 129), start
at one key, and include an empty sequence; local layers use window-only
pools whose earlier table entries all point at one NaN page; partition
counts 1, 2, 16 and automatic must agree.
"""
import numpy as np
import pytest
import torch

import rba_inputs as ri
import relative_position_bias_paged_amd as rba
from gpu_helpers import (LSE_MAX_ABS, assert_parity, device, errors, gpu_decode,
                         gpu_prefill, oracle_decode)

pytestmark = pytest.mark.gpu


def spec(hq, hkv, d, W, R, P, dtype=torch.bfloat16):
    return ri.LayerSpec(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, window=W, rel_extent=R,
                        page_size=P, dtype=dtype)


EDGE_LENS = [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 1000, 2049]

CASES = [
    # id, spec, lens, window-only pool
    ("global-gqa4", spec(32, 8, 128, 0, 1024, 64), EDGE_LENS, False),
    ("global-r64-clamp", spec(8, 2, 128, 0, 64, 64), EDGE_LENS, False),
    ("local-w512-windowpool", spec(32, 16, 128, 512, 512, 64), EDGE_LENS + [5000], True),
    ("local-w100-p16", spec(8, 4, 128, 100, 100, 16), EDGE_LENS, True),
    ("gqa8-headgroups", spec(16, 2, 128, 0, 300, 32), [5, 700, 64], False),
    ("gqa3-mha1", spec(3, 1, 128, 0, 50, 64), [90, 1, 300], False),
    ("mha", spec(4, 4, 128, 33, 40, 128), [1, 500, 129], False),
    ("d64", spec(8, 2, 64, 0, 128, 64), [100, 1, 777], False),
    ("r1", spec(4, 2, 128, 0, 1, 64), [300, 65], False),
    ("p256", spec(4, 1, 128, 0, 512, 256), [1000, 255, 257], False),
]


@pytest.mark.parametrize("splits", [1, 2, 16, 0])
@pytest.mark.parametrize("cid,sp,lens,wonly", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(cid, sp, lens, wonly, splits):
    dev = device()
    case = ri.make_decode(sp, lens, seed=len(cid) * 31 + splits, device=dev, window_only=wonly)
    out, lse = gpu_decode(case, num_splits=splits, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(case, want_lse=True)
    assert_parity(out, ref, sp.dtype, f"{cid} splits={splits}")
    assert np.max(np.abs(lse.cpu().double().numpy() - ref_lse)) <= LSE_MAX_ABS


def test_decode_fp32():
    dev = device()
    sp = spec(4, 2, 64, 0, 64, 16, dtype=torch.float32)
    case = ri.make_decode(sp, [1, 17, 300], seed=3, device=dev)
    out = gpu_decode(case)
    assert_parity(out, oracle_decode(case), torch.float32, "decode fp32")
    sp = spec(4, 1, 128, 40, 40, 32, dtype=torch.float32)
    case = ri.make_decode(sp, [100, 7], seed=4, device=dev, window_only=True)
    out = gpu_decode(case, num_splits=8)
    assert_parity(out, oracle_decode(case), torch.float32, "decode fp32 window")


def test_empty_sequence_gives_zero_row():
    dev = device()
    sp = spec(8, 2, 128, 0, 64, 64)
    case = ri.make_decode(sp, [10, 200], seed=9, device=dev)
    lens = torch.tensor([10, 0], dtype=torch.int32, device=dev)
    case0 = ri.DecodeCase(**{**case.__dict__, "seq_lens_dev": lens})
    for splits in (1, 4):
        out, lse = gpu_decode(case0, num_splits=splits, want_lse=True, max_seq_len=200)
        torch.cuda.synchronize()
        assert torch.all(out[1] == 0)
        assert torch.all(torch.isneginf(lse[1]))
        ref = oracle_decode(case, seqs=[0])
        assert_parity(out[:1], ref, torch.bfloat16, "row 0")


def test_workspace_contents_are_ignored():
    """Ragged lengths under 16 partitions: most sequences fill only some of
    them, and one is empty.  Partitions that hold no key write nothing, and
    the merge must not read their slots, so a workspace filled with NaN
    (0xFF bytes) beforehand must not change the result."""
    dev = device()
    sp = spec(32, 8, 128, 0, 1024, 64)
    lens = [9000, 1, 64, 65, 3000, 4097, 130, 2049, 17, 8191]
    case = ri.make_decode(sp, lens, seed=33, device=dev)
    empty = 4
    lens_dev = case.seq_lens_dev.clone()
    lens_dev[empty] = 0
    case0 = ri.DecodeCase(**{**case.__dict__, "seq_lens_dev": lens_dev})
    need = rba.decode_workspace_size(case.q, case.k_pool, case.v_pool, case.block_table,
                                     lens_dev, case.max_seq_len, case.bias, window=0,
                                     sm_scale=sp.scale(), num_splits=16)
    for fill in (0xFF, 0x00):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=dev)
        lse = torch.empty(case.q.shape[:2], dtype=torch.float32, device=dev)
        out = rba.decode(case.q, case.k_pool, case.v_pool, case.block_table, lens_dev,
                         case.max_seq_len, case.bias, window=0, sm_scale=sp.scale(),
                         num_splits=16, workspace=ws, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))
        keep = [b for b in range(len(lens)) if b != empty]
        ref, ref_lse = oracle_decode(case0, seqs=keep, want_lse=True)
        assert_parity(out[keep], ref, sp.dtype, f"ragged, workspace filled with {fill:#x}")
        assert np.max(np.abs(lse[keep].cpu().double().numpy() - ref_lse)) <= LSE_MAX_ABS


def test_long_partitions_plan():
    """Two partitions of 313 pages: the largest-first plan groups partition
    sizes into 256 classes by a shift, and a short sequence's partitions sit
    in other classes than the long one's."""
    dev = device()
    sp = spec(8, 2, 128, 0, 1024, 64)
    case = ri.make_decode(sp, [40000, 300, 20001], seed=41, device=dev)
    out, lse = gpu_decode(case, num_splits=2, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(case, want_lse=True)
    assert_parity(out, ref, sp.dtype, "two long partitions")
    assert np.max(np.abs(lse.cpu().double().numpy() - ref_lse)) <= LSE_MAX_ABS


def test_split_counts_agree():
    dev = device()
    sp = spec(32, 8, 128, 0, 1024, 64)
    case = ri.make_decode(sp, [9000, 4097, 64], seed=21, device=dev)
    outs = [gpu_decode(case, num_splits=s) for s in (1, 3, 16, 64)]
    for o in outs[1:]:
        max_abs, _ = errors(o, outs[0].double().cpu().numpy())
        assert max_abs <= 2e-2


def test_decode_page_table_bit_exact():
    """Two different placements of the same logical keys: identical output bits."""
    dev = device()
    sp = spec(16, 4, 128, 0, 256, 64)
    lens = [700, 64, 1300]
    a = ri.make_decode(sp, lens, seed=8, device=dev, shuffle=False)
    b = ri.make_decode(sp, lens, seed=8, device=dev, shuffle=True)
    assert not torch.equal(a.block_table, b.block_table)
    for splits in (1, 4):
        oa = gpu_decode(a, num_splits=splits)
        ob = gpu_decode(b, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_decode_is_last_prefill_row():
    """Decode at n keys equals the prefill output of position n-1 (same keys,
    same bias row), within the bf16 bar."""
    dev = device()
    sp = spec(8, 2, 128, 0, 128, 64)
    pre = ri.make_prefill(sp, [333, 64], seed=31, device=dev, num_pages=8)
    p_out = gpu_prefill(pre)
    last = torch.tensor([332, 333 + 63], device=dev)
    q = pre.q.index_select(0, last).contiguous()
    bias = pre.bias.index_select(0, last).contiguous()
    d_out = __import__("relative_position_bias_paged_amd").decode(
        q, pre.k_pool, pre.v_pool, pre.block_table, pre.seq_lens_dev, 333, bias,
        window=0, sm_scale=sp.scale(), num_splits=2)
    max_abs, _ = errors(d_out, p_out.index_select(0, last).double().cpu().numpy())
    assert max_abs <= 2e-2


@pytest.mark.parametrize("W,R", [(0, 1024), (300, 300)])
def test_decode_gqa_equals_repeated_mha(W, R):
    """GQA (4 query heads per KV head) against MHA over a pool whose K/V
    heads are repeated per query head: the same rows within the bf16 bar,
    and both meet the oracle."""
    dev = device()
    sp = spec(16, 4, 128, W, R, 64)
    case = ri.make_decode(sp, [1, 64, 65, 1000, 5000], seed=95, device=dev)
    G = sp.num_q_heads // sp.num_kv_heads
    k_mha = case.k_pool.repeat_interleave(G, dim=1).contiguous()
    v_mha = case.v_pool.repeat_interleave(G, dim=1).contiguous()
    o_gqa = gpu_decode(case)
    o_mha = gpu_decode(case, k_pool=k_mha, v_pool=v_mha)
    torch.cuda.synchronize()
    max_abs, mean_rel = errors(o_mha, o_gqa.double().cpu().numpy())
    assert max_abs <= 2e-2 and mean_rel <= 5e-3
    assert_parity(o_mha, oracle_decode(case), sp.dtype, "MHA twin")


def test_decode_global_equals_window_wider_than_sequence():
    """A global layer and a windowed layer whose window exceeds every
    context see the same keys: equal within the bf16 bar."""
    dev = device()
    lens = [1, 129, 3000, 7000]
    glob = ri.make_decode(spec(8, 2, 128, 0, 512, 64), lens, seed=97, device=dev)
    wide = ri.DecodeCase(**{**glob.__dict__, "spec": spec(8, 2, 128, 8192, 512, 64)})
    o_g = gpu_decode(glob)
    o_w = gpu_decode(wide)
    torch.cuda.synchronize()
    max_abs, mean_rel = errors(o_w, o_g.double().cpu().numpy())
    assert max_abs <= 2e-2 and mean_rel <= 5e-3
    assert_parity(o_w, oracle_decode(glob), torch.bfloat16, "wide window")


def test_nan_pages_outside_window_cannot_leak():
    """The window-only pool's page 0 is NaN and every pre-window table entry
    points at it; zeroing it must not change a single output bit."""
    dev = device()
    sp = spec(8, 4, 128, 128, 128, 64)
    case = ri.make_decode(sp, [1000, 129, 3000], seed=41, device=dev, window_only=True)
    assert torch.isnan(case.k_pool[0]).all()
    k0 = case.k_pool.clone()
    v0 = case.v_pool.clone()
    k0[0] = 0
    v0[0] = 0
    for splits in (1, 2):
        o1 = gpu_decode(case, num_splits=splits)
        o2 = gpu_decode(case, num_splits=splits, k_pool=k0, v_pool=v0)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("name", ["mixed-decode-256", "long-decode-32x131072"])
def test_full_size_workload_sampled(name):
    """The full-size decode workloads in the benchmark's launch configuration,
    checked against the oracle on sampled sequences (all heads)."""
    dev = device()
    w = ri.WORKLOADS[name]
    cases = ri.build_workload(name, dev)
    splits = w.get("num_splits", 0)
    g = torch.Generator().manual_seed(5)
    for key, case in cases.items():
        out = gpu_decode(case, num_splits=splits)
        torch.cuda.synchronize()
        B = len(case.seq_lens)
        seqs = sorted(set([0, B - 1] + torch.randint(0, B, (4,), generator=g).tolist()))
        ref = oracle_decode(case, seqs=seqs)
        sel = out.index_select(0, torch.tensor(seqs, device=dev))
        assert_parity(sel, ref, torch.bfloat16, f"{name}/{key}")
        del out
    del cases
    torch.cuda.empty_cache()
