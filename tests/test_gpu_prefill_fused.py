"""GPU parity of rba_prefill_fused, the prefill whose bias is formed in the
kernel from its projection, bias[t,h,d] = r[t,h,:] . W[:,d], against the CPU
oracle's projected prefill (the same definition in fp64, W in the pages'
[d_rel, R] layout; the kernel reads its transpose).

The kernel rounds the products it stages for band tiles to bf16, as the
bias tensors the streaming prefill reads are stored, so the bar is the bf16
one of the other prefill tests.  Cases span local and global layers, the
clamped-bucket region, windows shorter and longer than R, R = 1 and tiny R,
d_rel 16 and 32, GQA 1..8 (so 32..256 queries per head and work-group),
head_dim 64, page sizes 16..128, ragged and empty sequences, and prefill
over a cached history.  Windowed layers with an even GQA run 4-wave
work-groups (at head_dim 128 with the bias stage in the next K/V buffers),
odd ones 8-wave work-groups; both are covered.
"""
import zlib

import numpy as np
import pytest
import torch

import rba_inputs as ri
from gpu_helpers import (LSE_MAX_ABS, assert_parity, device, errors, gpu_prefill,
                         gpu_prefill_fused, oracle_prefill_projected, sample_positions)
import relative_position_bias_paged_amd as rba

pytestmark = pytest.mark.gpu


def spec(hq, hkv, d, W, R, P):
    return ri.LayerSpec(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, window=W, rel_extent=R,
                        page_size=P)


CASES = [
    # id, spec, key lens, new lens (None: no history), d_rel
    ("local-w512-r512", spec(4, 2, 128, 512, 512, 64), [700, 1300], None, 32),
    ("global-r1024-gqa4", spec(8, 2, 128, 0, 1024, 64), [2100], None, 32),
    ("global-r128-clamp-d16", spec(8, 2, 128, 0, 128, 64), [517, 1100], None, 16),
    ("window-below-extent-p16", spec(4, 2, 128, 100, 300, 16), [300, 450], None, 32),
    ("window-above-extent", spec(4, 1, 128, 300, 64, 64), [700], None, 16),
    ("mha-p128", spec(2, 2, 128, 0, 200, 128), [1000, 33], None, 32),
    ("gqa8", spec(8, 1, 128, 0, 256, 64), [333], None, 32),
    ("d64-local", spec(4, 2, 64, 192, 192, 64), [500, 129], None, 16),
    ("d64-global-d32", spec(4, 1, 64, 0, 96, 32), [400], None, 32),
    ("extent-one", spec(4, 2, 128, 0, 1, 64), [200], None, 16),
    ("extent-seven", spec(4, 2, 128, 0, 7, 64), [150], None, 32),
    ("ragged-empty", spec(4, 2, 128, 0, 64, 64), [0, 1, 65, 129], None, 32),
    ("history-local", spec(4, 2, 128, 512, 512, 64), [700, 1300], [130, 300], 32),
    ("history-global", spec(8, 2, 128, 0, 1024, 64), [2100], [257], 32),
    ("history-one-token", spec(4, 2, 128, 0, 300, 64), [1, 64, 65, 999], [1, 1, 1, 1], 16),
    ("local-mha-8-waves", spec(3, 3, 128, 256, 256, 64), [600, 257], None, 32),
    ("local-gqa3-8-waves-p16", spec(6, 2, 128, 300, 300, 16), [500], None, 16),
    ("local-gqa4-d64-history", spec(8, 2, 64, 128, 128, 64), [400, 700], [64, 333], 32),
    ("local-gqa2-p256-history", spec(4, 2, 128, 200, 256, 256), [900, 64], [450, 64], 16),
]


def _case(cid, sp, keys, new, d_rel, dev):
    return ri.make_projected(sp, keys, new, d_rel, seed=zlib.crc32(cid.encode()) % 100000,
                             device=dev)


@pytest.mark.parametrize("cid,sp,keys,new,d_rel", CASES, ids=[c[0] for c in CASES])
def test_prefill_fused_parity(cid, sp, keys, new, d_rel):
    dev = device()
    case = _case(cid, sp, keys, new, d_rel, dev)
    out, lse = gpu_prefill_fused(case, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_prefill_projected(case, want_lse=True)
    assert_parity(out, ref, torch.bfloat16, cid)
    g = lse.cpu().double().numpy()
    both_empty = np.isneginf(g) & np.isneginf(ref_lse)
    diff = np.zeros_like(g)
    np.subtract(g, ref_lse, out=diff, where=~both_empty)
    assert np.max(np.abs(diff), initial=0.0) <= LSE_MAX_ABS, cid


@pytest.mark.parametrize("W,R", [(0, 1024), (512, 512)])
def test_fused_matches_streamed_bias(W, R):
    """The fused kernel and the streaming one given the product rounded to bf16
    (formed here in fp32 from the same bf16 r and W) agree closely: both add
    the same bf16 bias, up to a rare product whose fp32 sums round apart."""
    dev = device()
    sp = spec(8, 2, 128, W, R, 64)
    case = ri.make_projected(sp, [1500, 777], None, 32, seed=61, device=dev)
    h = case.hist
    bias = torch.matmul(case.rel_r.float(), case.w_rel.float()).to(torch.bfloat16)
    streamed = ri.PrefillCase(spec=sp, seq_lens=h.new_lens, q=h.q, k_log=h.k_log, v_log=h.v_log,
                              bias=bias, cu_seqlens=h.cu_seqlens, seq_lens_dev=h.seq_lens_dev,
                              block_table=h.block_table, k_pool=h.k_pool, v_pool=h.v_pool)
    o_fused = gpu_prefill_fused(case)
    o_stream = gpu_prefill(streamed)
    torch.cuda.synchronize()
    max_abs, mean_rel = errors(o_fused, o_stream.double().cpu().numpy())
    assert max_abs <= 1e-2 and mean_rel <= 2e-3, (max_abs, mean_rel)


def test_fused_null_seq_lens_is_plain_prefill():
    """seq_lens NULL reads every sequence as holding exactly its new tokens:
    bit-identical to passing seq_lens equal to the lengths."""
    dev = device()
    case = ri.make_projected(spec(4, 2, 128, 256, 256, 64), [300, 65], None, 32, seed=67,
                             device=dev)
    o1 = gpu_prefill_fused(case)
    o2 = gpu_prefill_fused(case, seq_lens=None)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("name", ["fused-local-prefill-4x4096-drel32",
                                  "fused-global-prefill-2x16384-drel32"])
def test_fused_workload_sampled(name):
    """The fused benchmark workloads at full size, in the launch the bench
    times, checked on every head of at least 128 tokens per sequence: its
    first and last tokens, tile, window and clamp borders, and random ones."""
    dev = device()
    case = ri.build_workload(name, dev)["prefill"]
    out = gpu_prefill_fused(case)
    torch.cuda.synchronize()
    h = case.hist
    sp = h.spec
    g = torch.Generator().manual_seed(11)
    cu = h.cu_list()
    rows = []
    for b, L in enumerate(h.new_lens):
        for t in sample_positions(L, 128, g, window=sp.window, rel_extent=sp.rel_extent):
            rows += [(cu[b] + t, hh) for hh in range(sp.num_q_heads)]
    ref = oracle_prefill_projected(case, rows=rows)
    tok = torch.tensor([r[0] for r in rows], device=dev)
    hd = torch.tensor([r[1] for r in rows], device=dev)
    assert_parity(out[tok, hd], ref, torch.bfloat16, name)


def test_fused_rejects_fp32_pools():
    dev = device()
    sp = ri.LayerSpec(num_q_heads=4, num_kv_heads=2, head_dim=64, window=0, rel_extent=32,
                      page_size=16, dtype=torch.float32)
    case = ri.make_projected(sp, [40], None, 16, seed=3, device=dev)
    with pytest.raises(rba.RbaError):
        gpu_prefill_fused(case)
