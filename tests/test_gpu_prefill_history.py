"""GPU parity of rba_prefill over a cached history (chunked prefill, several
new tokens of a decode step) against the CPU oracle on the same inputs.

Sequence b holds n_b keys in the pool, the keys of its L_b new tokens
included; the new tokens are its last L_b positions.  Cases span history
lengths on and off the 64-key tile, one new token (the decode case), a
sequence without history next to ones with it, windows shorter and longer
than the new chunk, the clamped-bucket region, page sizes 16/64/128, GQA 1..4,
head_dim 64 and the fp32 path.
"""
import zlib

import numpy as np
import pytest
import torch

import rba_inputs as ri
from gpu_helpers import (LSE_MAX_ABS, assert_parity, device, errors, gpu_decode, gpu_prefill,
                         oracle_prefill_history, sample_positions)
import relative_position_bias_paged_amd as rba

pytestmark = pytest.mark.gpu


def spec(hq, hkv, d, W, R, P, dtype=torch.bfloat16, **kw):
    return ri.LayerSpec(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, window=W, rel_extent=R,
                        page_size=P, dtype=dtype, **kw)


CASES = [
    # id, spec, key lens, new lens
    ("local-w512-hist", spec(4, 2, 128, 512, 512, 64), [700, 1300], [130, 300]),
    ("local-w100-p16", spec(4, 2, 128, 100, 100, 16), [300, 450], [77, 1]),
    ("local-w64-long-chunk", spec(8, 2, 128, 64, 128, 64), [900], [600]),
    ("global-r1024-gqa4", spec(8, 2, 128, 0, 1024, 64), [2100], [257]),
    ("global-r128-clamp", spec(8, 2, 128, 0, 128, 64), [517, 1100], [1, 64]),
    ("global-p128-mha", spec(2, 2, 128, 0, 200, 128), [1000], [999]),
    ("mixed-history", spec(4, 1, 128, 0, 300, 64), [333, 90, 1024], [333, 17, 64]),
    ("tile-aligned-history", spec(4, 2, 128, 256, 256, 64), [640, 512], [128, 64]),
    ("d64-local", spec(4, 2, 64, 192, 192, 64), [500, 129], [100, 129]),
    ("d64-global", spec(4, 1, 64, 0, 96, 16), [400], [33]),
]


@pytest.mark.parametrize("cid,sp,keys,new", CASES, ids=[c[0] for c in CASES])
def test_prefill_history_parity(cid, sp, keys, new):
    dev = device()
    case = ri.make_prefill_history(sp, keys, new, seed=zlib.crc32(cid.encode()) % 100000,
                                   device=dev)
    out, lse = gpu_prefill(case, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_prefill_history(case, want_lse=True)
    assert_parity(out, ref, sp.dtype, cid)
    assert np.max(np.abs(lse.cpu().double().numpy() - ref_lse)) <= LSE_MAX_ABS, cid


def test_prefill_history_fp32():
    dev = device()
    sp = spec(4, 2, 64, 64, 64, 16, dtype=torch.float32, bias_std=0.5)
    case = ri.make_prefill_history(sp, [256, 100], [40, 100], seed=31, device=dev)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    assert_parity(out, oracle_prefill_history(case), torch.float32, "fp32 history")


@pytest.mark.parametrize("W,R", [(512, 512), (0, 1024)])
def test_chunked_equals_whole_prefill(W, R):
    """The last chunk of a sequence, prefilled over the rest as history, gives
    the rows a prefill of the whole sequence gives (both on the GPU)."""
    dev = device()
    sp = spec(8, 2, 128, W, R, 64)
    lens, new = [1500, 777], [300, 129]
    whole = ri.make_prefill(sp, lens, seed=37, device=dev, num_pages=40)
    chunk = ri.HistoryCase(
        spec=sp, new_lens=new, key_lens=lens,
        q=torch.cat([whole.q[c - m:c] for c, m in zip(whole.cu_list()[1:], new)]),
        k_log=whole.k_log, v_log=whole.v_log,
        bias=torch.cat([whole.bias[c - m:c] for c, m in zip(whole.cu_list()[1:], new)]),
        cu_seqlens=torch.tensor(ri._cumsum(new), dtype=torch.int32, device=dev),
        seq_lens_dev=whole.seq_lens_dev, block_table=whole.block_table,
        k_pool=whole.k_pool, v_pool=whole.v_pool)
    o_whole = gpu_prefill(whole)
    o_chunk = gpu_prefill(chunk)
    torch.cuda.synchronize()
    sel = torch.cat([o_whole[c - m:c] for c, m in zip(whole.cu_list()[1:], new)])
    max_abs, _ = errors(o_chunk, sel.double().cpu().numpy())
    assert max_abs <= 2e-2
    assert_parity(o_chunk, oracle_prefill_history(chunk), torch.bfloat16, "chunk")


@pytest.mark.parametrize("W,R", [(512, 512), (0, 1024)])
def test_one_new_token_equals_decode(W, R):
    """One new token per sequence through rba_prefill equals rba_decode on the
    same cache (both on the GPU), and both match the oracle."""
    dev = device()
    sp = spec(8, 2, 128, W, R, 64)
    lens = [1, 63, 64, 65, 1000, 2049]
    case = ri.make_prefill_history(sp, lens, [1] * len(lens), seed=41, device=dev)
    o_pre = gpu_prefill(case)
    dcase = ri.DecodeCase(spec=sp, seq_lens=lens, q=case.q, bias=case.bias,
                          seq_lens_dev=case.seq_lens_dev, block_table=case.block_table,
                          k_pool=case.k_pool, v_pool=case.v_pool, seed=0, window_only=False,
                          _kv_first_page=[0] * len(lens))
    o_dec = gpu_decode(dcase)
    torch.cuda.synchronize()
    max_abs, _ = errors(o_pre, o_dec.double().cpu().numpy())
    assert max_abs <= 2e-2
    assert_parity(o_pre, oracle_prefill_history(case), torch.bfloat16, "one token")


def test_null_seq_lens_is_plain_prefill():
    """seq_lens NULL reads every sequence as holding exactly its new tokens:
    the result is bit-identical to passing seq_lens equal to the lengths."""
    dev = device()
    sp = spec(4, 2, 128, 0, 256, 64)
    case = ri.make_prefill(sp, [300, 65], seed=43, device=dev, num_pages=8)
    o1 = gpu_prefill(case)
    o2 = rba.prefill(case.q, case.cu_seqlens, case.max_seqlen, case.k_pool, case.v_pool,
                     case.block_table, None, case.bias, window=sp.window, sm_scale=sp.scale())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# History lengths whose remainders mod 32 put a 64-key tile's smallest
# distance exactly at R-1 for some query block (R = 128: 30; R = 98: 0;
# R = 100: 2), next to others.
LAST_BUCKET_HIST = [0, 2, 30, 31, 33, 62, 97]
LAST_BUCKET_NEW = [160, 97, 130, 64, 1, 200, 150]


@pytest.mark.parametrize("W,R,dtype", [(128, 128, torch.bfloat16), (98, 98, torch.bfloat16),
                                       (100, 100, torch.bfloat16), (64, 128, torch.bfloat16),
                                       (300, 128, torch.bfloat16), (0, 128, torch.bfloat16),
                                       (100, 100, torch.float32)])
def test_dominant_last_bucket(W, R, dtype):
    """Bucket R-1 set to 6 in every bias row, the rest N(0, 1): the keys at
    distance R-1 and beyond that the window shows carry most of the softmax
    weight, so a wrong value for that bucket, or a lost key at distance
    exactly R-1 (a window of R keys ends there), moves those rows far past
    the bar."""
    dev = device()
    sp = spec(4, 2, 128, W, R, 64, dtype=dtype)
    keys = [h + n for h, n in zip(LAST_BUCKET_HIST, LAST_BUCKET_NEW)]
    case = ri.make_prefill_history(sp, keys, LAST_BUCKET_NEW, seed=7 * R + W, device=dev)
    case.bias[..., R - 1] = 6.0
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    assert_parity(out, oracle_prefill_history(case), dtype, f"W={W} R={R}")


@pytest.mark.parametrize("W", [128, 100])
def test_narrow_window_ignores_buckets_it_cannot_reach(W):
    """A window of W <= R keys never reaches a distance above W-1: bias
    columns W.. set to NaN change nothing, bit for bit, against the same
    layer with only W columns (bucket W-1 large, so that its use counts)."""
    dev = device()
    sp = spec(4, 2, 128, W, W, 64)
    keys = [h + n for h, n in zip(LAST_BUCKET_HIST, LAST_BUCKET_NEW)]
    case = ri.make_prefill_history(sp, keys, LAST_BUCKET_NEW, seed=W, device=dev)
    case.bias[..., W - 1] = 6.0
    wide_bias = torch.full((*case.bias.shape[:2], 2 * W + 8), float("nan"), dtype=case.bias.dtype,
                           device=dev)
    wide_bias[..., :W] = case.bias
    o1 = gpu_prefill(case)
    o2 = rba.prefill(case.q, case.cu_seqlens, case.max_seqlen, case.k_pool, case.v_pool,
                     case.block_table, case.seq_lens_dev, wide_bias, window=W,
                     sm_scale=sp.scale())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert_parity(o1, oracle_prefill_history(case), torch.bfloat16, f"W={W}")


@pytest.mark.parametrize("name", ["chunked-local-4x512-ctx4096", "chunked-global-2x2048-ctx16384"])
def test_chunked_workload_sampled(name):
    """The chunked-prefill benchmark workloads at full size, checked on every
    head of at least 128 new tokens per sequence: the first and last new
    tokens, tile edges, window and clamp borders (on positions), and random
    ones."""
    dev = device()
    case = ri.build_workload(name, dev)["prefill"]
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    sp = case.spec
    g = torch.Generator().manual_seed(5)
    cu = case.cu_list()
    rows = []
    for b, (n, L) in enumerate(zip(case.key_lens, case.new_lens)):
        for t in sample_positions(L, 128, g, window=sp.window, rel_extent=sp.rel_extent,
                                  offset=n - L):
            rows += [(cu[b] + t, h) for h in range(sp.num_q_heads)]
    ref = oracle_prefill_history(case, rows=rows)
    tok = torch.tensor([r[0] for r in rows], device=dev)
    hd = torch.tensor([r[1] for r in rows], device=dev)
    assert_parity(out[tok, hd], ref, torch.bfloat16, name)
