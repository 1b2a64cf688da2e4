"""Window-only local pools: each sequence owns a ring of
rba_window_ring_pages(window, page_size, max_new) pages, and its positional
block table maps page j to ring[j % ring_pages].  Keys older than the window
are overwritten as the sequence grows; no output depends on them (nor on
the ring slots no query of a call sees, whatever they hold): prefill never
loads them, decode loads the pages that hold them and masks them out.

Checked on the GPU against the oracle on the full logical keys: a local
layer prefilled chunk by chunk (append, then prefill over the history) into
a ring of O(window + chunk) pages, and decode steps (append one token, then
decode) at long contexts held in a ring of O(window) pages.
"""
import pytest
import torch

import oracle
import rba_inputs as ri
from gpu_helpers import assert_parity, device
import relative_position_bias_paged_amd as rba

pytestmark = pytest.mark.gpu


def _rings(B, ring, dev, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(B * ring, generator=g).to(torch.int32)
    return perm.view(B, ring).to(dev)


@pytest.mark.parametrize("chunk", [200, 64, 1])
def test_chunked_local_prefill_through_a_ring(chunk):
    dev = device()
    W, R, P, Hq, Hkv, D = 256, 256, 64, 8, 2, 128
    sp = ri.LayerSpec(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, window=W, rel_extent=R,
                      page_size=P)
    lens = [700, 413] if chunk > 1 else [300, 129]
    whole = ri.make_prefill(sp, lens, seed=81 + chunk, device="cpu")
    B = len(lens)
    ring = rba.window_ring_pages(W, P, chunk)
    assert ring == -(-(W + chunk - 1) // P) + 1
    rings = _rings(B, ring, dev, seed=chunk)
    max_pages = -(-max(lens) // P)
    table = rba.ring_block_table(rings, max_pages)
    k_pool = torch.full((B * ring, Hkv, P, D), float("nan"), dtype=sp.dtype, device=dev)
    v_pool = torch.full_like(k_pool, float("nan"))
    cu = whole.cu_list()
    out = torch.empty_like(whole.q, device=dev)
    done = [0] * B
    while any(d < n for d, n in zip(done, lens)):
        new = [min(chunk, n - d) for d, n in zip(done, lens)]
        after = [d + m for d, m in zip(done, new)]
        rows = torch.tensor([cu[b] + done[b] + i for b in range(B) for i in range(new[b])])
        seq_lens = torch.tensor(after, dtype=torch.int32, device=dev)
        cu_new = torch.tensor(ri._cumsum(new), dtype=torch.int32, device=dev)
        rba.kv_append(whole.k_log[rows].to(dev), whole.v_log[rows].to(dev), cu_new,
                      k_pool, v_pool, table, seq_lens)
        o = rba.prefill(whole.q[rows].to(dev), cu_new, max(new), k_pool, v_pool, table,
                        seq_lens, whole.bias[rows].to(dev), window=W, sm_scale=sp.scale())
        out[rows.to(dev)] = o
        done = after
    torch.cuda.synchronize()
    ref = oracle.prefill(whole.q, whole.k_log, whole.v_log, whole.bias, cu, window=W,
                         rel_extent=R, sm_scale=sp.scale())
    assert_parity(out, ref, torch.bfloat16, f"ring chunk {chunk}")


def test_decode_steps_through_a_ring():
    dev = device()
    W, R, P, Hq, Hkv, D = 512, 512, 64, 8, 2, 128
    scale = D ** -0.5
    lens0 = [5000, 20000, 777, 512]
    steps = 3
    B = len(lens0)
    ring = rba.window_ring_pages(W, P, 1)
    rings = _rings(B, ring, dev, seed=5)
    table = rba.ring_block_table(rings, -(-(max(lens0) + steps) // P))
    k_pool = torch.full((B * ring, Hkv, P, D), float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full_like(k_pool, float("nan"))
    g = torch.Generator(device="cpu").manual_seed(7)
    # logical keys of every position (the oracle reads them all; the kernels
    # only the last W, which are the ones appended into the ring)
    k_log = [torch.randn((n + steps, Hkv, D), generator=g).to(torch.bfloat16) for n in lens0]
    v_log = [torch.randn((n + steps, Hkv, D), generator=g).to(torch.bfloat16) for n in lens0]
    # fill the window before the first step: positions n-W+1 .. n-1
    first = [min(W - 1, n - 1) for n in lens0]
    rows_k = torch.cat([k_log[b][lens0[b] - 1 - first[b]:lens0[b] - 1] for b in range(B)])
    rows_v = torch.cat([v_log[b][lens0[b] - 1 - first[b]:lens0[b] - 1] for b in range(B)])
    rba.kv_append(rows_k.to(dev), rows_v.to(dev),
                  torch.tensor(ri._cumsum(first), dtype=torch.int32, device=dev), k_pool, v_pool,
                  table, torch.tensor([n - 1 for n in lens0], dtype=torch.int32, device=dev))
    for s in range(steps):
        n_now = [n + s for n in lens0]
        q = torch.randn((B, Hq, D), generator=g).to(torch.bfloat16)
        bias = torch.randn((B, Hq, R), generator=g).to(torch.bfloat16)
        seq_lens = torch.tensor(n_now, dtype=torch.int32, device=dev)
        newk = torch.stack([k_log[b][n_now[b] - 1] for b in range(B)])
        newv = torch.stack([v_log[b][n_now[b] - 1] for b in range(B)])
        rba.kv_append(newk.to(dev), newv.to(dev), torch.arange(B + 1, dtype=torch.int32, device=dev),
                      k_pool, v_pool, table, seq_lens)
        out = rba.decode(q.to(dev), k_pool, v_pool, table, seq_lens, max(n_now), bias.to(dev),
                         window=W, sm_scale=scale)
        torch.cuda.synchronize()
        ref = oracle.decode(q, torch.cat([k_log[b][:n_now[b]] for b in range(B)]),
                            torch.cat([v_log[b][:n_now[b]] for b in range(B)]), bias,
                            ri._cumsum(n_now), window=W, rel_extent=R, sm_scale=scale)
        assert_parity(out, ref, torch.bfloat16, f"ring decode step {s}")
    # the pool is O(window): ring pages per sequence, whatever the length
    assert k_pool.shape[0] == B * ring


@pytest.mark.parametrize("P", [16, 64])
@pytest.mark.parametrize("new", [1, 4])
def test_prefill_new_tokens_through_a_window_only_ring(P, new):
    """Prefill of a few new tokens over a ring that holds only the keys the
    call's queries can see (the rest of the ring is NaN, as after a fresh
    allocation).  Window starts fall off the 64-key tile.  The result matches
    the oracle on the full logical keys and is bit-identical to the same call
    on a twin ring whose unwritten slots hold zeros."""
    dev = device()
    W, R, Hq, Hkv, D = 512, 512, 8, 2, 128
    sp = ri.LayerSpec(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, window=W, rel_extent=R,
                      page_size=P)
    lens = [5000, 777, 1300, 515]
    B = len(lens)
    case = ri.make_prefill_history(sp, lens, [new] * B, seed=90 + P + new, device="cpu")
    ring = rba.window_ring_pages(W, P, new)
    rings = _rings(B, ring, dev, seed=P * 10 + new)
    table = rba.ring_block_table(rings, -(-max(lens) // P))
    k_pool = torch.full((B * ring, Hkv, P, D), float("nan"), dtype=sp.dtype, device=dev)
    v_pool = torch.full_like(k_pool, float("nan"))
    # the keys the call's queries see: positions n - new - W + 1 .. n - 1
    cu_kv = case.cu_kv_list()
    lo = [max(0, n - new - W + 1) for n in lens]
    rows = torch.cat([torch.arange(cu_kv[b] + lo[b], cu_kv[b + 1]) for b in range(B)])
    assert any((n - new - W + 1) % 64 for n in lens)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    rba.kv_append(case.k_log[rows].to(dev), case.v_log[rows].to(dev),
                  torch.tensor(ri._cumsum([n - l for n, l in zip(lens, lo)]), dtype=torch.int32,
                               device=dev),
                  k_pool, v_pool, table, seq_lens)
    assert torch.isnan(k_pool).any()
    q, bias = case.q.to(dev), case.bias.to(dev)
    cu_q = torch.tensor(case.cu_list(), dtype=torch.int32, device=dev)
    o_nan = rba.prefill(q, cu_q, new, k_pool, v_pool, table, seq_lens, bias, window=W,
                        sm_scale=sp.scale())
    o_zero = rba.prefill(q, cu_q, new, torch.nan_to_num(k_pool, nan=0.0),
                         torch.nan_to_num(v_pool, nan=0.0), table, seq_lens, bias, window=W,
                         sm_scale=sp.scale())
    torch.cuda.synchronize()
    ref = oracle.prefill_history(case.q, case.k_log, case.v_log, case.bias, case.cu_list(),
                                 cu_kv, window=W, rel_extent=R, sm_scale=sp.scale())
    assert_parity(o_nan, ref, torch.bfloat16, f"ring prefill P={P} new={new}")
    assert torch.equal(o_nan.view(torch.int16), o_zero.view(torch.int16))


@pytest.mark.parametrize("P", [16, 64])
def test_prefill_last_token_on_a_window_only_decode_pool(P):
    """One new token through rba_prefill on a window-only pool (every table
    entry before the window's first page points at one NaN page) equals
    rba_decode on the same pool, and both match the oracle."""
    dev = device()
    sp = ri.LayerSpec(num_q_heads=8, num_kv_heads=2, head_dim=128, window=300, rel_extent=300,
                      page_size=P)
    lens = [5000, 777, 301, 64, 1]
    case = ri.make_decode(sp, lens, seed=40 + P, device=dev, window_only=True)
    assert torch.isnan(case.k_pool[0]).all()
    cu = torch.arange(len(lens) + 1, dtype=torch.int32, device=dev)
    o_pre = rba.prefill(case.q, cu, 1, case.k_pool, case.v_pool, case.block_table,
                        case.seq_lens_dev, case.bias, window=sp.window, sm_scale=sp.scale())
    o_dec = rba.decode(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens_dev,
                       case.max_seq_len, case.bias, window=sp.window, sm_scale=sp.scale())
    torch.cuda.synchronize()
    ks, vs = zip(*(case.logical_kv(b) for b in range(len(lens))))
    ref = oracle.decode(case.q, torch.cat(ks), torch.cat(vs), case.bias, ri._cumsum(lens),
                        window=sp.window, rel_extent=sp.rel_extent, sm_scale=sp.scale())
    assert_parity(o_pre, ref, torch.bfloat16, f"prefill on window pool P={P}")
    assert_parity(o_dec, ref, torch.bfloat16, f"decode on window pool P={P}")
