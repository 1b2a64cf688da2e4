"""Window-only local pools: each sequence owns a ring of
rba_window_ring_pages(window, page_size, max_new) pages, and its positional
block table maps page j to ring[j % ring_pages].  Keys older than the window
are overwritten as the sequence grows; the kernels never read them.

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
