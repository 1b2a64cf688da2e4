"""GPU tests of rba_kv_append and of a decode step captured in a HIP graph.

The append must write exactly the new tokens' rows at their page-table
positions (checked bit for bit against a scatter written here with torch
indexing), leave rows with an out-of-range position or page id unwritten,
and feed a following decode that matches the oracle.  A captured append +
decode step is replayed several times, with new inputs copied into its
buffers between replays, and every replay is compared bit for bit with the
same step run eagerly and with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import rba_inputs as ri
from gpu_helpers import assert_parity, device, gpu_decode, random_pools
import relative_position_bias_paged_amd as rba

pytestmark = pytest.mark.gpu


def _reference_append(k_pool, v_pool, table, k_new, v_new, lens_before, new):
    """The same writes with plain torch indexing, one row at a time."""
    P = k_pool.shape[2]
    rk, rv = k_pool.clone(), v_pool.clone()
    tab = table.cpu()
    tok = 0
    for b, (n0, m) in enumerate(zip(lens_before, new)):
        for i in range(m):
            pos = n0 + i
            page = int(tab[b, pos // P])
            if 0 <= page < k_pool.shape[0]:
                rk[page, :, pos % P, :] = k_new[tok]
                rv[page, :, pos % P, :] = v_new[tok]
            tok += 1
    return rk, rv


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("dtype,D,P", [(torch.bfloat16, 128, 16), (torch.bfloat16, 64, 64),
                                       (torch.float32, 64, 32), (torch.float32, 128, 128)])
@pytest.mark.parametrize("Hkv", [4, 3, 1])     # odd counts leave a head group half full
def test_append_writes_exactly_the_new_rows(dtype, D, P, Hkv):
    dev = device()
    before = [0, 17, 64, 100, 31, 5]
    new = [5, 0, 1, 70, 33, 2]
    after = [a + b for a, b in zip(before, new)]
    k_pool, v_pool, table = random_pools(dev, dtype, Hkv, D, P, after, seed=int(D + P))
    g = torch.Generator(device="cpu").manual_seed(7)
    k_new = torch.randn((sum(new), Hkv, D), generator=g).to(dtype).to(dev)
    v_new = torch.randn((sum(new), Hkv, D), generator=g).to(dtype).to(dev)
    cu = torch.tensor(ri._cumsum(new), dtype=torch.int32, device=dev)
    lens = torch.tensor(after, dtype=torch.int32, device=dev)
    rk, rv = _reference_append(k_pool, v_pool, table, k_new, v_new, before, new)
    rba.kv_append(k_new, v_new, cu, k_pool, v_pool, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(_bits(k_pool), _bits(rk))
    assert torch.equal(_bits(v_pool), _bits(rv))


def test_append_skips_rows_outside_the_table_or_pool():
    dev = device()
    dtype, Hkv, D, P = torch.bfloat16, 2, 128, 16
    before, new = [10, 20, 0], [4, 3, 2]
    after = [a + b for a, b in zip(before, new)]
    k_pool, v_pool, table = random_pools(dev, dtype, Hkv, D, P, after, seed=3)
    # sequence 1: its page for the new rows is outside the pool
    table[1, 20 // P] = k_pool.shape[0] + 5
    g = torch.Generator(device="cpu").manual_seed(9)
    k_new = torch.randn((sum(new), Hkv, D), generator=g).to(dtype).to(dev)
    v_new = torch.randn((sum(new), Hkv, D), generator=g).to(dtype).to(dev)
    cu = torch.tensor(ri._cumsum(new), dtype=torch.int32, device=dev)
    # sequence 2: seq_lens so large that its positions fall past the table
    lens = torch.tensor([after[0], after[1], table.shape[1] * P + 10], dtype=torch.int32,
                        device=dev)
    rk, rv = _reference_append(k_pool, v_pool, table, k_new, v_new,
                               [before[0], before[1], 10 ** 6], [new[0], new[1], 0])
    rba.kv_append(k_new, v_new, cu, k_pool, v_pool, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(_bits(k_pool), _bits(rk))
    assert torch.equal(_bits(v_pool), _bits(rv))


@pytest.mark.parametrize("W,R", [(512, 512), (0, 1024)])
def test_append_then_decode_matches_oracle(W, R):
    """Decode after appending each sequence's last token (its pool slot
    poisoned first) matches the oracle on the logical keys."""
    dev = device()
    sp = ri.LayerSpec(num_q_heads=8, num_kv_heads=2, head_dim=128, window=W, rel_extent=R,
                      page_size=64)
    lens = [1, 64, 65, 300, 1500]
    case = ri.make_decode(sp, lens, seed=51, device=dev)
    P = sp.page_size
    ks, vs = [], []
    tab = case.block_table.cpu()
    for b, n in enumerate(lens):
        k, v = case.logical_kv(b)
        ks.append(k[n - 1])
        vs.append(v[n - 1])
        page = int(tab[b, (n - 1) // P])
        case.k_pool[page, :, (n - 1) % P, :] = float("nan")
        case.v_pool[page, :, (n - 1) % P, :] = float("nan")
    k_new = torch.stack(ks).to(dev)
    v_new = torch.stack(vs).to(dev)
    cu = torch.arange(len(lens) + 1, dtype=torch.int32, device=dev)
    rba.kv_append(k_new, v_new, cu, case.k_pool, case.v_pool, case.block_table, case.seq_lens_dev)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    k_all = torch.cat([case.logical_kv(b)[0] for b in range(len(lens))])
    v_all = torch.cat([case.logical_kv(b)[1] for b in range(len(lens))])
    ref = oracle.decode(case.q, k_all, v_all, case.bias, ri._cumsum(lens), window=W,
                        rel_extent=R, sm_scale=sp.scale())
    assert_parity(out, ref, torch.bfloat16, f"append+decode W={W}")


@pytest.mark.parametrize("W,R", [(96, 256), (0, 256)])
def test_graph_captured_decode_step(W, R):
    """Append + decode captured once in a HIP graph and replayed for three
    steps (new token inputs and seq_lens copied into the graph's buffers
    between replays): every replay equals the eager step bit for bit and
    matches the oracle."""
    dev = device()
    dtype, Hq, Hkv, D, P = torch.bfloat16, 8, 2, 128, 64
    scale = D ** -0.5
    lens0 = [100, 233, 64, 511]
    steps = 3
    B = len(lens0)
    cap = [n + steps for n in lens0]
    max_len = max(cap)
    k_pool, v_pool, table = random_pools(dev, dtype, Hkv, D, P, cap, seed=61)
    # logical keys: the initial ones are whatever the pool holds at 0 .. n0-1
    tab, kc, vc = table.cpu(), k_pool.cpu(), v_pool.cpu()
    k_log = [[kc[int(tab[b, s // P]), :, s % P, :] for s in range(n)] for b, n in enumerate(lens0)]
    v_log = [[vc[int(tab[b, s // P]), :, s % P, :] for s in range(n)] for b, n in enumerate(lens0)]
    gen = torch.Generator(device="cpu").manual_seed(71)
    step_in = []
    for s in range(steps):
        step_in.append(dict(
            q=torch.randn((B, Hq, D), generator=gen).to(dtype),
            bias=torch.randn((B, Hq, R), generator=gen).to(dtype),
            k=torch.randn((B, Hkv, D), generator=gen).to(dtype),
            v=torch.randn((B, Hkv, D), generator=gen).to(dtype),
            lens=torch.tensor([n + s + 1 for n in lens0], dtype=torch.int32)))

    def buffers():
        return dict(q=torch.empty((B, Hq, D), dtype=dtype, device=dev),
                    bias=torch.empty((B, Hq, R), dtype=dtype, device=dev),
                    k=torch.empty((B, Hkv, D), dtype=dtype, device=dev),
                    v=torch.empty((B, Hkv, D), dtype=dtype, device=dev),
                    lens=torch.empty((B,), dtype=torch.int32, device=dev),
                    out=torch.empty((B, Hq, D), dtype=dtype, device=dev))

    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    gb = buffers()
    gb["lens"].copy_(step_in[0]["lens"])
    gb["q"].copy_(step_in[0]["q"])
    gb["bias"].copy_(step_in[0]["bias"])
    need = rba.decode_workspace_size(gb["q"], k_pool, v_pool, table, gb["lens"], max_len, gb["bias"],
                                     window=W, sm_scale=scale)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    k_eager, v_eager = k_pool.clone(), v_pool.clone()

    def step(buf, kp, vp):
        rba.kv_append(buf["k"], buf["v"], cu, kp, vp, table, buf["lens"])
        rba.decode(buf["q"], kp, vp, table, buf["lens"], max_len, buf["bias"], window=W,
                   sm_scale=scale, workspace=ws, out=buf["out"])

    # run the kernels once outside the capture (on copies of the pools)
    warm = buffers()
    for name in ("q", "bias", "k", "v", "lens"):
        warm[name].copy_(step_in[0][name])
    step(warm, k_pool.clone(), v_pool.clone())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb, k_pool, v_pool)
    eb = buffers()
    for s in range(steps):
        for name in ("q", "bias", "k", "v", "lens"):
            gb[name].copy_(step_in[s][name])
            eb[name].copy_(step_in[s][name])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(eb, k_eager, v_eager)
        torch.cuda.synchronize()
        assert torch.equal(gb["out"].view(torch.int16), eb["out"].view(torch.int16)), s
        for b in range(B):
            k_log[b].append(step_in[s]["k"][b])
            v_log[b].append(step_in[s]["v"][b])
        lens_now = [n + s + 1 for n in lens0]
        k_all = torch.cat([torch.stack(k_log[b]) for b in range(B)])
        v_all = torch.cat([torch.stack(v_log[b]) for b in range(B)])
        ref = oracle.decode(step_in[s]["q"], k_all, v_all, step_in[s]["bias"],
                            ri._cumsum(lens_now), window=W, rel_extent=R, sm_scale=scale)
        assert_parity(gb["out"], ref, torch.bfloat16, f"graph step {s}")
    assert torch.equal(k_pool.view(torch.int16), k_eager.view(torch.int16))


def test_graph_captured_mtp_verify_step():
    """Multi-token verification step (append the 4 drafted tokens' K/V, then
    rba_decode_multi over the whole cache) captured once in a HIP graph and
    replayed for three steps with new inputs copied into its buffers: every
    replay equals the eager step bit for bit and matches the oracle's
    prefill over the history."""
    dev = device()
    dtype, Hq, Hkv, D, P, R, W, L = torch.bfloat16, 8, 2, 128, 64, 256, 0, 4
    scale = D ** -0.5
    lens0 = [100, 1900, 64, 511]
    steps = 3
    B = len(lens0)
    cap = [n + L * steps for n in lens0]
    max_len = max(cap)
    k_pool, v_pool, table = random_pools(dev, dtype, Hkv, D, P, cap, seed=81)
    tab, kc, vc = table.cpu(), k_pool.cpu(), v_pool.cpu()
    k_log = [[kc[int(tab[b, s // P]), :, s % P, :] for s in range(n)] for b, n in enumerate(lens0)]
    v_log = [[vc[int(tab[b, s // P]), :, s % P, :] for s in range(n)] for b, n in enumerate(lens0)]
    gen = torch.Generator(device="cpu").manual_seed(83)
    step_in = []
    for s in range(steps):
        step_in.append(dict(
            q=torch.randn((B * L, Hq, D), generator=gen).to(dtype),
            bias=torch.randn((B * L, Hq, R), generator=gen).to(dtype),
            k=torch.randn((B * L, Hkv, D), generator=gen).to(dtype),
            v=torch.randn((B * L, Hkv, D), generator=gen).to(dtype),
            lens=torch.tensor([n + L * (s + 1) for n in lens0], dtype=torch.int32)))

    def buffers():
        return dict(q=torch.empty((B * L, Hq, D), dtype=dtype, device=dev),
                    bias=torch.empty((B * L, Hq, R), dtype=dtype, device=dev),
                    k=torch.empty((B * L, Hkv, D), dtype=dtype, device=dev),
                    v=torch.empty((B * L, Hkv, D), dtype=dtype, device=dev),
                    lens=torch.empty((B,), dtype=torch.int32, device=dev),
                    out=torch.empty((B * L, Hq, D), dtype=dtype, device=dev))

    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device=dev)
    gb = buffers()
    for name in ("q", "bias", "lens"):
        gb[name].copy_(step_in[0][name])
    need = rba.decode_multi_workspace_size(gb["q"], L, k_pool, v_pool, table, gb["lens"], max_len,
                                           gb["bias"], window=W, sm_scale=scale, num_splits=4)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    k_eager, v_eager = k_pool.clone(), v_pool.clone()

    def step(buf, kp, vp):
        rba.kv_append(buf["k"], buf["v"], cu, kp, vp, table, buf["lens"])
        rba.decode_multi(buf["q"], L, kp, vp, table, buf["lens"], max_len, buf["bias"], window=W,
                         sm_scale=scale, num_splits=4, workspace=ws, out=buf["out"])

    warm = buffers()
    for name in ("q", "bias", "k", "v", "lens"):
        warm[name].copy_(step_in[0][name])
    step(warm, k_pool.clone(), v_pool.clone())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb, k_pool, v_pool)
    eb = buffers()
    for s in range(steps):
        for name in ("q", "bias", "k", "v", "lens"):
            gb[name].copy_(step_in[s][name])
            eb[name].copy_(step_in[s][name])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(eb, k_eager, v_eager)
        torch.cuda.synchronize()
        assert torch.equal(gb["out"].view(torch.int16), eb["out"].view(torch.int16)), s
        for b in range(B):
            for i in range(L):
                k_log[b].append(step_in[s]["k"][b * L + i])
                v_log[b].append(step_in[s]["v"][b * L + i])
        lens_now = [n + L * (s + 1) for n in lens0]
        k_all = torch.cat([torch.stack(k_log[b]) for b in range(B)])
        v_all = torch.cat([torch.stack(v_log[b]) for b in range(B)])
        ref = oracle.prefill_history(step_in[s]["q"], k_all, v_all, step_in[s]["bias"],
                                     list(range(0, B * L + 1, L)), ri._cumsum(lens_now), window=W,
                                     rel_extent=R, sm_scale=scale)
        assert_parity(gb["out"], ref, torch.bfloat16, f"graph mtp step {s}")
    assert torch.equal(k_pool.view(torch.int16), k_eager.view(torch.int16))
