"""GPU tests of prefill calls captured in a HIP graph.

A chunked-prefill step is captured once: append the chunk's K/V to the pages,
then attend its queries over the whole cache. The bias is streamed, or formed
in the kernel from its projection. The step is replayed for three chunks,
with each chunk's inputs and the new key counts copied into the graph's
buffers between replays. Every replay equals the same calls run eagerly, bit
for bit, and meets the oracle. The calls allocate nothing and read no device
data on the host, so the grid of each launch is fixed by host scalars
(max_seqlen) and the key counts are read on the device.
"""
import pytest
import torch

import oracle
import rba_inputs as ri
import relative_position_bias_paged_amd as rba
from gpu_helpers import assert_parity, device, random_pools

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["streamed-bias", "formed-bias"])
@pytest.mark.parametrize("W,R", [(0, 1024), (256, 256)])
def test_graph_captured_chunked_prefill(W, R, fused):
    dev = device()
    dtype, Hq, Hkv, D, P, L, d_rel = torch.bfloat16, 8, 2, 128, 64, 64, 32
    scale = D ** -0.5
    lens0 = [100, 300]
    steps, B = 3, len(lens0)
    cap = [n + steps * L for n in lens0]
    k_pool, v_pool, table = random_pools(dev, dtype, Hkv, D, P, cap, seed=91)
    tab, kc, vc = table.cpu(), k_pool.cpu(), v_pool.cpu()
    k_log = [[kc[int(tab[b, s // P]), :, s % P, :] for s in range(n)] for b, n in enumerate(lens0)]
    v_log = [[vc[int(tab[b, s // P]), :, s % P, :] for s in range(n)] for b, n in enumerate(lens0)]
    gen = torch.Generator(device="cpu").manual_seed(93)
    w_rel = torch.randn((d_rel, R), generator=gen).to(dtype)
    w_rel_t = w_rel.t().contiguous().to(dev)
    step_in = []
    for s in range(steps):
        step_in.append(dict(
            q=torch.randn((B * L, Hq, D), generator=gen).to(dtype),
            bias=(torch.randn((B * L, Hq, d_rel), generator=gen) if fused
                  else torch.randn((B * L, Hq, R), generator=gen)).to(dtype),
            k=torch.randn((B * L, Hkv, D), generator=gen).to(dtype),
            v=torch.randn((B * L, Hkv, D), generator=gen).to(dtype),
            lens=torch.tensor([n + (s + 1) * L for n in lens0], dtype=torch.int32)))
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device=dev)

    def buffers():
        return {name: torch.empty(t.shape, dtype=t.dtype, device=dev)
                for name, t in step_in[0].items()} | {
                    "out": torch.empty((B * L, Hq, D), dtype=dtype, device=dev)}

    def step(buf, kp, vp):
        rba.kv_append(buf["k"], buf["v"], cu, kp, vp, table, buf["lens"])
        if fused:
            rba.prefill_fused(buf["q"], cu, L, kp, vp, table, buf["lens"], buf["bias"], w_rel_t,
                              window=W, sm_scale=scale, out=buf["out"])
        else:
            rba.prefill(buf["q"], cu, L, kp, vp, table, buf["lens"], buf["bias"], window=W,
                        sm_scale=scale, out=buf["out"])

    # run the kernels once outside the capture (on copies of the pools)
    warm = buffers()
    for name, t in step_in[0].items():
        warm[name].copy_(t)
    step(warm, k_pool.clone(), v_pool.clone())
    torch.cuda.synchronize()
    gb = buffers()
    for name, t in step_in[0].items():
        gb[name].copy_(t)
    k_eager, v_eager = k_pool.clone(), v_pool.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb, k_pool, v_pool)
    eb = buffers()
    for s in range(steps):
        for name, t in step_in[s].items():
            gb[name].copy_(t)
            eb[name].copy_(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(eb, k_eager, v_eager)
        torch.cuda.synchronize()
        assert torch.equal(gb["out"].view(torch.int16), eb["out"].view(torch.int16)), s
        for b in range(B):
            k_log[b] += list(step_in[s]["k"][b * L:(b + 1) * L])
            v_log[b] += list(step_in[s]["v"][b * L:(b + 1) * L])
        lens_now = [n + (s + 1) * L for n in lens0]
        k_all = torch.cat([torch.stack(k_log[b]) for b in range(B)])
        v_all = torch.cat([torch.stack(v_log[b]) for b in range(B)])
        if fused:
            ref = oracle.prefill_projected(step_in[s]["q"], k_all, v_all, step_in[s]["bias"], w_rel,
                                           [0, L, 2 * L], ri._cumsum(lens_now), window=W,
                                           sm_scale=scale)
        else:
            ref = oracle.prefill_history(step_in[s]["q"], k_all, v_all, step_in[s]["bias"],
                                         [0, L, 2 * L], ri._cumsum(lens_now), window=W,
                                         rel_extent=R, sm_scale=scale)
        assert_parity(gb["out"], ref, torch.bfloat16, f"graph chunk {s}")
    assert torch.equal(k_pool.view(torch.int16), k_eager.view(torch.int16))
    assert torch.equal(v_pool.view(torch.int16), v_eager.view(torch.int16))
