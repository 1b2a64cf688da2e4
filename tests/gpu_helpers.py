"""Shared pieces of the GPU tests: running the HIP path, running the oracle
on the same seeded inputs, and the parity bar.

Tolerances (on the final output, against the fp64 oracle, unrounded):
  bf16: max |gpu - ref| <= 2e-2 and sum|gpu - ref| / sum|ref| <= 5e-3
  fp32: max |gpu - ref| <= 1e-5
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import rba_inputs as ri
import relative_position_bias_paged_amd as rba

BF16_MAX_ABS = 2e-2
BF16_MEAN_REL = 5e-3
F32_MAX_ABS = 1e-5
LSE_MAX_ABS = 2e-2


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def errors(gpu: torch.Tensor, ref: np.ndarray):
    g = gpu.detach().float().cpu().double().numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    diff = np.abs(g - ref)
    return float(diff.max(initial=0.0)), float(diff.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_parity(gpu: torch.Tensor, ref: np.ndarray, dtype, what=""):
    max_abs, mean_rel = errors(gpu, ref)
    if dtype == torch.float32:
        assert max_abs <= F32_MAX_ABS, f"{what}: max|d| {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max|d| {max_abs:.3e} > {BF16_MAX_ABS}"
        assert mean_rel <= BF16_MEAN_REL, f"{what}: mean rel {mean_rel:.3e} > {BF16_MEAN_REL}"
    return max_abs, mean_rel


def gpu_prefill(case: ri.PrefillCase, want_lse=False, block_table=None, k_pool=None, v_pool=None):
    sp = case.spec
    lse = None
    if want_lse:
        lse = torch.empty((case.total_tokens, sp.num_q_heads), dtype=torch.float32,
                          device=case.q.device)
    out = rba.prefill(case.q, case.cu_seqlens, case.max_seqlen,
                      case.k_pool if k_pool is None else k_pool,
                      case.v_pool if v_pool is None else v_pool,
                      case.block_table if block_table is None else block_table,
                      case.seq_lens_dev, case.bias, window=sp.window, sm_scale=sp.scale(),
                      lse=lse)
    return (out, lse) if want_lse else out


def oracle_prefill(case: ri.PrefillCase, rows=None, want_lse=False):
    sp = case.spec
    return oracle.prefill(case.q, case.k_log, case.v_log, case.bias, case.cu_list(),
                          window=sp.window, rel_extent=sp.rel_extent, sm_scale=sp.scale(),
                          rows=rows, want_lse=want_lse)


def oracle_prefill_history(case: ri.HistoryCase, rows=None, want_lse=False):
    sp = case.spec
    return oracle.prefill_history(case.q, case.k_log, case.v_log, case.bias, case.cu_list(),
                                  case.cu_kv_list(), window=sp.window, rel_extent=sp.rel_extent,
                                  sm_scale=sp.scale(), rows=rows, want_lse=want_lse)


def gpu_prefill_fused(case: ri.ProjectedCase, want_lse=False, seq_lens="case"):
    h = case.hist
    sp = h.spec
    lse = None
    if want_lse:
        lse = torch.empty((h.total_tokens, sp.num_q_heads), dtype=torch.float32,
                          device=h.q.device)
    out = rba.prefill_fused(h.q, h.cu_seqlens, h.max_seqlen, h.k_pool, h.v_pool, h.block_table,
                            h.seq_lens_dev if seq_lens == "case" else seq_lens, case.rel_r,
                            case.w_rel_t, window=sp.window, sm_scale=sp.scale(), lse=lse)
    return (out, lse) if want_lse else out


def oracle_prefill_projected(case: ri.ProjectedCase, rows=None, want_lse=False):
    h = case.hist
    sp = h.spec
    return oracle.prefill_projected(h.q, h.k_log, h.v_log, case.rel_r, case.w_rel, h.cu_list(),
                                    h.cu_kv_list(), window=sp.window, sm_scale=sp.scale(),
                                    rows=rows, want_lse=want_lse)


def gpu_decode(case: ri.DecodeCase, num_splits=0, want_lse=False, block_table=None,
               k_pool=None, v_pool=None, max_seq_len=None):
    sp = case.spec
    lse = None
    if want_lse:
        lse = torch.empty(case.q.shape[:2], dtype=torch.float32, device=case.q.device)
    out = rba.decode(case.q, case.k_pool if k_pool is None else k_pool,
                     case.v_pool if v_pool is None else v_pool,
                     case.block_table if block_table is None else block_table,
                     case.seq_lens_dev, case.max_seq_len if max_seq_len is None else max_seq_len,
                     case.bias, window=sp.window, sm_scale=sp.scale(), num_splits=num_splits,
                     lse=lse)
    return (out, lse) if want_lse else out


def oracle_decode(case: ri.DecodeCase, seqs=None, heads=None, want_lse=False):
    """Oracle rows for the given sequences (all by default) and heads.

    Returns an array [len(seqs), len(heads), D] (and lse [len(seqs), len(heads)]).
    """
    sp = case.spec
    B = len(case.seq_lens)
    seqs = list(range(B)) if seqs is None else list(seqs)
    heads = list(range(sp.num_q_heads)) if heads is None else list(heads)
    ks, vs, cu = [], [], [0]
    for b in seqs:
        k, v = case.logical_kv(b)
        ks.append(k)
        vs.append(v)
        cu.append(cu[-1] + case.seq_lens[b])
    k = torch.cat(ks, 0)
    v = torch.cat(vs, 0)
    idx = torch.tensor(seqs, dtype=torch.long, device=case.q.device)
    q = case.q.index_select(0, idx)
    bias = case.bias.index_select(0, idx)
    rows = [(i, h) for i in range(len(seqs)) for h in heads]
    res = oracle.decode(q, k, v, bias, cu, window=sp.window, rel_extent=sp.rel_extent,
                        sm_scale=sp.scale(), rows=rows, want_lse=want_lse)
    if want_lse:
        out, lse = res
        return (out.reshape(len(seqs), len(heads), -1), lse.reshape(len(seqs), len(heads)))
    return res.reshape(len(seqs), len(heads), -1)


def sample_positions(L: int, count: int, gen: torch.Generator, window: int = 0,
                     rel_extent: int = 0, offset: int = 0):
    """Sorted query indices in [0, L): every tile and border case the kernels
    special-case (sequence start and end, 32/64-query and 64-key tile edges,
    the window edge, the clamp border t - s = R - 1 for the first key), then
    random ones until ``count`` are chosen.  ``offset`` is the position of
    index 0 (prefill over a history): borders are placed on positions."""
    pos = {0, 1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 127, 128, 129, 191, 192, 255, 256}
    for edge in (window, rel_extent):
        if edge > 0:
            pos |= {edge - 2, edge - 1, edge, edge + 1, edge + 63, edge + 64, 2 * edge - 1}
    idx = {p - offset for p in pos} | {L - 65, L - 64, L - 33, L - 32, L - 2, L - 1}
    idx = {i for i in idx if 0 <= i < L}
    while len(idx) < min(count, L):
        idx.add(int(torch.randint(0, L, (1,), generator=gen)))
    return sorted(idx)


def random_pools(dev, dtype, Hkv, D, P, lens_after, spare_pages=3, seed=0):
    """Random pools (no NaN) and a shuffled table with room for lens_after."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    pages_per = [max(1, -(-n // P)) for n in lens_after]
    num_pages = sum(pages_per) + spare_pages
    perm = torch.randperm(num_pages, generator=g)
    table = torch.zeros((len(lens_after), max(pages_per)), dtype=torch.int32)
    off = 0
    for b, npg in enumerate(pages_per):
        table[b, :npg] = perm[off:off + npg].to(torch.int32)
        off += npg
    k_pool = torch.randn((num_pages, Hkv, P, D), generator=g).to(dtype).to(dev)
    v_pool = torch.randn((num_pages, Hkv, P, D), generator=g).to(dtype).to(dev)
    return k_pool, v_pool, table.to(dev)
