"""Seeded synthetic inputs for relative-position-bias paged attention.

This module only draws random tensors and lays them out; it computes nothing
of the attention itself.  Both the HIP library's callers (tests, bench, smoke)
and the CPU oracle take their inputs from here.

Layouts produced (the C ABI in include/rba.h documents the same):
  q        [T, Hq, D]  (prefill, tokens of all sequences back to back)
           [B, Hq, D]  (decode, one query per sequence)
  bias     [T, Hq, R] / [B, Hq, R]
  k_pool, v_pool  [num_pages, Hkv, P, D], one page = P consecutive key
           positions of one sequence, head-major inside the page
  block_table     int32 [B, max_pages]; entry j is the pool page holding key
           positions j*P .. j*P+P-1; entries past a sequence's last page are 0
  seq_lens        int32 [B]; keys held for each sequence
  k_log, v_log    logical K/V, token-major [sum_b n_b, Hkv, D], for the oracle

Recipe: float tensors are N(0,1) (the tiny fp32 case draws its bias with
standard deviation 0.5) and are cast to the workload dtype before either side
sees them.  Page placements and context lengths come from a CPU generator with
the workload's seed.  Pool pages that no sequence owns, and the slots past the
end of a sequence's last page, are filled with NaN so that a stray read shows
up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

POISON = float("nan")


@dataclasses.dataclass
class LayerSpec:
    """One attention layer's geometry."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int          # <= 0: full causal
    rel_extent: int
    page_size: int
    dtype: torch.dtype = torch.bfloat16
    sm_scale: Optional[float] = None
    bias_std: float = 1.0

    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass
class PrefillCase:
    spec: LayerSpec
    seq_lens: List[int]
    q: torch.Tensor
    k_log: torch.Tensor
    v_log: torch.Tensor
    bias: torch.Tensor
    cu_seqlens: torch.Tensor      # int32 [B+1], device
    seq_lens_dev: torch.Tensor    # int32 [B], device
    block_table: torch.Tensor     # int32 [B, max_pages], device
    k_pool: torch.Tensor
    v_pool: torch.Tensor

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seq_lens)) if self.seq_lens else 0

    def cu_list(self) -> List[int]:
        cu = [0]
        for n in self.seq_lens:
            cu.append(cu[-1] + n)
        return cu


@dataclasses.dataclass
class DecodeCase:
    """Decode inputs.  q and bias hold q_len rows per sequence (row b*q_len
    + i is sequence b's token at position n_b - q_len + i); q_len 1 is the
    single-token decode, [B, Hq, D] / [B, Hq, R]."""
    spec: LayerSpec
    seq_lens: List[int]
    q: torch.Tensor
    bias: torch.Tensor
    seq_lens_dev: torch.Tensor
    block_table: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    seed: int
    window_only: bool
    _kv_first_page: List[int]     # first page index whose contents are real
    q_len: int = 1

    @property
    def max_seq_len(self) -> int:
        return int(max(self.seq_lens)) if self.seq_lens else 0

    def logical_kv(self, b: int):
        """Logical K/V [n_b, Hkv, D] of sequence b, on the CPU.

        Regenerated from the per-sequence seed (same device as the pool, so
        the values are the ones scattered into the pool); positions whose page
        is not real (window-only pools) are NaN.
        """
        k, v = _seq_kv(self.spec, self.seed, b, self.seq_lens[b], self.q.device)
        k, v = k.cpu(), v.cpu()
        first = self._kv_first_page[b] * self.spec.page_size
        if first > 0:
            k[:first] = POISON
            v[:first] = POISON
        return k, v


def _cpu_gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _dev_gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, gen, device, dtype, std=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def _scatter_pages(pool: torch.Tensor, pages: torch.Tensor, kv: torch.Tensor, P: int):
    """Write logical rows kv [n, Hkv, D] into pool pages ``pages`` (in order)."""
    n, Hkv, D = kv.shape
    npg = pages.numel()
    padded = torch.full((npg * P, Hkv, D), POISON, dtype=kv.dtype, device=kv.device)
    padded[:n] = kv
    pool[pages.to(pool.device).long()] = padded.view(npg, P, Hkv, D).permute(0, 2, 1, 3)


def make_prefill(spec: LayerSpec, seq_lens: List[int], seed: int, device="cpu",
                 num_pages: Optional[int] = None, shuffle: bool = True) -> PrefillCase:
    """Prefill inputs: each sequence's keys are its own tokens (no history)."""
    P = spec.page_size
    B = len(seq_lens)
    T = int(sum(seq_lens))
    g = _dev_gen(seed, device)
    q = _randn((T, spec.num_q_heads, spec.head_dim), g, device, spec.dtype)
    k_log = _randn((T, spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    v_log = _randn((T, spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    bias = _randn((T, spec.num_q_heads, spec.rel_extent), g, device, spec.dtype,
                  std=spec.bias_std)

    pages_per = [max(1, -(-n // P)) for n in seq_lens]
    needed = int(sum(pages_per))
    if num_pages is None:
        num_pages = needed
    if num_pages < needed:
        raise ValueError("pool too small")
    cg = _cpu_gen(seed)
    perm = torch.randperm(num_pages, generator=cg) if shuffle else torch.arange(num_pages)
    max_pages = max(pages_per) if pages_per else 1
    table = torch.zeros((max(B, 1), max_pages), dtype=torch.int32)
    k_pool = torch.full((num_pages, spec.num_kv_heads, P, spec.head_dim), POISON,
                        dtype=spec.dtype, device=device)
    v_pool = torch.full_like(k_pool, POISON)
    off = 0
    tok = 0
    for b, n in enumerate(seq_lens):
        pg = perm[off:off + pages_per[b]]
        table[b, :pages_per[b]] = pg.to(torch.int32)
        if n > 0:
            _scatter_pages(k_pool, pg, k_log[tok:tok + n], P)
            _scatter_pages(v_pool, pg, v_log[tok:tok + n], P)
        off += pages_per[b]
        tok += n
    cu = [0]
    for n in seq_lens:
        cu.append(cu[-1] + n)
    return PrefillCase(
        spec=spec, seq_lens=list(seq_lens), q=q, k_log=k_log, v_log=v_log, bias=bias,
        cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device),
        seq_lens_dev=torch.tensor(list(seq_lens) or [0], dtype=torch.int32, device=device)[:B],
        block_table=table.to(device), k_pool=k_pool, v_pool=v_pool)


@dataclasses.dataclass
class HistoryCase:
    """Prefill of new tokens over a cached history: sequence b holds
    key_lens[b] keys in the pool (its new tokens' keys included) and this
    call's new_lens[b] tokens are its last positions."""
    spec: LayerSpec
    new_lens: List[int]
    key_lens: List[int]
    q: torch.Tensor               # [sum new, Hq, D]
    k_log: torch.Tensor           # [sum keys, Hkv, D], sequences back to back
    v_log: torch.Tensor
    bias: torch.Tensor            # [sum new, Hq, R]
    cu_seqlens: torch.Tensor      # int32 [B+1] over the new tokens, device
    seq_lens_dev: torch.Tensor    # int32 [B] keys per sequence, device
    block_table: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor

    @property
    def total_tokens(self) -> int:
        return int(sum(self.new_lens))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.new_lens)) if self.new_lens else 0

    def cu_list(self) -> List[int]:
        return _cumsum(self.new_lens)

    def cu_kv_list(self) -> List[int]:
        return _cumsum(self.key_lens)


def _cumsum(lens):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    return cu


def make_prefill_history(spec: LayerSpec, key_lens: List[int], new_lens: List[int], seed: int,
                         device="cpu", num_pages: Optional[int] = None,
                         shuffle: bool = True, with_bias: bool = True) -> HistoryCase:
    """Prefill inputs over a history: all key_lens[b] keys of each sequence
    are in shuffled pool pages; queries and bias rows exist for the last
    new_lens[b] positions only (with_bias False: no bias tensor)."""
    if any(m > n for m, n in zip(new_lens, key_lens)):
        raise ValueError("more new tokens than keys")
    P = spec.page_size
    B = len(key_lens)
    g = _dev_gen(seed, device)
    q = _randn((int(sum(new_lens)), spec.num_q_heads, spec.head_dim), g, device, spec.dtype)
    k_log = _randn((int(sum(key_lens)), spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    v_log = _randn((int(sum(key_lens)), spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    bias = (_randn((int(sum(new_lens)), spec.num_q_heads, spec.rel_extent), g, device, spec.dtype,
                   std=spec.bias_std) if with_bias else None)
    pages_per = [max(1, -(-n // P)) for n in key_lens]
    needed = int(sum(pages_per))
    if num_pages is None:
        num_pages = needed
    if num_pages < needed:
        raise ValueError("pool too small")
    cg = _cpu_gen(seed)
    perm = torch.randperm(num_pages, generator=cg) if shuffle else torch.arange(num_pages)
    table = torch.zeros((max(B, 1), max(pages_per) if pages_per else 1), dtype=torch.int32)
    k_pool = torch.full((num_pages, spec.num_kv_heads, P, spec.head_dim), POISON,
                        dtype=spec.dtype, device=device)
    v_pool = torch.full_like(k_pool, POISON)
    off = 0
    tok = 0
    for b, n in enumerate(key_lens):
        pg = perm[off:off + pages_per[b]]
        table[b, :pages_per[b]] = pg.to(torch.int32)
        if n > 0:
            _scatter_pages(k_pool, pg, k_log[tok:tok + n], P)
            _scatter_pages(v_pool, pg, v_log[tok:tok + n], P)
        off += pages_per[b]
        tok += n
    return HistoryCase(
        spec=spec, new_lens=list(new_lens), key_lens=list(key_lens), q=q, k_log=k_log,
        v_log=v_log, bias=bias,
        cu_seqlens=torch.tensor(_cumsum(new_lens), dtype=torch.int32, device=device),
        seq_lens_dev=torch.tensor(list(key_lens) or [0], dtype=torch.int32, device=device)[:B],
        block_table=table.to(device), k_pool=k_pool, v_pool=v_pool)


@dataclasses.dataclass
class ProjectedCase:
    """Prefill whose bias is given by its projection: rel_r [sum new, Hq,
    d_rel] and w_rel [d_rel, R] (w_rel_t = its transpose, the layout the
    fused kernel reads).  ``hist`` holds everything else (its bias is None)."""
    hist: HistoryCase
    rel_r: torch.Tensor
    w_rel: torch.Tensor
    w_rel_t: torch.Tensor

    @property
    def spec(self) -> LayerSpec:
        return self.hist.spec

    @property
    def d_rel(self) -> int:
        return int(self.w_rel.shape[0])


def make_projected(spec: LayerSpec, key_lens: List[int], new_lens: Optional[List[int]],
                   d_rel: int, seed: int, device="cpu", num_pages: Optional[int] = None,
                   r_std: float = 1.0) -> ProjectedCase:
    """Inputs of the fused prefill.  r ~ N(0, r_std^2) and W ~ N(0, (bias_std /
    (r_std sqrt(d_rel)))^2), so the bias r . W has the spread bias_std of the
    stored bias tensors; new_lens None: no history (every key is a query)."""
    new = list(key_lens) if new_lens is None else list(new_lens)
    hist = make_prefill_history(spec, list(key_lens), new, seed, device=device,
                                num_pages=num_pages, with_bias=False)
    g = _dev_gen(seed + 7919, device)
    rel_r = _randn((int(sum(new)), spec.num_q_heads, d_rel), g, device, spec.dtype, std=r_std)
    w_rel = _randn((d_rel, spec.rel_extent), g, device, spec.dtype,
                   std=spec.bias_std / (r_std * math.sqrt(d_rel)))
    return ProjectedCase(hist=hist, rel_r=rel_r, w_rel=w_rel, w_rel_t=w_rel.t().contiguous())


@dataclasses.dataclass
class AppendCase:
    """New tokens' keys and values to write into shuffled pool pages; the
    sequences hold key_lens[b] keys after the append."""
    spec: LayerSpec
    new_lens: List[int]
    key_lens: List[int]
    k_new: torch.Tensor           # [sum new, Hkv, D]
    v_new: torch.Tensor
    cu_new: torch.Tensor          # int32 [B+1], device
    seq_lens_dev: torch.Tensor    # int32 [B] keys after the append, device
    block_table: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor


def make_append(spec: LayerSpec, key_lens: List[int], new_lens: List[int], seed: int,
                device="cpu") -> AppendCase:
    P = spec.page_size
    g = _dev_gen(seed, device)
    T = int(sum(new_lens))
    k_new = _randn((T, spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    v_new = _randn((T, spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    pages_per = [max(1, -(-n // P)) for n in key_lens]
    num_pages = int(sum(pages_per))
    perm = torch.randperm(num_pages, generator=_cpu_gen(seed))
    table = torch.zeros((len(key_lens), max(pages_per)), dtype=torch.int32)
    off = 0
    for b, npg in enumerate(pages_per):
        table[b, :npg] = perm[off:off + npg].to(torch.int32)
        off += npg
    k_pool = torch.zeros((num_pages, spec.num_kv_heads, P, spec.head_dim), dtype=spec.dtype,
                         device=device)
    return AppendCase(spec=spec, new_lens=list(new_lens), key_lens=list(key_lens), k_new=k_new,
                      v_new=v_new,
                      cu_new=torch.tensor(_cumsum(new_lens), dtype=torch.int32, device=device),
                      seq_lens_dev=torch.tensor(key_lens, dtype=torch.int32, device=device),
                      block_table=table.to(device), k_pool=k_pool, v_pool=torch.zeros_like(k_pool))


def _seq_kv(spec: LayerSpec, seed: int, b: int, n: int, device):
    g = _dev_gen(seed * 1_000_003 + 7919 * (b + 1), device)
    k = _randn((n, spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    v = _randn((n, spec.num_kv_heads, spec.head_dim), g, device, spec.dtype)
    return k, v


def make_decode(spec: LayerSpec, seq_lens: List[int], seed: int, device="cpu",
                window_only: bool = False, shuffle: bool = True, q_len: int = 1) -> DecodeCase:
    """Decode inputs: sequence b holds n_b keys; its q_len queries sit at
    n_b - q_len .. n_b - 1 (one query at n_b - 1 by default).

    With ``window_only`` (local layers) only the pages covering the keys the
    queries see (the last ``window + q_len - 1`` positions) hold real keys;
    every earlier table entry points to pool page 0, which is NaN-filled and
    must never influence the output.
    """
    P = spec.page_size
    B = len(seq_lens)
    g = _dev_gen(seed, device)
    q = _randn((B * q_len, spec.num_q_heads, spec.head_dim), g, device, spec.dtype)
    bias = _randn((B * q_len, spec.num_q_heads, spec.rel_extent), g, device, spec.dtype,
                  std=spec.bias_std)

    pages_per = [max(1, -(-n // P)) for n in seq_lens]
    first_real = []
    for n, npg in zip(seq_lens, pages_per):
        if window_only and spec.window > 0:
            first_real.append(max(0, n - q_len - spec.window + 1) // P)
        else:
            first_real.append(0)
    real_per = [npg - f for npg, f in zip(pages_per, first_real)]
    reserve = 1 if window_only else 0
    num_pages = reserve + int(sum(real_per))
    cg = _cpu_gen(seed)
    perm = (torch.randperm(num_pages - reserve, generator=cg) if shuffle
            else torch.arange(num_pages - reserve)) + reserve
    max_pages = max(pages_per) if pages_per else 1
    table = torch.zeros((max(B, 1), max_pages), dtype=torch.int32)
    k_pool = torch.empty((num_pages, spec.num_kv_heads, P, spec.head_dim),
                         dtype=spec.dtype, device=device)
    v_pool = torch.empty_like(k_pool)
    if reserve:
        k_pool[0] = POISON
        v_pool[0] = POISON
    off = 0
    for b, n in enumerate(seq_lens):
        pg = perm[off:off + real_per[b]]
        table[b, first_real[b]:pages_per[b]] = pg.to(torch.int32)
        k, v = _seq_kv(spec, seed, b, n, device)
        lo = first_real[b] * P
        _scatter_pages(k_pool, pg, k[lo:], P)
        _scatter_pages(v_pool, pg, v[lo:], P)
        del k, v
        off += real_per[b]
    return DecodeCase(
        spec=spec, seq_lens=list(seq_lens), q=q, bias=bias,
        seq_lens_dev=torch.tensor(list(seq_lens), dtype=torch.int32, device=device),
        block_table=table.to(device), k_pool=k_pool, v_pool=v_pool, seed=seed,
        window_only=window_only, _kv_first_page=first_real, q_len=q_len)


# ---------------------------------------------------------------------------
# The five named workloads (sizes of the layers described on the pages: local
# layers window 512 with 16 KV heads, global layers full causal with 8 KV heads
# and a 1024-bucket bias, 32 query heads, head_dim 128, 64-token pages).

LOCAL = dict(num_q_heads=32, num_kv_heads=16, head_dim=128, window=512,
             rel_extent=512, page_size=64)
GLOBAL = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, window=0,
              rel_extent=1024, page_size=64)

WORKLOADS = {
    "tiny-local-prefill-fp32": dict(
        kind="prefill", seed=1001, seq_lens=[256], num_pages=16, shuffle=False,
        spec=LayerSpec(num_q_heads=4, num_kv_heads=2, head_dim=64, window=64,
                       rel_extent=64, page_size=16, dtype=torch.float32,
                       bias_std=0.5)),
    "local-prefill-4x4096": dict(
        kind="prefill", seed=1002, seq_lens=[4096] * 4, num_pages=512, shuffle=True,
        spec=LayerSpec(**LOCAL)),
    "global-prefill-2x16384": dict(
        kind="prefill", seed=1003, seq_lens=[16384] * 2, num_pages=512, shuffle=True,
        spec=LayerSpec(**GLOBAL)),
    "mixed-decode-256": dict(
        kind="mixed-decode", seed=1004, batch=256, ctx_lo=1024, ctx_hi=32768,
        local=LayerSpec(**LOCAL), glob=LayerSpec(**GLOBAL)),
    "long-decode-32x131072": dict(
        kind="decode", seed=1005, seq_lens=[131072] * 32, num_splits=16,
        spec=LayerSpec(**GLOBAL)),
    # verification of drafted tokens (multi-token prediction): 4 new tokens
    # per sequence over the long-decode cache shape, 8 partitions of 16384 keys
    "mtp-verify-32x131072-q4": dict(
        kind="mtp-verify", seed=1011, seq_lens=[131072] * 32, q_len=4, num_splits=8,
        spec=LayerSpec(**GLOBAL)),
    # K/V append of a prefill chunk: 8 sequences, 2048 new tokens each onto
    # 2048 cached ones, local-layer pools
    "kv-append-8x2048": dict(
        kind="append", seed=1008, key_lens=[4096] * 8, new_lens=[2048] * 8,
        spec=LayerSpec(**LOCAL)),
    # chunked prefill: the last chunk of each sequence over the cached rest
    "chunked-local-4x512-ctx4096": dict(
        kind="prefill-history", seed=1006, key_lens=[4096] * 4, new_lens=[512] * 4,
        num_pages=512, spec=LayerSpec(**LOCAL)),
    "chunked-global-2x2048-ctx16384": dict(
        kind="prefill-history", seed=1007, key_lens=[16384] * 2, new_lens=[2048] * 2,
        num_pages=512, spec=LayerSpec(**GLOBAL)),
    # the two prefill layers with the bias formed from its projection
    # r [T, Hq, d_rel] . W [d_rel, R] in the kernel (d_rel is not stated on
    # the pages; 32 here)
    "fused-local-prefill-4x4096-drel32": dict(
        kind="prefill-projected", seed=1009, seq_lens=[4096] * 4, num_pages=512, d_rel=32,
        spec=LayerSpec(**LOCAL)),
    "fused-global-prefill-2x16384-drel32": dict(
        kind="prefill-projected", seed=1010, seq_lens=[16384] * 2, num_pages=512, d_rel=32,
        spec=LayerSpec(**GLOBAL)),
}


def mixed_decode_lengths(seed: int, batch: int, lo: int, hi: int) -> List[int]:
    """Context lengths uniform in [lo, hi] (inclusive), from the CPU generator."""
    g = _cpu_gen(seed + 17)
    return torch.randint(lo, hi + 1, (batch,), generator=g).tolist()


def build_workload(name: str, device="cpu"):
    """Materialise a named workload.  Returns a dict of cases."""
    w = WORKLOADS[name]
    if w["kind"] == "prefill":
        return {"prefill": make_prefill(w["spec"], w["seq_lens"], w["seed"], device,
                                        num_pages=w["num_pages"], shuffle=w["shuffle"])}
    if w["kind"] == "decode":
        return {"decode": make_decode(w["spec"], w["seq_lens"], w["seed"], device)}
    if w["kind"] == "mtp-verify":
        return {"verify": make_decode(w["spec"], w["seq_lens"], w["seed"], device,
                                      q_len=w["q_len"])}
    if w["kind"] == "append":
        return {"append": make_append(w["spec"], w["key_lens"], w["new_lens"], w["seed"], device)}
    if w["kind"] == "prefill-history":
        return {"prefill": make_prefill_history(w["spec"], w["key_lens"], w["new_lens"], w["seed"],
                                                device, num_pages=w["num_pages"])}
    if w["kind"] == "prefill-projected":
        return {"prefill": make_projected(w["spec"], w["seq_lens"], None, w["d_rel"], w["seed"],
                                          device, num_pages=w["num_pages"])}
    if w["kind"] == "mixed-decode":
        lens = mixed_decode_lengths(w["seed"], w["batch"], w["ctx_lo"], w["ctx_hi"])
        return {
            "local": make_decode(w["local"], lens, w["seed"], device, window_only=True),
            "global": make_decode(w["glob"], lens, w["seed"] + 100, device),
        }
    raise KeyError(name)
