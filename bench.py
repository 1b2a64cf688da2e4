"""Benchmark of relative-position-bias paged attention on one MI355X.

One step = one pass of the hot path over one batch of the headline workload:
the global full-causal layer prefill of 2 sequences x 16384 tokens (32 query
heads, 8 KV heads, head_dim 128, bias [T, 32, 1024] bf16 with distances
clamped to bucket 1023, 64-token pages under a shuffled 512-page table).
Inputs are synthetic, seeded, and resident in HBM before timing starts.

Printed: one JSON line.  Its top level is the headline: prefill TFLOP/s, a
roofline object for the kernel (algorithmic FLOPs over the HIP-event time of
the launches, on the stream they run on, against the bf16 matrix peak; the
HBM traffic and MFMA-busy fraction recorded by rocprofv3 for this kernel
source, if any), the parity of the timed output against the CPU oracle on
rows sampled without replacement, and the oracle's own throughput on those
rows (cpu_baseline).  "secondary" holds one object per other workload with
the same fields (decode lines in KV-read GB/s against HBM).  Every line warms
up for a fixed stretch of device time, not only a step count: the GPU takes
10-20 ms of back-to-back work to settle its clocks.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak (the fp32 path is plain FMA)
# Highest HBM read rate measured on the box for a plain linear read of a
# 17 GB pool with non-temporal loads (best grid): the practical ceiling a
# streaming decode kernel can reach, next to the 8 TB/s nameplate.
MEASURED_READ_CEILING_GBS = 6600.0
RIDGE_FLOP_PER_BYTE = 315.0
HEADLINE = "global-prefill-2x16384"
SECONDARY = ["local-prefill-4x4096", "tiny-local-prefill-fp32", "mixed-decode-256",
             "long-decode-32x131072", "mtp-verify-32x131072-q4", "chunked-local-4x512-ctx4096",
             "chunked-global-2x2048-ctx16384", "kv-append-8x2048",
             "fused-local-prefill-4x4096-drel32", "fused-global-prefill-2x16384-drel32"]
BF16_MAX_ABS, BF16_MEAN_REL, F32_MAX_ABS = 2e-2, 5e-3, 1e-5


# ---------------------------------------------------------------------------
# algorithmic work (visible pairs only; every byte counted once)

def visible_prefill_pairs(L: int, W: int) -> int:
    if W > 0 and L > W:
        return W * (W + 1) // 2 + (L - W) * W
    return L * (L + 1) // 2


def bias_entries_prefill(L: int, W: int, R: int) -> int:
    cap = min(W, R) if W > 0 else R
    if L > cap:
        return cap * (cap + 1) // 2 + (L - cap) * cap
    return L * (L + 1) // 2


def prefill_work(case):
    sp = case.spec
    D, Hq, Hkv, W, R = sp.head_dim, sp.num_q_heads, sp.num_kv_heads, sp.window, sp.rel_extent
    es = 2 if str(sp.dtype) == "torch.bfloat16" else 4
    pairs = sum(visible_prefill_pairs(L, W) for L in case.seq_lens)
    T = case.total_tokens
    flops = 4 * D * Hq * pairs
    byt = (T * Hq * D * es * 2                      # q read, out written
           + T * Hkv * D * es * 2                   # k, v
           + Hq * es * sum(bias_entries_prefill(L, W, R) for L in case.seq_lens))
    return flops, byt


def prefill_history_work(case):
    """Prefill over a cached history: query positions n-L .. n-1 of each
    sequence; keys visible to any of them are read once."""
    sp = case.spec
    D, Hq, Hkv, W, R = sp.head_dim, sp.num_q_heads, sp.num_kv_heads, sp.window, sp.rel_extent
    es = 2 if str(sp.dtype) == "torch.bfloat16" else 4
    pairs = bias_entries = kv_keys = 0
    for n, L in zip(case.key_lens, case.new_lens):
        for p in range(n - L, n):
            vis = min(p + 1, W) if W > 0 else p + 1
            pairs += vis
            bias_entries += min(vis, R)
        kv_keys += n - (max(0, n - L - W + 1) if W > 0 else 0)
    T = case.total_tokens
    flops = 4 * D * Hq * pairs
    byt = T * Hq * D * es * 2 + kv_keys * Hkv * D * es * 2 + Hq * es * bias_entries
    return flops, byt


def prefill_projected_work(case):
    """Prefill with the bias formed from its projection: the attention of
    prefill_history_work, plus 2*d_rel FLOPs per bias entry a row uses; the
    bias bytes become those of r [T, Hq, d_rel] and W [d_rel, R]."""
    h = case.hist
    sp = h.spec
    es = 2
    flops, byt = prefill_history_work(h)
    bias_entries = 0
    W, R = sp.window, sp.rel_extent
    for n, L in zip(h.key_lens, h.new_lens):
        for p in range(n - L, n):
            vis = min(p + 1, W) if W > 0 else p + 1
            bias_entries += min(vis, R)
    byt -= sp.num_q_heads * es * bias_entries
    byt += case.rel_r.numel() * es + case.w_rel.numel() * es
    flops += 2 * case.d_rel * sp.num_q_heads * bias_entries
    return flops, byt


def decode_work(case):
    """Single-token (q_len 1) or multi-token decode: K and V of the keys any
    of a sequence's queries sees, once, plus q, out and the bias entries."""
    sp = case.spec
    D, Hq, Hkv, W, R = sp.head_dim, sp.num_q_heads, sp.num_kv_heads, sp.window, sp.rel_extent
    ql = getattr(case, "q_len", 1)
    es = 2
    flops = byt = 0
    for n in case.seq_lens:
        keys = 0
        for i in range(ql):
            p = n - ql + i
            vis = min(p + 1, W) if W > 0 else p + 1
            flops += 4 * D * Hq * vis
            byt += Hq * min(vis, R) * es
        lo = max(0, n - ql - W + 1) if W > 0 else 0
        keys = n - lo
        byt += keys * Hkv * D * es * 2
    byt += len(case.seq_lens) * ql * Hq * D * es * 2
    return flops, byt


# ---------------------------------------------------------------------------
# recorded profiler figures (only when taken on the current kernel source)

def source_hash(*names):
    """Hash of kernel sources together with their compile flags: counters
    taken on another build of the same source do not describe this one."""
    from relative_position_bias_paged_amd import build as hip_build
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "relative_position_bias_paged_amd", "csrc", n), "rb") as f:
            h.update(f.read())
        h.update(" ".join(hip_build.EXTRA_FLAGS.get(n, [])).encode())
    return h.hexdigest()


def _recorded(path, workload, kernel_source, key):
    """kernel_source: one source file, or a tuple of the sources whose
    kernels a step launches."""
    path = os.path.join(ROOT, "profiles", path)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    sources = kernel_source if isinstance(kernel_source, tuple) else (kernel_source,)
    if not rec or rec.get("source_sha256") != source_hash(*sources):
        return None
    return rec.get(key)


def recorded_traffic(workload: str, kernel_source: str):
    """HBM bytes per step from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, if they were taken on the current kernel source; else None."""
    return _recorded("traffic.json", workload, kernel_source, "traffic_bytes")


def recorded_mfma_busy(workload: str, kernel_source: str):
    """SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES) from the
    committed rocprofv3 counter run, if taken on the current source."""
    return _recorded("sq_counters.json", workload, kernel_source, "mfma_busy")


# ---------------------------------------------------------------------------
# timing

def time_steps(step, steps: int, warmup: int, torch, min_warm_ms: float = 0.0):
    """Run warmup (at least `warmup` steps, and at least `min_warm_ms` of
    back-to-back work), then `steps` timed steps.  Returns (wall ms per
    step, event-timed ms per step: the timed region's device time over the
    steps, gaps between launches included, warm-up steps run, warm-up ms)."""
    t0 = time.perf_counter()
    done = 0
    for _ in range(warmup):
        step()
        done += 1
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        while (time.perf_counter() - t0) * 1e3 < min_warm_ms:
            for _ in range(max(1, warmup)):
                step()
                done += 1
            torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3
    # one event pair around the whole timed region: an event pair around
    # every step would put its own records between the launches
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = start.elapsed_time(end) / steps
    return wall, ev, done, warm_ms


# ---------------------------------------------------------------------------
# parity and the oracle's own speed on a sample (after the timed region)

def _errors(gpu, ref):
    import numpy as np
    g = gpu.detach().float().cpu().double().numpy().reshape(ref.shape)
    diff = np.abs(g - ref)
    return {"max_abs": float(diff.max(initial=0.0)),
            "mean_rel": float(diff.sum() / max(float(np.abs(ref).sum()), 1e-300)),
            "finite": bool(np.isfinite(g).all())}


def _within(err, dtype_is_f32):
    if dtype_is_f32:
        return err["finite"] and err["max_abs"] <= F32_MAX_ABS
    return err["finite"] and err["max_abs"] <= BF16_MAX_ABS and err["mean_rel"] <= BF16_MEAN_REL


def _threads_default():
    return int(os.environ.get("OMP_NUM_THREADS", "0") or 0)


def prefill_oracle_sample(kind, case, out, budget_s, seed):
    """The oracle, as it stands, on (token, head) rows drawn WITHOUT
    replacement from the whole workload, sized to about budget_s of work.
    Returns (parity of the GPU output on those rows, the oracle's speed)."""
    import numpy as np
    import torch

    import oracle

    orc = oracle.default()
    if kind == "prefill-projected":
        h = case.hist
        sp = h.spec
        cu, key_lens, new_lens = h.cu_list(), h.key_lens, h.new_lens
        args = (h.q.cpu(), h.k_log.cpu(), h.v_log.cpu(), case.rel_r.cpu(), case.w_rel.cpu(),
                cu, h.cu_kv_list())

        def run(rows):
            return orc.prefill_projected(*args, window=sp.window, sm_scale=sp.scale(), rows=rows)
    elif kind == "prefill-history":
        sp = case.spec
        cu, key_lens, new_lens = case.cu_list(), case.key_lens, case.new_lens
        args = (case.q.cpu(), case.k_log.cpu(), case.v_log.cpu(), case.bias.cpu(), cu,
                case.cu_kv_list())

        def run(rows):
            return orc.prefill_history(*args, window=sp.window, rel_extent=sp.rel_extent,
                                       sm_scale=sp.scale(), rows=rows)
    else:
        sp = case.spec
        cu = case.cu_list()
        key_lens = new_lens = case.seq_lens
        args = (case.q.cpu(), case.k_log.cpu(), case.v_log.cpu(), case.bias.cpu(), cu)

        def run(rows):
            return orc.prefill(*args, window=sp.window, rel_extent=sp.rel_extent,
                               sm_scale=sp.scale(), rows=rows)
    Hq, D, W, R = sp.num_q_heads, sp.head_dim, sp.window, sp.rel_extent
    T = int(cu[-1])
    d_rel = case.d_rel if kind == "prefill-projected" else 0

    def rows_flops(rows):
        f = 0
        for tok, _ in rows:
            b = int(np.searchsorted(cu, tok, side="right")) - 1
            p = key_lens[b] - new_lens[b] + (tok - cu[b])
            vis = min(p + 1, W) if W > 0 else p + 1
            f += 4 * D * vis + 2 * d_rel * min(vis, R)
        return f

    order = torch.randperm(T * Hq, generator=torch.Generator().manual_seed(seed)).tolist()
    probe = [(i // Hq, i % Hq) for i in order[:64]]
    t0 = time.perf_counter()
    run(probe)
    dt = time.perf_counter() - t0
    n = int(min(T * Hq, max(64, 64 * budget_s / max(dt, 1e-4))))
    rows = [(i // Hq, i % Hq) for i in order[:n]]
    t0 = time.perf_counter()
    ref = run(rows)
    dt = time.perf_counter() - t0
    tok = torch.tensor([r[0] for r in rows], device=out.device)
    hd = torch.tensor([r[1] for r in rows], device=out.device)
    err = _errors(out[tok, hd], ref)
    err.update(rows=n, of=T * Hq, within_tolerance=_within(err, str(sp.dtype) == "torch.float32"))
    speed = {"value": rows_flops(rows) / dt / 1e12, "unit": "TFLOP/s",
             "cores": orc.threads_used, "kind": "oracle", "seconds": round(dt, 2),
             "sample": f"{n} (token, head) rows of {T * Hq}, drawn without replacement; "
                       f"fp64, full score rows"}
    return err, speed


def decode_oracle_sample(cases, outs, budget_s, seed):
    """The oracle on whole sequences (every head) drawn without replacement
    from each decode case, sized to about budget_s of work.  Returns (parity
    over every sampled row, the oracle's KV-read speed)."""
    import numpy as np
    import torch

    import oracle
    orc = oracle.default()
    g = torch.Generator().manual_seed(seed)
    per_case = max(1.0, budget_s / max(1, len(cases)))
    diffs = []
    refs = []
    nbytes = 0
    total_s = 0.0
    seqs_used = {}
    for key, c in cases.items():
        sp = c.spec
        B = len(c.seq_lens)
        ql = getattr(c, "q_len", 1)
        order = torch.randperm(B, generator=g).tolist()
        spent = 0.0
        used = 0
        for b in order:
            if spent >= per_case and used > 0:
                break
            k, v = c.logical_kv(b)
            n = c.seq_lens[b]
            rows_q = c.q[b * ql:(b + 1) * ql]
            rows_b = c.bias[b * ql:(b + 1) * ql]
            t0 = time.perf_counter()
            if ql == 1:
                ref = orc.decode(rows_q, k, v, rows_b, [0, n], window=sp.window,
                                 rel_extent=sp.rel_extent, sm_scale=sp.scale())
            else:
                ref = orc.prefill_history(rows_q, k, v, rows_b, [0, ql], [0, n],
                                          window=sp.window, rel_extent=sp.rel_extent,
                                          sm_scale=sp.scale())
            dt = time.perf_counter() - t0
            spent += dt
            used += 1
            gpu = outs[key][b * ql:(b + 1) * ql].float().cpu().double().numpy()
            diffs.append(np.abs(gpu - ref).ravel())
            refs.append(np.abs(ref).ravel())
            lo = max(0, n - ql - sp.window + 1) if sp.window > 0 else 0
            nbytes += (n - lo) * sp.num_kv_heads * sp.head_dim * 2 * 2
        total_s += spent
        seqs_used[key] = f"{used} of {B}"
    d = np.concatenate(diffs)
    r = np.concatenate(refs)
    err = {"max_abs": float(d.max(initial=0.0)), "mean_rel": float(d.sum() / max(r.sum(), 1e-300)),
           "finite": bool(np.isfinite(d).all()), "sequences": seqs_used}
    err["within_tolerance"] = _within(err, False)
    speed = {"value": nbytes / total_s / 1e9, "unit": "GB/s", "cores": orc.threads_used,
             "kind": "oracle", "seconds": round(total_s, 2),
             "sample": "whole sequences (every head), drawn without replacement: "
                       + ", ".join(f"{k} {v}" for k, v in seqs_used.items())
                       + "; fp64, full score rows"}
    return err, speed


# ---------------------------------------------------------------------------
# one line per workload

def _roofline(flops, byt, ev_ms, workload, source, kernel, force=None):
    tf = flops / (ev_ms * 1e-3) / 1e12
    gbs = byt / (ev_ms * 1e-3) / 1e9
    bound = force or ("mfma" if flops / byt >= RIDGE_FLOP_PER_BYTE else "hbm")
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    elif bound == "alu":
        roof = {"bound": "alu", "achieved": round(tf, 3), "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 5)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": recorded_traffic(workload, source),
                 "mfma_busy": recorded_mfma_busy(workload, source),
                 "kernel": kernel, "kernel_ms": round(ev_ms, 5),
                 "algorithmic_bytes": byt, "algorithmic_flops": flops,
                 "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
    return roof


def line(name, args, torch, rba, ri, oracle_budget):
    """Build one workload, time it, then check it against the oracle."""
    w = ri.WORKLOADS[name]
    kind = w["kind"]
    cases = ri.build_workload(name, torch.device("cuda:0"))
    res = {"workload": name}
    if kind == "append":
        c = cases["append"]
        es = 2 if str(c.spec.dtype) == "torch.bfloat16" else 4
        byt = 2 * 2 * c.k_new.numel() * es          # K and V, each read once and written once

        def step():
            rba.kv_append(c.k_new, c.v_new, c.cu_new, c.k_pool, c.v_pool, c.block_table,
                          c.seq_lens_dev)

        wall, ev, wsteps, wms = time_steps(step, args.steps, args.warmup, torch, args.min_warm_ms)
        gbs = byt / (ev * 1e-3) / 1e9
        # parity: every appended row, read back through the page table by torch
        P = c.spec.page_size
        ok = True
        cu = [0]
        for m in c.new_lens:
            cu.append(cu[-1] + m)
        for b, (n, m) in enumerate(zip(c.key_lens, c.new_lens)):
            pos = torch.arange(n - m, n, device=c.k_pool.device)
            pages = c.block_table[b].long()[pos // P]
            ok &= bool(torch.equal(c.k_pool[pages, :, pos % P], c.k_new[cu[b]:cu[b + 1]]))
            ok &= bool(torch.equal(c.v_pool[pages, :, pos % P], c.v_new[cu[b]:cu[b + 1]]))
        res.update(metric="K/V append GB/s", value=round(gbs, 1), unit="GB/s",
                   ms_per_step=round(wall, 4), warmup_steps=wsteps, warmup_ms=round(wms, 1),
                   roofline=_roofline(0, byt, ev, name, "kv_append.hip", "kv_append_kernel<false>",
                                      force="hbm"),
                   parity={"bit_exact": ok, "rows": int(c.k_new.shape[0]),
                           "check": "every appended row read back through the page table"},
                   oracle=None)
    elif kind in ("prefill", "prefill-history", "prefill-projected"):
        case = cases["prefill"]
        work = {"prefill": prefill_work, "prefill-history": prefill_history_work,
                "prefill-projected": prefill_projected_work}[kind]
        flops, byt = work(case)
        h = case.hist if kind == "prefill-projected" else case
        sp = h.spec
        out = torch.empty_like(h.q)
        if kind == "prefill-projected":
            def step():
                rba.prefill_fused(h.q, h.cu_seqlens, h.max_seqlen, h.k_pool, h.v_pool,
                                  h.block_table, h.seq_lens_dev, case.rel_r, case.w_rel_t,
                                  window=sp.window, sm_scale=sp.scale(), out=out)
            nw = 4 if sp.window > 0 and (sp.num_q_heads // sp.num_kv_heads) % 2 == 0 else 8
            kernel = (f"prefill_bf16_kernel<{sp.head_dim}, {nw} waves, d_rel {case.d_rel}> "
                      "(bias formed in the kernel)")
        else:
            def step():
                rba.prefill(h.q, h.cu_seqlens, h.max_seqlen, h.k_pool, h.v_pool, h.block_table,
                            h.seq_lens_dev, h.bias, window=sp.window, sm_scale=sp.scale(),
                            out=out)
            kernel = ("prefill_f32_kernel" if str(sp.dtype) == "torch.float32"
                      else f"prefill_bf16_kernel<{sp.head_dim}, {4 if sp.window > 0 else 8} waves>")
        wall, ev, wsteps, wms = time_steps(step, args.steps, args.warmup, torch, args.min_warm_ms)
        f32 = str(sp.dtype) == "torch.float32"
        src = "attn_f32.hip" if f32 else "prefill_bf16.hip"
        roof = _roofline(flops, byt, ev, name, src, kernel, force="alu" if f32 else None)
        res.update(metric="prefill attn TFLOP/s", value=round(flops / (wall * 1e-3) / 1e12, 3),
                   unit="TFLOP/s", ms_per_step=round(wall, 5), warmup_steps=wsteps,
                   warmup_ms=round(wms, 1), roofline=roof,
                   hbm_gbs=round(byt / (ev * 1e-3) / 1e9, 1))
        if oracle_budget > 0:
            torch.cuda.synchronize()
            err, speed = prefill_oracle_sample(kind, case, out, oracle_budget, seed=12345)
            res.update(parity=err, oracle=speed)
    else:
        flops = byt = 0
        for c in cases.values():
            f, b = decode_work(c)
            flops += f
            byt += b
        outs = {k: torch.empty_like(c.q) for k, c in cases.items()}
        if kind == "mtp-verify":
            c = cases["verify"]
            sp = c.spec
            need = rba.decode_multi_workspace_size(c.q, c.q_len, c.k_pool, c.v_pool,
                                                   c.block_table, c.seq_lens_dev, c.max_seq_len,
                                                   c.bias, window=sp.window, sm_scale=sp.scale(),
                                                   num_splits=w.get("num_splits", 0))
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=c.q.device)

            def step():
                rba.decode_multi(c.q, c.q_len, c.k_pool, c.v_pool, c.block_table, c.seq_lens_dev,
                                 c.max_seq_len, c.bias, window=sp.window, sm_scale=sp.scale(),
                                 num_splits=w.get("num_splits", 0), workspace=ws,
                                 out=outs["verify"])
            kernel = "decode_multi_kernel<128> (+ plan_kernel, merge_kernel<128>)"
            src = ("decode_multi.hip", "decode_bf16.hip")
            splits = {"verify": rba.decode_multi_num_splits(
                c.q, c.q_len, c.k_pool, c.v_pool, c.block_table, c.seq_lens_dev, c.max_seq_len,
                c.bias, window=sp.window, sm_scale=sp.scale(), num_splits=w.get("num_splits", 0))}
        else:
            splits_req = w.get("num_splits", 0)
            ws = {}
            for key, c in cases.items():
                sp = c.spec
                need = rba.decode_workspace_size(c.q, c.k_pool, c.v_pool, c.block_table,
                                                 c.seq_lens_dev, c.max_seq_len, c.bias,
                                                 window=sp.window, sm_scale=sp.scale(),
                                                 num_splits=splits_req)
                ws[key] = torch.empty(max(need, 1), dtype=torch.uint8, device=c.q.device)

            def step():
                for key, c in cases.items():
                    sp = c.spec
                    rba.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens_dev,
                               c.max_seq_len, c.bias, window=sp.window, sm_scale=sp.scale(),
                               num_splits=splits_req, workspace=ws[key], out=outs[key])
            kernel = "decode_bf16_kernel<128> (+ plan_kernel, merge_kernel<128>)"
            src = "decode_bf16.hip"
            splits = {k: rba.decode_num_splits(c.q, c.k_pool, c.v_pool, c.block_table,
                                               c.seq_lens_dev, c.max_seq_len, c.bias,
                                               window=c.spec.window, sm_scale=c.spec.scale(),
                                               num_splits=splits_req)
                      for k, c in cases.items()}
        wall, ev, wsteps, wms = time_steps(step, args.steps, args.warmup, torch, args.min_warm_ms)
        gbs = byt / (ev * 1e-3) / 1e9
        roof = _roofline(flops, byt, ev, name, src, kernel, force="hbm")
        roof["measured_read_ceiling_gbs"] = MEASURED_READ_CEILING_GBS
        roof["frac_of_measured_ceiling"] = round(gbs / MEASURED_READ_CEILING_GBS, 4)
        res.update(metric="decode KV-read GB/s", value=round(gbs, 1), unit="GB/s",
                   ms_per_step=round(wall, 4), warmup_steps=wsteps, warmup_ms=round(wms, 1),
                   roofline=roof, splits=splits)
        if oracle_budget > 0:
            torch.cuda.synchronize()
            err, speed = decode_oracle_sample(cases, outs, oracle_budget, seed=54321)
            res.update(parity=err, oracle=speed)
    del cases
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warm-ms", type=float, default=60.0,
                    help="every line warms up for at least this much back-to-back work")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (parity and CPU speed) of every line")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the headline's cpu_baseline sample")
    ap.add_argument("--line-cpu-budget", type=float, default=2.0,
                    help="seconds of oracle work per secondary line")
    ap.add_argument("--copy-calibration-gib", type=int, default=0,
                    help="only run a plain device copy of this many GiB, three times "
                         "(the known-size kernel that scales FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the attention "
              "kernels shard by sequence and KV head with no exchange, so a multi-GPU figure "
              "is the one-GPU figure times N and is not measured here.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_gib > 0:
        import torch
        n = args.copy_calibration_gib << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 3
        print(json.dumps({"copy_calibration_bytes": n, "launches": 4,
                          "read_plus_write_GBps": round(2 * n / dt / 1e9, 1)}), flush=True)
        return

    import torch

    import rba_inputs as ri
    import relative_position_bias_paged_amd as rba

    rba.load()
    head_budget = 0.0 if args.no_cpu_baseline else args.cpu_budget
    main_line = line(args.workload, args, torch, rba, ri, head_budget)
    w = ri.WORKLOADS[args.workload]
    cfg = {"workload": args.workload, "parallelism": "single GPU"}
    for k in ("seq_lens", "key_lens", "new_lens"):
        if k in w:
            v = w[k]
            cfg["sequences"] = len(v)
            cfg[k[:-1]] = v[0] if len(set(v)) == 1 else v
    for k in ("batch", "q_len", "num_splits", "d_rel"):
        if k in w:
            cfg[k] = w[k]
    sp = w.get("spec")
    if sp is not None:
        cfg.update(q_heads=sp.num_q_heads, kv_heads=sp.num_kv_heads, head_dim=sp.head_dim,
                   window=sp.window, rel_extent=sp.rel_extent, page_size=sp.page_size)
    result = {
        "metric": "prefill attn TFLOP/s + decode KV-read GB/s (% MI355X peak), rel-bias paged",
        "value": main_line["value"], "unit": main_line["unit"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_steps_run": main_line["warmup_steps"], "warmup_ms": main_line["warmup_ms"],
        "ms_per_step": main_line["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if sp is not None and str(sp.dtype) == "torch.float32" else "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v/bias, shuffled page placement)",
        "config": cfg,
        "roofline": main_line["roofline"],
    }
    if "parity" in main_line:
        result["parity"] = main_line["parity"]
    if main_line.get("oracle"):
        result["cpu_baseline"] = main_line["oracle"]
    if not args.no_secondary:
        budget = 0.0 if args.no_cpu_baseline else args.line_cpu_budget
        result["secondary"] = [line(n, args, torch, rba, ri, budget)
                               for n in SECONDARY if n != args.workload and n in ri.WORKLOADS]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
