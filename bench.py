"""Benchmark of relative-position-bias paged attention on one MI355X.

One step = one pass of the hot path over one batch of the headline workload:
the local sliding-window layer prefill of 4 sequences x 4096 tokens (32 query
heads, 16 KV heads, head_dim 128, window 512, bias [T, 32, 512] bf16, 64-token
pages placed by a shuffled 512-page pool).  Inputs are synthetic, seeded, and
resident in HBM before timing starts.

Printed: one JSON line with the throughput (prefill TFLOP/s), a roofline
object for the kernel (achieved algorithmic GB/s against HBM peak, from HIP
events on the launch stream), the CPU oracle timed on a bounded sample of the
same workload, and the other four-layer workloads (global-layer prefill,
mixed and long-context decode) measured more briefly under "secondary".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MAIN = "local-prefill-4x4096"
SECONDARY = ["global-prefill-2x16384", "mixed-decode-256", "long-decode-32x131072",
             "chunked-local-4x512-ctx4096", "chunked-global-2x2048-ctx16384", "kv-append-8x2048",
             "fused-local-prefill-4x4096-drel32", "fused-global-prefill-2x16384-drel32"]
RIDGE_FLOP_PER_BYTE = 315.0


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
    sp = case.spec
    D, Hq, Hkv, W, R = sp.head_dim, sp.num_q_heads, sp.num_kv_heads, sp.window, sp.rel_extent
    es = 2
    flops = 0
    byt = 0
    for n in case.seq_lens:
        vis = min(n, W) if W > 0 else n
        flops += 4 * D * Hq * vis
        byt += vis * Hkv * D * es * 2 + Hq * min(vis, R) * es
    B = len(case.seq_lens)
    byt += B * Hq * D * es * 2
    return flops, byt


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


def recorded_traffic(workload: str, kernel_source: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_sha256") != source_hash(kernel_source):
        return None
    return rec.get("traffic_bytes")


# ---------------------------------------------------------------------------
# timing

def time_steps(step, steps: int, warmup: int, torch, min_warm_ms: float = 0.0):
    """Run warmup (at least `warmup` steps, and at least `min_warm_ms` of
    back-to-back work), then `steps` timed steps.  Returns (wall ms per
    step, event-timed ms per step: the timed region's device time over the
    steps, gaps between launches included)."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        while (time.perf_counter() - t0) * 1e3 < min_warm_ms:
            for _ in range(max(1, warmup)):
                step()
            torch.cuda.synchronize()
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
    return wall, ev


def cpu_baseline(case, budget_s: float):
    """The oracle, as it stands, on a random sample of the workload's rows."""
    import numpy as np
    import torch

    import oracle

    sp = case.spec
    cu = case.cu_list()
    q, k, v, bias = case.q.cpu(), case.k_log.cpu(), case.v_log.cpu(), case.bias.cpu()
    g = torch.Generator().manual_seed(12345)
    T, Hq = case.total_tokens, sp.num_q_heads

    def rows_flops(rows):
        f = 0
        for tok, _ in rows:
            b = int(np.searchsorted(cu, tok, side="right")) - 1
            t = tok - cu[b]
            vis = min(t + 1, sp.window) if sp.window > 0 else t + 1
            f += 4 * sp.head_dim * vis
        return f

    def draw(n):
        toks = torch.randint(0, T, (n,), generator=g).tolist()
        hs = torch.randint(0, Hq, (n,), generator=g).tolist()
        return list(zip(toks, hs))

    orc = oracle.default()
    probe = draw(256)
    t0 = time.perf_counter()
    orc.prefill(q, k, v, bias, cu, window=sp.window, rel_extent=sp.rel_extent,
                sm_scale=sp.scale(), rows=probe)
    dt = time.perf_counter() - t0
    n = max(256, int(256 * budget_s / max(dt, 1e-3)))
    rows = draw(n)
    t0 = time.perf_counter()
    orc.prefill(q, k, v, bias, cu, window=sp.window, rel_extent=sp.rel_extent,
                sm_scale=sp.scale(), rows=rows)
    dt = time.perf_counter() - t0
    return {"value": rows_flops(rows) / dt / 1e12, "unit": "TFLOP/s",
            "cores": orc.threads_used, "kind": "oracle",
            "sample": f"{n} random (token, head) rows of {T * Hq}; fp64, full score rows, "
                      f"{dt:.1f} s"}


# ---------------------------------------------------------------------------

def run_prefill(case, steps, warmup, torch, rba, min_warm_ms=0.0):
    sp = case.spec
    out = torch.empty_like(case.q)

    def step():
        rba.prefill(case.q, case.cu_seqlens, case.max_seqlen, case.k_pool, case.v_pool,
                    case.block_table, case.seq_lens_dev, case.bias, window=sp.window,
                    sm_scale=sp.scale(), out=out)

    return time_steps(step, steps, warmup, torch, min_warm_ms)


def run_prefill_fused(case, steps, warmup, torch, rba, min_warm_ms=0.0):
    h = case.hist
    sp = h.spec
    out = torch.empty_like(h.q)

    def step():
        rba.prefill_fused(h.q, h.cu_seqlens, h.max_seqlen, h.k_pool, h.v_pool, h.block_table,
                          h.seq_lens_dev, case.rel_r, case.w_rel_t, window=sp.window,
                          sm_scale=sp.scale(), out=out)

    return time_steps(step, steps, warmup, torch, min_warm_ms)


def run_decode(cases, splits, steps, warmup, torch, rba, min_warm_ms=0.0):
    ws = {}
    outs = {}
    for key, c in cases.items():
        sp = c.spec
        need = rba.decode_workspace_size(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens_dev,
                                         c.max_seq_len, c.bias, window=sp.window,
                                         sm_scale=sp.scale(), num_splits=splits)
        ws[key] = torch.empty(max(need, 1), dtype=torch.uint8, device=c.q.device)
        outs[key] = torch.empty_like(c.q)

    def step():
        for key, c in cases.items():
            sp = c.spec
            rba.decode(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens_dev, c.max_seq_len,
                       c.bias, window=sp.window, sm_scale=sp.scale(), num_splits=splits,
                       workspace=ws[key], out=outs[key])

    return time_steps(step, steps, warmup, torch, min_warm_ms)


def secondary(name, torch, rba, ri, steps, warmup, min_warm_ms=0.0):
    w = ri.WORKLOADS[name]
    cases = ri.build_workload(name, torch.device("cuda:0"))
    if w["kind"] == "append":
        c = cases["append"]
        es = 2 if str(c.spec.dtype) == "torch.bfloat16" else 4
        byt = 2 * 2 * c.k_new.numel() * es          # K and V, each read once and written once

        def step():
            rba.kv_append(c.k_new, c.v_new, c.cu_new, c.k_pool, c.v_pool, c.block_table,
                          c.seq_lens_dev)

        wall, ev = time_steps(step, steps, warmup, torch, min_warm_ms)
        gbs = byt / (ev * 1e-3) / 1e9
        return {"workload": name, "metric": "K/V append GB/s", "value": round(gbs, 1),
                "unit": "GB/s", "ms_per_step": round(wall, 4), "kernel_ms": round(ev, 4),
                "algorithmic_bytes": byt,
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    if w["kind"] in ("prefill", "prefill-history", "prefill-projected"):
        case = cases["prefill"]
        work = {"prefill": prefill_work, "prefill-history": prefill_history_work,
                "prefill-projected": prefill_projected_work}[w["kind"]]
        flops, byt = work(case)
        if w["kind"] == "prefill-projected":
            wall, ev = run_prefill_fused(case, steps, warmup, torch, rba, min_warm_ms)
        else:
            wall, ev = run_prefill(case, steps, warmup, torch, rba, min_warm_ms)
        tf = flops / (ev * 1e-3) / 1e12
        gbs = byt / (ev * 1e-3) / 1e9
        if w["kind"] != "prefill" and flops / byt < RIDGE_FLOP_PER_BYTE:
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
        else:
            roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        res = {"workload": name, "metric": "prefill attn TFLOP/s", "value": round(tf, 2),
               "unit": "TFLOP/s", "ms_per_step": round(wall, 4), "kernel_ms": round(ev, 4),
               "roofline": roof, "hbm_gbs": round(gbs, 1),
               "algorithmic_flops": flops, "algorithmic_bytes": byt}
    else:
        splits = w.get("num_splits", 0)
        flops = byt = 0
        for c in cases.values():
            f, b = decode_work(c)
            flops += f
            byt += b
        wall, ev = run_decode(cases, splits, steps, warmup, torch, rba, min_warm_ms)
        gbs = byt / (ev * 1e-3) / 1e9
        res = {"workload": name, "metric": "decode KV-read GB/s", "value": round(gbs, 1),
               "unit": "GB/s", "ms_per_step": round(wall, 4), "step_event_ms": round(ev, 4),
               "algorithmic_bytes": byt,
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
               "splits": {k: rba.decode_num_splits(c.q, c.k_pool, c.v_pool, c.block_table,
                                                   c.seq_lens_dev, c.max_seq_len, c.bias,
                                                   window=c.spec.window, sm_scale=c.spec.scale(),
                                                   num_splits=splits)
                          for k, c in cases.items()}}
    del cases
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU takes some 10-20 ms of back-to-back work to reach its steady
    # clocks; the default warm-up covers that (about 15 ms on the headline)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=MAIN)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the cpu_baseline sample")
    ap.add_argument("--copy-calibration-gib", type=int, default=0,
                    help="only run a plain device copy of this many GiB, three times "
                         "(the known-size kernel that scales FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

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

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the attention "
              "kernels shard by sequence and KV head with no exchange, so a multi-GPU figure "
              "is the one-GPU figure times N and is not measured here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rba_inputs as ri
    import relative_position_bias_paged_amd as rba

    rba.load()
    dev = torch.device("cuda:0")
    w = ri.WORKLOADS[args.workload]
    base = {
        "metric": "prefill attn TFLOP/s + decode KV-read GB/s (% MI355X peak), rel-bias paged",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v/bias, shuffled page placement)",
    }
    if w["kind"] == "append":
        res = secondary(args.workload, torch, rba, ri, args.steps, args.warmup)
        result = dict(base, metric=res["metric"], value=res["value"], unit="GB/s",
                      ms_per_step=res["ms_per_step"],
                      config={"workload": args.workload, "parallelism": "single GPU"},
                      roofline=dict(res["roofline"],
                                    traffic=recorded_traffic(args.workload, "kv_append.hip"),
                                    kernel="kv_append_kernel",
                                    kernel_ms=res["kernel_ms"],
                                    algorithmic_bytes=res["algorithmic_bytes"]))
        print(json.dumps(result), flush=True)
        return
    if w["kind"] in ("prefill-history", "prefill-projected"):
        res = secondary(args.workload, torch, rba, ri, args.steps, args.warmup)
        fused = w["kind"] == "prefill-projected"
        kernel = ("prefill_bf16_kernel<128, 8 waves, d_rel 32> (bias formed in the kernel)" if fused
                  else "prefill_bf16_kernel<128>")
        result = dict(base, value=res["value"], unit="TFLOP/s", ms_per_step=res["ms_per_step"],
                      config={"workload": args.workload, "parallelism": "single GPU"},
                      roofline=dict(res["roofline"],
                                    traffic=(recorded_traffic(args.workload, "prefill_bf16.hip")
                                             if fused else None),
                                    kernel=kernel,
                                    kernel_ms=res["kernel_ms"],
                                    algorithmic_bytes=res["algorithmic_bytes"],
                                    algorithmic_flops=res["algorithmic_flops"]))
        print(json.dumps(result), flush=True)
        return
    if w["kind"] != "prefill":
        # a decode workload as the main line: throughput in KV-read GB/s
        res = secondary(args.workload, torch, rba, ri, args.steps, args.warmup)
        result = dict(base, value=res["value"], unit="GB/s", ms_per_step=res["ms_per_step"],
                      config={"workload": args.workload, "parallelism": "single GPU",
                              "splits": res["splits"]},
                      roofline=dict(res["roofline"], traffic=recorded_traffic(args.workload,
                                                                              "decode_bf16.hip"),
                                    kernel="decode_bf16_kernel<128> (+ merge_kernel<128>)",
                                    step_ms=res["step_event_ms"],
                                    algorithmic_bytes=res["algorithmic_bytes"]))
        print(json.dumps(result), flush=True)
        return
    case = ri.build_workload(args.workload, dev)["prefill"]
    sp = case.spec
    flops, byt = prefill_work(case)
    wall, ev = run_prefill(case, args.steps, args.warmup, torch, rba)
    tflops = flops / (wall * 1e-3) / 1e12
    achieved = byt / (ev * 1e-3) / 1e9
    local = sp.window > 0
    result = dict(base, **{
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(wall, 5),
        "config": {"workload": args.workload, "sequences": len(case.seq_lens),
                   "seq_len": case.max_seqlen, "q_heads": sp.num_q_heads,
                   "kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "window": sp.window,
                   "rel_extent": sp.rel_extent, "page_size": sp.page_size,
                   "parallelism": "single GPU"},
    })
    mfma = flops / (ev * 1e-3) / 1e12
    if local:   # the bias stream makes this layer HBM-bound (142 FLOP/B < ridge)
        result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        result["roofline"] = {"bound": "mfma", "achieved": round(mfma, 2),
                              "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(mfma / MFMA_BF16_PEAK_TFLOPS, 4)}
    result["roofline"].update({
        "traffic": recorded_traffic(args.workload, "prefill_bf16.hip"),
        "kernel": "prefill_bf16_kernel<128>", "kernel_ms": round(ev, 5),
        "algorithmic_bytes": byt, "algorithmic_flops": flops,
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "mfma_frac": round(mfma / MFMA_BF16_PEAK_TFLOPS, 4)})
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    del case
    torch.cuda.empty_cache()
    if not args.no_secondary:
        # after the oracle's pause the clocks have dropped again: each short
        # secondary warms for a fixed stretch of work, not just a step count
        result["secondary"] = [secondary(n, torch, rba, ri, steps=max(5, args.steps // 5),
                                         warmup=max(2, args.warmup // 5), min_warm_ms=30.0)
                               for n in SECONDARY if n != args.workload]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
