"""Host checks of the synthetic inputs: page layout, geometry, seeding."""
import json
import os

import torch

import rba_inputs as ri

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_workload_geometry_matches_pages():
    with open(os.path.join(GOLDEN, "pages_geometry.json")) as f:
        geo = json.load(f)
    loc = ri.WORKLOADS["local-prefill-4x4096"]["spec"]
    glo = ri.WORKLOADS["global-prefill-2x16384"]["spec"]
    assert loc.window == geo["local_window"]["value"]
    assert loc.num_kv_heads == geo["local_kv_heads"]["value"]
    assert glo.num_kv_heads == geo["global_kv_heads"]["value"]
    assert glo.window <= 0 and geo["global_window_left"]["value"] == -1
    assert glo.rel_extent == geo["global_rel_extent"]["value"]
    ex = geo["bias_shape_example"]
    mib = ex["tokens"] * ex["local_heads"] * ex["rel_extent"] * ex["dtype_bytes"] / 2**20
    assert mib == ex["approx_mib"]
    mixed = ri.WORKLOADS["mixed-decode-256"]
    assert mixed["local"].window == 512 and mixed["glob"].rel_extent == 1024


def test_prefill_pages_hold_logical_tokens():
    spec = ri.LayerSpec(num_q_heads=4, num_kv_heads=2, head_dim=8, window=0,
                        rel_extent=4, page_size=4, dtype=torch.float32)
    case = ri.make_prefill(spec, [9, 4], seed=5, num_pages=8, shuffle=True)
    table = case.block_table.cpu()
    tok = 0
    for b, n in enumerate(case.seq_lens):
        for s in range(n):
            page = int(table[b, s // 4])
            assert torch.equal(case.k_pool[page, :, s % 4], case.k_log[tok + s])
            assert torch.equal(case.v_pool[page, :, s % 4], case.v_log[tok + s])
        # the slots past the last key of the last page are NaN poison
        last = int(table[b, (n - 1) // 4])
        for s in range(n, -(-n // 4) * 4):
            assert torch.isnan(case.k_pool[last, :, s % 4]).all()
        tok += n
    used = set(int(x) for x in table.flatten() if True)
    # pool pages nobody owns stay poisoned
    owned = {int(table[0, j]) for j in range(3)} | {int(table[1, 0])}
    for p in range(8):
        if p not in owned:
            assert torch.isnan(case.k_pool[p]).all()
    assert used


def test_decode_window_only_pool():
    spec = ri.LayerSpec(num_q_heads=4, num_kv_heads=2, head_dim=8, window=6,
                        rel_extent=6, page_size=4, dtype=torch.float32)
    case = ri.make_decode(spec, [3, 17, 8], seed=9, window_only=True)
    table = case.block_table.cpu()
    assert torch.isnan(case.k_pool[0]).all()
    for b, n in enumerate(case.seq_lens):
        k, v = case.logical_kv(b)
        lo = max(0, n - 6)
        first = lo // 4
        for j in range(first):
            assert int(table[b, j]) == 0
        for s in range(first * 4, n):
            page = int(table[b, s // 4])
            assert page != 0
            assert torch.equal(case.k_pool[page, :, s % 4], k[s])
            assert torch.equal(case.v_pool[page, :, s % 4], v[s])
        assert torch.isnan(k[:first * 4]).all()


def test_seeded_inputs_repeat():
    spec = ri.LayerSpec(num_q_heads=2, num_kv_heads=1, head_dim=4, window=0,
                        rel_extent=3, page_size=2, dtype=torch.bfloat16)
    a = ri.make_prefill(spec, [5], seed=3)
    b = ri.make_prefill(spec, [5], seed=3)
    assert torch.equal(a.q, b.q) and torch.equal(a.bias, b.bias)
    assert torch.equal(a.block_table, b.block_table)
    assert torch.equal(a.k_pool.nan_to_num(7.0), b.k_pool.nan_to_num(7.0))


def test_mixed_decode_lengths_in_range():
    lens = ri.mixed_decode_lengths(1004, 256, 1024, 32768)
    assert len(lens) == 256 and min(lens) >= 1024 and max(lens) <= 32768
