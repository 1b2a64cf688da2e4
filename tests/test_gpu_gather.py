"""GPU tests of rba_kv_gather, the reverse of rba_kv_append, and of the
page-table check rba_check_page_table.

De-paging whole sequences through shuffled page tables returns, byte for
byte, the logical K/V the pools were filled from. This covers page sizes
below, at and above the 64-key tile, and lengths on both sides of page
borders (the positional page table of the TensorRT-LLM PR #17860 page). A
window-only decode pool gives back its last W positions. A gather with the
arguments of an append returns the appended rows. Rows whose position or page
id is out of range are left unwritten. The page-table check counts exactly the
reachable entries that name no pool page, against a plain Python count.
"""
import random

import pytest
import torch

import rba_inputs as ri
import relative_position_bias_paged_amd as rba
from gpu_helpers import device, random_pools

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.contiguous().view(torch.uint8)


def _cu(lens, dev):
    return torch.tensor(ri._cumsum(lens), dtype=torch.int32, device=dev)


@pytest.mark.parametrize("dtype,D,P,Hkv", [(torch.bfloat16, 128, 64, 8), (torch.bfloat16, 64, 16, 2),
                                           (torch.float32, 64, 16, 3), (torch.bfloat16, 128, 256, 1),
                                           (torch.float32, 128, 32, 4)])
def test_gather_depages_whole_sequences(dtype, D, P, Hkv):
    dev = device()
    sp = ri.LayerSpec(num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D, window=0, rel_extent=8,
                      page_size=P, dtype=dtype)
    lens = [1, P - 1, P, P + 1, 2 * P - 1, 2 * P + 1, 700]
    needed = sum(max(1, -(-n // P)) for n in lens)
    case = ri.make_prefill(sp, lens, seed=P + D + Hkv, device=dev, num_pages=needed + 7,
                           shuffle=True)
    k, v = rba.kv_gather(case.cu_seqlens, case.total_tokens, case.k_pool, case.v_pool,
                         case.block_table, case.seq_lens_dev)
    torch.cuda.synchronize()
    assert torch.equal(_bytes(k), _bytes(case.k_log))
    assert torch.equal(_bytes(v), _bytes(case.v_log))


def test_gather_window_only_decode_pool():
    """A local layer's window-only pool (earlier table entries point at one
    NaN page): the last min(n, W) positions of each sequence come back."""
    dev = device()
    W = 512
    sp = ri.LayerSpec(num_q_heads=32, num_kv_heads=16, head_dim=128, window=W, rel_extent=W,
                      page_size=64)
    lens = [5, 511, 512, 513, 3000, 4097]
    case = ri.make_decode(sp, lens, seed=41, device=dev, window_only=True)
    assert torch.isnan(case.k_pool).any()
    last = [min(n, W) for n in lens]
    k, v = rba.kv_gather(_cu(last, dev), sum(last), case.k_pool, case.v_pool, case.block_table,
                         case.seq_lens_dev)
    torch.cuda.synchronize()
    ref_k, ref_v = [], []
    for b, n in enumerate(lens):
        kb, vb = case.logical_kv(b)
        ref_k.append(kb[n - last[b]:])
        ref_v.append(vb[n - last[b]:])
    ref_k, ref_v = torch.cat(ref_k), torch.cat(ref_v)
    assert not torch.isnan(ref_k.float()).any()
    assert torch.equal(_bytes(k.cpu()), _bytes(ref_k))
    assert torch.equal(_bytes(v.cpu()), _bytes(ref_v))


@pytest.mark.parametrize("dtype,D,P,Hkv", [(torch.bfloat16, 128, 16, 3), (torch.float32, 64, 64, 2)])
def test_gather_after_append_returns_the_rows(dtype, D, P, Hkv):
    dev = device()
    before = [0, 17, 64, 100, 31, 5]
    new = [5, 0, 1, 70, 33, 2]
    after = [a + b for a, b in zip(before, new)]
    k_pool, v_pool, table = random_pools(dev, dtype, Hkv, D, P, after, seed=11)
    g = torch.Generator(device="cpu").manual_seed(13)
    k_new = torch.randn((sum(new), Hkv, D), generator=g).to(dtype).to(dev)
    v_new = torch.randn((sum(new), Hkv, D), generator=g).to(dtype).to(dev)
    cu = _cu(new, dev)
    lens = torch.tensor(after, dtype=torch.int32, device=dev)
    rba.kv_append(k_new, v_new, cu, k_pool, v_pool, table, lens)
    k, v = rba.kv_gather(cu, sum(new), k_pool, v_pool, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(_bytes(k), _bytes(k_new))
    assert torch.equal(_bytes(v), _bytes(v_new))


def test_gather_leaves_unreachable_rows_unwritten():
    dev = device()
    dtype, Hkv, D, P = torch.bfloat16, 2, 128, 16
    lens_list = [30, 40, 8]
    k_pool, v_pool, table = random_pools(dev, dtype, Hkv, D, P, lens_list, seed=17)
    # sequence 1: the page of positions 16..31 is outside the pool
    table[1, 1] = k_pool.shape[0] + 5
    # sequence 2: a key count so large that its positions fall past the table
    lens = torch.tensor([30, 40, table.shape[1] * P + 10], dtype=torch.int32, device=dev)
    rows = [30, 40, 8]
    sentinel = 7.0
    k_out = torch.full((sum(rows), Hkv, D), sentinel, dtype=dtype, device=dev)
    v_out = torch.full_like(k_out, sentinel)
    rba.kv_gather(_cu(rows, dev), sum(rows), k_pool, v_pool, table, lens, k_out=k_out, v_out=v_out)
    torch.cuda.synchronize()
    tab = table.cpu()
    for b, n in enumerate(rows):
        for i in range(n):
            r = sum(rows[:b]) + i
            unreachable = (b == 1 and 16 <= i < 32) or b == 2
            if unreachable:
                assert (k_out[r] == sentinel).all() and (v_out[r] == sentinel).all(), (b, i)
            else:
                page = int(tab[b, i // P])
                assert torch.equal(_bytes(k_out[r]), _bytes(k_pool[page, :, i % P])), (b, i)
                assert torch.equal(_bytes(v_out[r]), _bytes(v_pool[page, :, i % P])), (b, i)


def _count_bad(table, lens, num_pages, P, window, max_new):
    """Reachable entries naming no pool page, counted in plain Python."""
    bad = 0
    for b, n in enumerate(lens):
        n = max(n, 0)
        if n == 0:
            continue
        lo = max(0, n - max_new - window + 1) if window > 0 else 0
        for j in range(lo // P, (n - 1) // P + 1):
            if j >= len(table[b]) or not 0 <= table[b][j] < num_pages:
                bad += 1
    return bad


def test_check_page_table_cases():
    dev = device()
    P, num_pages = 16, 40
    table = [[(7 * b + j) % num_pages for j in range(8)] for b in range(5)]
    table[0][2] = -1                  # reachable on a global layer
    table[1][7] = num_pages           # past sequence 1's keys: unreachable
    table[3][0] = num_pages + 9       # before the window of a long sequence
    lens = [40, 100, 8 * P + 20, 8 * P, -3]    # sequence 2 runs past the table
    t = torch.tensor(table, dtype=torch.int32, device=dev)
    n = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = torch.full((1,), 12345, dtype=torch.int32, device=dev)   # no zeroing needed
    for window, max_new in ((0, 1), (40, 1), (40, 8), (1000, 1)):
        got = rba.check_page_table(t, n, num_pages, P, window=window, max_new=max_new, out=out)
        torch.cuda.synchronize()
        ref = _count_bad(table, lens, num_pages, P, window, max_new)
        assert int(got.item()) == ref, (window, max_new, int(got.item()), ref)
    assert _count_bad(table, lens, num_pages, P, 0, 1) == 1 + 2 + 1   # -1, two past the table, window-free
    empty = rba.check_page_table(t[:0], n[:0], num_pages, P)
    torch.cuda.synchronize()
    assert int(empty.item()) == 0


@pytest.mark.parametrize("seed", range(6))
def test_check_page_table_random(seed):
    dev = device()
    rng = random.Random(seed)
    P = rng.choice([16, 64, 256])
    B, max_pages, num_pages = rng.randint(1, 40), rng.randint(1, 70), rng.randint(1, 500)
    table = [[rng.randrange(num_pages) if rng.random() > 0.05 else rng.choice([-1, num_pages, 10 ** 6])
              for _ in range(max_pages)] for _ in range(B)]
    lens = [rng.choice([0, 1, P, P + 1, rng.randint(1, max_pages * P), max_pages * P + 5])
            for _ in range(B)]
    window = rng.choice([0, 0, 1, 17, 512])
    max_new = rng.choice([1, 1, 4, 100])
    got = rba.check_page_table(torch.tensor(table, dtype=torch.int32, device=dev),
                               torch.tensor(lens, dtype=torch.int32, device=dev), num_pages, P,
                               window=window, max_new=max_new)
    torch.cuda.synchronize()
    assert int(got.item()) == _count_bad(table, lens, num_pages, P, window, max_new)
