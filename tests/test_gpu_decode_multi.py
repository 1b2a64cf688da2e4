"""GPU parity of rba_decode_multi (q_len new tokens per sequence over a long
cache, page-aligned partitions with an LSE merge) against the oracle's
prefill over a history, which computes the same rows from their definition.

Cases: q_len 2..16 (so 16, 8, 4, 2 and 1 query heads per wave, and partial
head groups when G is not a multiple of 16 / q_len), GQA 1..8, local layers
on window-only pools whose earlier table entries all point at one NaN page,
the clamped-bucket region, sequences no longer than q_len, lengths on both
sides of page borders, page sizes 16..256, head_dim 64, and partition counts
1, 2, 16 and automatic.
"""
import numpy as np
import pytest
import torch

import oracle
import rba_inputs as ri
import relative_position_bias_paged_amd as rba
from gpu_helpers import LSE_MAX_ABS, assert_parity, device, errors, gpu_decode

pytestmark = pytest.mark.gpu


def spec(hq, hkv, d, W, R, P):
    return ri.LayerSpec(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, window=W, rel_extent=R,
                        page_size=P)


EDGE = [4, 5, 15, 16, 17, 63, 64, 65, 127, 129, 1000, 2049]

CASES = [
    # id, spec, lens, q_len, window-only pool
    ("global-gqa4-q4", spec(32, 8, 128, 0, 1024, 64), EDGE, 4, False),
    ("global-gqa4-q2", spec(32, 8, 128, 0, 1024, 64), [2, 3, 64, 65, 3000], 2, False),
    ("global-gqa4-q8", spec(32, 8, 128, 0, 1024, 64), [8, 9, 64, 200, 1500], 8, False),
    ("global-q16-mha", spec(4, 4, 128, 0, 256, 64), [16, 17, 300], 16, False),
    ("global-r64-clamp-q3", spec(8, 2, 128, 0, 64, 32), EDGE, 3, False),
    ("gqa8-q4-two-groups", spec(16, 2, 128, 0, 300, 64), [4, 700, 64], 4, False),
    ("gqa3-q5-partial-group", spec(6, 2, 128, 0, 100, 16), [5, 90, 333], 5, False),
    ("local-w512-q4-windowpool", spec(32, 16, 128, 512, 512, 64), EDGE + [5000], 4, True),
    ("local-w100-p16-q7", spec(8, 4, 128, 100, 100, 16), EDGE + [777], 7, True),
    ("local-w300-r64-q4", spec(8, 2, 128, 300, 64, 64), [4, 400, 1200], 4, False),
    ("d64-q4", spec(8, 2, 64, 0, 128, 64), [4, 100, 777], 4, False),
    ("p256-q2", spec(4, 1, 128, 0, 512, 256), [1000, 255, 257], 2, False),
]


def oracle_multi(case, seqs=None):
    """Oracle rows [len(seqs) * q_len, Hq, D] and lse, from the prefill over
    each sequence's history (the q_len tokens are its last positions)."""
    sp = case.spec
    L = case.q_len
    seqs = range(len(case.seq_lens)) if seqs is None else seqs
    outs, lses = [], []
    for b in seqs:
        k, v = case.logical_kv(b)
        n = case.seq_lens[b]
        o, l = oracle.prefill_history(case.q[b * L:(b + 1) * L], k, v,
                                      case.bias[b * L:(b + 1) * L], [0, L], [0, n],
                                      window=sp.window, rel_extent=sp.rel_extent,
                                      sm_scale=sp.scale(), want_lse=True)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


def gpu_multi(case, splits=0, want_lse=True, **kw):
    sp = case.spec
    lse = torch.empty(case.q.shape[:2], dtype=torch.float32, device=case.q.device)
    out = rba.decode_multi(case.q, case.q_len, case.k_pool, case.v_pool, case.block_table,
                           case.seq_lens_dev, case.max_seq_len, case.bias, window=sp.window,
                           sm_scale=sp.scale(), num_splits=splits, lse=lse, **kw)
    return (out, lse) if want_lse else out


@pytest.mark.parametrize("splits", [1, 2, 16, 0])
@pytest.mark.parametrize("cid,sp,lens,q_len,wonly", CASES, ids=[c[0] for c in CASES])
def test_decode_multi_parity(cid, sp, lens, q_len, wonly, splits):
    dev = device()
    lens = [n for n in lens if n >= q_len]      # a sequence holds its new tokens' keys
    case = ri.make_decode(sp, lens, seed=len(cid) * 17 + splits, device=dev, window_only=wonly,
                          q_len=q_len)
    if wonly:
        assert torch.isnan(case.k_pool[0]).all()
    out, lse = gpu_multi(case, splits)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_multi(case)
    assert_parity(out, ref, torch.bfloat16, f"{cid} splits={splits}")
    assert np.max(np.abs(lse.cpu().double().numpy() - ref_lse)) <= LSE_MAX_ABS


@pytest.mark.parametrize("W,R", [(512, 512), (0, 1024)])
def test_decode_multi_equals_prefill_over_history(W, R):
    """The same rows through rba_prefill over the history (both on the GPU)."""
    dev = device()
    sp = spec(8, 2, 128, W, R, 64)
    lens, L = [4, 65, 1000, 3000], 4
    case = ri.make_decode(sp, lens, seed=71, device=dev, q_len=L)
    o_multi = gpu_multi(case, want_lse=False)
    cu = torch.arange(0, L * len(lens) + 1, L, dtype=torch.int32, device=dev)
    o_pre = rba.prefill(case.q, cu, L, case.k_pool, case.v_pool, case.block_table,
                        case.seq_lens_dev, case.bias, window=W, sm_scale=sp.scale())
    torch.cuda.synchronize()
    max_abs, mean_rel = errors(o_multi, o_pre.double().cpu().numpy())
    assert max_abs <= 2e-2 and mean_rel <= 5e-3


def test_q_len_one_is_decode():
    """q_len 1 is rba_decode: bit-identical output and LSE."""
    dev = device()
    sp = spec(32, 8, 128, 0, 1024, 64)
    case = ri.make_decode(sp, [1, 64, 65, 5000], seed=73, device=dev)
    o1, l1 = gpu_multi(case, 0)
    o2, l2 = gpu_decode(case, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_page_table_bit_exact():
    """Identity and shuffled page tables over the same logical K/V give the
    bitwise-identical output."""
    dev = device()
    sp = spec(32, 8, 128, 0, 1024, 64)
    lens = [700, 3000, 4]
    a = ri.make_decode(sp, lens, seed=75, device=dev, q_len=4, shuffle=False)
    b = ri.make_decode(sp, lens, seed=75, device=dev, q_len=4, shuffle=True)
    assert not torch.equal(a.block_table, b.block_table)
    oa = gpu_multi(a, 8, want_lse=False)
    ob = gpu_multi(b, 8, want_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_masked_slots_cannot_leak():
    """NaN in every pool slot no query sees (the tails of the sequences' last
    pages) leaves the output bit-identical to a twin holding zeros there."""
    dev = device()
    sp = spec(8, 2, 128, 0, 256, 64)
    case = ri.make_decode(sp, [100, 650, 4], seed=77, device=dev, q_len=4)
    o_nan = gpu_multi(case, 2, want_lse=False)
    z = ri.DecodeCase(**{**case.__dict__, "k_pool": torch.nan_to_num(case.k_pool, nan=0.0),
                         "v_pool": torch.nan_to_num(case.v_pool, nan=0.0)})
    o_zero = gpu_multi(z, 2, want_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o_nan.view(torch.int16), o_zero.view(torch.int16))


def test_decode_multi_errors():
    dev = device()
    sp = spec(8, 2, 128, 0, 256, 64)
    case = ri.make_decode(sp, [100], seed=79, device=dev, q_len=17)
    with pytest.raises(rba.RbaError):
        gpu_multi(case)
    f32 = ri.LayerSpec(num_q_heads=4, num_kv_heads=2, head_dim=64, window=0, rel_extent=32,
                       page_size=16, dtype=torch.float32)
    case = ri.make_decode(f32, [40], seed=81, device=dev, q_len=2)
    with pytest.raises(rba.RbaError):
        gpu_multi(case)


def test_mtp_verify_workload_sampled():
    """The mtp-verify benchmark workload at full size, in the launch the bench
    times: every head of every token of three sampled sequences."""
    dev = device()
    case = ri.build_workload("mtp-verify-32x131072-q4", dev)["verify"]
    out = gpu_multi(case, ri.WORKLOADS["mtp-verify-32x131072-q4"]["num_splits"], want_lse=False)
    torch.cuda.synchronize()
    seqs = [0, 13, 31]
    ref, _ = oracle_multi(case, seqs)
    L = case.q_len
    sel = torch.cat([out[b * L:(b + 1) * L] for b in seqs])
    assert_parity(sel, ref, torch.bfloat16, "mtp-verify")
