"""rba_decode_noalloc (the decode for callers that cannot allocate, its
workspace in the library's static per-GPU array) against rba_decode with a
caller workspace: the same kernels and partition plan, so the outputs and
LSE must be bit-identical, and both within the bf16 bar of the oracle.
Two calls in a row, the second on a smaller input, so the second runs over
the first call's leftovers in the shared array."""
import numpy as np
import pytest
import torch

import rba_inputs as ri
import relative_position_bias_paged_amd as rba
from gpu_helpers import LSE_MAX_ABS, assert_parity, device, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu


def _noalloc(case, splits):
    sp = case.spec
    out = torch.empty_like(case.q)
    lse = torch.empty(case.q.shape[:2], dtype=torch.float32, device=case.q.device)
    rba.decode_noalloc(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens_dev,
                       case.max_seq_len, case.bias, window=sp.window, sm_scale=sp.scale(),
                       num_splits=splits, out=out, lse=lse)
    return out, lse


def test_noalloc_decode_matches_decode_twice():
    dev = device()
    glob = ri.LayerSpec(num_q_heads=32, num_kv_heads=8, head_dim=128, window=0, rel_extent=1024,
                        page_size=64)
    runs = [
        # a large call: 48 sequences up to 20000 keys, 16 partitions
        (ri.make_decode(glob, [20000 - 397 * i for i in range(48)], seed=501, device=dev), 16),
        # then a smaller one, automatic partitions, lengths around page edges
        (ri.make_decode(glob, [1, 63, 64, 65, 129, 3000], seed=502, device=dev), 0),
    ]
    for i, (case, splits) in enumerate(runs):
        need = rba.decode_workspace_size(case.q, case.k_pool, case.v_pool, case.block_table,
                                         case.seq_lens_dev, case.max_seq_len, case.bias,
                                         window=0, sm_scale=glob.scale(), num_splits=splits)
        assert 0 < need <= rba.DECODE_SCRATCH_BYTES
        out, lse = _noalloc(case, splits)
        ref_out, ref_lse = gpu_decode(case, num_splits=splits, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"call {i}"
        assert torch.equal(lse, ref_lse), f"call {i}"
        seqs = list(range(0, len(case.seq_lens), 7))
        ref, ref_l = oracle_decode(case, seqs=seqs, want_lse=True)
        idx = torch.tensor(seqs, device=dev)
        assert_parity(out[idx], ref, torch.bfloat16, f"noalloc call {i}")
        assert np.max(np.abs(lse[idx].cpu().double().numpy() - ref_l)) <= LSE_MAX_ABS


def test_noalloc_local_layer_window_pool():
    """A local layer on a window-only pool (one partition, no workspace) and
    then a global layer with partitions: both through the same entry point."""
    dev = device()
    loc = ri.LayerSpec(num_q_heads=32, num_kv_heads=16, head_dim=128, window=512,
                       rel_extent=512, page_size=64)
    case = ri.make_decode(loc, [5000, 700, 513, 1], seed=503, device=dev, window_only=True)
    out, _ = _noalloc(case, 0)
    ref = gpu_decode(case)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert_parity(out, oracle_decode(case), torch.bfloat16, "noalloc local")
