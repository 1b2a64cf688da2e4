"""The C ABI on the host: the library loads, exports every symbol that
include/rba.h declares, and rejects bad arguments before enqueuing anything.

No call here reaches a kernel launch: every one fails host validation first
(or only queries sizes), so these tests run without a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

import relative_position_bias_paged_amd as rba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rba.h")
FAKE = 1 << 20          # a non-null, 16-byte aligned stand-in address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rba_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(rba.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = rba.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rba.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (rba_\w+)", out))
    assert set(declared_functions()) <= exported
    # nothing else of ours leaks out
    assert exported == set(declared_functions())


def _layer(hq=32, hkv=8, d=128, page=64, R=1024, W=0, scale=0.088, dtype=rba.RBA_BF16,
           seqs=2, max_pages=256, pages=512, kp=FAKE, vp=FAKE, table=FAKE, lens=FAKE):
    kv = rba.rba_kv_cache(kp, vp, hkv, d, dtype)
    pt = rba.rba_page_table(table, lens, seqs, max_pages, page, pages)
    prm = rba.rba_attn_params(hq, W, R, scale)
    return kv, pt, prm


def _prefill(kv, pt, prm, q=FAKE, cu=FAKE, T=100, max_len=50, bias=FAKE, out=FAKE, lse=None):
    return rba.load().rba_prefill(q, cu, T, max_len, ctypes.byref(kv), ctypes.byref(pt), bias,
                                  ctypes.byref(prm), out, lse, None)


def _prefill_fused(kv, pt, prm, q=FAKE, cu=FAKE, T=100, max_len=50, r=FAKE, w=FAKE, d_rel=32,
                   out=FAKE, lse=None):
    return rba.load().rba_prefill_fused(q, cu, T, max_len, ctypes.byref(kv), ctypes.byref(pt), r,
                                        w, d_rel, ctypes.byref(prm), out, lse, None)


def _decode(kv, pt, prm, q=FAKE, max_len=1000, bias=FAKE, splits=0, ws=None, ws_bytes=0,
            out=FAKE, lse=None):
    return rba.load().rba_decode(q, ctypes.byref(kv), ctypes.byref(pt), max_len, bias,
                                 ctypes.byref(prm), splits, ws, ws_bytes, out, lse, None)


@pytest.mark.parametrize("change,expected", [
    (dict(hq=30, hkv=8), rba.RBA_ERR_INVALID_ARG),        # Hq % Hkv != 0
    (dict(hkv=0), rba.RBA_ERR_INVALID_ARG),
    (dict(page=48), rba.RBA_ERR_INVALID_ARG),             # not a power of two
    (dict(page=0), rba.RBA_ERR_INVALID_ARG),
    (dict(R=0), rba.RBA_ERR_INVALID_ARG),
    (dict(scale=0.0), rba.RBA_ERR_INVALID_ARG),
    (dict(scale=-1.0), rba.RBA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), rba.RBA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), rba.RBA_ERR_INVALID_ARG),
    (dict(dtype=7), rba.RBA_ERR_INVALID_ARG),
    (dict(d=0), rba.RBA_ERR_INVALID_ARG),
    (dict(d=96), rba.RBA_ERR_UNSUPPORTED),
    (dict(d=256), rba.RBA_ERR_UNSUPPORTED),
    (dict(page=8), rba.RBA_ERR_UNSUPPORTED),
    (dict(page=2048), rba.RBA_ERR_UNSUPPORTED),
    (dict(kp=0), rba.RBA_ERR_INVALID_ARG),
    (dict(vp=FAKE + 2), rba.RBA_ERR_INVALID_ARG),         # misaligned pool
    (dict(table=0), rba.RBA_ERR_INVALID_ARG),
    (dict(max_pages=0), rba.RBA_ERR_INVALID_ARG),
    (dict(pages=0), rba.RBA_ERR_INVALID_ARG),
    (dict(seqs=-1), rba.RBA_ERR_INVALID_ARG),
])
def test_layer_validation(change, expected):
    kv, pt, prm = _layer(**change)
    assert _prefill(kv, pt, prm) == expected
    assert _decode(kv, pt, prm) == expected


@pytest.mark.parametrize("kwargs", [
    dict(q=0), dict(cu=0), dict(bias=0), dict(out=0), dict(q=FAKE + 8), dict(bias=FAKE + 2),
    dict(out=FAKE + 4), dict(lse=FAKE + 2), dict(T=-1), dict(max_len=-3),
    dict(max_len=256 * 64 + 1),                          # beyond the page table's reach
])
def test_prefill_argument_errors(kwargs):
    kv, pt, prm = _layer()
    assert _prefill(kv, pt, prm, **kwargs) == rba.RBA_ERR_INVALID_ARG


def test_prefill_key_positions_below_2_pow_29():
    # the page table reaches 2^29 keys: refused before any launch
    kv, pt, prm = _layer(max_pages=1 << 23)
    assert _prefill(kv, pt, prm) == rba.RBA_ERR_UNSUPPORTED
    assert _prefill_fused(kv, pt, prm) == rba.RBA_ERR_UNSUPPORTED


def test_prefill_bias_rows_of_a_wave_within_2_gib():
    # 32 rows of one head span (31 * Hq + 1) * R elements: refused when that
    # reaches 2 GiB, before any launch (the fused variant reads no bias tensor)
    kv, pt, prm = _layer(hq=64, hkv=8, R=1 << 20)
    assert _prefill(kv, pt, prm) == rba.RBA_ERR_UNSUPPORTED


def test_prefill_empty_is_noop():
    kv, pt, prm = _layer()
    assert _prefill(kv, pt, prm, q=0, cu=0, bias=0, out=0, T=0) == rba.RBA_OK
    kv, pt, prm = _layer(seqs=0)
    assert _prefill(kv, pt, prm, q=0, cu=0, bias=0, out=0) == rba.RBA_OK


@pytest.mark.parametrize("kwargs,expected", [
    (dict(q=0), rba.RBA_ERR_INVALID_ARG),
    (dict(cu=0), rba.RBA_ERR_INVALID_ARG),
    (dict(r=0), rba.RBA_ERR_INVALID_ARG),
    (dict(w=0), rba.RBA_ERR_INVALID_ARG),
    (dict(out=0), rba.RBA_ERR_INVALID_ARG),
    (dict(r=FAKE + 8), rba.RBA_ERR_INVALID_ARG),
    (dict(w=FAKE + 2), rba.RBA_ERR_INVALID_ARG),
    (dict(d_rel=0), rba.RBA_ERR_INVALID_ARG),
    (dict(d_rel=-16), rba.RBA_ERR_INVALID_ARG),
    (dict(d_rel=64), rba.RBA_ERR_UNSUPPORTED),
    (dict(d_rel=24), rba.RBA_ERR_UNSUPPORTED),
    (dict(T=-1), rba.RBA_ERR_INVALID_ARG),
    (dict(max_len=256 * 64 + 1), rba.RBA_ERR_INVALID_ARG),
])
def test_prefill_fused_argument_errors(kwargs, expected):
    kv, pt, prm = _layer()
    assert _prefill_fused(kv, pt, prm, **kwargs) == expected


def test_prefill_fused_needs_bf16_pools():
    kv, pt, prm = _layer(dtype=rba.RBA_F32)
    assert _prefill_fused(kv, pt, prm) == rba.RBA_ERR_UNSUPPORTED


def test_prefill_fused_shares_the_layer_checks():
    kv, pt, prm = _layer(hq=30, hkv=8)
    assert _prefill_fused(kv, pt, prm) == rba.RBA_ERR_INVALID_ARG
    kv, pt, prm = _layer(d=96)
    assert _prefill_fused(kv, pt, prm) == rba.RBA_ERR_UNSUPPORTED


def test_prefill_fused_empty_is_noop():
    kv, pt, prm = _layer()
    assert _prefill_fused(kv, pt, prm, T=0, q=0, r=0, w=0, out=0) == rba.RBA_OK


@pytest.mark.parametrize("kwargs", [
    dict(q=0), dict(bias=0), dict(out=0), dict(q=FAKE + 2), dict(max_len=-1), dict(splits=-2),
    dict(max_len=256 * 64 + 1),
])
def test_decode_argument_errors(kwargs):
    kv, pt, prm = _layer()
    assert _decode(kv, pt, prm, **kwargs) == rba.RBA_ERR_INVALID_ARG


def test_decode_needs_seq_lens():
    kv, pt, prm = _layer(lens=0)
    assert _decode(kv, pt, prm) == rba.RBA_ERR_INVALID_ARG


def test_decode_workspace_errors():
    kv, pt, prm = _layer(seqs=32, max_pages=2048, pages=65536)
    lib = rba.load()
    need = lib.rba_decode_workspace_size(ctypes.byref(kv), ctypes.byref(pt), 131072,
                                         ctypes.byref(prm), 16)
    assert need > 0
    assert _decode(kv, pt, prm, max_len=131072, splits=16) == rba.RBA_ERR_WORKSPACE
    assert _decode(kv, pt, prm, max_len=131072, splits=16, ws=FAKE, ws_bytes=need - 1) == \
        rba.RBA_ERR_WORKSPACE
    assert _decode(kv, pt, prm, max_len=131072, splits=16, ws=FAKE + 16, ws_bytes=need) == \
        rba.RBA_ERR_WORKSPACE


def test_decode_split_plan():
    lib = rba.load()

    def plan(max_len, splits, **kw):
        kv, pt, prm = _layer(**kw)
        n = lib.rba_decode_num_splits(ctypes.byref(kv), ctypes.byref(pt), max_len,
                                      ctypes.byref(prm), splits)
        ws = lib.rba_decode_workspace_size(ctypes.byref(kv), ctypes.byref(pt), max_len,
                                           ctypes.byref(prm), splits)
        return n, ws

    # long-context global decode: 16 requested partitions of 128 pages each
    n, ws = plan(131072, 16, seqs=32, max_pages=2048, pages=65536)
    assert n == 16
    rows = 32 * 32
    # partial outputs and LSE, each 256-byte aligned, then the largest-first
    # plan: two int32 per (sequence, partition)
    assert ws == rows * 16 * 128 * 4 + rows * 16 * 4 + 32 * 16 * 8
    # one partition: no workspace
    assert plan(4096, 1, seqs=4)[1] == 0
    # never more partitions than pages
    assert plan(100, 64, seqs=4)[0] == 2
    # local layer: the visible window spans at most 9 pages of 64
    n, _ = plan(32768, 0, seqs=256, hkv=16, W=512, R=512, max_pages=512, pages=70000)
    assert n == 1
    # automatic split of a global layer at batch 256 and 32K context
    n, _ = plan(32768, 0, seqs=256, max_pages=512, pages=70000)
    assert 1 < n <= 256
    # fp32 runs unpartitioned
    assert plan(131072, 16, seqs=32, max_pages=2048, pages=65536, dtype=rba.RBA_F32) == (1, 0)
    # invalid arguments report 0
    assert plan(1000, 0, hq=31) == (0, 0)


# rba_kv_gather shares rba_kv_append's argument checks (the same mapping,
# copied the other way)
COPIES = ["rba_kv_append", "rba_kv_gather"]


def _append(kv, pt, k=FAKE, v=FAKE, cu=FAKE, total=10, fn="rba_kv_append"):
    return getattr(rba.load(), fn)(k, v, cu, total, ctypes.byref(kv), ctypes.byref(pt), None)


@pytest.mark.parametrize("kwargs,expected", [
    (dict(k=None), rba.RBA_ERR_INVALID_ARG),
    (dict(v=None), rba.RBA_ERR_INVALID_ARG),
    (dict(cu=None), rba.RBA_ERR_INVALID_ARG),
    (dict(k=FAKE + 4), rba.RBA_ERR_INVALID_ARG),
    (dict(total=-1), rba.RBA_ERR_INVALID_ARG),
])
@pytest.mark.parametrize("fn", COPIES)
def test_append_argument_errors(kwargs, expected, fn):
    kv, pt, _ = _layer()
    assert _append(kv, pt, fn=fn, **kwargs) == expected


@pytest.mark.parametrize("fn", COPIES)
def test_append_layer_errors(fn):
    kv, pt, _ = _layer(lens=None)
    assert _append(kv, pt, fn=fn) == rba.RBA_ERR_INVALID_ARG   # seq_lens is required
    kv, pt, _ = _layer(page=48)
    assert _append(kv, pt, fn=fn) == rba.RBA_ERR_INVALID_ARG   # page size not a power of two
    kv, pt, _ = _layer(d=96)
    assert _append(kv, pt, fn=fn) == rba.RBA_ERR_UNSUPPORTED
    kv, pt, _ = _layer(page=2048)
    assert _append(kv, pt, fn=fn) == rba.RBA_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", COPIES)
def test_append_empty_is_noop(fn):
    kv, pt, _ = _layer()
    assert _append(kv, pt, k=None, v=None, cu=None, total=0, fn=fn) == rba.RBA_OK
    kv, pt, _ = _layer(seqs=0)
    assert _append(kv, pt, k=None, total=5, fn=fn) == rba.RBA_OK


_LAYOUT_C = r"""
#include <stdio.h>
#include "rba.h"
#define F(s, f) printf("%s %s %zu\n", #s, #f, offsetof(s, f))
int main(void) {
  printf("rba_page_table * %zu\n", sizeof(rba_page_table));
  F(rba_page_table, block_table); F(rba_page_table, seq_lens); F(rba_page_table, num_seqs);
  F(rba_page_table, max_pages_per_seq); F(rba_page_table, page_size); F(rba_page_table, num_pages);
  printf("rba_kv_cache * %zu\n", sizeof(rba_kv_cache));
  F(rba_kv_cache, k_pool); F(rba_kv_cache, v_pool); F(rba_kv_cache, num_kv_heads);
  F(rba_kv_cache, head_dim); F(rba_kv_cache, dtype);
  printf("rba_attn_params * %zu\n", sizeof(rba_attn_params));
  F(rba_attn_params, num_q_heads); F(rba_attn_params, window); F(rba_attn_params, rel_extent);
  F(rba_attn_params, sm_scale);
  printf("enum * %zu\n", sizeof(rba_status) + 0 * sizeof(rba_dtype));
  return 0;
}
"""


def test_struct_layouts_match_the_header(tmp_path):
    """The binding's ctypes structs against the header compiled as C (gcc):
    every size and field offset agrees, so a C caller and the binding pass
    the same bytes."""
    src = tmp_path / "layout.c"
    src.write_text(_LAYOUT_C)
    exe = tmp_path / "layout"
    inc = os.path.join(ROOT, "include")
    res = subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", inc,
                          "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    seen = 0
    for line in filter(None, out):
        name, field, value = line.split()
        if name == "enum":
            assert int(value) == ctypes.sizeof(ctypes.c_int)
            continue
        cls = getattr(rba, name)
        if field == "*":
            assert ctypes.sizeof(cls) == int(value), name
        else:
            assert getattr(cls, field).offset == int(value), (name, field)
        seen += 1
    assert seen == 18


def test_c_abi_check_program_builds(tmp_path):
    """The plain-C check program of the GPU tests compiles and links against
    the header, librba.so, the oracle's library and the HIP runtime."""
    import sys
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import c_abi_build
    out = c_abi_build.build(str(tmp_path / "c_abi_check"))
    assert os.path.getsize(out) > 0


def test_check_page_table_argument_errors():
    lib = rba.load()
    _, pt, _ = _layer()

    def call(p=pt, window=0, max_new=1, out=FAKE):
        return lib.rba_check_page_table(ctypes.byref(p) if p is not None else None, window, max_new,
                                        out, None)

    assert call(p=None) == rba.RBA_ERR_INVALID_ARG
    assert call(out=None) == rba.RBA_ERR_INVALID_ARG
    assert call(max_new=0) == rba.RBA_ERR_INVALID_ARG
    _, bad_page, _ = _layer(page=48)
    assert call(p=bad_page) == rba.RBA_ERR_INVALID_ARG
    _, no_lens, _ = _layer(lens=None)
    assert call(p=no_lens) == rba.RBA_ERR_INVALID_ARG


def test_window_ring_pages():
    # window 512, 64-token pages, one new token: 512 positions span 9 pages
    assert rba.window_ring_pages(512, 64, 1) == 9
    # a 512-token chunk over a 512 window: 1023 positions, up to 17 pages
    assert rba.window_ring_pages(512, 64, 512) == 17
    assert rba.window_ring_pages(100, 16, 1) == 8
    assert rba.window_ring_pages(0, 64, 1) == 0          # full causal: no ring
    assert rba.window_ring_pages(512, 48, 1) == 0        # not a power of two
    assert rba.window_ring_pages(512, 64, 0) == 0
    # brute force: every start position of a span lies in at most that many pages
    for W, P, m in ((512, 64, 1), (100, 16, 7), (64, 64, 64), (33, 32, 1)):
        span = W + m - 1
        worst = max((s + span - 1) // P - s // P + 1 for s in range(4 * P))
        assert rba.window_ring_pages(W, P, m) >= worst
        assert rba.window_ring_pages(W, P, m) <= worst + 1


def test_ring_block_table_is_positional():
    import torch
    rings = torch.tensor([[7, 3, 9], [0, 1, 2]], dtype=torch.int32)
    t = rba.ring_block_table(rings, 8)
    assert t.tolist() == [[7, 3, 9, 7, 3, 9, 7, 3], [0, 1, 2, 0, 1, 2, 0, 1]]
    # against the definition, on a larger random ring set
    g = torch.Generator().manual_seed(1)
    rings = torch.randperm(5 * 9, generator=g).to(torch.int32).view(5, 9)
    t = rba.ring_block_table(rings, 40)
    for b in range(5):
        for j in range(40):
            assert int(t[b, j]) == int(rings[b, j % 9])


def test_ring_block_table_errors():
    lib = rba.load()
    buf = (ctypes.c_int32 * 8)()
    assert lib.rba_ring_block_table(buf, 2, 0, 4, buf) == rba.RBA_ERR_INVALID_ARG
    assert lib.rba_ring_block_table(buf, -1, 3, 4, buf) == rba.RBA_ERR_INVALID_ARG
    assert lib.rba_ring_block_table(None, 2, 3, 4, buf) == rba.RBA_ERR_INVALID_ARG
    assert lib.rba_ring_block_table(buf, 2, 3, 4, None) == rba.RBA_ERR_INVALID_ARG
    assert lib.rba_ring_block_table(None, 0, 3, 4, None) == rba.RBA_OK


def _decode_noalloc(kv, pt, prm, q=FAKE, max_len=1000, bias=FAKE, splits=0, out=FAKE, lse=None):
    return rba.load().rba_decode_noalloc(q, ctypes.byref(kv), ctypes.byref(pt), max_len, bias,
                                         ctypes.byref(prm), splits, out, lse, None)


def test_decode_noalloc_host_checks():
    """The allocation-free decode shares rba_decode's checks and rejects a call
    whose workspace would not fit the static per-GPU array, before any
    device work (so these run without a GPU)."""
    kv, pt, prm = _layer(hq=30, hkv=8)
    assert _decode_noalloc(kv, pt, prm) == rba.RBA_ERR_INVALID_ARG
    kv, pt, prm = _layer()
    assert _decode_noalloc(kv, pt, prm, q=0) == rba.RBA_ERR_INVALID_ARG
    kv, pt, prm = _layer(lens=0)
    assert _decode_noalloc(kv, pt, prm) == rba.RBA_ERR_INVALID_ARG
    # 1024 sequences x 32 heads x 64 partitions of fp32 partials: 1 GiB
    kv, pt, prm = _layer(seqs=1024, max_pages=2048, pages=1 << 20)
    lib = rba.load()
    need = lib.rba_decode_workspace_size(ctypes.byref(kv), ctypes.byref(pt), 131072,
                                         ctypes.byref(prm), 64)
    assert need > rba.DECODE_SCRATCH_BYTES
    assert _decode_noalloc(kv, pt, prm, max_len=131072, splits=64) == rba.RBA_ERR_WORKSPACE
    kv, pt, prm = _layer(seqs=0)
    assert _decode_noalloc(kv, pt, prm, q=0, bias=0, out=0) == rba.RBA_OK


def test_scratch_limit_matches_header():
    text = open(HEADER).read()
    import re as _re
    m = _re.search(r"#define RBA_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == rba.DECODE_SCRATCH_BYTES


def _decode_multi(kv, pt, prm, q=FAKE, q_len=4, max_len=1000, bias=FAKE, splits=0, ws=None,
                  ws_bytes=0, out=FAKE, lse=None):
    return rba.load().rba_decode_multi(q, q_len, ctypes.byref(kv), ctypes.byref(pt), max_len,
                                       bias, ctypes.byref(prm), splits, ws, ws_bytes, out, lse,
                                       None)


@pytest.mark.parametrize("kwargs,expected", [
    (dict(q=0), rba.RBA_ERR_INVALID_ARG),
    (dict(bias=0), rba.RBA_ERR_INVALID_ARG),
    (dict(out=0), rba.RBA_ERR_INVALID_ARG),
    (dict(q_len=0), rba.RBA_ERR_INVALID_ARG),
    (dict(q_len=-2), rba.RBA_ERR_INVALID_ARG),
    (dict(q_len=17), rba.RBA_ERR_UNSUPPORTED),
    (dict(max_len=3), rba.RBA_ERR_INVALID_ARG),          # shorter than the new tokens
    (dict(max_len=256 * 64 + 1), rba.RBA_ERR_INVALID_ARG),
    (dict(splits=-1), rba.RBA_ERR_INVALID_ARG),
])
def test_decode_multi_argument_errors(kwargs, expected):
    kv, pt, prm = _layer()
    assert _decode_multi(kv, pt, prm, **kwargs) == expected


def test_decode_multi_layer_checks_and_dtype():
    kv, pt, prm = _layer(hq=30, hkv=8)
    assert _decode_multi(kv, pt, prm) == rba.RBA_ERR_INVALID_ARG
    kv, pt, prm = _layer(dtype=rba.RBA_F32)
    assert _decode_multi(kv, pt, prm) == rba.RBA_ERR_UNSUPPORTED   # fp32: prefill over history
    kv, pt, prm = _layer(seqs=0)
    assert _decode_multi(kv, pt, prm, q=0, bias=0, out=0) == rba.RBA_OK


def test_decode_multi_plan_and_workspace():
    lib = rba.load()

    def plan(q_len, max_len, splits, **kw):
        kv, pt, prm = _layer(**kw)
        n = lib.rba_decode_multi_num_splits(q_len, ctypes.byref(kv), ctypes.byref(pt), max_len,
                                            ctypes.byref(prm), splits)
        ws = lib.rba_decode_multi_workspace_size(q_len, ctypes.byref(kv), ctypes.byref(pt),
                                                 max_len, ctypes.byref(prm), splits)
        return n, ws

    # 32 sequences of 131072 keys, 4 new tokens each, 8 partitions: partials
    # and LSE for 32*4*32 rows, then the (sequence, partition) plan
    n, ws = plan(4, 131072, 8, seqs=32, max_pages=2048, pages=65536)
    rows = 32 * 4 * 32
    assert n == 8
    assert ws == rows * 8 * 128 * 4 + rows * 8 * 4 + 32 * 8 * 8
    # q_len 1 plans like rba_decode
    kv, pt, prm = _layer(seqs=32, max_pages=2048, pages=65536)
    one = lib.rba_decode_workspace_size(ctypes.byref(kv), ctypes.byref(pt), 131072,
                                        ctypes.byref(prm), 16)
    assert plan(1, 131072, 16, seqs=32, max_pages=2048, pages=65536) == (16, one)
    # a local layer's queries see window + q_len - 1 keys: at most 10 pages of 64
    n, _ = plan(8, 32768, 64, seqs=4, hkv=16, W=512, R=512, max_pages=512, pages=3000)
    assert n == 10
    assert plan(4, 1000, 0, hq=31) == (0, 0)
    assert plan(17, 1000, 0) == (0, 0)


def test_status_strings():
    for code, name in [(0, "RBA_OK"), (1, "RBA_ERR_INVALID_ARG"), (2, "RBA_ERR_UNSUPPORTED"),
                       (3, "RBA_ERR_WORKSPACE"), (4, "RBA_ERR_HIP")]:
        assert rba.status_string(code) == name
    assert rba.status_string(99) == "RBA_UNKNOWN_STATUS"


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rba.prefill(q, torch.zeros(2, dtype=torch.int32), 4,
                    torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16),
                    torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16),
                    torch.zeros((1, 1), dtype=torch.int32), None,
                    torch.zeros((4, 2, 8), dtype=torch.bfloat16), window=0, sm_scale=0.1)
