"""Python binding of librba: paged attention with a learned relative-position
bias on AMD Instinct MI355X (gfx950).

This module only marshals arguments: it checks tensor placement, dtypes and
shapes, turns them into the C structs of ``include/rba.h`` and calls the
library on the current HIP stream.  Every step of the computation runs in the
HIP kernels of ``librba.so``; there is no fallback.  If the library has not
been built (``__graft_entry__.build()`` or ``python -m
relative_position_bias_paged_amd.build``) any call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["prefill", "prefill_fused", "decode", "decode_noalloc", "decode_num_splits",
           "decode_workspace_size", "decode_multi", "decode_multi_num_splits",
           "decode_multi_workspace_size", "kv_append", "kv_gather", "check_page_table", "window_ring_pages", "ring_block_table",
           "status_string", "RbaError", "library_path", "load", "DECODE_SCRATCH_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librba.so")

RBA_OK = 0
RBA_ERR_INVALID_ARG = 1
RBA_ERR_UNSUPPORTED = 2
RBA_ERR_WORKSPACE = 3
RBA_ERR_HIP = 4

RBA_BF16 = 0
RBA_F32 = 1

# every symbol include/rba.h declares
EXPORTED = ("rba_prefill", "rba_prefill_fused", "rba_decode", "rba_decode_noalloc",
            "rba_decode_num_splits", "rba_decode_workspace_size", "rba_decode_multi",
            "rba_decode_multi_num_splits", "rba_decode_multi_workspace_size", "rba_kv_append",
            "rba_kv_gather", "rba_check_page_table", "rba_window_ring_pages", "rba_ring_block_table", "rba_status_string")

# RBA_DECODE_SCRATCH_BYTES of include/rba.h: the workspace limit of rba_decode_noalloc
DECODE_SCRATCH_BYTES = 64 << 20


class rba_page_table(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p),
                ("num_seqs", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32),
                ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class rba_kv_cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p),
                ("v_pool", ctypes.c_void_p),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int)]


class rba_attn_params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32),
                ("window", ctypes.c_int32),
                ("rel_extent", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class RbaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load librba.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    lib.rba_prefill.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                P(rba_kv_cache), P(rba_page_table), ctypes.c_void_p,
                                P(rba_attn_params), ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]
    lib.rba_prefill.restype = ctypes.c_int
    lib.rba_prefill_fused.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_int32, P(rba_kv_cache), P(rba_page_table),
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      P(rba_attn_params), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.rba_prefill_fused.restype = ctypes.c_int
    lib.rba_decode.argtypes = [ctypes.c_void_p, P(rba_kv_cache), P(rba_page_table), ctypes.c_int32,
                               ctypes.c_void_p, P(rba_attn_params), ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p]
    lib.rba_decode.restype = ctypes.c_int
    lib.rba_decode_noalloc.argtypes = [ctypes.c_void_p, P(rba_kv_cache), P(rba_page_table),
                                       ctypes.c_int32, ctypes.c_void_p, P(rba_attn_params),
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.rba_decode_noalloc.restype = ctypes.c_int
    lib.rba_decode_multi.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(rba_kv_cache),
                                     P(rba_page_table), ctypes.c_int32, ctypes.c_void_p,
                                     P(rba_attn_params), ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.rba_decode_multi.restype = ctypes.c_int
    for fn, res in (("rba_decode_multi_num_splits", ctypes.c_int32),
                    ("rba_decode_multi_workspace_size", ctypes.c_size_t)):
        getattr(lib, fn).argtypes = [ctypes.c_int32, P(rba_kv_cache), P(rba_page_table),
                                     ctypes.c_int32, P(rba_attn_params), ctypes.c_int32]
        getattr(lib, fn).restype = res
    lib.rba_ring_block_table.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p]
    lib.rba_ring_block_table.restype = ctypes.c_int
    lib.rba_decode_num_splits.argtypes = [P(rba_kv_cache), P(rba_page_table), ctypes.c_int32,
                                          P(rba_attn_params), ctypes.c_int32]
    lib.rba_decode_num_splits.restype = ctypes.c_int32
    lib.rba_decode_workspace_size.argtypes = [P(rba_kv_cache), P(rba_page_table), ctypes.c_int32,
                                              P(rba_attn_params), ctypes.c_int32]
    lib.rba_decode_workspace_size.restype = ctypes.c_size_t
    lib.rba_kv_append.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                  P(rba_kv_cache), P(rba_page_table), ctypes.c_void_p]
    lib.rba_kv_append.restype = ctypes.c_int
    lib.rba_kv_gather.argtypes = lib.rba_kv_append.argtypes
    lib.rba_kv_gather.restype = ctypes.c_int
    lib.rba_check_page_table.argtypes = [P(rba_page_table), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.rba_check_page_table.restype = ctypes.c_int
    lib.rba_window_ring_pages.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.rba_window_ring_pages.restype = ctypes.c_int32
    lib.rba_status_string.argtypes = [ctypes.c_int]
    lib.rba_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().rba_status_string(int(status)).decode()


# --------------------------------------------------------------------------
# marshalling helpers

_DTYPES = {torch.bfloat16: RBA_BF16, torch.float32: RBA_F32}


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _structs(k_pool, v_pool, block_table, seq_lens, num_q_heads, window, rel_extent, sm_scale):
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool must both be [num_pages, Hkv, page_size, head_dim]")
    if k_pool.dtype not in _DTYPES or v_pool.dtype != k_pool.dtype:
        raise TypeError("k_pool / v_pool must be bf16 or fp32 and match")
    num_pages, hkv, page, hd = k_pool.shape
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, max_pages_per_seq]")
    kv = rba_kv_cache(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), hkv, hd, _DTYPES[k_pool.dtype])
    pt = rba_page_table(_dev(block_table, "block_table", torch.int32),
                        _dev(seq_lens, "seq_lens", torch.int32) if seq_lens is not None else None,
                        block_table.shape[0], block_table.shape[1], page, num_pages)
    prm = rba_attn_params(int(num_q_heads), int(window), int(rel_extent), float(sm_scale))
    return kv, pt, prm


def _check(status: int, where: str):
    if status != RBA_OK:
        raise RbaError(status, where)


# --------------------------------------------------------------------------
# entry points (same names as the C ABI, without the rba_ prefix)

def prefill(q: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
            k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
            seq_lens: Optional[torch.Tensor], bias: torch.Tensor, *, window: int,
            sm_scale: float, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rba_prefill: q [T,Hq,D], bias [T,Hq,R], pools [pages,Hkv,P,D]; returns out [T,Hq,D]."""
    lib = load()
    if q.dim() != 3 or bias.dim() != 3 or bias.shape[:2] != q.shape[:2]:
        raise ValueError("q must be [T,Hq,D] and bias [T,Hq,R]")
    T, hq, hd = q.shape
    kv, pt, prm = _structs(k_pool, v_pool, block_table, seq_lens, hq, window, bias.shape[2], sm_scale)
    if q.dtype != k_pool.dtype or bias.dtype != k_pool.dtype:
        raise TypeError("q, bias and the pools must share one dtype")
    if hd != k_pool.shape[3]:
        raise ValueError("head_dim of q and pools differ")
    if cu_seqlens.numel() != block_table.shape[0] + 1:
        raise ValueError("cu_seqlens must have num_seqs + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lse_ptr = None
    if lse is not None:
        if lse.shape != (T, hq):
            raise ValueError("lse must be [T, Hq]")
        lse_ptr = _dev(lse, "lse", torch.float32)
    st = lib.rba_prefill(_dev(q, "q"), _dev(cu_seqlens, "cu_seqlens", torch.int32), T,
                         int(max_seqlen), ctypes.byref(kv), ctypes.byref(pt),
                         _dev(bias, "bias"), ctypes.byref(prm), _dev(out, "out"), lse_ptr,
                         _stream(stream))
    _check(st, "rba_prefill")
    return out


def prefill_fused(q: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                  k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                  seq_lens: Optional[torch.Tensor], rel_r: torch.Tensor, w_rel_t: torch.Tensor,
                  *, window: int, sm_scale: float, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rba_prefill_fused: the bias formed in the kernel from rel_r [T,Hq,d_rel] and
    w_rel_t [R,d_rel] (W transposed); returns out [T,Hq,D]."""
    lib = load()
    if q.dim() != 3 or rel_r.dim() != 3 or rel_r.shape[:2] != q.shape[:2]:
        raise ValueError("q must be [T,Hq,D] and rel_r [T,Hq,d_rel]")
    if w_rel_t.dim() != 2 or w_rel_t.shape[1] != rel_r.shape[2]:
        raise ValueError("w_rel_t must be [R, d_rel] with the d_rel of rel_r")
    T, hq, hd = q.shape
    R, d_rel = w_rel_t.shape
    kv, pt, prm = _structs(k_pool, v_pool, block_table, seq_lens, hq, window, R, sm_scale)
    for name, t in (("q", q), ("rel_r", rel_r), ("w_rel_t", w_rel_t)):
        if t.dtype != k_pool.dtype:
            raise TypeError(f"{name} and the pools must share one dtype")
    if hd != k_pool.shape[3]:
        raise ValueError("head_dim of q and pools differ")
    if cu_seqlens.numel() != block_table.shape[0] + 1:
        raise ValueError("cu_seqlens must have num_seqs + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lse_ptr = None
    if lse is not None:
        if lse.shape != (T, hq):
            raise ValueError("lse must be [T, Hq]")
        lse_ptr = _dev(lse, "lse", torch.float32)
    st = lib.rba_prefill_fused(_dev(q, "q"), _dev(cu_seqlens, "cu_seqlens", torch.int32), T,
                               int(max_seqlen), ctypes.byref(kv), ctypes.byref(pt),
                               _dev(rel_r, "rel_r"), _dev(w_rel_t, "w_rel_t"), int(d_rel),
                               ctypes.byref(prm), _dev(out, "out"), lse_ptr, _stream(stream))
    _check(st, "rba_prefill_fused")
    return out


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, cu_new: torch.Tensor,
              k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
              seq_lens: torch.Tensor, *, stream=None) -> None:
    """rba_kv_append: k_new/v_new [total_new,Hkv,D] into the pools; seq_lens
    are the key counts after the append (the new tokens are the last ones)."""
    lib = load()
    if k_new.dim() != 3 or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must both be [total_new, Hkv, head_dim]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise TypeError("new keys/values and the pools must share one dtype")
    if k_new.shape[1:] != (k_pool.shape[1], k_pool.shape[3]):
        raise ValueError("k_new heads/head_dim differ from the pool")
    if cu_new.numel() != block_table.shape[0] + 1:
        raise ValueError("cu_new must have num_seqs + 1 entries")
    if seq_lens is None:
        raise ValueError("seq_lens is required")
    kv, pt, _ = _structs(k_pool, v_pool, block_table, seq_lens, k_pool.shape[1], 0, 1, 1.0)
    st = lib.rba_kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                           _dev(cu_new, "cu_new", torch.int32), int(k_new.shape[0]),
                           ctypes.byref(kv), ctypes.byref(pt), _stream(stream))
    _check(st, "rba_kv_append")


def kv_gather(cu_rows: torch.Tensor, total_rows: int, k_pool: torch.Tensor, v_pool: torch.Tensor,
              block_table: torch.Tensor, seq_lens: torch.Tensor, *, k_out=None, v_out=None,
              stream=None):
    """rba_kv_gather: the K/V rows of positions n_b - L_b .. n_b - 1 of each
    sequence (L_b rows per cu_rows), read out of the pool pages into
    [total_rows, Hkv, D] tensors, which are returned (allocated unless
    given).  cu_rows = prefix sums of seq_lens de-pages every sequence."""
    lib = load()
    if cu_rows.numel() != block_table.shape[0] + 1:
        raise ValueError("cu_rows must have num_seqs + 1 entries")
    if seq_lens is None:
        raise ValueError("seq_lens is required")
    shape = (int(total_rows), k_pool.shape[1], k_pool.shape[3])
    if k_out is None:
        k_out = torch.empty(shape, dtype=k_pool.dtype, device=k_pool.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=v_pool.dtype, device=v_pool.device)
    if tuple(k_out.shape) != shape or tuple(v_out.shape) != shape:
        raise ValueError(f"k_out and v_out must both be {list(shape)}")
    if k_out.dtype != k_pool.dtype or v_out.dtype != k_pool.dtype:
        raise TypeError("outputs and the pools must share one dtype")
    kv, pt, _ = _structs(k_pool, v_pool, block_table, seq_lens, k_pool.shape[1], 0, 1, 1.0)
    st = lib.rba_kv_gather(_dev(k_out, "k_out"), _dev(v_out, "v_out"),
                           _dev(cu_rows, "cu_rows", torch.int32), int(total_rows),
                           ctypes.byref(kv), ctypes.byref(pt), _stream(stream))
    _check(st, "rba_kv_gather")
    return k_out, v_out


def check_page_table(block_table: torch.Tensor, seq_lens: torch.Tensor, num_pages: int,
                     page_size: int, *, window: int = 0, max_new: int = 1, out=None,
                     stream=None) -> torch.Tensor:
    """rba_check_page_table: the number of table entries a call with up to
    max_new new tokens per sequence could reach that do not name a pool page,
    as a device int32 tensor of one element (``out`` if given)."""
    lib = load()
    if block_table.dim() != 2 or seq_lens is None or seq_lens.numel() != block_table.shape[0]:
        raise ValueError("block_table must be [num_seqs, max_pages] and seq_lens [num_seqs]")
    if out is None:
        out = torch.empty((1,), dtype=torch.int32, device=block_table.device)
    pt = rba_page_table(_dev(block_table, "block_table", torch.int32),
                        _dev(seq_lens, "seq_lens", torch.int32), block_table.shape[0],
                        block_table.shape[1], int(page_size), int(num_pages))
    st = lib.rba_check_page_table(ctypes.byref(pt), int(window), int(max_new),
                                  _dev(out, "out", torch.int32), _stream(stream))
    _check(st, "rba_check_page_table")
    return out


def window_ring_pages(window: int, page_size: int, max_new: int = 1) -> int:
    """rba_window_ring_pages: pages per sequence of a window-only pool."""
    return int(load().rba_window_ring_pages(int(window), int(page_size), int(max_new)))


def ring_block_table(rings: torch.Tensor, max_pages_per_seq: int) -> torch.Tensor:
    """rba_ring_block_table: the positional block table over per-sequence
    page rings, entry j of sequence b = rings[b][j % ring_pages].  rings:
    int32 [num_seqs, ring_pages] (any device; the C helper runs on a host
    copy); returns int32 [num_seqs, max_pages_per_seq] on the same device."""
    if rings.dim() != 2 or rings.dtype != torch.int32:
        raise ValueError("rings must be int32 [num_seqs, ring_pages]")
    host = rings.detach().to("cpu").contiguous()
    table = torch.empty((host.shape[0], int(max_pages_per_seq)), dtype=torch.int32)
    st = load().rba_ring_block_table(host.data_ptr(), host.shape[0], host.shape[1],
                                     int(max_pages_per_seq), table.data_ptr())
    _check(st, "rba_ring_block_table")
    return table.to(rings.device)


def _decode_structs(q, k_pool, v_pool, block_table, seq_lens, bias, window, sm_scale):
    if q.dim() != 3 or bias.dim() != 3 or bias.shape[:2] != q.shape[:2]:
        raise ValueError("q must be [B,Hq,D] and bias [B,Hq,R]")
    return _structs(k_pool, v_pool, block_table, seq_lens, q.shape[1], window,
                    bias.shape[2], sm_scale)


def decode_num_splits(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, bias, *,
                      window: int, sm_scale: float, num_splits: int = 0) -> int:
    lib = load()
    kv, pt, prm = _decode_structs(q, k_pool, v_pool, block_table, seq_lens, bias, window, sm_scale)
    return int(lib.rba_decode_num_splits(ctypes.byref(kv), ctypes.byref(pt), int(max_seq_len),
                                         ctypes.byref(prm), int(num_splits)))


def decode_workspace_size(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, bias, *,
                          window: int, sm_scale: float, num_splits: int = 0) -> int:
    lib = load()
    kv, pt, prm = _decode_structs(q, k_pool, v_pool, block_table, seq_lens, bias, window, sm_scale)
    return int(lib.rba_decode_workspace_size(ctypes.byref(kv), ctypes.byref(pt), int(max_seq_len),
                                             ctypes.byref(prm), int(num_splits)))


def decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
           block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
           bias: torch.Tensor, *, window: int, sm_scale: float, num_splits: int = 0,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rba_decode: q [B,Hq,D], bias [B,Hq,R]; returns out [B,Hq,D].

    ``workspace`` (a uint8 device tensor) is allocated with torch when not
    given and the call needs one.
    """
    lib = load()
    kv, pt, prm = _decode_structs(q, k_pool, v_pool, block_table, seq_lens, bias, window, sm_scale)
    if q.dtype != k_pool.dtype or bias.dtype != k_pool.dtype:
        raise TypeError("q, bias and the pools must share one dtype")
    need = int(lib.rba_decode_workspace_size(ctypes.byref(kv), ctypes.byref(pt), int(max_seq_len),
                                             ctypes.byref(prm), int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lse_ptr = None
    if lse is not None:
        if lse.shape != q.shape[:2]:
            raise ValueError("lse must be [B, Hq]")
        lse_ptr = _dev(lse, "lse", torch.float32)
    st = lib.rba_decode(_dev(q, "q"), ctypes.byref(kv), ctypes.byref(pt), int(max_seq_len),
                        _dev(bias, "bias"), ctypes.byref(prm), int(num_splits), ws_ptr, ws_bytes,
                        _dev(out, "out"), lse_ptr, _stream(stream))
    _check(st, "rba_decode")
    return out


def decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                   bias: torch.Tensor, *, window: int, sm_scale: float, out: torch.Tensor,
                   num_splits: int = 0, lse: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """rba_decode_noalloc: rba_decode with its workspace in the library's
    static per-GPU array (at most DECODE_SCRATCH_BYTES).  ``out`` (and
    ``lse``) are the caller's: nothing is allocated here or in the call.
    Calls that may overlap on one GPU race on that array."""
    lib = load()
    kv, pt, prm = _decode_structs(q, k_pool, v_pool, block_table, seq_lens, bias, window, sm_scale)
    if q.dtype != k_pool.dtype or bias.dtype != k_pool.dtype:
        raise TypeError("q, bias and the pools must share one dtype")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lse_ptr = None
    if lse is not None:
        if lse.shape != q.shape[:2]:
            raise ValueError("lse must be [B, Hq]")
        lse_ptr = _dev(lse, "lse", torch.float32)
    st = lib.rba_decode_noalloc(_dev(q, "q"), ctypes.byref(kv), ctypes.byref(pt),
                                int(max_seq_len), _dev(bias, "bias"), ctypes.byref(prm),
                                int(num_splits), _dev(out, "out"), lse_ptr, _stream(stream))
    _check(st, "rba_decode_noalloc")
    return out


def _multi_structs(q, q_len, k_pool, v_pool, block_table, seq_lens, bias, window, sm_scale):
    if q.dim() != 3 or bias.dim() != 3 or bias.shape[:2] != q.shape[:2]:
        raise ValueError("q must be [B*q_len,Hq,D] and bias [B*q_len,Hq,R]")
    if q_len < 1 or q.shape[0] != block_table.shape[0] * q_len:
        raise ValueError("q must hold q_len rows per sequence of the block table")
    return _structs(k_pool, v_pool, block_table, seq_lens, q.shape[1], window, bias.shape[2],
                    sm_scale)


def decode_multi_num_splits(q, q_len, k_pool, v_pool, block_table, seq_lens, max_seq_len, bias, *,
                            window: int, sm_scale: float, num_splits: int = 0) -> int:
    lib = load()
    kv, pt, prm = _multi_structs(q, q_len, k_pool, v_pool, block_table, seq_lens, bias, window,
                                 sm_scale)
    return int(lib.rba_decode_multi_num_splits(int(q_len), ctypes.byref(kv), ctypes.byref(pt),
                                               int(max_seq_len), ctypes.byref(prm),
                                               int(num_splits)))


def decode_multi_workspace_size(q, q_len, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                                bias, *, window: int, sm_scale: float, num_splits: int = 0) -> int:
    lib = load()
    kv, pt, prm = _multi_structs(q, q_len, k_pool, v_pool, block_table, seq_lens, bias, window,
                                 sm_scale)
    return int(lib.rba_decode_multi_workspace_size(int(q_len), ctypes.byref(kv), ctypes.byref(pt),
                                                   int(max_seq_len), ctypes.byref(prm),
                                                   int(num_splits)))


def decode_multi(q: torch.Tensor, q_len: int, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                 bias: torch.Tensor, *, window: int, sm_scale: float, num_splits: int = 0,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rba_decode_multi: q [B*q_len,Hq,D], bias [B*q_len,Hq,R]; sequence b's
    q_len tokens are its last positions.  Returns out [B*q_len,Hq,D].
    ``workspace`` (uint8 device tensor) is allocated with torch when not
    given and the call needs one."""
    lib = load()
    kv, pt, prm = _multi_structs(q, q_len, k_pool, v_pool, block_table, seq_lens, bias, window,
                                 sm_scale)
    if q.dtype != k_pool.dtype or bias.dtype != k_pool.dtype:
        raise TypeError("q, bias and the pools must share one dtype")
    need = int(lib.rba_decode_multi_workspace_size(int(q_len), ctypes.byref(kv), ctypes.byref(pt),
                                                   int(max_seq_len), ctypes.byref(prm),
                                                   int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lse_ptr = None
    if lse is not None:
        if lse.shape != q.shape[:2]:
            raise ValueError("lse must be [B*q_len, Hq]")
        lse_ptr = _dev(lse, "lse", torch.float32)
    st = lib.rba_decode_multi(_dev(q, "q"), int(q_len), ctypes.byref(kv), ctypes.byref(pt),
                              int(max_seq_len), _dev(bias, "bias"), ctypes.byref(prm),
                              int(num_splits), ws_ptr, ws_bytes, _dev(out, "out"), lse_ptr,
                              _stream(stream))
    _check(st, "rba_decode_multi")
    return out
