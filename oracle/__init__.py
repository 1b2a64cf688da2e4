"""CPU oracle for relative-position-bias paged attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and the
two share no code: this side is plain C (``rba_oracle.c``) compiled with gcc,
computing in fp64 from the inputs exactly as stored, and reading K/V from
logical (un-paged) token-major tensors.

The definition it writes out, and the passages it follows, are in the header
of ``rba_oracle.c``.  Every function here is pinned by the CPU tests (brute
force on tiny inputs, closed forms, invariants, a library special case).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rba_oracle.c")
_LIB = os.path.join(_HERE, "librba_oracle.so")

F32 = 0
BF16 = 1

def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _as_stored(x: torch.Tensor):
    """Contiguous CPU tensor in its stored dtype, plus the oracle dtype code."""
    x = x.detach().to("cpu").contiguous()
    if x.dtype == torch.bfloat16:
        return x, BF16
    if x.dtype == torch.float32:
        return x, F32
    raise TypeError(f"oracle takes bf16 or fp32 tensors, got {x.dtype}")


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _arr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


class Oracle:
    """ctypes front of one compiled oracle library."""

    def __init__(self, lib_path: str = _LIB):
        if lib_path == _LIB and (not os.path.exists(_LIB)
                                 or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(lib_path)
        args = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_double, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int]
        for name in ("rba_oracle_prefill", "rba_oracle_decode"):
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        hist = lib.rba_oracle_prefill_history
        hist.argtypes = args[:6] + [ctypes.c_void_p] + args[6:]
        hist.restype = ctypes.c_int
        proj = lib.rba_oracle_prefill_projected
        proj.argtypes = ([ctypes.c_int] + [ctypes.c_void_p] * 7
                         + [ctypes.c_int] * 6 + [ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                                                 ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int])
        proj.restype = ctypes.c_int
        self._lib = lib
        self.threads_used = 0

    def _run(self, fn, q, k, v, bias, cu, window, rel_extent, sm_scale, rows,
             want_lse, num_threads, cu_kv=None):
        q, dt = _as_stored(q)
        k, dk = _as_stored(k)
        v, dv = _as_stored(v)
        bias, db = _as_stored(bias)
        if len({dt, dk, dv, db}) != 1:
            raise TypeError("q, k, v and bias must share one dtype")
        N, Hq, D = q.shape
        Hkv = k.shape[1]
        R = bias.shape[2]
        if R != rel_extent:
            raise ValueError("bias last dim must equal rel_extent")
        cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
        rows_arr = None
        if rows is not None:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
            n_rows = rows_arr.shape[0]
        else:
            n_rows = N * Hq
        out = np.zeros((n_rows, D), dtype=np.float64)
        lse = np.zeros((n_rows,), dtype=np.float64) if want_lse else None
        if cu_kv is None:
            used = fn(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _arr(cu), len(cu) - 1,
                      Hq, Hkv, D, R, int(window), float(sm_scale), _arr(rows_arr),
                      n_rows, _arr(out), _arr(lse), int(num_threads))
        else:
            ckv = np.ascontiguousarray(np.asarray(cu_kv, dtype=np.int64))
            if len(ckv) != len(cu):
                raise ValueError("cu_q and cu_kv must describe the same sequences")
            used = fn(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _arr(cu), _arr(ckv),
                      len(cu) - 1, Hq, Hkv, D, R, int(window), float(sm_scale),
                      _arr(rows_arr), n_rows, _arr(out), _arr(lse), int(num_threads))
        if used < 0:
            raise ValueError("oracle rejected its arguments")
        self.threads_used = used
        if rows is None:
            out = out.reshape(N, Hq, D)
            if lse is not None:
                lse = lse.reshape(N, Hq)
        return (out, lse) if want_lse else out

    def prefill(self, q, k, v, bias, cu_seqlens, *, window: int, rel_extent: int,
                sm_scale: float, rows=None, want_lse: bool = False,
                num_threads: int = 0):
        """Reference prefill.

        q [T,Hq,D], k/v [T,Hkv,D] logical (token-major, sequences back to
        back), bias [T,Hq,R], cu_seqlens [B+1].  ``rows``: optional (token,
        head) pairs.  Returns out fp64 [T,Hq,D] (or [n_rows,D]) and, if asked,
        lse fp64 [T,Hq] (or [n_rows]).
        """
        return self._run(self._lib.rba_oracle_prefill, q, k, v, bias, cu_seqlens,
                         window, rel_extent, sm_scale, rows, want_lse, num_threads)

    def prefill_history(self, q, k, v, bias, cu_q, cu_kv, *, window: int, rel_extent: int,
                        sm_scale: float, rows=None, want_lse: bool = False,
                        num_threads: int = 0):
        """Reference prefill over a cached history.

        k/v [sum n_b, Hkv, D] hold all n_b logical keys of each sequence back
        to back (cu_kv [B+1]); q [sum L_b, Hq, D] and bias [sum L_b, Hq, R]
        hold this call's L_b query tokens (cu_q [B+1]), which are the last
        L_b positions of their sequence.  ``rows``: optional (query token,
        head) pairs.
        """
        return self._run(self._lib.rba_oracle_prefill_history, q, k, v, bias, cu_q,
                         window, rel_extent, sm_scale, rows, want_lse, num_threads,
                         cu_kv=cu_kv)

    def prefill_projected(self, q, k, v, rel_r, w_rel, cu_q, cu_kv=None, *, window: int,
                          sm_scale: float, rows=None, want_lse: bool = False,
                          num_threads: int = 0):
        """Prefill whose bias is the projection bias[t,h,d] = sum_k rel_r[t,h,k] w_rel[k,d],
        formed in fp64 and rounded once (ties to even) to the inputs' dtype.

        rel_r [sum L_b, Hq, d_rel], w_rel [d_rel, R] (the pages' layout); the
        rest as ``prefill`` (cu_kv None) or ``prefill_history`` (cu_kv given).
        """
        q, dt = _as_stored(q)
        k, dk = _as_stored(k)
        v, dv = _as_stored(v)
        rel_r, dr = _as_stored(rel_r)
        w_rel, dw = _as_stored(w_rel)
        if len({dt, dk, dv, dr, dw}) != 1:
            raise TypeError("q, k, v, rel_r and w_rel must share one dtype")
        N, Hq, D = q.shape
        Hkv = k.shape[1]
        d_rel, R = w_rel.shape
        if rel_r.shape != (N, Hq, d_rel):
            raise ValueError("rel_r must be [T, Hq, d_rel] with the d_rel of w_rel")
        cu = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int64))
        ckv = None
        if cu_kv is not None:
            ckv = np.ascontiguousarray(np.asarray(cu_kv, dtype=np.int64))
            if len(ckv) != len(cu):
                raise ValueError("cu_q and cu_kv must describe the same sequences")
        rows_arr = None
        if rows is not None:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
            n_rows = rows_arr.shape[0]
        else:
            n_rows = N * Hq
        out = np.zeros((n_rows, D), dtype=np.float64)
        lse = np.zeros((n_rows,), dtype=np.float64) if want_lse else None
        used = self._lib.rba_oracle_prefill_projected(
            dt, _ptr(q), _ptr(k), _ptr(v), _ptr(rel_r), _ptr(w_rel), _arr(cu), _arr(ckv),
            len(cu) - 1, Hq, Hkv, D, R, int(window), d_rel, float(sm_scale), _arr(rows_arr),
            n_rows, _arr(out), _arr(lse), int(num_threads))
        if used < 0:
            raise ValueError("oracle rejected its arguments")
        self.threads_used = used
        if rows is None:
            out = out.reshape(N, Hq, D)
            if lse is not None:
                lse = lse.reshape(N, Hq)
        return (out, lse) if want_lse else out

    def decode(self, q, k, v, bias, cu_kv, *, window: int, rel_extent: int,
               sm_scale: float, rows=None, want_lse: bool = False,
               num_threads: int = 0):
        """Reference single-token decode.

        q [B,Hq,D]; k/v [sum n_b, Hkv, D] hold the logical keys of the B
        sequences back to back (cu_kv [B+1]); the query of sequence b sits at
        position n_b - 1.  bias [B,Hq,R].  ``rows``: optional (sequence, head)
        pairs.
        """
        return self._run(self._lib.rba_oracle_decode, q, k, v, bias, cu_kv,
                         window, rel_extent, sm_scale, rows, want_lse, num_threads)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def prefill(*args, **kwargs):
    return default().prefill(*args, **kwargs)


def decode(*args, **kwargs):
    return default().decode(*args, **kwargs)


def prefill_history(*args, **kwargs):
    return default().prefill_history(*args, **kwargs)


def prefill_projected(*args, **kwargs):
    return default().prefill_projected(*args, **kwargs)
