"""CPU oracle for indexed sparse attention (DSA) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the
two share no code: the oracle is plain C (``oracle.c``, fp64 direct loops,
a full sort for Top-K, a two-pass softmax) built into ``liboracle.so`` and
called here through ctypes.

Functions take a ``synth.Workload`` (or any object with the same fields)
and return fp64 numpy arrays:

  index_scores(w)          -> scores [B,T,Lmax] (NaN where not visible)
  mx_quantize(v)           -> (E8M0 byte, E4M3 element values) of one group
  topk(w, scores)          -> (idx [B,T,K] ascending, -1 padded; count [B,T])
  sparse_mla(w, idx)       -> (out [B,T,H,Dv], lse [B,T,H])
  forward(w)               -> dict with all of the above

``want`` (bool [B,T]) restricts the work to a subset of queries; rows not
wanted are left untouched (zero for fresh arrays).

Parity status of each function is documented in the test that pins it
(tests/test_oracle_pins.py).  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# (DSA_ORACLE_LIBRARY: another build of oracle.c, e.g. a sanitised one)
_LIB_PATH = os.environ.get("DSA_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int64),
        ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double),
        ("q_idx_dtype", ctypes.c_int32), ("idx_key_dtype", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
    ]


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(_Dims)
        lib.oracle_index_scores.argtypes = [D, P, P, P, P, P, P, P]
        lib.oracle_topk.argtypes = [D, P, P, P, P, P]
        lib.oracle_sparse_mla.argtypes = [D, P, P, P, P, P, P, P, P]
        lib.oracle_attention_weights.argtypes = [D, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, P]
        for f in (lib.oracle_index_scores, lib.oracle_topk, lib.oracle_sparse_mla,
                  lib.oracle_attention_weights):
            f.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_quantize.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_quantize.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_mx_quantize.argtypes = [P, ctypes.c_int, P, P]
        lib.oracle_mx_quantize.restype = None
        _lib = lib
    return _lib


def _p(a) -> Optional[int]:
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dims(w) -> _Dims:
    return _Dims(w.batch, w.q_len, w.max_seq_len, w.idx_heads, w.idx_dim, w.heads, w.qk_dim,
                 w.v_dim, w.top_k, float(w.softmax_scale), w.q_idx_dtype, w.idx_key_dtype,
                 w.q_dtype, w.kv_dtype)


def _want(w, want):
    if want is None:
        return None
    a = np.ascontiguousarray(np.asarray(want, dtype=np.uint8).reshape(w.batch, w.q_len))
    return a


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def e4m3_quantize(x: float) -> float:
    return _load().oracle_e4m3_quantize(x)


def e8m0_value(e: int) -> float:
    return _load().oracle_e8m0_value(e)


def mx_quantize(values) -> tuple:
    """MX quantisation of one group of at most 32 values to E4M3 elements.

    Returns (E8M0 scale byte, element values as float64); the group's
    dequantised values are ``elements * 2**(byte - 127)``.
    """
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64).ravel())
    assert 1 <= v.size <= 32
    e = np.zeros(1, np.uint8)
    out = np.zeros(v.size, np.float64)
    _load().oracle_mx_quantize(_p(v), v.size, _p(e), _p(out))
    return int(e[0]), out


def index_scores(w, want=None) -> np.ndarray:
    d = _dims(w)
    out = np.zeros((w.batch, w.q_len, w.max_seq_len), np.float64)
    wt = _want(w, want)
    rc = _load().oracle_index_scores(ctypes.byref(d), _p(w.q_idx), _p(w.head_w), _p(w.k_idx),
                                     _p(w.k_scale), _p(w.seq_lens), _p(wt), _p(out))
    assert rc == 0
    return out


def topk(w, scores: np.ndarray, want=None):
    d = _dims(w)
    idx = np.full((w.batch, w.q_len, w.top_k), -1, np.int32)
    cnt = np.zeros((w.batch, w.q_len), np.int32)
    wt = _want(w, want)
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    rc = _load().oracle_topk(ctypes.byref(d), _p(scores), _p(w.seq_lens), _p(wt), _p(idx), _p(cnt))
    assert rc == 0
    return idx, cnt


def sparse_mla(w, idx: np.ndarray, want=None):
    d = _dims(w)
    out = np.zeros((w.batch, w.q_len, w.heads, w.v_dim), np.float64)
    lse = np.zeros((w.batch, w.q_len, w.heads), np.float64)
    wt = _want(w, want)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert idx.shape == (w.batch, w.q_len, w.top_k)
    rc = _load().oracle_sparse_mla(ctypes.byref(d), _p(w.q), _p(w.kv), _p(w.kv_scale), _p(idx),
                                   _p(w.seq_lens), _p(wt), _p(out), _p(lse))
    assert rc == 0
    return out, lse


def attention_weights(w, idx: np.ndarray, b: int, t: int, h: int) -> np.ndarray:
    d = _dims(w)
    p = np.zeros(w.top_k, np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    rc = _load().oracle_attention_weights(ctypes.byref(d), _p(w.q), _p(w.kv), _p(w.kv_scale),
                                          _p(idx), _p(w.seq_lens), b, t, h, _p(p))
    assert rc == 0
    return p


def forward(w, want=None) -> dict:
    s = index_scores(w, want)
    idx, cnt = topk(w, s, want)
    out, lse = sparse_mla(w, idx, want)
    return {"scores": s, "idx": idx, "count": cnt, "out": out, "lse": lse}


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().oracle_num_threads())
