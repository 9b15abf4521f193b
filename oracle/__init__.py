"""fp64 CPU oracle for split-KV decode attention (ctypes over fd_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers allowed.  The product path never imports
this package, and this package imports nothing from the product.

Every function takes numpy arrays.  Half-precision inputs are passed as their
raw uint16 bit patterns together with a dtype name ("f32", "f16", "bf16"), and
the C side decodes them exactly to double.  Layouts follow the decode problem
of the pages ("FlashDecoding 数学推导" §2.1.1; "adv04: Flash-Decoding" §4):
q [batch, heads_q, d], K/V [batch, max_kv_len, heads_kv, d].

Pinned by tests/test_oracle_pins.py and tests/test_oracle_decoders.py against
the pages' worked examples, closed forms, invariants and an mpmath brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile fd_oracle.c with gcc (plain C11, OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        L = ctypes.c_long
        lib.oracle_attention.argtypes = [I, P, P, P, P, I, I, I, I, I, D, I, P, P, P]
        lib.oracle_attention.restype = I
        lib.oracle_split_partials.argtypes = [I, P, P, P, P, I, I, I, I, I, D, I, I, P, P, P, P]
        lib.oracle_split_partials.restype = I
        lib.oracle_combine.argtypes = [P, P, L, I, I, P, P]
        lib.oracle_combine.restype = None
        lib.oracle_combine_mlo.argtypes = [P, P, P, L, I, I, P, P, P]
        lib.oracle_combine_mlo.restype = None
        lib.oracle_merge2.argtypes = [P, D, P, D, I, P, P]
        lib.oracle_merge2.restype = None
        lib.oracle_softmax.argtypes = [P, I, P]
        lib.oracle_softmax.restype = None
        lib.oracle_online_softmax.argtypes = [P, I, P, P]
        lib.oracle_online_softmax.restype = None
        lib.oracle_tile_incremental.argtypes = [P, P, P, I, I, D, P, P, P]
        lib.oracle_tile_incremental.restype = None
        lib.oracle_decode.argtypes = [I, P, ctypes.c_size_t, P]
        lib.oracle_decode.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = I
        lib.oracle_set_threads.argtypes = [I]
        lib.oracle_set_threads.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _raw(a: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want:
        raise TypeError(f"oracle expects {np.dtype(want).name} storage for {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _lens(kv_lens, batch):
    if kv_lens is None:
        return None
    lens = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
    if lens.shape != (batch,):
        raise ValueError("kv_lens must have shape [batch]")
    return lens


def _shapes(q, k, v):
    if q.ndim != 3 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("expected q [batch, heads_q, d] and K/V [batch, N, heads_kv, d]")
    batch, heads_q, d = q.shape
    kb, n_max, heads_kv, kd = k.shape
    if kb != batch or kd != d or heads_q % heads_kv:
        raise ValueError("inconsistent q/K/V shapes")
    return batch, heads_q, heads_kv, n_max, d


def threads() -> int:
    return _load().oracle_max_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def decode(dtype: str, raw: np.ndarray) -> np.ndarray:
    """Exact decode of stored elements to float64."""
    raw = _raw(raw, dtype)
    out = np.empty(raw.shape, dtype=np.float64)
    _load().oracle_decode(_DTYPES[dtype], _ptr(raw), raw.size, _ptr(out))
    return out


def attention(dtype, q, k, v, kv_lens=None, scale=None, rows=None):
    """Plain full-row softmax attention in fp64.

    Returns (o [R, d], lse [R]) for R = batch*heads_q rows in (b, hq) order,
    or for the given rows, an int array of (b, hq) pairs of shape [R, 2].
    """
    q, k, v = _raw(q, dtype), _raw(k, dtype), _raw(v, dtype)
    batch, heads_q, heads_kv, n_max, d = _shapes(q, k, v)
    lens = _lens(kv_lens, batch)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        nr, rows_arr = batch * heads_q, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        nr = rows_arr.shape[0]
        if nr and (rows_arr[:, 0].min() < 0 or rows_arr[:, 0].max() >= batch
                   or rows_arr[:, 1].min() < 0 or rows_arr[:, 1].max() >= heads_q):
            raise ValueError("row index out of range")
    o = np.empty((nr, d), dtype=np.float64)
    lse = np.empty((nr,), dtype=np.float64)
    rc = _load().oracle_attention(_DTYPES[dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(lens), batch,
                                  heads_q, heads_kv, n_max, d, float(scale), nr, _ptr(rows_arr),
                                  _ptr(o), _ptr(lse))
    if rc:
        raise MemoryError("oracle_attention: scratch allocation failed")
    return o, lse


def split_partials(dtype, q, k, v, kv_lens, num_splits, split_len, scale=None, with_mlo=False):
    """Per-split LSE pairs (o_part [batch, Hq, B, d], lse_part [batch, Hq, B]).

    With with_mlo=True also returns the triple's m and l ([batch, Hq, B] each).
    """
    q, k, v = _raw(q, dtype), _raw(k, dtype), _raw(v, dtype)
    batch, heads_q, heads_kv, n_max, d = _shapes(q, k, v)
    lens = _lens(kv_lens, batch)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o_part = np.empty((batch, heads_q, num_splits, d), dtype=np.float64)
    lse_part = np.empty((batch, heads_q, num_splits), dtype=np.float64)
    m_part = np.empty_like(lse_part) if with_mlo else None
    l_part = np.empty_like(lse_part) if with_mlo else None
    rc = _load().oracle_split_partials(_DTYPES[dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(lens),
                                       batch, heads_q, heads_kv, n_max, d, float(scale),
                                       int(num_splits), int(split_len), _ptr(o_part),
                                       _ptr(lse_part), _ptr(m_part), _ptr(l_part))
    if rc:
        raise MemoryError("oracle_split_partials: scratch allocation failed")
    if with_mlo:
        return o_part, lse_part, m_part, l_part
    return o_part, lse_part


def combine(o_part, lse_part):
    """LSE merge over the split axis: ([..., B, d], [..., B]) -> ([..., d], [...])."""
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    *lead, nb, d = o_part.shape
    if tuple(lse_part.shape) != (*lead, nb):
        raise ValueError("lse_part must match o_part without its last axis")
    rows = int(np.prod(lead)) if lead else 1
    o = np.empty((*lead, d), dtype=np.float64)
    lse = np.empty(tuple(lead), dtype=np.float64)
    _load().oracle_combine(_ptr(o_part), _ptr(lse_part), rows, nb, d, _ptr(o), _ptr(lse))
    return o, lse


def combine_mlo(o_part, m_part, l_part):
    """m/l/o merge over the split axis -> (o, m_global, l_global)."""
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    m_part = np.ascontiguousarray(m_part, dtype=np.float64)
    l_part = np.ascontiguousarray(l_part, dtype=np.float64)
    *lead, nb, d = o_part.shape
    rows = int(np.prod(lead)) if lead else 1
    o = np.empty((*lead, d), dtype=np.float64)
    mg = np.empty(tuple(lead), dtype=np.float64)
    lg = np.empty(tuple(lead), dtype=np.float64)
    _load().oracle_combine_mlo(_ptr(o_part), _ptr(m_part), _ptr(l_part), rows, nb, d, _ptr(o),
                               _ptr(mg), _ptr(lg))
    return o, mg, lg


def merge2(o1, s1, o2, s2):
    """Stable two-operand LSE merge (o1, S1) (+) (o2, S2) -> (o, S)."""
    o1 = np.ascontiguousarray(o1, dtype=np.float64)
    o2 = np.ascontiguousarray(o2, dtype=np.float64)
    o = np.empty_like(o1)
    s = ctypes.c_double()
    _load().oracle_merge2(_ptr(o1), float(s1), _ptr(o2), float(s2), o1.size, _ptr(o),
                          ctypes.byref(s))
    return o, s.value


def softmax(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    p = np.empty_like(x)
    _load().oracle_softmax(_ptr(x), x.size, _ptr(p))
    return p


def online_softmax(x):
    """Running (m_j, d_j) of the online-softmax recurrence for j = 1..n."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    m = np.empty_like(x)
    dd = np.empty_like(x)
    _load().oracle_online_softmax(_ptr(x), x.size, _ptr(m), _ptr(dd))
    return m, dd


def tile_incremental(q, kmat, vmat, scale):
    """Running (m_j, l_j, o_j) of the incremental per-tile update."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    kmat = np.ascontiguousarray(kmat, dtype=np.float64)
    vmat = np.ascontiguousarray(vmat, dtype=np.float64)
    n, d = kmat.shape
    m = np.empty(n)
    ell = np.empty(n)
    o = np.empty((n, d))
    _load().oracle_tile_incremental(_ptr(q), _ptr(kmat), _ptr(vmat), n, d, float(scale), _ptr(m),
                                    _ptr(ell), _ptr(o))
    return m, ell, o
