"""fp64 CPU oracle for the Gemma 4 interleaved attention block.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the benchmark's
CPU-baseline leg are its only users; the HIP library never imports, links or
calls it.  The arithmetic lives in ``oracle.c`` (plain loops, fp64, two-pass
softmax); this module only marshals numpy arrays into it.

Array conventions (row-major, contiguous):
  prefill  q [B,S,Hq,d], k/v [B,S,Hkv,d], pos [B,S] int32
  decode   q [B,Hq,d], k_cache/v_cache [B,Hkv,C,d], pos [B] int32
  decode_multi q [B,L,Hq,d], caches as decode, pos [B] (last query's position)
  fill_cache k/v [B,S,Hkv,d], pos [B,S] -> caches [B,Hkv,C,d]
Inputs are float32, or bf16 given as their uint16 bit patterns; outputs fp64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def load(path):
    """Open an oracle shared library at path and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P, I, D, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
    lib.g4o_prefill.argtypes = [P, P, P, I, P, I, I, I, I, I, I, D, D, P, L, P]
    lib.g4o_prefill.restype = I
    lib.g4o_decode.argtypes = [P, P, P, I, P, I, I, I, I, I, I, D, D, P]
    lib.g4o_decode.restype = I
    lib.g4o_decode_multi.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, D, D, P]
    lib.g4o_decode_multi.restype = I
    lib.g4o_fill_cache.argtypes = [P, P, I, P, I, I, I, I, I, I, P, P]
    lib.g4o_fill_cache.restype = I
    lib.g4o_probs.argtypes = [P, P, I, P, I, I, I, I, I, I, D, D, I, I, I, P]
    lib.g4o_probs.restype = I
    lib.g4o_rope.argtypes = [P, I, I, D, D]
    lib.g4o_rope.restype = None
    lib.g4o_nrot.argtypes = [I, D]
    lib.g4o_nrot.restype = I
    return lib


def _lib(lib=None):
    global _LIB
    if lib is not None:
        return lib
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(
                os.path.join(_HERE, "oracle.c")):
            _build.build()
        _LIB = load(path)
    return _LIB


def _in(a):
    """Return (contiguous array, dtype code): 0 = float32, 1 = bf16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def nrot(d, p, lib=None):
    return _lib(lib).g4o_nrot(int(d), float(p))


def rope(x, theta, p, pos, lib=None):
    """R(pos) applied to a copy of the fp64 head vector x (pairs t < n_rot)."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    _lib(lib).g4o_rope(_ptr(y), d, nrot(d, p, lib), float(theta), float(pos))
    return y


def prefill(q, k, v, pos, window, theta, p, rows=None, lib=None):
    """Causal (optionally windowed) attention; v is k for the K=V layer.

    rows: None for every row (out [B,S,Hq,d]) or flattened ids b*S+i
    (out [len(rows),Hq,d]).
    """
    q, dt = _in(q)
    k, dk = _in(k)
    v, dv = _in(v)
    if not (dt == dk == dv):
        raise TypeError("q, k, v must share a dtype")
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, d) and v.shape == k.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert pos.shape == (B, S)
    if rows is None:
        out = np.empty((B, S, Hq, d), np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, Hq, d), np.float64)
        rp, nr = _ptr(rows), rows.size
    rc = _lib(lib).g4o_prefill(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(pos), B, S, Hq, Hkv, d,
                            int(window), float(theta), float(p), rp, nr, _ptr(out))
    if rc != 0:
        raise ValueError(f"g4o_prefill failed ({rc})")
    return out


def probs(q, k, pos, window, theta, p, b, i, h, lib=None):
    """Softmax probability row of query (b, i, h) over all S keys."""
    q, dt = _in(q)
    k, dk = _in(k)
    assert dt == dk
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    out = np.empty(S, np.float64)
    rc = _lib(lib).g4o_probs(_ptr(q), _ptr(k), dt, _ptr(pos), B, S, Hq, Hkv, d, int(window),
                          float(theta), float(p), int(b), int(i), int(h), _ptr(out))
    if rc != 0:
        raise ValueError(f"g4o_probs failed ({rc})")
    return out


def decode(q, k_cache, v_cache, pos, window, theta, p, lib=None):
    """One query token per sequence against a raw KV cache (v_cache None: K=V)."""
    q, dt = _in(q)
    k_cache, dk = _in(k_cache)
    if v_cache is not None:
        v_cache, dv = _in(v_cache)
        assert dv == dk and v_cache.shape == k_cache.shape
    assert dt == dk
    B, Hq, d = q.shape
    _, Hkv, C, _ = k_cache.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert pos.shape == (B,)
    out = np.empty((B, Hq, d), np.float64)
    rc = _lib(lib).g4o_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), dt, _ptr(pos), B, Hq, Hkv, d,
                           C, int(window), float(theta), float(p), _ptr(out))
    if rc != 0:
        raise ValueError(f"g4o_decode failed ({rc})")
    return out


def decode_multi(q, k_cache, v_cache, pos, window, theta, p, lib=None):
    """L query tokens per sequence (q [B,L,Hq,d]; pos [B] = last query's position)."""
    q, dt = _in(q)
    k_cache, dk = _in(k_cache)
    if v_cache is not None:
        v_cache, dv = _in(v_cache)
        assert dv == dk and v_cache.shape == k_cache.shape
    assert dt == dk
    B, L, Hq, d = q.shape
    _, Hkv, C, _ = k_cache.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert pos.shape == (B,)
    out = np.empty((B, L, Hq, d), np.float64)
    rc = _lib(lib).g4o_decode_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), dt, _ptr(pos), B, L,
                                    Hq, Hkv, d, C, int(window), float(theta), float(p), _ptr(out))
    if rc != 0:
        raise ValueError(f"g4o_decode_multi failed ({rc})")
    return out


def fill_cache(k, v, pos, k_cache, v_cache, window, lib=None):
    """Copies of k_cache (and v_cache) with the prefill rows k, v [B,S,Hkv,d] written in."""
    k, dk = _in(k)
    kc = np.array(k_cache, copy=True, order="C")
    assert kc.dtype == k.dtype
    vc = None
    if v is not None:
        v, dv = _in(v)
        assert dv == dk and v.shape == k.shape
        vc = np.array(v_cache, copy=True, order="C")
        assert vc.dtype == v.dtype and vc.shape == kc.shape
    B, S, Hkv, d = k.shape
    _, Hkv2, C, d2 = kc.shape
    assert (Hkv2, d2) == (Hkv, d) and kc.shape[0] == B
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert pos.shape == (B, S)
    rc = _lib(lib).g4o_fill_cache(_ptr(k), _ptr(v), k.dtype.itemsize, _ptr(pos), B, S, Hkv, d, C,
                                  int(window), _ptr(kc), _ptr(vc))
    if rc != 0:
        raise ValueError(f"g4o_fill_cache failed ({rc})")
    return kc, vc
