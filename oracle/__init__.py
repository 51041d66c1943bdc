"""fp64 CPU oracle for the Gemma 4 interleaved attention block.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the benchmark's
CPU-baseline leg are its only users; the HIP library never imports, links or
calls it.  The arithmetic lives in ``oracle.c`` (plain loops, fp64, two-pass
softmax); this module only marshals numpy arrays into it.

Array conventions (row-major, contiguous):
  prefill  q [B,S,Hq,d], k/v [B,S,Hkv,d], pos [B,S] int32
  decode   q [B,Hq,d], k_cache/v_cache [B,Hkv,C,d], pos [B] int32
  decode_multi q [B,L,Hq,d], caches as decode, pos [B] (last query's position)
  fill_cache k/v [B,S,Hkv,d], pos [B,S] -> caches [B,Hkv,C,d]; with separate
             values the cached keys are turned at their positions
  fp8 caches  uint8 E4M3 codes [B,Hkv,C,d] with float32 scales [Hkv]
  vision_prefill q [B,S,Hq,d], k/v [B,S,Hkv,d], pos2 [B,S,2] (w, h), lengths [B]
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
    lib.g4o_rotate_rows.argtypes = [P, I, P, L, I, I, D, D, P]
    lib.g4o_rotate_rows.restype = I
    lib.g4o_nrot.argtypes = [I, D]
    lib.g4o_nrot.restype = I
    lib.g4o_vision_prefill.argtypes = [P, P, P, I, P, P, I, I, I, I, I, D, P, L, P]
    lib.g4o_vision_prefill.restype = I
    lib.g4o_e4m3_value.argtypes = [I]
    lib.g4o_e4m3_value.restype = D
    lib.g4o_e4m3_encode.argtypes = [ctypes.c_float]
    lib.g4o_e4m3_encode.restype = I
    lib.g4o_quantize_e4m3.argtypes = [P, I, P, L, I, I, P]
    lib.g4o_quantize_e4m3.restype = I
    lib.g4o_threads.argtypes = []
    lib.g4o_threads.restype = I
    lib.g4o_set_threads.argtypes = [I]
    lib.g4o_set_threads.restype = None
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


def _in(a, f64=False):
    """Return (contiguous array, dtype code): 0 = float32, 1 = bf16 bits, 2 = float64
    (float64 only where f64 is set: decode of dequantized caches)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    if f64 and a.dtype == np.float64:
        return a, 2
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def threads(lib=None):
    """Threads the oracle's OpenMP loops use."""
    return int(_lib(lib).g4o_threads())


def set_threads(n, lib=None):
    """Use n threads in the oracle's OpenMP loops from now on."""
    _lib(lib).g4o_set_threads(int(n))


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
    """One query token per sequence against a KV cache.  With v_cache, k_cache
    holds the keys already turned at their positions (what fill_cache writes);
    v_cache None: K=V, k_cache holds the raw tensor.  float32, bf16 bits or
    float64 (all three arrays alike).  v_cache given as k_cache itself is K=V."""
    if v_cache is k_cache:
        v_cache = None
    q, dt = _in(q, f64=True)
    k_cache, dk = _in(k_cache, f64=True)
    if v_cache is not None:
        v_cache, dv = _in(v_cache, f64=True)
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
    """L query tokens per sequence (q [B,L,Hq,d]; pos [B] = last query's position).
    Caches as for decode (v_cache given as k_cache itself is K=V)."""
    if v_cache is k_cache:
        v_cache = None
    q, dt = _in(q, f64=True)
    k_cache, dk = _in(k_cache, f64=True)
    if v_cache is not None:
        v_cache, dv = _in(v_cache, f64=True)
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


def rotate_rows(x, pos, theta, p, lib=None):
    """fp64 R(pos[b, i]) x[b, i, h] for x [B, S, H, d] (float32, bf16 bits or
    float64) and pos [B, S]: each head vector turned at its token's position."""
    x, dt = _in(x, f64=True)
    B, S, H, d = x.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert pos.shape == (B, S)
    out = np.empty(x.shape, np.float64)
    rc = _lib(lib).g4o_rotate_rows(_ptr(x), dt, _ptr(pos), B * S, H, d, float(theta), float(p),
                                   _ptr(out))
    if rc != 0:
        raise ValueError(f"g4o_rotate_rows failed ({rc})")
    return out


def f64_to_bf16_bits(x):
    """bf16 bit patterns of fp64 values, rounded once to the nearest bf16 (8
    significant bits), ties to even; overflow gives infinity.  (Below 2^-126,
    bf16's subnormal range, this keeps 8 significant bits instead of the
    coarser subnormal grid; turned keys never get there.)"""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)  # x = m 2^e, 1/2 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _turned_keys(k, pos, theta, p, lib):
    """The keys a cache with separate values holds: k turned at its positions,
    rounded to k's element type (float32 or bf16 bits)."""
    if theta is None or p is None:
        raise ValueError("a cache with separate values holds turned keys: pass theta and p")
    r = rotate_rows(k, pos, theta, p, lib)
    if k.dtype == np.float32:
        return r.astype(np.float32)
    if k.dtype == np.uint16:
        return f64_to_bf16_bits(r)
    raise TypeError(f"keys to turn must be float32 or bf16 bits, got {k.dtype}")


def fill_cache(k, v, pos, k_cache, v_cache, window, theta=None, p=None, lib=None):
    """Copies of k_cache (and v_cache) with the prefill rows k, v [B,S,Hkv,d] written in
    (float32, bf16 bits, or uint8 E4M3 codes).  With separate values (v given,
    float rows), the keys are first turned at their positions with theta and
    p and rounded to their element type; otherwise bytes are copied unchanged."""
    k = np.ascontiguousarray(k)
    if v is not None and k.dtype != np.uint8:
        k = _turned_keys(k, pos, theta, p, lib)
    return _place(k, v, pos, k_cache, v_cache, window, lib)


def _place(k, v, pos, k_cache, v_cache, window, lib=None):
    """The rows k (and v) placed into copies of the caches, bytes unchanged."""
    k = np.ascontiguousarray(k)
    assert k.dtype in (np.float32, np.uint16, np.uint8), k.dtype
    kc = np.array(k_cache, copy=True, order="C")
    assert kc.dtype == k.dtype
    vc = None
    if v is not None:
        v = np.ascontiguousarray(v)
        assert v.dtype == k.dtype and v.shape == k.shape
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


def e4m3_values(lib=None):
    """fp64 value of every E4M3 code 0..255 (NaN for 0x7F and 0xFF)."""
    L = _lib(lib)
    return np.array([L.g4o_e4m3_value(c) for c in range(256)], np.float64)


def e4m3_encode(x, lib=None):
    """E4M3 code of each float32 value of x (round to nearest even, saturating)."""
    L = _lib(lib)
    x = np.asarray(x, np.float32)
    return np.array([L.g4o_e4m3_encode(float(v)) for v in x.ravel()],
                    np.int64).astype(np.uint8).reshape(x.shape)


def quantize_e4m3(x, scale, lib=None):
    """E4M3 codes of x [..., Hkv, d] (float32 or bf16 bits) divided by scale[Hkv]."""
    x, dt = _in(x)
    scale = np.ascontiguousarray(scale, np.float32)
    Hkv, d = x.shape[-2:]
    assert scale.shape == (Hkv,)
    out = np.empty(x.shape, np.uint8)
    rc = _lib(lib).g4o_quantize_e4m3(_ptr(x), dt, _ptr(scale), x.size // (Hkv * d), Hkv, d,
                                     _ptr(out))
    if rc != 0:
        raise ValueError(f"g4o_quantize_e4m3 failed ({rc})")
    return out


def dequantize_e4m3(codes, scale, lib=None):
    """fp64 values code_value * scale[h] of an E4M3 cache [B, Hkv, C, d] (exact)."""
    scale = np.asarray(scale, np.float32).astype(np.float64)
    return e4m3_values(lib)[np.asarray(codes, np.uint8)] * scale[None, :, None, None]


def fill_cache_fp8(k, v, pos, k_cache, v_cache, window, k_scale, v_scale, theta=None, p=None,
                   lib=None):
    """fill_cache into E4M3 caches: with separate values the keys are turned
    at their positions and rounded to float32 first; the rows are quantized
    with the per-KV-head scales, then placed as the plain fill places bytes."""
    k = np.ascontiguousarray(k)
    if v is not None:
        if theta is None or p is None:
            raise ValueError("a cache with separate values holds turned keys: pass theta and p")
        k = rotate_rows(k, pos, theta, p, lib).astype(np.float32)
    kq = quantize_e4m3(k, k_scale, lib)
    vq = None if v is None else quantize_e4m3(v, v_scale, lib)
    return _place(kq, vq, pos, k_cache, v_cache, window, lib=lib)


def decode_fp8(q, k_codes, v_codes, k_scale, v_scale, pos, window, theta, p, lib=None):
    """decode_multi over E4M3 caches (v_codes None: K=V, values use k_scale):
    the caches are dequantized exactly in fp64 and decoded as decode_multi
    reads them (with separate values the key codes are of turned keys;
    v_codes given as k_codes itself is K=V)."""
    if v_codes is k_codes:
        v_codes = None
    kc = dequantize_e4m3(k_codes, k_scale, lib)
    vc = None if v_codes is None else dequantize_e4m3(v_codes, v_scale, lib)
    qf = np.asarray(q)
    qf = bf16_bits_to_f64(qf) if qf.dtype == np.uint16 else qf.astype(np.float64)
    return decode_multi(qf, kc, vc, pos, window, theta, p, lib=lib)


def bf16_bits_to_f64(bits):
    """Exact fp64 values of bf16 bit patterns."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def vision_prefill(q, k, v, pos2, theta, lengths=None, rows=None, lib=None):
    """Bidirectional attention with 2D RoPE over the patches of each image
    (pos2 [B,S,2] = (w, h) per patch; lengths [B] valid patches, None = S).

    rows: None for every row (out [B,S,Hq,d]) or flattened ids b*S+i
    (out [len(rows),Hq,d]).  Rows of padding patches are zero.
    """
    q, dt = _in(q)
    k, dk = _in(k)
    v, dv = _in(v)
    if not (dt == dk == dv):
        raise TypeError("q, k, v must share a dtype")
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, d) and v.shape == k.shape
    pos2 = np.ascontiguousarray(pos2, dtype=np.int32)
    assert pos2.shape == (B, S, 2)
    ln = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    assert ln is None or ln.shape == (B,)
    if rows is None:
        out = np.empty((B, S, Hq, d), np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, Hq, d), np.float64)
        rp, nr = _ptr(rows), rows.size
    rc = _lib(lib).g4o_vision_prefill(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(pos2), _ptr(ln), B, S,
                                      Hq, Hkv, d, float(theta), rp, nr, _ptr(out))
    if rc != 0:
        raise ValueError(f"g4o_vision_prefill failed ({rc})")
    return out
