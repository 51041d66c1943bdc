"""libg4attn: Gemma 4 interleaved attention (sliding-window local layers and
K=V / p-RoPE global layers) on AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/g4attn.h.  It only checks and
marshals torch tensors (device memory) and passes torch's current HIP stream;
every step of the computation runs in the library's HIP kernels.  There is no
CPU or PyTorch fallback: if the library is missing, calls raise.

Layouts (contiguous): prefill q/out [B,S,Hq,d], k/v/kv [B,S,Hkv,d], pos [B,S]
int32; decode q/out [B,Hq,d], caches [B,Hkv,capacity,d], pos [B] int32; fp8
caches hold one E4M3 code per element with float32 scales [Hkv].
"""
from ._lib import lib as _g4lib

F32, BF16 = 0, 1
STATUS = {0: "G4A_OK", -1: "G4A_EINVAL", -2: "G4A_EUNSUPPORTED", -3: "G4A_EALIGN",
          -4: "G4A_EWORKSPACE", -5: "G4A_EHIP"}


class G4AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _g4lib().g4attn_strerror(status).decode()
        if status == -5:
            msg += f" (hipError {_g4lib().g4attn_last_hip_error()})"
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _torch():
    import torch
    return torch


def _code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _out(like_shape, out, out_dtype, device):
    torch = _torch()
    if out is not None:
        return out
    dt = torch.float32 if out_dtype in (None, F32, torch.float32) else torch.bfloat16
    return torch.empty(like_shape, dtype=dt, device=device)


def _check(rc, where):
    if rc != 0:
        raise G4AttnError(rc, where)


def prefill_workspace_bytes(B, S, Hkv, d, p, in_dtype=BF16):
    return int(_g4lib().g4attn_prefill_workspace_bytes(B, S, Hkv, d, float(p), int(in_dtype)))


def _workspace(need, workspace, device):
    if workspace is None:
        return _torch().empty(max(need, 16), dtype=_torch().uint8, device=device)
    return workspace


def _nbytes(t):
    return t.numel() * t.element_size()


def local_prefill(q, k, v, pos, window, theta=1e4, p=1.0, out=None, out_dtype=None,
                  workspace=None):
    """Causal sliding-window attention, separate K and V (g4attn_local_prefill)."""
    _dev(q, k, v, pos, out, workspace)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    out = _out((B, S, Hq, d), out, out_dtype, q.device)
    ws = _workspace(prefill_workspace_bytes(B, S, Hkv, d, p, _code(q)), workspace, q.device)
    rc = _g4lib().g4attn_local_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(pos), B, S, Hq,
                                     Hkv, d, int(window), float(theta), float(p), _code(q),
                                     _code(out), _ptr(ws), _nbytes(ws), _stream())
    _check(rc, "g4attn_local_prefill")
    return out


def global_prefill(q, kv, pos, window=0, theta=1e6, p=0.25, out=None, out_dtype=None,
                   workspace=None):
    """Causal attention with keys identical to values (g4attn_global_prefill)."""
    _dev(q, kv, pos, out, workspace)
    B, S, Hq, d = q.shape
    Hkv = kv.shape[2]
    out = _out((B, S, Hq, d), out, out_dtype, q.device)
    ws = _workspace(prefill_workspace_bytes(B, S, Hkv, d, p, _code(q)), workspace, q.device)
    rc = _g4lib().g4attn_global_prefill(_ptr(q), _ptr(kv), _ptr(out), _ptr(pos), B, S, Hq, Hkv, d,
                                      int(window), float(theta), float(p), _code(q), _code(out),
                                      _ptr(ws), _nbytes(ws), _stream())
    _check(rc, "g4attn_global_prefill")
    return out


def vision_prefill(q, k, v, pos2, theta=1e4, lengths=None, out=None, out_dtype=None,
                   workspace=None):
    """Vision-encoder attention (g4attn_vision_prefill): every patch of an
    image sees every valid patch of the image, with 2D RoPE driven by
    pos2 [B, S, 2] = (w, h).  lengths [B] int32 (None: all S valid); rows of
    padding patches are zero.  bf16 q, k, v with d = 256."""
    _dev(q, k, v, pos2, lengths, out, workspace)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    out = _out(q.shape, out, out_dtype, q.device)
    workspace = _workspace(prefill_workspace_bytes(B, S, Hkv, d, 1.0, _code(q)), workspace,
                           q.device)
    rc = _g4lib().g4attn_vision_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(pos2),
                                        _ptr(lengths), B, S, Hq, Hkv, d, float(theta), _code(q),
                                        _code(out), _ptr(workspace), _nbytes(workspace),
                                        _stream())
    _check(rc, "g4attn_vision_prefill")
    return out


def decode_workspace_bytes(B, Hq, Hkv, d, capacity, window):
    return int(_g4lib().g4attn_decode_workspace_bytes(B, Hq, Hkv, d, capacity, window))


def decode(q, k_cache, v_cache, pos, window, theta, p, out=None, workspace=None,
           out_dtype=None):
    """One query token per sequence against a raw KV cache (g4attn_decode).

    v_cache None means K=V; window > 0 is a ring cache of `window` slots.
    """
    torch = _torch()
    _dev(q, k_cache, v_cache, pos, out, workspace)
    B, Hq, d = q.shape
    _, Hkv, C, _ = k_cache.shape
    out = _out((B, Hq, d), out, out_dtype, q.device)
    workspace = _workspace(decode_workspace_bytes(B, Hq, Hkv, d, C, window), workspace,
                           q.device)
    nbytes = _nbytes(workspace)
    rc = _g4lib().g4attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(pos), B, Hq,
                              Hkv, d, C, int(window), float(theta), float(p), _code(q),
                              _code(out), _ptr(workspace), nbytes, _stream())
    _check(rc, "g4attn_decode")
    return out


def decode_multi_workspace_bytes(B, q_len, Hq, Hkv, d, capacity, window):
    return _g4lib().g4attn_decode_multi_workspace_bytes(B, q_len, Hq, Hkv, d, capacity,
                                                        int(window))


def decode_multi(q, k_cache, v_cache, pos, window, theta, p, out=None, workspace=None,
                 out_dtype=None):
    """q_len query tokens per sequence at once (g4attn_decode_multi).

    q is [B, q_len, Hq, d]; pos [B] is the position of the last token; a ring
    (window > 0) needs capacity >= window + q_len - 1.
    """
    torch = _torch()
    _dev(q, k_cache, v_cache, pos, out, workspace)
    B, L, Hq, d = q.shape
    _, Hkv, C, _ = k_cache.shape
    out = _out((B, L, Hq, d), out, out_dtype, q.device)
    workspace = _workspace(decode_multi_workspace_bytes(B, L, Hq, Hkv, d, C, window), workspace,
                           q.device)
    nbytes = _nbytes(workspace)
    rc = _g4lib().g4attn_decode_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(pos),
                                    B, L, Hq, Hkv, d, C, int(window), float(theta), float(p),
                                    _code(q), _code(out), _ptr(workspace), nbytes, _stream())
    _check(rc, "g4attn_decode_multi")
    return out


def fill_cache(k, v, pos, k_cache, v_cache, window):
    """Write prefill rows k, v [B, S, Hkv, d] into the caches (g4attn_fill_cache).

    v None means K=V (only k_cache is written); window > 0 is a ring.
    """
    _dev(k, v, pos, k_cache, v_cache)
    B, S, Hkv, d = k.shape
    C = k_cache.shape[2]
    rc = _g4lib().g4attn_fill_cache(_ptr(k), _ptr(v), _ptr(pos), B, S, Hkv, d, _ptr(k_cache),
                                  _ptr(v_cache), C, int(window), _code(k), _stream())
    _check(rc, "g4attn_fill_cache")
    return k_cache, v_cache


def _fp8_cache(t):
    if t is not None and t.element_size() != 1:
        raise TypeError(f"fp8 caches hold one byte per element (uint8 or float8_e4m3fn), got {t.dtype}")


def _scales(*ts):
    torch = _torch()
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"scales must be float32, got {t.dtype}")


def fill_cache_fp8(k, v, pos, k_cache, v_cache, window, k_scale, v_scale=None):
    """Quantize prefill rows k, v [B, S, Hkv, d] (bf16 or f32) into E4M3 caches
    [B, Hkv, capacity, d] (g4attn_fill_cache_fp8): code = E4M3(x / scale[h]).

    v None means K=V (only k_cache is written, v_scale unused).
    """
    _dev(k, v, pos, k_cache, v_cache, k_scale, v_scale)
    _fp8_cache(k_cache)
    _fp8_cache(v_cache)
    _scales(k_scale, v_scale)
    B, S, Hkv, d = k.shape
    C = k_cache.shape[2]
    rc = _g4lib().g4attn_fill_cache_fp8(_ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _ptr(pos),
                                        B, S, Hkv, d, _ptr(k_cache), _ptr(v_cache), C,
                                        int(window), _code(k), _stream())
    _check(rc, "g4attn_fill_cache_fp8")
    return k_cache, v_cache


def decode_fp8_workspace_bytes(B, q_len, Hq, Hkv, d, capacity, window):
    return int(_g4lib().g4attn_decode_fp8_workspace_bytes(B, q_len, Hq, Hkv, d, capacity, window))


def decode_fp8(q, k_cache, v_cache, k_scale, v_scale, pos, window, theta, p, out=None,
               workspace=None, out_dtype=None):
    """Decode of q_len query tokens over E4M3 caches (g4attn_decode_fp8).

    q is bf16 [B, q_len, Hq, d]; caches [B, Hkv, capacity, d] hold one code
    per element (uint8 or float8_e4m3fn); k_scale, v_scale are float32 [Hkv];
    v_cache None means K=V (values are k_cache with k_scale).
    """
    _dev(q, k_cache, v_cache, k_scale, v_scale, pos, out, workspace)
    _fp8_cache(k_cache)
    _fp8_cache(v_cache)
    _scales(k_scale, v_scale)
    if _code(q) != BF16:
        raise TypeError("decode_fp8 takes a bfloat16 query")
    B, L, Hq, d = q.shape
    _, Hkv, C, _ = k_cache.shape
    out = _out((B, L, Hq, d), out, out_dtype, q.device)
    workspace = _workspace(decode_fp8_workspace_bytes(B, L, Hq, Hkv, d, C, window), workspace,
                           q.device)
    rc = _g4lib().g4attn_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                    _ptr(v_scale), _ptr(out), _ptr(pos), B, L, Hq, Hkv, d, C,
                                    int(window), float(theta), float(p), _code(out),
                                    _ptr(workspace), _nbytes(workspace), _stream())
    _check(rc, "g4attn_decode_fp8")
    return out


def strerror(status):
    return _g4lib().g4attn_strerror(int(status)).decode()
