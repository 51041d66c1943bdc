"""The C-ABI library: it loads without a GPU, exports every symbol the header
declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import attention_g4attn_amd._lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "g4attn.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(g4attn_\w+)\s*\(", text)))


def test_header_lists_the_binding_signatures():
    assert header_functions() == sorted(L.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (g4attn_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else leaks out of the C ABI
    assert exported == set(header_functions())


def test_strerror_and_codes():
    lib = L.lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.g4attn_strerror(code)
    assert lib.g4attn_strerror(7) == b"unknown status"
    assert lib.g4attn_last_hip_error() == 0


# Fake, aligned, never dereferenced device addresses: every call below must
# fail validation before touching memory or the HIP runtime.
A = 1 << 20


def local(**kw):
    args = dict(q=A, k=2 * A, v=3 * A, out=4 * A, pos=5 * A, B=1, S=8, Hq=4, Hkv=2, d=256,
                window=4, theta=1e4, p=1.0, i=1, o=0, ws=6 * A, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return L.lib().g4attn_local_prefill(*args.values())


def glob(**kw):
    args = dict(q=A, kv=2 * A, out=4 * A, pos=5 * A, B=1, S=8, Hq=8, Hkv=1, d=512, window=0,
                theta=1e6, p=0.25, i=1, o=0, ws=6 * A, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return L.lib().g4attn_global_prefill(*args.values())


def dec(**kw):
    args = dict(q=A, k=2 * A, v=None, out=4 * A, pos=5 * A, B=2, Hq=16, Hkv=2, d=512,
                capacity=1024, window=0, theta=1e6, p=0.25, i=1, o=0, ws=6 * A,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return L.lib().g4attn_decode(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(out=None), -1),
    (dict(pos=None), -1), (dict(B=-1), -1), (dict(S=-2), -1), (dict(Hq=0), -1),
    (dict(Hkv=0), -1), (dict(Hq=5), -1), (dict(d=255), -1), (dict(window=-1), -1),
    (dict(theta=0.0), -1), (dict(theta=float("nan")), -1), (dict(p=1.5), -1),
    (dict(p=-0.1), -1), (dict(p=float("nan")), -1), (dict(i=2), -1), (dict(o=3), -1),
    (dict(d=128), -2), (dict(Hq=6, Hkv=2), -2), (dict(Hq=32, Hkv=2), -2), (dict(i=0, o=1), -2),
    (dict(q=A + 8), -3), (dict(out=4 * A + 4), -3), (dict(pos=5 * A + 2), -3),
    (dict(ws=None), -4), (dict(ws_bytes=8 * 2 * 256 * 2 - 1), -4), (dict(ws=6 * A + 8), -3),
])
def test_local_prefill_validation(kw, code):
    assert local(**kw) == code


def test_empty_inputs_are_noops():
    assert local(B=0, q=None, k=None, v=None, out=None, pos=None) == 0
    assert local(S=0, q=None, k=None, v=None, out=None, pos=None) == 0
    assert glob(S=0, q=None, kv=None, out=None, pos=None) == 0
    assert dec(B=0, q=None, k=None, out=None, pos=None, ws=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(kv=None), -1), (dict(d=384), -2), (dict(Hq=24, Hkv=1), -2), (dict(kv=2 * A + 1), -3),
    (dict(ws=None), -4), (dict(ws_bytes=8 * 128 * 2 - 1), -4),
])
def test_global_prefill_validation(kw, code):
    assert glob(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(capacity=0), -1), (dict(window=512, capacity=1024), -1), (dict(q=None), -1),
    (dict(k=None), -1), (dict(pos=None), -1), (dict(B=-1), -1), (dict(d=100), -1 + 0 * 2),
    (dict(d=96), -2), (dict(ws=None), -4), (dict(ws_bytes=100), -4), (dict(ws=6 * A + 4), -3),
    (dict(v=3 * A + 2), -3),
])
def test_decode_validation(kw, code):
    if kw.get("d") == 100:
        code = -2  # even but not a supported head dim
    assert dec(**kw) == code


def test_prefill_workspace_size():
    f = L.lib().g4attn_prefill_workspace_bytes
    # rotated slab [B, S, Hkv, slab dims] bf16: 128 dims when d = 512 and <= 64 pairs turn
    assert f(1, 262144, 2, 512, 0.25, 1) == 262144 * 2 * 128 * 2
    assert f(2, 1000, 8, 256, 1.0, 1) == 2 * 1000 * 8 * 256 * 2
    assert f(1, 100, 4, 512, 0.5, 1) == 100 * 4 * 512 * 2
    assert f(1, 100, 4, 512, 0.25, 0) == 0  # f32 inputs need none
    assert f(1, 100, 4, 512, 1.5, 1) == 0


def test_workspace_size():
    f = L.lib().g4attn_decode_workspace_bytes
    assert f(64, 16, 2, 512, 65536, 0) == 64 * 16 * 64 * (512 + 2) * 4  # 1024-row chunks
    assert f(64, 16, 8, 256, 512, 512) == 64 * 16 * 1 * (256 + 2) * 4  # one 512-slot chunk
    assert f(1, 16, 8, 256, 1024, 512) == 0  # ring capacity must equal the window
    assert f(1, 0, 8, 256, 512, 512) == 0


def decm(**kw):
    args = dict(q=A, k=2 * A, v=3 * A, out=4 * A, pos=5 * A, B=2, q_len=4, Hq=16, Hkv=8, d=256,
                capacity=515, window=512, theta=1e4, p=1.0, i=1, o=0, ws=6 * A,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return L.lib().g4attn_decode_multi(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q_len=0), -1), (dict(q_len=9), -1), (dict(capacity=514), -1),  # ring < W + q_len - 1
    (dict(capacity=0), -1), (dict(q=None), -1), (dict(pos=None), -1), (dict(B=-1), -1),
    (dict(d=96), -2), (dict(Hq=48), -2), (dict(ws=None), -4), (dict(ws_bytes=100), -4),
    (dict(out=4 * A + 4), -3),
])
def test_decode_multi_validation(kw, code):
    assert decm(**kw) == code


def test_decode_multi_workspace_size():
    f = L.lib().g4attn_decode_multi_workspace_bytes
    g = L.lib().g4attn_decode_workspace_bytes
    # one token equals plain decode; a ring is one chunk of its whole capacity
    assert f(64, 1, 16, 2, 512, 65536, 0) == g(64, 16, 2, 512, 65536, 0)
    assert f(64, 4, 16, 8, 256, 515, 512) == 64 * 4 * 16 * 1 * (256 + 2) * 4
    assert f(2, 3, 16, 2, 512, 4096, 0) == 2 * 3 * 16 * 4 * (512 + 2) * 4
    assert f(2, 4, 16, 8, 256, 514, 512) == 0  # ring too small for 4 tokens
    assert f(2, 9, 16, 8, 256, 600, 512) == 0  # at most 8 tokens


def fill(**kw):
    args = dict(k=A, v=2 * A, pos=3 * A, B=1, S=16, Hkv=8, d=256, kc=4 * A, vc=5 * A,
                capacity=512, window=512, theta=1e4, p=1.0, dtype=1, stream=None)
    args.update(kw)
    return L.lib().g4attn_fill_cache(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(pos=None), -1), (dict(kc=None), -1), (dict(vc=None), -1),
    (dict(B=-1), -1), (dict(Hkv=0), -1), (dict(capacity=0), -1), (dict(window=-1), -1),
    (dict(dtype=5), -2), (dict(d=4), -2),  # 8 bytes a row: not whole 16-byte chunks
    (dict(k=A + 2), -3), (dict(kc=4 * A + 8), -3),
    (dict(theta=0.0), -1), (dict(theta=float("inf")), -1), (dict(p=-0.5), -1), (dict(p=2.0), -1),
    (dict(theta=0.0, v=None), -1),  # checked for K=V too
    (dict(d=1024), -2),             # keys turned with d > 512
])
def test_fill_cache_validation(kw, code):
    assert fill(**kw) == code


def test_fill_cache_turn_limit_applies_only_when_keys_turn():
    # d = 1024 is refused only where keys would be turned: K=V copies, and
    # p = 0 turns nothing (these reach the alignment check and stop there)
    assert fill(d=1024, v=None, k=A + 2) == -3
    assert fill(d=1024, p=0.0, k=A + 2) == -3


def test_fill_cache_empty_is_noop():
    assert fill(S=0, k=None, v=None, pos=None, kc=None, vc=None) == 0
    assert fill(B=0, k=None, v=None, pos=None, kc=None, vc=None) == 0


def decf(**kw):
    args = dict(q=A, k=2 * A, v=3 * A, ks=7 * A, vs=8 * A, out=4 * A, pos=5 * A, B=2, q_len=1,
                Hq=16, Hkv=2, d=512, capacity=65536, window=0, theta=1e6, p=0.25, o=0, ws=6 * A,
                ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return L.lib().g4attn_decode_fp8(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q_len=0), -1), (dict(q_len=9), -1), (dict(capacity=0), -1), (dict(B=-1), -1),
    (dict(q=None), -1), (dict(pos=None), -1), (dict(ks=None), -1), (dict(vs=None), -1),
    (dict(window=512, capacity=512, q_len=2), -1),  # ring < W + q_len - 1
    (dict(theta=0.0), -1), (dict(p=1.5), -1), (dict(o=7), -1),
    (dict(d=128), -2), (dict(Hq=24), -2),
    (dict(ws=None), -4), (dict(ws_bytes=100), -4),
    (dict(ks=7 * A + 4), -3), (dict(out=4 * A + 2), -3), (dict(k=2 * A + 1), -3),
])
def test_decode_fp8_validation(kw, code):
    assert decf(**kw) == code


def test_decode_fp8_k_equals_v_needs_no_value_scale():
    # v NULL is K=V: a missing v_scale is fine, so the call gets as far as the
    # workspace check (which fails here on purpose, before any launch)
    assert decf(v=None, vs=None, ws_bytes=100) == -4
    assert decf(v=2 * A, vs=None, ws_bytes=100) == -4  # v == k is K=V too


def test_decode_fp8_empty_is_noop():
    assert decf(B=0, q=None, k=None, v=None, ks=None, vs=None, out=None, pos=None, ws=None) == 0


def test_decode_fp8_workspace_size():
    f = L.lib().g4attn_decode_fp8_workspace_bytes
    assert f(64, 1, 16, 2, 512, 65536, 0) == 64 * 16 * 64 * (512 + 2) * 4  # 1024-row chunks
    assert f(64, 1, 16, 8, 256, 512, 512) == 64 * 16 * 1 * (256 + 2) * 4  # one chunk per ring
    assert f(64, 4, 16, 8, 256, 515, 512) == 64 * 4 * 16 * 1 * (256 + 2) * 4
    assert f(2, 4, 16, 8, 256, 514, 512) == 0  # ring too small for 4 tokens
    assert f(2, 9, 16, 8, 256, 600, 512) == 0


def fill8(**kw):
    args = dict(k=A, v=2 * A, ks=6 * A, vs=7 * A, pos=3 * A, B=1, S=16, Hkv=8, d=256, kc=4 * A,
                vc=5 * A, capacity=512, window=512, theta=1e4, p=1.0, dtype=1, stream=None)
    args.update(kw)
    return L.lib().g4attn_fill_cache_fp8(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(pos=None), -1), (dict(kc=None), -1), (dict(vc=None), -1),
    (dict(ks=None), -1), (dict(vs=None), -1), (dict(B=-1), -1), (dict(Hkv=0), -1),
    (dict(capacity=0), -1), (dict(window=-1), -1),
    (dict(dtype=5), -2), (dict(d=24), -2),  # rows must be whole 16-code chunks
    (dict(k=A + 2), -3), (dict(kc=4 * A + 8), -3), (dict(vs=7 * A + 4), -3),
    (dict(theta=-1.0), -1), (dict(p=1.5), -1), (dict(d=1024), -2),
])
def test_fill_cache_fp8_validation(kw, code):
    assert fill8(**kw) == code


def test_fill_cache_fp8_empty_is_noop():
    assert fill8(S=0, k=None, v=None, ks=None, vs=None, pos=None, kc=None, vc=None) == 0


def vis(**kw):
    args = dict(q=A, k=2 * A, v=3 * A, out=4 * A, pos=5 * A, ln=6 * A, B=2, S=100, Hq=8, Hkv=8,
                d=256, theta=1e4, i=1, o=0, ws=7 * A, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return L.lib().g4attn_vision_prefill(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(pos=None), -1), (dict(out=None), -1),
    (dict(B=-1), -1), (dict(Hq=12), -1), (dict(theta=0.0), -1), (dict(o=5), -1),
    (dict(d=512), -2), (dict(d=128), -2), (dict(i=0, o=0), -2), (dict(Hq=24, Hkv=2), -2),
    (dict(ws=None), -4), (dict(ws_bytes=1000), -4),
    (dict(ln=6 * A + 4), -3), (dict(pos=5 * A + 8), -3),
])
def test_vision_prefill_validation(kw, code):
    assert vis(**kw) == code


def test_vision_prefill_lengths_may_be_null_and_empty_is_noop():
    assert vis(ln=None, ws_bytes=1000) == -4  # passes the other checks
    assert vis(S=0, q=None, k=None, v=None, out=None, pos=None, ln=None, ws=None) == 0
    assert vis(B=0, q=None, k=None, v=None, out=None, pos=None, ln=None, ws=None) == 0


def test_prefill_rejects_key_rows_past_the_24_bit_row_offset():
    """The bf16 prefill kernels compute a key row's offset inside a tile with a
    24-bit multiply, so Hkv * d * 2 must stay below 2^24 bytes."""
    big = 1 << 14  # Hkv * 512 * 2 = 2^24 at d = 512; 2^23 at d = 256 still fits
    assert glob(Hq=big * 8, Hkv=big) == -2
    assert glob(Hq=(big - 1) * 8, Hkv=big - 1, ws=None) == -4  # fits; fails on the workspace
    assert local(Hq=2 * big, Hkv=big, ws=None) == -4  # d = 256: 2^23 bytes fit
    assert local(Hq=4 * big, Hkv=2 * big) == -2
    assert vis(Hq=2 * big, Hkv=2 * big) == -2


def dec_noalloc(**kw):
    args = dict(q=A, k=2 * A, v=None, out=4 * A, pos=5 * A, B=16, Hq=16, Hkv=2, d=512,
                capacity=65536, window=0, theta=1e6, p=0.25, i=1, o=0, stream=None)
    args.update(kw)
    return L.lib().g4attn_decode_noalloc(*args.values())


@pytest.mark.parametrize("kw,code", [
    # partials past the fixed 64 MiB scratch: 64 x 16 heads x 64 chunks x 514 x 4 B
    (dict(B=64), -6), (dict(B=8, capacity=262144), -6),
    (dict(q=None), -1), (dict(pos=None), -1), (dict(out=None), -1), (dict(B=-1), -1),
    (dict(capacity=0), -1), (dict(window=512, capacity=1024), -1), (dict(Hq=5), -1),
    (dict(d=384), -2), (dict(Hq=48, Hkv=3, B=2), -2), (dict(i=0, o=1), -2),
])
def test_decode_noalloc_validation(kw, code):
    """Rejected before any HIP call, the size check first."""
    assert dec_noalloc(**kw) == code


def test_decode_noalloc_empty_batch_is_noop():
    assert dec_noalloc(B=0, q=None, k=None, out=None, pos=None) == 0
