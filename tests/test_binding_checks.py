"""The Python binding rejects tensors whose dtype or shape does not match the
call before anything reaches the C ABI, which sees only pointers and sizes
(CPU only: the metadata checks run before the device-placement check, so CPU
tensors with the right metadata fail on placement instead)."""
import pytest
import torch

import attention_g4attn_amd as g4

bf, f32, i32, i64 = torch.bfloat16, torch.float32, torch.int32, torch.int64


def T(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


PLACEMENT = "GPU memory"


def local_args(**kw):
    a = dict(q=T(1, 8, 4, 256), k=T(1, 8, 2, 256), v=T(1, 8, 2, 256), pos=T(1, 8, dtype=i32),
             window=4)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(pos=T(1, 8, dtype=i64)), TypeError, "pos"),
    (dict(pos=T(8, dtype=i32)), ValueError, "pos"),
    (dict(k=T(1, 8, 2, 256, dtype=f32)), TypeError, "k"),
    (dict(v=T(1, 8, 2, 128)), ValueError, "v"),
    (dict(v=T(1, 8, 1, 256)), ValueError, "v"),
    (dict(k=T(1, 7, 2, 256)), ValueError, "k"),
    (dict(out=T(1, 8, 4, 128, dtype=f32)), ValueError, "out"),
    (dict(out=T(1, 8, 4, 256, dtype=torch.float16)), TypeError, "out"),
    (dict(q=T(1, 8, 4, 256, dtype=torch.float16)), TypeError, "q"),
])
def test_local_prefill_checks(kw, exc, msg):
    with pytest.raises(exc, match=msg):
        g4.local_prefill(**local_args(**kw))


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(pos=T(1, 16, dtype=i64)), TypeError, "pos"),
    (dict(kv=T(1, 16, 1, 256)), ValueError, "kv"),
    (dict(kv=T(1, 16, 1, 512, dtype=f32)), TypeError, "kv"),
    (dict(out=T(1, 16, 8, 512, dtype=f32)[:, :8]), ValueError, "out"),
])
def test_global_prefill_checks(kw, exc, msg):
    a = dict(q=T(1, 16, 8, 512), kv=T(1, 16, 1, 512), pos=T(1, 16, dtype=i32))
    a.update(kw)
    with pytest.raises(exc, match=msg):
        g4.global_prefill(**a)


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(pos2=T(2, 10, dtype=i32)), ValueError, "pos2"),
    (dict(pos2=T(2, 10, 2, dtype=i64)), TypeError, "pos2"),
    (dict(lengths=T(3, dtype=i32)), ValueError, "lengths"),
    (dict(lengths=T(2, dtype=i64)), TypeError, "lengths"),
    (dict(v=T(2, 10, 4, 128)), ValueError, "v"),
])
def test_vision_prefill_checks(kw, exc, msg):
    a = dict(q=T(2, 10, 8, 256), k=T(2, 10, 4, 256), v=T(2, 10, 4, 256),
             pos2=T(2, 10, 2, dtype=i32))
    a.update(kw)
    with pytest.raises(exc, match=msg):
        g4.vision_prefill(**a)


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(pos=T(3, dtype=i64)), TypeError, "pos"),
    (dict(pos=T(3, 1, dtype=i32)), ValueError, "pos"),
    (dict(k_cache=T(3, 2, 64, 256)), ValueError, "k_cache"),
    (dict(k_cache=T(3, 2, 64, 512, dtype=f32)), TypeError, "k_cache"),
    (dict(v_cache=T(3, 2, 32, 512)), ValueError, "v_cache"),
    (dict(out=T(3, 16, 256, dtype=f32)), ValueError, "out"),
])
def test_decode_checks(kw, exc, msg):
    a = dict(q=T(3, 16, 512), k_cache=T(3, 2, 64, 512), v_cache=None, pos=T(3, dtype=i32),
             window=0, theta=1e6, p=0.25)
    a.update(kw)
    with pytest.raises(exc, match=msg):
        g4.decode(**a)


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(out=T(3, 2, 16, 512, dtype=f32)), ValueError, "out"),
    (dict(q=T(3, 16, 512)), ValueError, "q"),
    (dict(k_cache=T(3, 2, 64, 256)), ValueError, "k_cache"),
])
def test_decode_multi_checks(kw, exc, msg):
    a = dict(q=T(3, 4, 16, 512), k_cache=T(3, 2, 64, 512), v_cache=None, pos=T(3, dtype=i32),
             window=0, theta=1e6, p=0.25)
    a.update(kw)
    with pytest.raises(exc, match=msg):
        g4.decode_multi(**a)


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(k_cache=T(1, 8, 32, 256, dtype=f32)), TypeError, "k_cache"),
    (dict(v_cache=T(1, 8, 16, 256)), ValueError, "v_cache"),
    (dict(v_cache=None), ValueError, "v_cache"),
    (dict(pos=T(1, 16, dtype=i64)), TypeError, "pos"),
    (dict(v=T(1, 16, 4, 256)), ValueError, "v"),
    (dict(theta=None), ValueError, "turned keys"),
    (dict(p=None), ValueError, "turned keys"),
])
def test_fill_cache_checks(kw, exc, msg):
    a = dict(k=T(1, 16, 8, 256), v=T(1, 16, 8, 256), pos=T(1, 16, dtype=i32),
             k_cache=T(1, 8, 32, 256), v_cache=T(1, 8, 32, 256), window=32, theta=1e4, p=1.0)
    a.update(kw)
    with pytest.raises(exc, match=msg):
        g4.fill_cache(**a)


u8 = torch.uint8


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(k_cache=T(1, 8, 32, 256)), TypeError, "k_cache"),
    (dict(k_scale=T(4, dtype=f32)), ValueError, "scale"),
    (dict(k_scale=T(8, dtype=bf)), TypeError, "scale"),
    (dict(v_scale=None), ValueError, "v_scale"),
    (dict(theta=None), ValueError, "turned keys"),
])
def test_fill_cache_fp8_checks(kw, exc, msg):
    a = dict(k=T(1, 16, 8, 256), v=T(1, 16, 8, 256), pos=T(1, 16, dtype=i32),
             k_cache=T(1, 8, 32, 256, dtype=u8), v_cache=T(1, 8, 32, 256, dtype=u8), window=32,
             k_scale=T(8, dtype=f32), v_scale=T(8, dtype=f32), theta=1e4, p=1.0)
    a.update(kw)
    with pytest.raises(exc, match=msg):
        g4.fill_cache_fp8(**a)


@pytest.mark.parametrize("kw,exc,msg", [
    ({}, ValueError, PLACEMENT),
    (dict(q=T(2, 1, 16, 512, dtype=f32)), TypeError, "bfloat16"),
    (dict(k_cache=T(2, 2, 64, 256, dtype=u8)), ValueError, "k_cache"),
    (dict(k_scale=T(3, dtype=f32)), ValueError, "scale"),
    (dict(pos=T(2, dtype=i64)), TypeError, "pos"),
    (dict(out=T(2, 1, 16, 512, dtype=torch.float16)), TypeError, "out"),
])
def test_decode_fp8_checks(kw, exc, msg):
    a = dict(q=T(2, 1, 16, 512), k_cache=T(2, 2, 64, 512, dtype=u8), v_cache=None,
             k_scale=T(2, dtype=f32), v_scale=None, pos=T(2, dtype=i32), window=0, theta=1e6,
             p=0.25)
    a.update(kw)
    with pytest.raises(exc, match=msg):
        g4.decode_fp8(**a)
