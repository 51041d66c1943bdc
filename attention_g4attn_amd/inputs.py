"""Seeded synthetic inputs and workload shapes.

Shared by the tests, the benchmark and the oracle side alike; holds none of
the attention arithmetic.  Every tensor is N(0, 1) drawn with a torch.Generator
on the device that will hold it, seeded 1000*workload + 10*layer + tensor
(q = 1, k or kv = 2, v = 3), then rounded to the input dtype.  Positions are
0..S-1.  The shapes follow the layer geometry the pages give for Gemma 4:
local layers with a 512/1024 window, 2 query heads per KV head and head dim
256; global layers with 8 query heads per KV head, head dim 512, K=V and
p = 0.25 ("Guia visual do Gemma 4", sections "Intercalacao de camadas de
atencao", "GQA", "Tecnica K=V", "p-RoPE"; techtoday page, attention section);
contexts up to 256K ("Visao geral do modelo Gemma 4", section "Recursos").
"""
from dataclasses import dataclass

import torch

LOCAL_THETA, GLOBAL_THETA = 1.0e4, 1.0e6


@dataclass(frozen=True)
class Layer:
    kind: str  # "local" (separate K, V) or "global" (K = V)
    B: int
    S: int
    Hq: int
    Hkv: int
    d: int
    window: int
    theta: float
    p: float


def local(B, S, Hq=16, Hkv=8, d=256, window=1024):
    return Layer("local", B, S, Hq, Hkv, d, window, LOCAL_THETA, 1.0)


def global_(B, S, Hq=16, Hkv=2, d=512):
    return Layer("global", B, S, Hq, Hkv, d, 0, GLOBAL_THETA, 0.25)


# Workloads (sizes of one GPU's share at the model's real shapes).
TINY_LOCAL = Layer("local", 1, 128, 4, 2, 256, 32, LOCAL_THETA, 1.0)  # fp32 inputs
TINY_GLOBAL = Layer("global", 1, 128, 8, 1, 512, 0, GLOBAL_THETA, 0.25)  # fp32 inputs
LOCAL_PREFILL = local(4, 8192)                                        # bf16
GLOBAL_PREFILL = Layer("global", 1, 32768, 32, 4, 512, 0, GLOBAL_THETA, 0.25)
GROUP_S = 262144
GROUP_LOCAL = local(1, GROUP_S)      # x5 per group
GROUP_GLOBAL = global_(1, GROUP_S)   # x1 per group


@dataclass(frozen=True)
class DecodeLayer:
    kind: str
    B: int
    Hq: int
    Hkv: int
    d: int
    capacity: int
    window: int  # > 0: ring cache of `window` slots
    theta: float
    p: float


DECODE_LOCAL = DecodeLayer("local", 64, 16, 8, 256, 512, 512, LOCAL_THETA, 1.0)
DECODE_GLOBAL = DecodeLayer("global", 64, 16, 2, 512, 65536, 0, GLOBAL_THETA, 0.25)
DECODE_LEN_RANGE = (4096, 65536)  # cache lengths, uniform, inclusive


def seed(workload, layer, tensor):
    return 1000 * workload + 10 * layer + tensor


def randn(shape, seed_, dtype, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed_)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def positions(B, S, device, offset=0):
    return (torch.arange(S, dtype=torch.int32, device=device) + offset).repeat(B, 1).contiguous()


def prefill_inputs(layer: Layer, workload, index, dtype, device, offset=0):
    """q, k, v (v is k for a global layer), pos."""
    q = randn((layer.B, layer.S, layer.Hq, layer.d), seed(workload, index, 1), dtype, device)
    k = randn((layer.B, layer.S, layer.Hkv, layer.d), seed(workload, index, 2), dtype, device)
    v = k if layer.kind == "global" else randn((layer.B, layer.S, layer.Hkv, layer.d),
                                               seed(workload, index, 3), dtype, device)
    return q, k, v, positions(layer.B, layer.S, device, offset)


def decode_lengths(B, seed_=4009, lo=DECODE_LEN_RANGE[0], hi=DECODE_LEN_RANGE[1]):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_)
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)


def decode_inputs(layer: DecodeLayer, workload, index, dtype, device, lengths=None):
    """q [B,Hq,d], k_cache, v_cache (None for K=V), pos [B] int32, lengths [B].

    Ring caches are full: every slot holds a token.  A linear cache holds
    lengths[b] tokens; the rows beyond are filled with NaN, which the kernels
    must never read.  The query token is the last cached one: pos = length - 1.
    """
    B = layer.B
    if lengths is None:
        lengths = decode_lengths(B)
    lengths = lengths.to(torch.int64)
    q = randn((B, layer.Hq, layer.d), seed(workload, index, 1), dtype, device)
    shape = (B, layer.Hkv, layer.capacity, layer.d)
    k = torch.empty(shape, dtype=dtype, device=device)
    v = None if layer.kind == "global" else torch.empty(shape, dtype=dtype, device=device)
    for b in range(B):  # per-sequence draws keep the temporary small
        k[b] = randn(shape[1:], seed(workload, index, 2) * 100003 + b, dtype, device)
        if v is not None:
            v[b] = randn(shape[1:], seed(workload, index, 3) * 100003 + b, dtype, device)
        if layer.window == 0:
            L = int(lengths[b])
            k[b, :, L:] = float("nan")
    pos = (lengths - 1).to(torch.int32).to(device)
    return q, k, v, pos, lengths


def e4m3_codes(shape, seed_, device, spread=8.0):
    """E4M3 codes (uint8) of N(0, spread^2) draws, through torch's float8_e4m3fn
    cast (|x| stays far below 448 for spread 8, so nothing saturates)."""
    x = randn(shape, seed_, torch.float32, device) * spread
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def kv_scales(Hkv, seed_, device, lo=0.08, hi=0.16):
    """Per-KV-head cache scales, uniform in [lo, hi): code values of spread 8
    times these are about N(0, 1)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_)
    return (lo + (hi - lo) * torch.rand(Hkv, generator=g, dtype=torch.float32)).to(device)


def decode_inputs_fp8(layer: DecodeLayer, workload, index, device, lengths=None, q_len=1):
    """q [B, q_len, Hq, d] bf16, E4M3 caches [B, Hkv, capacity, d] uint8 (v None
    for K=V), k_scale, v_scale [Hkv] float32 (v_scale None for K=V), pos [B]
    int32 (last query's position), lengths [B].  As decode_inputs: ring caches
    are full; a linear cache holds lengths[b] tokens and NaN codes (0x7F) past
    them, which the kernels must never read."""
    B = layer.B
    if lengths is None:
        lengths = decode_lengths(B)
    lengths = lengths.to(torch.int64)
    q = randn((B, q_len, layer.Hq, layer.d), seed(workload, index, 1), torch.bfloat16, device)
    shape = (B, layer.Hkv, layer.capacity, layer.d)
    k = torch.empty(shape, dtype=torch.uint8, device=device)
    v = None if layer.kind == "global" else torch.empty(shape, dtype=torch.uint8, device=device)
    for b in range(B):
        k[b] = e4m3_codes(shape[1:], seed(workload, index, 2) * 100003 + b, device)
        if v is not None:
            v[b] = e4m3_codes(shape[1:], seed(workload, index, 3) * 100003 + b, device)
        if layer.window == 0:
            k[b, :, int(lengths[b]):] = 0x7F
    ks = kv_scales(layer.Hkv, seed(workload, index, 4), device)
    vs = None if v is None else kv_scales(layer.Hkv, seed(workload, index, 5), device)
    pos = (lengths - 1).to(torch.int32).to(device)
    return q, k, v, ks, vs, pos, lengths


# Vision encoder: images as grids of 16x16-pixel patches, at most 9 x budget
# patches for a soft-token budget of 70 .. 1120 ("Guia visual do Gemma 4",
# sections "Encoder de visao" and "Suporte a resolucao variavel").  The pages
# give no head geometry for the encoder: 8 heads of dim 256 (MHA).
@dataclass(frozen=True)
class VisionLayer:
    grids: tuple  # (w, h) patch grid of each image; S = the largest w*h
    Hq: int = 8
    Hkv: int = 8
    d: int = 256
    theta: float = LOCAL_THETA

    @property
    def B(self):
        return len(self.grids)

    @property
    def S(self):
        return max(w * h for w, h in self.grids)


VISION_280 = VisionLayer(((60, 42), (42, 60), (56, 45), (48, 52)))  # budget 280: <= 2520 patches
VISION_1120 = VisionLayer(((120, 84),))                              # budget 1120: 10080 patches


def vision_positions(layer: VisionLayer, device):
    """pos2 [B, S, 2] int32 = (w, h) of each patch in raster order (rows of
    the grid one after the other), zeros past an image's patches; lengths [B]."""
    B, S = layer.B, layer.S
    pos = torch.zeros((B, S, 2), dtype=torch.int32)
    lengths = torch.empty(B, dtype=torch.int32)
    for b, (w, h) in enumerate(layer.grids):
        n = w * h
        i = torch.arange(n, dtype=torch.int32)
        pos[b, :n, 0] = i % w
        pos[b, :n, 1] = i // w
        lengths[b] = n
    return pos.to(device), lengths.to(device)


def vision_inputs(layer: VisionLayer, workload, dtype, device):
    """q [B,S,Hq,d], k, v [B,S,Hkv,d], pos2 [B,S,2], lengths [B]."""
    B, S = layer.B, layer.S
    q = randn((B, S, layer.Hq, layer.d), seed(workload, 0, 1), dtype, device)
    k = randn((B, S, layer.Hkv, layer.d), seed(workload, 0, 2), dtype, device)
    v = randn((B, S, layer.Hkv, layer.d), seed(workload, 0, 3), dtype, device)
    pos2, lengths = vision_positions(layer, device)
    return q, k, v, pos2, lengths
