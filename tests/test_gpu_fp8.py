"""Low-precision (FP8 E4M3) KV caches through the C ABI, against the fp64 oracle
(GPU).

- g4attn_fill_cache_fp8 quantizes: its codes are compared with
  oracle.fill_cache_fp8 (bf16 and fp32 inputs; ring, wrapped ring, linear and
  K=V caches; quotients that saturate, that fall in the subnormal range, and
  that sit exactly halfway between two codes) bit for bit, except the turned
  keys of caches with separate values (fp32 turn on the GPU, exact in the
  oracle): a quotient next to a rounding boundary may take the neighbouring
  code there.
- g4attn_decode_fp8 is compared element by element with oracle.decode_fp8 on
  the same codes and scales: ring and linear caches, K=V and separate K/V at
  d = 256 and 512, G = 1 to 8, 1 to 8 query tokens (1 to 4 column blocks),
  several 1024-row chunks (merge kernel), ragged last tiles, bf16 output,
  positions out of range (NaN rows).
- Closed loop: prefill rows -> fill_cache_fp8 -> decode_fp8 matches the
  oracle's fill (as above) and decode of the same rows.
- Full size: batch-64 decode at the local ring-512 and the global 64K shapes,
  every sequence checked; the fill of a 256K-token global prefill, sampled
  rows checked bit for bit.
The codes are widened exactly, so the decode tolerance is the bf16 one (max
|err| <= 1e-2, mean <= 1e-3).
"""
import numpy as np
import pytest
import torch

import attention_g4attn_amd as g4
import oracle
from attention_g4attn_amd import inputs
from tests.helpers import assert_parity, to_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def np8(t):
    return None if t is None else t.detach().contiguous().cpu().numpy()


def halfway_inputs(shape, scale, dtype):
    """Values x with x / scale exactly halfway between two neighbouring E4M3
    values (scale a power of two, so the quotient is exact)."""
    v = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double()
    mid = ((v[:-1] + v[1:]) / 2)
    n = int(np.prod(shape))
    idx = torch.arange(n) % mid.numel()
    sign = 1 - 2 * ((torch.arange(n) // mid.numel()) % 2)
    x = (mid[idx] * sign * scale).reshape(shape)
    return x.to(dtype).to(DEV)


def assert_turned_codes(got, want, what):
    """Codes of turned keys: equal, or neighbouring codes (no code value lies
    between theirs) where the GPU's fp32 turn and the oracle's exact one put
    the quotient on either side of a rounding boundary; rare."""
    vals = oracle.e4m3_values()
    grid = np.unique(vals[np.isfinite(vals)])
    g, w = vals[got], vals[want]
    lo, hi = np.minimum(g, w), np.maximum(g, w)
    between = np.searchsorted(grid, hi, "left") - np.searchsorted(grid, lo, "right")
    assert ((got == want) | (between == 0)).all(), f"{what}: codes more than one step apart"
    assert (got != want).mean() < 0.01, f"{what}: {(got != want).mean():.3%} of key codes differ"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("case", ["ring", "ring-wrap", "linear", "linear-kv", "halfway"])
def test_fill_cache_fp8_parity(case, dtype):
    B, Hkv, d = 2, 3, 256
    if case == "ring":
        S, C, W, off, kv = 40, 64, 64, 0, False
    elif case == "ring-wrap":
        S, C, W, off, kv = 150, 64, 60, 37, False
    elif case == "linear":
        S, C, W, off, kv = 50, 45, 0, -3, False
    else:
        S, C, W, off, kv = 33, 80, 0, 10, True
    if case == "halfway":
        ks = torch.tensor([0.25, 1.0, 4.0], device=DEV)
        vs = ks
        k = halfway_inputs((B, S, Hkv, d), 1.0, dtype) * ks.cpu().to(dtype).to(DEV)[None, None, :, None]
        v = None
    else:
        # N(0, 40^2) against scales 0.05 .. 0.3: quotients from the subnormal
        # range to far beyond 448 (saturated)
        ks = torch.tensor([0.05, 0.11, 0.3], device=DEV)
        vs = torch.tensor([0.07, 0.2, 0.013], device=DEV)
        k = inputs.randn((B, S, Hkv, d), 511, torch.float32, DEV).mul_(40).to(dtype)
        v = None if kv else inputs.randn((B, S, Hkv, d), 512, torch.float32,
                                         DEV).mul_(40).to(dtype)
    pos = inputs.positions(B, S, DEV, off)
    kc = torch.full((B, Hkv, C, d), 0x5A, dtype=torch.uint8, device=DEV)
    vc = None if v is None else torch.full((B, Hkv, C, d), 0xA5, dtype=torch.uint8, device=DEV)
    want_k, want_v = oracle.fill_cache_fp8(to_oracle(k), None if v is None else to_oracle(v),
                                           pos.cpu().numpy(), np8(kc), np8(vc), W, np8(ks),
                                           None if v is None else np8(vs), 1e4, 1.0)
    print(f"fill_cache_fp8 {case} {dtype}", flush=True)
    g4.fill_cache_fp8(k, v, pos, kc, vc, W, ks, None if v is None else vs, 1e4, 1.0)
    torch.cuda.synchronize()
    if v is None:
        assert np.array_equal(np8(kc), want_k)
        return
    assert np.array_equal(np8(vc), want_v)
    assert_turned_codes(np8(kc), want_k, f"{case} {dtype}")


def oracle_fp8(q, kc, vc, ks, vs, pos, window, theta, p):
    """oracle.decode_fp8 one sequence at a time over only the rows it may read
    (a linear cache is cut after the last query's row), so a full-size cache is
    never dequantized whole."""
    q, kc, vc = to_oracle(q), np8(kc), np8(vc)
    ks, vs = np8(ks), np8(vs)
    pos = pos.cpu().numpy()
    out = np.empty(q.shape, np.float64)
    for b in range(q.shape[0]):
        P = int(pos[b])
        rows = kc.shape[2] if window > 0 or P < 0 or P >= kc.shape[2] else P + 1
        out[b] = oracle.decode_fp8(q[b:b + 1], kc[b:b + 1, :, :rows],
                                   None if vc is None else vc[b:b + 1, :, :rows], ks, vs,
                                   pos[b:b + 1], window, theta, p)[0]
    return out


# name, layer for L, token counts
CASES = [
    # local ring, G = 2, separate K/V at d = 256: capacity exactly window + L - 1
    ("local-ring-min", lambda L: inputs.DecodeLayer("local", 3, 16, 8, 256, 64 + L - 1, 64,
                                                    1e4, 1.0), (1, 3, 8)),
    ("local-ring-512", lambda L: inputs.DecodeLayer("local", 2, 16, 8, 256, 512 + L - 1, 512,
                                                    1e4, 1.0), (1, 4)),
    # global K=V linear, G = 8, p-RoPE: several 1024-row chunks, 1 to 4 column blocks
    ("global-kv", lambda L: inputs.DecodeLayer("global", 2, 16, 2, 512, 3000, 0, 1e6, 0.25),
     (1, 2, 3, 8)),
    # global K=V with G = 4 and G = 1 at d = 256 (K=V tiles of 8 KB)
    ("global-g4", lambda L: inputs.DecodeLayer("global", 2, 8, 2, 512, 1500, 0, 1e6, 0.25),
     (1,)),
    ("kv-d256-g1", lambda L: inputs.DecodeLayer("global", 2, 4, 4, 256, 700, 0, 1e6, 1.0),
     (2,)),
    # separate K/V at d = 512, every pair turning, G = 4
    ("sep512", lambda L: inputs.DecodeLayer("local", 2, 8, 2, 512, 300, 0, 1e4, 1.0), (1, 5)),
    # K=V rings with p-RoPE: keys past the ring's wrap take the second per-tile angle
    ("kv-ring-p25", lambda L: inputs.DecodeLayer("global", 3, 16, 2, 512, 70 + L - 1, 64, 1e6,
                                                 0.25), (1, 4)),
    # K=V at d = 256 with 32 of 64 table pairs turning (per-pair select)
    ("kv-d256-p25", lambda L: inputs.DecodeLayer("global", 2, 16, 2, 256, 900, 0, 1e4, 0.25),
     (1, 2)),
]
PARAMS = [(name, mk, L) for name, mk, Ls in CASES for L in Ls]


def run_fp8(layer, L, lengths, workload, out_dtype=None):
    q, kc, vc, ks, vs, pos, _ = inputs.decode_inputs_fp8(layer, workload, 0, DEV, lengths, L)
    print(f"decode_fp8 {layer} L={L} lengths={lengths.tolist()}", flush=True)
    out = g4.decode_fp8(q, kc, vc, ks, vs, pos, layer.window, layer.theta, layer.p,
                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle_fp8(q, kc, vc, ks, vs, pos, layer.window, layer.theta, layer.p)
    return out, ref


@pytest.mark.parametrize("name,mk,L", PARAMS, ids=[f"{c[0]}-L{c[2]}" for c in PARAMS])
def test_decode_fp8_parity(name, mk, L):
    layer = mk(L)
    if layer.window > 0:  # a short sequence, a full ring, a ring wrapped several times
        lengths = torch.tensor([L, layer.capacity - 1, 5 * layer.capacity + 3][:layer.B])
    else:                 # ragged tails inside a tile, a chunk edge, the whole cache
        lengths = torch.tensor([L + 1, layer.capacity, 1025][:layer.B])
        lengths = lengths.clamp(max=layer.capacity)
    out, ref = run_fp8(layer, L, lengths, 60 + L)
    assert torch.isfinite(out).all()
    assert_parity(out, ref, torch.bfloat16, f"{name} L={L}")


def test_decode_fp8_bf16_output():
    layer = inputs.DecodeLayer("global", 2, 16, 2, 512, 2100, 0, 1e6, 0.25)
    out, ref = run_fp8(layer, 3, torch.tensor([2100, 40]), 70, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    got = out.float().cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= 1e-2 + 2.0 ** -8 * np.abs(ref))


@pytest.mark.parametrize("window", [0, 32])
def test_decode_fp8_positions_out_of_range_nan(window):
    """Tokens at negative positions, and a linear cache's sequence whose last
    token lies past the cache, give NaN rows; the others are unaffected."""
    C = 40 if window else 100
    layer = inputs.DecodeLayer("local", 3, 4, 2, 256, C + 3 if window else C, window, 1e4, 1.0)
    q, kc, vc, ks, vs, _, _ = inputs.decode_inputs_fp8(layer, 71, 0, DEV,
                                                       torch.tensor([C, C, C]), 4)
    pos = torch.tensor([1, 30, C + 5 if window == 0 else 77], dtype=torch.int32, device=DEV)
    out = g4.decode_fp8(q, kc, vc, ks, vs, pos, window, 1e4, 1.0)
    torch.cuda.synchronize()
    assert torch.isnan(out[0, :2]).all() and torch.isfinite(out[0, 2:]).all()
    assert torch.isfinite(out[1]).all()
    if window == 0:
        assert torch.isnan(out[2]).all()
    ref = oracle_fp8(q, kc, vc, ks, vs, pos, window, 1e4, 1.0)
    assert_parity(out[0, 2:], ref[0, 2:], torch.bfloat16, "valid tokens")
    assert_parity(out[1], ref[1], torch.bfloat16, "sequence 1")


def test_decode_fp8_many_sequences_mixed_lengths():
    """70 sequences over a 3-chunk linear K=V cache, lengths from 1 to the
    capacity and out-of-range positions (the grid maps workgroups only onto
    chunks with visible rows)."""
    layer = inputs.DecodeLayer("global", 70, 8, 1, 512, 2200, 0, 1e6, 0.25)
    g = torch.Generator()
    g.manual_seed(6)
    lengths = torch.randint(1, layer.capacity + 1, (layer.B,), generator=g)
    lengths[:3] = torch.tensor([1, 1024, layer.capacity])
    q, kc, _, ks, _, pos, _ = inputs.decode_inputs_fp8(layer, 74, 0, DEV, lengths)
    bad = [3, 63, 64, 69]
    pos[bad] = torch.tensor([-1, layer.capacity, -9, layer.capacity + 1],
                            dtype=torch.int32, device=DEV)
    out = g4.decode_fp8(q, kc, None, ks, None, pos, 0, layer.theta, layer.p)
    torch.cuda.synchronize()
    good = [b for b in range(layer.B) if b not in bad]
    assert torch.isnan(out[bad]).all()
    ref = oracle_fp8(q[good], kc[good], None, ks, None, pos[good], 0, layer.theta, layer.p)
    assert_parity(out[good], ref, torch.bfloat16, "70 sequences")


@pytest.mark.parametrize("kind", ["local", "global"])
def test_prefill_rows_fill_fp8_decode_closed_loop(kind):
    """Prefill rows quantized into the cache as a prompt and then new tokens;
    the codes match the oracle's (turned keys up to a neighbouring code), and
    decoding the new tokens at once equals the oracle's decode of its codes."""
    L = 4
    if kind == "local":
        layer = inputs.Layer("local", 2, 300, 16, 8, 256, 64, 1e4, 1.0)
        C = layer.window + L - 1
    else:
        layer = inputs.Layer("global", 1, 300, 16, 2, 512, 0, 1e6, 0.25)
        C = 512
    q, k, v, pos = inputs.prefill_inputs(layer, 98, 0, torch.bfloat16, DEV)
    S, kv = layer.S, kind == "global"
    ks = inputs.kv_scales(layer.Hkv, 98, DEV, 0.01, 0.02)  # N(0,1) rows -> codes up to ~400
    vs = None if kv else inputs.kv_scales(layer.Hkv, 99, DEV, 0.01, 0.02)
    kc = torch.full((layer.B, layer.Hkv, C, layer.d), 0x7F, dtype=torch.uint8, device=DEV)
    vc = None if kv else kc.clone()
    ok, ov = np8(kc), np8(vc)
    for sl in (slice(0, S - L), slice(S - L, S)):
        kk, vv, pp = k[:, sl].contiguous(), None if kv else v[:, sl].contiguous(), \
            pos[:, sl].contiguous()
        g4.fill_cache_fp8(kk, vv, pp, kc, vc, layer.window, ks, vs, layer.theta, layer.p)
        ok, ov = oracle.fill_cache_fp8(to_oracle(kk), None if kv else to_oracle(vv),
                                       pp.cpu().numpy(), ok, ov, layer.window, np8(ks), np8(vs),
                                       layer.theta, layer.p)
    last = torch.full((layer.B,), S - 1, dtype=torch.int32, device=DEV)
    print(f"fp8 closed loop {layer} C={C}", flush=True)
    out = g4.decode_fp8(q[:, S - L:].contiguous(), kc, vc, ks, vs, last, layer.window,
                        layer.theta, layer.p)
    torch.cuda.synchronize()
    if kv:
        assert np.array_equal(np8(kc), ok)
    else:
        assert np.array_equal(np8(vc), ov)
        assert_turned_codes(np8(kc), ok, f"closed loop {kind}")
    ref = oracle.decode_fp8(to_oracle(q[:, S - L:]), ok, ov, np8(ks), np8(vs),
                            last.cpu().numpy(), layer.window, layer.theta, layer.p)
    assert_parity(out, ref, torch.bfloat16, f"fp8 closed loop {kind}")


@pytest.mark.parametrize("layer", [inputs.DECODE_LOCAL, inputs.DECODE_GLOBAL],
                         ids=["local-ring512", "global-kv-linear65536"])
def test_decode_fp8_batch64_full_size(layer):
    lengths = inputs.decode_lengths(layer.B)
    out, ref = run_fp8(layer, 1, lengths, 4)
    assert torch.isfinite(out).all()
    mx, mean = assert_parity(out, ref, torch.bfloat16, f"fp8 {layer}")
    print(f"  max {mx:.2e} mean {mean:.2e}", flush=True)


def test_fill_fp8_group_global_prefill_s262144_sampled_rows():
    """The fill the benchmark times: a 256K-token K=V prefill into a linear
    fp8 cache; sampled token rows compared bit for bit."""
    layer = inputs.GROUP_GLOBAL
    _, k, _, pos = inputs.prefill_inputs(layer, 5, 5, torch.bfloat16, DEV)
    ks = inputs.kv_scales(layer.Hkv, 5, DEV, 0.01, 0.02)
    kc = torch.empty((1, layer.Hkv, layer.S, layer.d), dtype=torch.uint8, device=DEV)
    print(f"fill fp8 {layer}", flush=True)
    g4.fill_cache_fp8(k, None, pos, kc, None, 0, ks)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 511, 512, 100000, layer.S // 2, layer.S - 2, layer.S - 1}
                           | set(np.random.default_rng(3).choice(layer.S, 24, replace=False)
                                 .tolist())), np.int64)
    want = oracle.quantize_e4m3(to_oracle(k[0, torch.as_tensor(rows, device=DEV)]), np8(ks))
    got = kc[0][:, torch.as_tensor(rows, device=DEV)].permute(1, 0, 2).contiguous()
    assert np.array_equal(np8(got), want)


def test_decode_fp8_ring_at_large_positions():
    """Ring decode at positions near 2^24 (the queries' angle reduction at
    large arguments; the keys are cached turned), 3 query tokens, G = 2."""
    layer = inputs.DecodeLayer("local", 2, 16, 8, 256, 64 + 2, 64, 1e4, 1.0)
    q, kc, vc, ks, vs, _, _ = inputs.decode_inputs_fp8(layer, 73, 0, DEV,
                                                       torch.tensor([66, 66]), 3)
    pos = torch.tensor([(1 << 24) - 5, (1 << 24) + 12345], dtype=torch.int32, device=DEV)
    out = g4.decode_fp8(q, kc, vc, ks, vs, pos, layer.window, layer.theta, layer.p)
    torch.cuda.synchronize()
    ref = oracle_fp8(q, kc, vc, ks, vs, pos, layer.window, layer.theta, layer.p)
    assert torch.isfinite(out).all()
    assert_parity(out, ref, torch.bfloat16, "fp8 ring at large positions")
