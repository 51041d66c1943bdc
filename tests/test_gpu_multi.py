"""Cache fill and decode of several query tokens per sequence, through the C ABI,
against the fp64 oracle (GPU).

- g4attn_fill_cache places rows: compared with oracle.fill_cache, bit for bit
  for values, K=V rows and untouched slots; the turned keys of a cache with
  separate values (fp32 turn on the GPU, exact then rounded once in the
  oracle) to one bf16 unit in the last place, or a few fp32 ones.
- g4attn_decode_multi is compared element by element with oracle.decode_multi on
  the same caches, across ring and linear caches, K=V and separate K/V, the
  one-wave d = 512 path, one to four 16-column blocks (G * q_len up to 64),
  several cache chunks (merge kernel), fp32 inputs and bf16 outputs.
- Closed loop: prefill, fill the cache with the prompt and then the new
  tokens, decode the new tokens at once: equals the oracle's prefill rows.
- Full size, at the benchmark's shapes: 4-token decode of batch 64 over the
  515-slot rings and the 64K K=V cache (12 sampled sequences compared), and
  the fill of the 256K-token K=V prefill (sampled rows, bit for bit).
Tolerances as for the other parity tests (bf16: max 1e-2, mean 1e-3; f32 1e-4).
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


def _cache_pair(layer, dtype, seed_):
    shape = (layer.B, layer.Hkv, layer.capacity, layer.d)
    k = inputs.randn(shape, seed_, dtype, DEV)
    v = None if layer.kind == "global" else inputs.randn(shape, seed_ + 1, dtype, DEV)
    return k, v


def assert_turned_keys(got, want, dtype, written, what):
    """Turned keys: equal but for the last rounding.  bf16: the GPU rounds its
    fp32 turn, the oracle the exact one, so they may land one unit in the
    last place (2^-7 relative) apart, rarely; f32: within a few fp32 units
    (the fp32 sine, cosine and products differ from the exact ones in the
    last bits of most keys)."""
    g, w = np.asarray(got, np.float64), np.asarray(want, np.float64)
    rel = 2.0 ** -7 if dtype == torch.bfloat16 else 4e-7
    bad = np.abs(g - w) > rel * np.abs(w) + 1e-6
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} keys off by more than 1 ulp"
    if dtype == torch.bfloat16:
        differ = (g != w)[written]
        assert differ.mean() < 0.02, f"{what}: {differ.mean():.3%} of turned keys differ"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("case", ["ring", "ring-wrap", "linear", "linear-kv", "ring-p25"])
def test_fill_cache_parity(case, dtype):
    B, Hkv, d = 2, 3, 256
    if case == "ring":        # short prompt into a larger ring
        S, C, W, off, kv = 40, 64, 64, 0, False
    elif case == "ring-wrap": # more tokens than slots: the last C land, wrapped
        S, C, W, off, kv = 150, 64, 60, 37, False
    elif case == "linear":    # some positions past the cache and negative ones skipped
        S, C, W, off, kv = 50, 45, 0, -3, False
    elif case == "ring-p25":  # p-RoPE at large positions: only the first pairs turn
        S, C, W, off, kv = 30, 64, 64, 200000, False
    else:
        S, C, W, off, kv = 33, 80, 0, 10, True
    theta, p = (1e6, 0.25) if case == "ring-p25" else (1e4, 1.0)
    k = inputs.randn((B, S, Hkv, d), 501, dtype, DEV)
    v = None if kv else inputs.randn((B, S, Hkv, d), 502, dtype, DEV)
    pos = inputs.positions(B, S, DEV, off)
    kc = torch.full((B, Hkv, C, d), 7.0, dtype=dtype, device=DEV)
    vc = None if kv else torch.full((B, Hkv, C, d), -3.0, dtype=dtype, device=DEV)
    want_k, want_v = oracle.fill_cache(to_oracle(k), None if kv else to_oracle(v),
                                       pos.cpu().numpy(), to_oracle(kc),
                                       None if kv else to_oracle(vc), W, theta, p)
    print(f"fill_cache {case} {dtype}", flush=True)
    g4.fill_cache(k, v, pos, kc, vc, W, theta, p)
    torch.cuda.synchronize()
    if kv:
        assert np.array_equal(to_oracle(kc), want_k)
        return
    assert np.array_equal(to_oracle(vc), want_v)
    got = kc.float().cpu().numpy()
    want = (torch.from_numpy(want_k.view(np.int16)).view(torch.bfloat16).float().numpy()
            if dtype == torch.bfloat16 else want_k)
    written = (to_oracle(vc) != to_oracle(torch.full_like(vc, -3.0)))
    assert np.array_equal(got[~written], want[~written])  # slots not written keep their bytes
    assert_turned_keys(got, want, dtype, written, f"{case} {dtype}")


def _run_multi(layer, L, dtype, lengths, seed_, out_dtype=None):
    kc, vc = _cache_pair(layer, dtype, seed_)
    if layer.window == 0:  # rows past each sequence are never read
        for b in range(layer.B):
            kc[b, :, int(lengths[b]):] = float("nan")
    q = inputs.randn((layer.B, L, layer.Hq, layer.d), seed_ + 2, dtype, DEV)
    pos = (lengths - 1).to(torch.int32).to(DEV)
    print(f"decode_multi {layer} L={L} {dtype} lengths={lengths.tolist()}", flush=True)
    out = g4.decode_multi(q, kc, vc, pos, layer.window, layer.theta, layer.p,
                          out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.decode_multi(to_oracle(q), to_oracle(kc), None if vc is None else to_oracle(vc),
                              pos.cpu().numpy(), layer.window, layer.theta, layer.p)
    return out, ref


# kind, B, Hq, Hkv, d, capacity, window, theta, p
MULTI = [
    # local ring, G = 2: capacity exactly window + L - 1
    ("local-ring-min", lambda L: inputs.DecodeLayer("local", 3, 16, 8, 256, 64 + L - 1, 64,
                                                    1e4, 1.0), (1, 3, 8)),
    # local ring of 512 slots plus room for the draft tokens (with one token,
    # the 7 oldest slots hold keys before the window)
    ("local-ring-512", lambda L: inputs.DecodeLayer("local", 2, 16, 8, 256, 519, 512, 1e4, 1.0),
     (1, 4, 8)),
    # global K=V linear cache, G = 8: 1 to 4 column blocks, several 1024-row chunks
    ("global-kv", lambda L: inputs.DecodeLayer("global", 2, 16, 2, 512, 3000, 0, 1e6, 0.25),
     (1, 2, 3, 8)),
    # separate K/V at d = 512 (one-wave path), G = 4, every pair turning
    ("local-sep512", lambda L: inputs.DecodeLayer("local", 2, 8, 2, 512, 300, 0, 1e4, 1.0),
     (4, 5)),
]
CASES = [(name, mk, L) for name, mk, Ls in MULTI for L in Ls]


@pytest.mark.parametrize("name,mk,L", CASES, ids=[f"{c[0]}-L{c[2]}" for c in CASES])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_multi_parity(name, mk, L, dtype):
    layer = mk(L)
    if layer.window > 0:
        lengths = torch.tensor([L, layer.capacity - 1, 5 * layer.capacity + 3][:layer.B])
    else:
        lengths = torch.tensor([L + 1, layer.capacity, 1700][:layer.B])
    out, ref = _run_multi(layer, L, dtype, lengths, 700 + 10 * L)
    assert_parity(out, ref, dtype, f"{name} L={L}")


# K=V with more than 16 (token, head) columns: every column block is computed
# by one workgroup whose waves split the head dims (ring caches are one chunk
# and written in place; linear caches go through the merge kernel)
MANY_COLUMNS = [
    # ring of 70 slots at window 64, G = 8, 5 tokens: 40 columns in 3 blocks
    ("kv-ring-g8-L5", lambda: inputs.DecodeLayer("global", 3, 16, 2, 512, 70, 64, 1e6, 0.25), 5),
    # G = 4, d = 256, every pair turning, 6 tokens: 24 columns in 2 blocks
    ("kv-g4-d256-L6", lambda: inputs.DecodeLayer("global", 3, 8, 2, 256, 2100, 0, 1e4, 1.0), 6),
    # G = 8, 7 tokens: 56 columns in 4 blocks, 2 chunks
    ("kv-g8-L7", lambda: inputs.DecodeLayer("global", 3, 16, 2, 512, 1500, 0, 1e6, 0.25), 7),
]


@pytest.mark.parametrize("name,mk,L", MANY_COLUMNS, ids=[c[0] for c in MANY_COLUMNS])
@pytest.mark.parametrize("out_dtype", [None, torch.bfloat16], ids=["f32out", "bf16out"])
def test_decode_multi_many_columns_one_pass(name, mk, L, out_dtype):
    layer = mk()
    if layer.window > 0:  # a short sequence, a full ring, a wrapped ring
        lengths = torch.tensor([L, layer.capacity - 1, 5 * layer.capacity + 3])
    else:  # a sequence shorter than the tokens (NaN rows), one chunk edge, the capacity
        lengths = torch.tensor([L - 2, 1025, layer.capacity])
    out, ref = _run_multi(layer, L, torch.bfloat16, lengths, 1300 + L, out_dtype=out_dtype)
    got = out.float()
    if layer.window == 0:  # tokens 0, 1 of sequence 0 sit at negative positions
        assert torch.isnan(got[0, :2]).all() and torch.isfinite(got[0, 2:]).all()
        got, ref = got[:, 2:], ref[:, 2:]
    assert torch.isfinite(got).all()
    if out_dtype is None:
        assert_parity(got, ref, torch.bfloat16, f"{name}")
    else:
        g = got.cpu().double().numpy()
        assert np.all(np.abs(g - ref) <= 1e-2 + 2.0 ** -8 * np.abs(ref))


def test_decode_multi_bf16_output():
    layer = inputs.DecodeLayer("global", 2, 16, 2, 512, 2100, 0, 1e6, 0.25)
    out, ref = _run_multi(layer, 3, torch.bfloat16, torch.tensor([2100, 40]), 900,
                          out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    got = out.float().cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= 1e-2 + 2.0 ** -8 * np.abs(ref))


def test_decode_multi_many_sequences_two_column_blocks():
    """70 sequences (two 64-sequence scans of the grid numbering), 3 tokens of
    G = 8 heads (two column blocks), a 3-chunk K=V cache, lengths from 3 to the
    capacity and two positions past it (NaN rows)."""
    layer = inputs.DecodeLayer("global", 70, 16, 2, 512, 2100, 0, 1e6, 0.25)
    g = torch.Generator()
    g.manual_seed(11)
    lengths = torch.randint(3, layer.capacity + 1, (layer.B,), generator=g)
    lengths[:3] = torch.tensor([3, 1024, layer.capacity])
    kc, _ = _cache_pair(layer, torch.bfloat16, 960)
    q = inputs.randn((layer.B, 3, layer.Hq, layer.d), 962, torch.bfloat16, DEV)
    pos = (lengths - 1).to(torch.int32).to(DEV)
    bad = [64, 69]
    pos[bad] = layer.capacity + 3
    out = g4.decode_multi(q, kc, None, pos, 0, layer.theta, layer.p)
    torch.cuda.synchronize()
    assert torch.isnan(out[bad]).all()
    good = [b for b in range(layer.B) if b not in bad]
    ref = oracle.decode_multi(to_oracle(q[good]), to_oracle(kc[good]), None,
                              pos[good].cpu().numpy(), 0, layer.theta, layer.p)
    assert_parity(out[good], ref, torch.bfloat16, "70 sequences, 3 tokens")


@pytest.mark.parametrize("window", [0, 32])
def test_decode_multi_negative_token_positions_nan(window):
    """pos = 1 with 4 tokens: tokens 0 and 1 sit at -2 and -1 and give NaN rows."""
    C = 40 if window else 100
    layer = inputs.DecodeLayer("local", 2, 4, 2, 256, C, window, 1e4, 1.0)
    kc, vc = _cache_pair(layer, torch.bfloat16, 950)
    q = inputs.randn((2, 4, 4, 256), 951, torch.bfloat16, DEV)
    pos = torch.tensor([1, 30], dtype=torch.int32, device=DEV)
    out = g4.decode_multi(q, kc, vc, pos, window, 1e4, 1.0)
    torch.cuda.synchronize()
    assert torch.isnan(out[0, :2]).all() and torch.isfinite(out[0, 2:]).all()
    assert torch.isfinite(out[1]).all()
    ref = oracle.decode_multi(to_oracle(q), to_oracle(kc), to_oracle(vc), pos.cpu().numpy(),
                              window, 1e4, 1.0)
    assert_parity(out[0, 2:], ref[0, 2:], torch.bfloat16, "valid tokens")


@pytest.mark.parametrize("kind", ["local", "global"])
def test_prefill_fill_cache_decode_closed_loop(kind):
    """Prefill S tokens; fill the cache with the first S-L as a prompt and the
    last L as new tokens; decoding the L tokens at once gives the prefill rows."""
    L = 4
    if kind == "local":
        layer = inputs.Layer("local", 2, 300, 16, 8, 256, 64, 1e4, 1.0)
        C = layer.window + L - 1
    else:
        layer = inputs.Layer("global", 1, 300, 16, 2, 512, 0, 1e6, 0.25)
        C = 512
    q, k, v, pos = inputs.prefill_inputs(layer, 97, 0, torch.bfloat16, DEV)
    S = layer.S
    kv = kind == "global"
    kc = torch.full((layer.B, layer.Hkv, C, layer.d), float("nan"), dtype=torch.bfloat16,
                    device=DEV)
    vc = None if kv else torch.full_like(kc, float("nan"))
    print(f"closed loop {layer} C={C}", flush=True)
    g4.fill_cache(k[:, :S - L].contiguous(), None if kv else v[:, :S - L].contiguous(),
                  pos[:, :S - L].contiguous(), kc, vc, layer.window, layer.theta, layer.p)
    g4.fill_cache(k[:, S - L:].contiguous(), None if kv else v[:, S - L:].contiguous(),
                  pos[:, S - L:].contiguous(), kc, vc, layer.window, layer.theta, layer.p)
    out = g4.decode_multi(q[:, S - L:].contiguous(), kc, vc,
                          torch.full((layer.B,), S - 1, dtype=torch.int32, device=DEV),
                          layer.window, layer.theta, layer.p)
    torch.cuda.synchronize()
    rows = np.array([b * S + i for b in range(layer.B) for i in range(S - L, S)], np.int64)
    ref = oracle.prefill(to_oracle(q), to_oracle(k), to_oracle(v), pos.cpu().numpy(),
                         layer.window, layer.theta, layer.p, rows=rows)
    ref = ref.reshape(layer.B, L, layer.Hq, layer.d)
    assert_parity(out, ref, torch.bfloat16, f"closed loop {kind}")


@pytest.mark.parametrize("kind", ["local-ring515", "global-kv-linear65536"])
def test_decode_multi_full_size_sampled_sequences(kind):
    """4 query tokens per sequence at the benchmark's shapes (batch 64); every
    output of 12 sampled sequences compared (the GPU computes all 64)."""
    L = 4
    if kind.startswith("local"):
        base = inputs.DECODE_LOCAL
        layer = inputs.DecodeLayer(base.kind, base.B, base.Hq, base.Hkv, base.d,
                                   base.window + L - 1, base.window, base.theta, base.p)
    else:
        layer = inputs.DECODE_GLOBAL
    lengths = inputs.decode_lengths(layer.B)
    _, kc, vc, pos, _ = inputs.decode_inputs(layer, 62, 0, torch.bfloat16, DEV, lengths)
    q = inputs.randn((layer.B, L, layer.Hq, layer.d), 6201, torch.bfloat16, DEV)
    print(f"decode_multi full size {kind}", flush=True)
    out = g4.decode_multi(q, kc, vc, pos, layer.window, layer.theta, layer.p)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    seqs = sorted({0, layer.B - 1} | set(np.random.default_rng(63).choice(layer.B, 10, replace=False)
                                          .tolist()))
    for b in seqs:
        P = int(pos[b])
        rows = layer.capacity if layer.window > 0 else P + 1  # the rows a linear cache holds
        ref = oracle.decode_multi(to_oracle(q[b:b + 1]), to_oracle(kc[b:b + 1, :, :rows]),
                                  None if vc is None else to_oracle(vc[b:b + 1, :, :rows]),
                                  pos[b:b + 1].cpu().numpy(), layer.window, layer.theta, layer.p)
        assert_parity(out[b:b + 1], ref, torch.bfloat16, f"{kind} b={b}")


def test_fill_cache_group_global_prefill_s262144_sampled_rows():
    """The fill the benchmark times: the 256K-token K=V rows into a linear
    cache; sampled rows compared bit for bit with the oracle's fill."""
    gl = inputs.global_(1, inputs.GROUP_S)
    k = inputs.randn((gl.B, gl.S, gl.Hkv, gl.d), 6201, torch.bfloat16, DEV)
    p = inputs.positions(gl.B, gl.S, DEV)
    kc = torch.empty((gl.B, gl.Hkv, gl.S, gl.d), dtype=torch.bfloat16, device=DEV)
    print("fill_cache full size", flush=True)
    g4.fill_cache(k, None, p, kc, None, 0)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 4095, 4096, gl.S // 2, gl.S - 1}
                           | set(np.random.default_rng(64).choice(gl.S, 26, replace=False)
                                 .tolist())), np.int64)
    sub_k = k[:, torch.as_tensor(rows, device=DEV)].contiguous()       # [1, n, Hkv, d]
    sub_p = torch.arange(rows.size, dtype=torch.int32)[None].numpy()   # slot i for row i
    want, _ = oracle.fill_cache(to_oracle(sub_k), None, sub_p,
                                np.zeros((1, gl.Hkv, rows.size, gl.d), np.uint16), None, 0)
    got = kc[:, :, torch.as_tensor(rows, device=DEV)].contiguous()
    assert np.array_equal(to_oracle(got), want)
