"""HIP kernels vs the fp64 oracle, element by element, through the C ABI.

Sizes keep the oracle to seconds while spanning several query tiles (16 tokens
for d=512/G=8 ... 128 tokens for G=1), several 32-key KV tiles and ragged
tails.  Tolerances: fp32 inputs max |err| <= 1e-4; bf16 inputs max |err| <=
1e-2 and mean |err| <= 1e-3, measured on fp32 outputs.
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


def run_prefill(layer, dtype, offset=0, window=None, out_dtype=None, wl=90, idx=0):
    q, k, v, pos = inputs.prefill_inputs(layer, wl, idx, dtype, DEV, offset)
    W = layer.window if window is None else window
    print(f"prefill {layer} {dtype} W={W} offset={offset}", flush=True)
    if layer.kind == "global":
        out = g4.global_prefill(q, k, pos, W, layer.theta, layer.p, out_dtype=out_dtype)
    else:
        out = g4.local_prefill(q, k, v, pos, W, layer.theta, layer.p, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, (q, k, v, pos, W)


def oracle_prefill(layer, q, k, v, pos, W, rows=None):
    return oracle.prefill(to_oracle(q), to_oracle(k), to_oracle(v), pos.cpu().numpy(), W,
                          layer.theta, layer.p, rows=rows)


def test_tiny_fp32_local_and_global():
    for layer in (inputs.TINY_LOCAL, inputs.TINY_GLOBAL):
        out, (q, k, v, pos, W) = run_prefill(layer, torch.float32, wl=1)
        ref = oracle_prefill(layer, q, k, v, pos, W)
        assert_parity(out, ref, torch.float32, str(layer))


SMALL = [
    # kind, B, S, Hq, Hkv, d, window, theta, p
    inputs.Layer("global", 1, 300, 8, 1, 512, 0, 1e6, 0.25),
    inputs.Layer("global", 2, 77, 16, 2, 512, 0, 1e6, 0.25),
    inputs.Layer("local", 2, 333, 4, 2, 256, 64, 1e4, 1.0),
    inputs.Layer("local", 1, 700, 16, 8, 256, 256, 1e4, 1.0),
    inputs.Layer("local", 1, 200, 2, 2, 256, 1, 1e4, 1.0),
    inputs.Layer("global", 1, 150, 4, 1, 256, 0, 1e6, 0.5),
    inputs.Layer("local", 1, 190, 8, 2, 512, 40, 1e4, 0.25),
    inputs.Layer("global", 1, 129, 2, 1, 512, 0, 1e4, 0.0),
    inputs.Layer("local", 1, 100, 4, 4, 256, 0, 1e4, 0.25),
    inputs.Layer("local", 1, 170, 4, 2, 512, 70, 1e4, 0.5),   # separate K/V, d=512, 128 pairs turn
    inputs.Layer("global", 1, 140, 8, 1, 512, 0, 1e6, 1.0),   # K=V, every pair turns
    inputs.Layer("global", 1, 203, 8, 2, 512, 0, 1e6, 0.25),  # G=4: 32 tokens per workgroup
    inputs.Layer("global", 1, 211, 8, 1, 512, 96, 1e6, 0.25),  # window on the K=V path
    inputs.Layer("local", 1, 1100, 8, 4, 256, 512, 1e4, 1.0),  # small-model window 512
    # window not a multiple of the 32-key tile: spans of 34 tiles visited in
    # rotated order, a short span at the start, a ragged last query tile
    inputs.Layer("local", 2, 2500, 4, 2, 256, 1000, 1e4, 1.0),
]


@pytest.mark.parametrize("layer", SMALL, ids=lambda l: f"{l.kind}-S{l.S}-G{l.Hq // l.Hkv}-d{l.d}-W{l.window}-p{l.p}")
def test_bf16_prefill_small(layer):
    out, (q, k, v, pos, W) = run_prefill(layer, torch.bfloat16)
    ref = oracle_prefill(layer, q, k, v, pos, W)
    assert_parity(out, ref, torch.bfloat16, str(layer))


@pytest.mark.parametrize("layer", [SMALL[0], SMALL[2]], ids=["global", "local"])
def test_bf16_prefill_fp32_path_for_f32_inputs_small(layer):
    out, (q, k, v, pos, W) = run_prefill(layer, torch.float32)
    ref = oracle_prefill(layer, q, k, v, pos, W)
    assert_parity(out, ref, torch.float32, str(layer))


def test_caller_workspace_of_queried_size_with_stale_contents():
    """The key-slab workspace needs no initialisation: NaN bytes left in it by
    an earlier user do not reach the output."""
    for layer in (SMALL[0], SMALL[3]):
        q, k, v, pos = inputs.prefill_inputs(layer, 91, 0, torch.bfloat16, DEV)
        need = g4.prefill_workspace_bytes(layer.B, layer.S, layer.Hkv, layer.d, layer.p)
        ws = torch.full((need // 2,), float("nan"), dtype=torch.bfloat16, device=DEV)
        W = layer.window
        if layer.kind == "global":
            out = g4.global_prefill(q, k, pos, W, layer.theta, layer.p, workspace=ws)
        else:
            out = g4.local_prefill(q, k, v, pos, W, layer.theta, layer.p, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out, oracle_prefill(layer, q, k, v, pos, W), torch.bfloat16, str(layer))
        with pytest.raises(g4.G4AttnError, match="EWORKSPACE"):
            g4.global_prefill(q, k, pos, W, layer.theta, layer.p, workspace=ws[:need // 2 - 8]) \
                if layer.kind == "global" else \
                g4.local_prefill(q, k, v, pos, W, layer.theta, layer.p, workspace=ws[:need // 2 - 8])


def test_large_positions_offset():
    """Positions near 2^18: rotation angles must stay accurate."""
    layer = inputs.Layer("global", 1, 160, 8, 1, 512, 0, 1e6, 0.25)
    out, (q, k, v, pos, W) = run_prefill(layer, torch.bfloat16, offset=200000)
    assert_parity(out, oracle_prefill(layer, q, k, v, pos, W), torch.bfloat16, "offset global")
    layer = inputs.Layer("local", 1, 160, 4, 2, 256, 48, 1e4, 1.0)
    out, (q, k, v, pos, W) = run_prefill(layer, torch.bfloat16, offset=261000)
    assert_parity(out, oracle_prefill(layer, q, k, v, pos, W), torch.bfloat16, "offset local")


@pytest.mark.parametrize("layer", [SMALL[0], SMALL[2], SMALL[5]],
                         ids=["global-d512", "local-d256", "kv-d256"])
def test_bf16_output(layer):
    """bf16 output: the d = 512 epilogue stores from the accumulators, the
    d = 256 one stages whole rows through LDS first (ragged S included)."""
    out, (q, k, v, pos, W) = run_prefill(layer, torch.bfloat16, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ref = oracle_prefill(layer, q, k, v, pos, W)
    got = out.float().cpu().double().numpy()
    # bf16 storage adds at most half an ulp of the output: 2^-9 relative
    assert np.all(np.abs(got - ref) <= 1e-2 + 2.0 ** -8 * np.abs(ref))


def test_window_ge_seq_equals_global_and_k_equals_v_paths():
    layer = inputs.Layer("local", 1, 260, 8, 1, 512, 0, 1e6, 0.25)
    q, k, v, pos = inputs.prefill_inputs(layer, 91, 0, torch.bfloat16, DEV)
    a = g4.global_prefill(q, k, pos, 0, 1e6, 0.25)
    b = g4.global_prefill(q, k, pos, 260, 1e6, 0.25)
    c = g4.local_prefill(q, k, k.clone(), pos, 0, 1e6, 0.25)  # separate-V path fed v := k
    d = g4.global_prefill(q, k, pos, 0, 1e6, 0.25)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, d), "not deterministic"
    assert (a - c).abs().max().item() <= 1e-6


def test_unread_tail_and_guard_band():
    """Output rows are written exactly; memory past the output stays untouched."""
    layer = inputs.Layer("global", 1, 45, 8, 1, 512, 0, 1e6, 0.25)
    q, k, v, pos = inputs.prefill_inputs(layer, 92, 0, torch.bfloat16, DEV)
    n = 1 * 45 * 8 * 512
    buf = torch.full((n + 4096,), float("nan"), device=DEV)
    out = buf[:n].view(1, 45, 8, 512)
    g4.global_prefill(q, k, pos, 0, 1e6, 0.25, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.isnan(buf[n:]).all()


# ---------------------------------------------------------------- decode ----

def run_decode(layer, dtype, lengths, wl=95):
    q, kc, vc, pos, lengths = inputs.decode_inputs(layer, wl, 0, dtype, DEV, lengths)
    print(f"decode {layer} {dtype} lengths={lengths.tolist()[:8]}", flush=True)
    out = g4.decode(q, kc, vc, pos, layer.window, layer.theta, layer.p)
    torch.cuda.synchronize()
    ref = oracle.decode(to_oracle(q), to_oracle(kc), None if vc is None else to_oracle(vc),
                        pos.cpu().numpy(), layer.window, layer.theta, layer.p)
    return out, ref


DEC = [
    inputs.DecodeLayer("global", 4, 16, 2, 512, 3000, 0, 1e6, 0.25),
    inputs.DecodeLayer("local", 4, 16, 8, 256, 512, 512, 1e4, 1.0),
    inputs.DecodeLayer("local", 3, 8, 4, 256, 96, 96, 1e4, 1.0),
    inputs.DecodeLayer("global", 3, 8, 1, 512, 700, 0, 1e6, 0.25),
    # a 1024-slot ring: one chunk of 64 tiles for four waves, G = 1
    inputs.DecodeLayer("local", 4, 4, 4, 256, 1024, 1024, 1e4, 1.0),
    # separate K and V at d = 512 (one-wave path), every pair turning, G = 4
    inputs.DecodeLayer("local", 3, 8, 2, 512, 256, 256, 1e4, 1.0),
    # separate K and V in a linear cache (no window)
    inputs.DecodeLayer("local", 3, 4, 2, 256, 700, 0, 1e4, 1.0),
]


@pytest.mark.parametrize("layer", DEC, ids=lambda l: f"{l.kind}-C{l.capacity}-G{l.Hq // l.Hkv}")
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_small(layer, dtype):
    if layer.window > 0:
        lengths = torch.tensor([1, layer.window - 1, layer.window, 5 * layer.window + 3][:layer.B])
    else:
        C = layer.capacity
        lengths = torch.tensor([1, min(2049, C // 2 + 1), C, min(1500, C - 3)][:layer.B])
    out, ref = run_decode(layer, dtype, lengths)
    assert_parity(out, ref, dtype, str(layer))


@pytest.mark.parametrize("layer", [DEC[1], DEC[0]], ids=["local-direct", "global-merge"])
def test_decode_bf16_output(layer):
    lengths = torch.tensor([1, 300, layer.capacity, 77])
    q, kc, vc, pos, _ = inputs.decode_inputs(layer, 98, 0, torch.bfloat16, DEV, lengths)
    out = g4.decode(q, kc, vc, pos, layer.window, layer.theta, layer.p, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ref = oracle.decode(to_oracle(q), to_oracle(kc), None if vc is None else to_oracle(vc),
                        pos.cpu().numpy(), layer.window, layer.theta, layer.p)
    got = out.float().cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= 1e-2 + 2.0 ** -8 * np.abs(ref))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_value_cache_given_as_the_key_cache_is_k_equals_v(dtype):
    """v_cache passed as k_cache itself is K=V: the keys are read raw and
    turned (a separate value cache would mean keys cached turned), the same
    result as v_cache = None, on the GPU and in the oracle.  (Two decodes of
    the same inputs may differ slightly: waves claim tiles at run time, so a
    column's reference max, against which P is rounded to bf16, and the
    order the partials are summed in vary; about 1e-4 here.)"""
    layer = inputs.DecodeLayer("global", 2, 16, 2, 512, 1500, 0, 1e6, 0.25)
    lengths = torch.tensor([1500, 37])
    q, kc, _, pos, _ = inputs.decode_inputs(layer, 97, 0, dtype, DEV, lengths)
    print(f"decode v_cache=k_cache {dtype}", flush=True)
    a = g4.decode(q, kc, None, pos, 0, layer.theta, layer.p)
    b = g4.decode(q, kc, kc, pos, 0, layer.theta, layer.p)
    torch.cuda.synchronize()
    # reading the keys as cached turned would move the scores by O(1)
    assert (a - b).abs().max().item() <= 2e-3
    qo, ko, po = to_oracle(q), to_oracle(kc), pos.cpu().numpy()
    ref = oracle.decode(qo, ko, None, po, 0, layer.theta, layer.p)
    assert np.array_equal(oracle.decode(qo, ko, ko, po, 0, layer.theta, layer.p), ref)
    assert_parity(b, ref, dtype, "v_cache = k_cache")


def test_decode_ring_bad_positions_nan():
    """The ring path finishes rows in place: a negative position gives NaN there too."""
    layer = inputs.DecodeLayer("local", 3, 4, 2, 256, 512, 512, 1e4, 1.0)
    q, kc, vc, pos, _ = inputs.decode_inputs(layer, 99, 0, torch.bfloat16, DEV,
                                             torch.tensor([10, 600, 3]))
    pos = torch.tensor([-1, 599, -7], dtype=torch.int32, device=DEV)
    out = g4.decode(q, kc, vc, pos, 512, 1e4, 1.0)
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.isfinite(out[1]).all() and torch.isnan(out[2]).all()


@pytest.mark.parametrize("S", [1, 31, 33])
def test_prefill_short_sequences(S):
    for layer in (inputs.Layer("global", 2, S, 8, 1, 512, 0, 1e6, 0.25),
                  inputs.Layer("local", 2, S, 4, 2, 256, 16, 1e4, 1.0)):
        out, (q, k, v, pos, W) = run_prefill(layer, torch.bfloat16, wl=94)
        assert_parity(out, oracle_prefill(layer, q, k, v, pos, W), torch.bfloat16, str(layer))


def test_decode_bad_positions_nan():
    layer = inputs.DecodeLayer("global", 3, 8, 1, 512, 64, 0, 1e6, 0.25)
    q, kc, vc, pos, _ = inputs.decode_inputs(layer, 96, 0, torch.bfloat16, DEV,
                                             torch.tensor([10, 10, 10]))
    pos = torch.tensor([-1, 64, 5], dtype=torch.int32, device=DEV)
    out = g4.decode(q, kc, None, pos, 0, 1e6, 0.25)
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.isnan(out[1]).all() and torch.isfinite(out[2]).all()


def test_decode_many_sequences_mixed_lengths():
    """130 sequences (the grid's unit numbering scans them 64 at a time) over a
    3-chunk linear cache: lengths from 1 to the capacity, and positions past
    the cache or negative.  Workgroups map densely onto the chunks that hold
    visible rows; every good row must match and every bad one be NaN."""
    layer = inputs.DecodeLayer("global", 130, 8, 1, 512, 2500, 0, 1e6, 0.25)
    g = torch.Generator()
    g.manual_seed(5)
    lengths = torch.randint(1, layer.capacity + 1, (layer.B,), generator=g)
    lengths[:4] = torch.tensor([1, 1024, 1025, layer.capacity])
    q, kc, _, pos, _ = inputs.decode_inputs(layer, 93, 0, torch.bfloat16, DEV, lengths)
    bad = [5, 64, 65, 129]
    pos[bad] = torch.tensor([-1, layer.capacity, -7, layer.capacity + 4000],
                            dtype=torch.int32, device=DEV)
    out = g4.decode(q, kc, None, pos, 0, layer.theta, layer.p)
    torch.cuda.synchronize()
    good = [b for b in range(layer.B) if b not in bad]
    assert torch.isnan(out[bad]).all()
    ref = oracle.decode(to_oracle(q[good]), to_oracle(kc[good]), None,
                        pos[good].cpu().numpy(), 0, layer.theta, layer.p)
    assert_parity(out[good], ref, torch.bfloat16, "130 sequences")


def test_decode_equals_last_prefill_row():
    S = 517
    layer = inputs.Layer("global", 1, S, 16, 2, 512, 0, 1e6, 0.25)
    q, k, v, pos = inputs.prefill_inputs(layer, 97, 0, torch.bfloat16, DEV)
    pre = g4.global_prefill(q, k, pos, 0, 1e6, 0.25)
    cache = k.permute(0, 2, 1, 3).contiguous()
    dec = g4.decode(q[:, S - 1].contiguous(), cache, None,
                    torch.tensor([S - 1], dtype=torch.int32, device=DEV), 0, 1e6, 0.25)
    torch.cuda.synchronize()
    assert (dec - pre[:, S - 1]).abs().max().item() <= 1e-2


@pytest.mark.parametrize("kind", ["global", "local"])
def test_score_far_above_first_tile_takes_exact_path(kind):
    """A key whose score lies ~130 (base 2) above the row's first visible tile
    sends the row to the exact recompute path; the result must still match."""
    if kind == "global":
        layer = inputs.Layer("global", 1, 200, 8, 1, 512, 0, 1e6, 0.25)
    else:
        layer = inputs.Layer("local", 1, 300, 4, 2, 256, 128, 1e4, 1.0)
    q, k, v, pos = inputs.prefill_inputs(layer, 93, 0, torch.bfloat16, DEV)
    q = torch.ones_like(q)
    k = k.clone()
    k[:, :64] = 0          # rows' first tiles score exactly 0
    k[:, 150] = 8.0        # scores of key 150 are ~100 natural units
    if kind == "global":
        v = k
        out = g4.global_prefill(q, k, pos, 0, layer.theta, layer.p)
    else:
        out = g4.local_prefill(q, k, v, pos, layer.window, layer.theta, layer.p)
    torch.cuda.synchronize()
    ref = oracle_prefill(layer, q, k, v, pos, layer.window)
    assert_parity(out, ref, torch.bfloat16, f"overflow {kind}")
