"""HIP kernels vs the fp64 oracle at the full workload sizes, through the C ABI,
in the launch configuration the benchmark times (same entry points, same
seeded inputs, fp32 outputs).

The local prefill of B=4, S=8192 (window 1024) and decode are compared on every
output.  For the longer layers the oracle recomputes a deterministic sample of
query rows one by one (all heads of each row): the first rows, the rows around
the window edge, rows on both sides of query-tile and key-tile boundaries, the
last row, and seeded random rows.
Tolerance: bf16 inputs, max |err| <= 1e-2 and mean |err| <= 1e-3.
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


def sample_rows(S, W, n_random, seed, tile=128):
    rows = {0, 1, 2, S - 1, S - 2}
    if W > 0:
        rows |= {W - 2, W - 1, W, W + 1}
    for t in (tile, 2 * tile, S // 2 // tile * tile, (S - 1) // tile * tile):
        rows |= {t - 1, t, t + 1}
    for t in (32, 64, 96):  # key-tile edges inside the first query tile
        rows |= {t - 1, t}
    rng = np.random.default_rng(seed)
    rows |= set(int(r) for r in rng.choice(S, n_random, replace=False))
    return np.array(sorted(r for r in rows if 0 <= r < S), dtype=np.int64)


def check_prefill(layer, workload, index, n_random, seed, batches=None):
    q, k, v, pos = inputs.prefill_inputs(layer, workload, index, torch.bfloat16, DEV)
    print(f"fullsize prefill {layer} workload={workload} layer={index}", flush=True)
    ws = torch.empty(max(16, g4.prefill_workspace_bytes(layer.B, layer.S, layer.Hkv, layer.d,
                                                        layer.p)), dtype=torch.uint8, device=DEV)
    if layer.kind == "global":
        out = g4.global_prefill(q, k, pos, layer.window, layer.theta, layer.p, workspace=ws)
    else:
        out = g4.local_prefill(q, k, v, pos, layer.window, layer.theta, layer.p, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    S = layer.S
    ids = []
    for b in (range(layer.B) if batches is None else batches):
        ids.extend(b * S + sample_rows(S, layer.window, n_random, seed + b))
    ids = np.array(ids, dtype=np.int64)
    qh, kh = to_oracle(q), to_oracle(k)
    vh = kh if layer.kind == "global" else to_oracle(v)
    ref = oracle.prefill(qh, kh, vh, pos.cpu().numpy(), layer.window, layer.theta, layer.p,
                         rows=ids)
    got = out.view(layer.B * S, layer.Hq, layer.d)[torch.as_tensor(ids, device=DEV)]
    mx, mean = assert_parity(got, ref, torch.bfloat16, f"{layer} rows={len(ids)}")
    print(f"  rows {len(ids)}: max {mx:.2e} mean {mean:.2e}", flush=True)


def test_local_prefill_b4_s8192_every_row():
    """Every output row of the local prefill workload (B=4, S=8192, 16/8 heads,
    d=256, window 1024) against the oracle (5.2e11 oracle FLOPs)."""
    layer = inputs.LOCAL_PREFILL
    q, k, v, pos = inputs.prefill_inputs(layer, 2, 0, torch.bfloat16, DEV)
    print(f"fullsize prefill {layer} workload=2 layer=0 (every row)", flush=True)
    ws = torch.empty(g4.prefill_workspace_bytes(layer.B, layer.S, layer.Hkv, layer.d, layer.p),
                     dtype=torch.uint8, device=DEV)
    out = g4.local_prefill(q, k, v, pos, layer.window, layer.theta, layer.p, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ref = oracle.prefill(to_oracle(q), to_oracle(k), to_oracle(v), pos.cpu().numpy(),
                         layer.window, layer.theta, layer.p)
    mx, mean = assert_parity(out, ref, torch.bfloat16, f"{layer} every row")
    print(f"  rows {layer.B * layer.S}: max {mx:.2e} mean {mean:.2e}", flush=True)


def test_global_prefill_s32768():
    check_prefill(inputs.GLOBAL_PREFILL, 3, 0, n_random=12, seed=31)


def test_small_model_local_layer_window512_s131072():
    """The local layer of the small model sizes: window 512 at 128K context."""
    check_prefill(inputs.local(1, 131072, window=512), 8, 0, n_random=24, seed=81)


def test_group_local_layer_s262144():
    check_prefill(inputs.GROUP_LOCAL, 5, 0, n_random=32, seed=51)


def test_group_global_layer_s262144():
    layer = inputs.GROUP_GLOBAL
    q, k, _, pos = inputs.prefill_inputs(layer, 5, 5, torch.bfloat16, DEV)
    print(f"fullsize prefill {layer} workload=5 layer=5", flush=True)
    ws = torch.empty(g4.prefill_workspace_bytes(1, layer.S, layer.Hkv, layer.d, layer.p),
                     dtype=torch.uint8, device=DEV)
    out = g4.global_prefill(q, k, pos, 0, layer.theta, layer.p, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    # rows near the start are cheap for the oracle; the last rows see 2^18 keys.
    # Fixed rows at the starts and ends of query tiles (16 tokens) and key
    # tiles (32 keys), plus seeded random rows over the whole sequence.
    S = layer.S
    fixed = {0, 1, 15, 16, 17, 31, 32, 4095, 4096, 100000, S // 2, S - 33, S - 17, S - 16, S - 1}
    rnd = np.random.default_rng(55).choice(S, 20, replace=False)
    ids = np.array(sorted(fixed | {int(r) for r in rnd}), dtype=np.int64)
    ref = oracle.prefill(to_oracle(q), to_oracle(k), to_oracle(k), pos.cpu().numpy(), 0,
                         layer.theta, layer.p, rows=ids)
    got = out.view(S, layer.Hq, layer.d)[torch.as_tensor(ids, device=DEV)]
    mx, mean = assert_parity(got, ref, torch.bfloat16, f"{layer} rows={len(ids)}")
    print(f"  rows {len(ids)}: max {mx:.2e} mean {mean:.2e}", flush=True)


@pytest.mark.parametrize("layer", [inputs.DECODE_LOCAL, inputs.DECODE_GLOBAL],
                         ids=["local-ring512", "global-kv-linear65536"])
def test_decode_batch64(layer):
    lengths = inputs.decode_lengths(layer.B)
    q, kc, vc, pos, _ = inputs.decode_inputs(layer, 4, 0, torch.bfloat16, DEV, lengths)
    print(f"fullsize decode {layer}", flush=True)
    out = g4.decode(q, kc, vc, pos, layer.window, layer.theta, layer.p)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ref = oracle.decode(to_oracle(q), to_oracle(kc), None if vc is None else to_oracle(vc),
                        pos.cpu().numpy(), layer.window, layer.theta, layer.p)
    mx, mean = assert_parity(out, ref, torch.bfloat16, str(layer))
    print(f"  max {mx:.2e} mean {mean:.2e}", flush=True)


def test_decode_batch64_ring1024():
    """Local decode of the large model sizes: window 1024, a full 1024-slot
    ring per (sequence, KV head), batch 64, every sequence checked."""
    layer = inputs.DecodeLayer("local", 64, 16, 8, 256, 1024, 1024, inputs.LOCAL_THETA, 1.0)
    lengths = inputs.decode_lengths(layer.B)
    q, kc, vc, pos, _ = inputs.decode_inputs(layer, 84, 0, torch.bfloat16, DEV, lengths)
    print(f"fullsize decode {layer}", flush=True)
    out = g4.decode(q, kc, vc, pos, layer.window, layer.theta, layer.p)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ref = oracle.decode(to_oracle(q), to_oracle(kc), to_oracle(vc), pos.cpu().numpy(),
                        layer.window, layer.theta, layer.p)
    mx, mean = assert_parity(out, ref, torch.bfloat16, str(layer))
    print(f"  max {mx:.2e} mean {mean:.2e}", flush=True)


def test_decode_global_256k_context():
    """Global K=V decode over a 262144-row linear cache with lengths drawn up
    to the context (8 sequences, so the oracle stays within seconds)."""
    layer = inputs.DecodeLayer("global", 8, 16, 2, 512, 262144, 0, inputs.GLOBAL_THETA, 0.25)
    lengths = inputs.decode_lengths(layer.B, 4011, 4096, 262144)
    lengths[0] = 262144  # one sequence fills the cache
    q, kc, _, pos, _ = inputs.decode_inputs(layer, 85, 0, torch.bfloat16, DEV, lengths)
    print(f"fullsize decode {layer} lengths={lengths.tolist()}", flush=True)
    out = g4.decode(q, kc, None, pos, 0, layer.theta, layer.p)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ref = oracle.decode(to_oracle(q), to_oracle(kc), None, pos.cpu().numpy(), 0, layer.theta,
                        layer.p)
    mx, mean = assert_parity(out, ref, torch.bfloat16, str(layer))
    print(f"  max {mx:.2e} mean {mean:.2e}", flush=True)
