"""g4attn_decode_noalloc (partials in the library's fixed device scratch)
against g4attn_decode (partials in a caller workspace), through the C ABI, on
consecutive calls that reuse the scratch, the later ones smaller; the oracle
checks both.  Tolerance as every bf16 decode: max |err| <= 1e-2 and mean
|err| <= 1e-3."""
import pytest
import torch

import attention_g4attn_amd as g4
import oracle
from attention_g4attn_amd import inputs
from tests.helpers import assert_parity, errors, to_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"

CALLS = [  # (layer, lengths): each call smaller than the one before
    (inputs.DecodeLayer("global", 16, 16, 2, 512, 65536, 0, inputs.GLOBAL_THETA, 0.25),
     inputs.decode_lengths(16, 4021, 4096, 65536)),
    (inputs.DecodeLayer("global", 5, 16, 2, 512, 3000, 0, inputs.GLOBAL_THETA, 0.25),
     torch.tensor([3000, 1, 1025, 2048, 2999])),
    (inputs.DecodeLayer("local", 64, 16, 8, 256, 512, 512, inputs.LOCAL_THETA, 1.0),
     inputs.decode_lengths(64)),
    (inputs.DecodeLayer("local", 3, 4, 2, 256, 512, 512, inputs.LOCAL_THETA, 1.0),
     torch.tensor([600, 512, 4096])),
]


def test_noalloc_decode_matches_workspace_decode_on_consecutive_calls():
    for i, (layer, lengths) in enumerate(CALLS):
        print(f"noalloc call {i}: {layer} lengths={lengths.tolist()[:6]}", flush=True)
        q, kc, vc, pos, _ = inputs.decode_inputs(layer, 130 + i, 0, torch.bfloat16, DEV, lengths)
        ref_ws = g4.decode(q, kc, vc, pos, layer.window, layer.theta, layer.p)
        got = torch.full(ref_ws.shape, float("nan"), dtype=torch.float32, device=DEV)
        g4.decode_noalloc(q, kc, vc, pos, layer.window, layer.theta, layer.p, out=got)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        mx, mean = errors(got, ref_ws.double().cpu().numpy())
        # the bf16 decode's bar; the two can differ by more than rounding
        # noise because waves claim cache tiles dynamically, so each wave's
        # partial (and the bf16 rounding of its P) differs from run to run
        assert mx <= 1e-2 and mean <= 1e-3, (i, mx, mean)
        ref = oracle.decode(to_oracle(q), to_oracle(kc), None if vc is None else to_oracle(vc),
                            pos.cpu().numpy(), layer.window, layer.theta, layer.p)
        assert_parity(got, ref, torch.bfloat16, f"noalloc call {i}")


def test_noalloc_decode_bf16_output_and_bad_positions():
    layer = inputs.DecodeLayer("global", 4, 16, 2, 512, 2048, 0, inputs.GLOBAL_THETA, 0.25)
    q, kc, _, pos, _ = inputs.decode_inputs(layer, 140, 0, torch.bfloat16, DEV,
                                            torch.tensor([2048, 700, 1, 1500]))
    pos[1] = -1          # a bad position gives a NaN row
    pos[2] = 5000        # past the linear cache: NaN row
    got = torch.zeros((4, 16, 512), dtype=torch.bfloat16, device=DEV)
    g4.decode_noalloc(q, kc, None, pos, 0, layer.theta, layer.p, out=got)
    ref_ws = g4.decode(q, kc, None, pos, 0, layer.theta, layer.p, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.isnan(got[1].float()).all() and torch.isnan(got[2].float()).all()
    for b in (0, 3):
        mx, _ = errors(got[b], ref_ws[b].double().cpu().numpy())
        assert mx <= 1e-2, (b, mx)


def test_noalloc_decode_rejects_partials_past_the_scratch():
    layer = inputs.DECODE_GLOBAL  # batch 64 over 65536 rows: 135 MB of partials
    q = torch.zeros((layer.B, layer.Hq, layer.d), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros(layer.B, dtype=torch.int32, device=DEV)
    out = torch.empty((layer.B, layer.Hq, layer.d), dtype=torch.float32, device=DEV)
    big = torch.empty((layer.B, layer.Hkv, 65536, layer.d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(g4.G4AttnError, match="G4A_ESCRATCH"):
        g4.decode_noalloc(q, big, None, pos, 0, layer.theta, layer.p, out=out)
