"""Vision-encoder attention (2D RoPE, no causal mask) through the C ABI against
the fp64 oracle (GPU).

- Small and medium shapes, every row compared: G = 1, 2, 8; sequence lengths
  that leave ragged key tiles and partial workgroups; padded images (lengths
  below S, down to an image with no patch); random and raster grid positions;
  fp32 and bf16 outputs; a batch of eight images (sampled rows).
- A score far above the row's first tile takes the exact recompute path.
- Full size: budget-280 batch (4 images up to 2520 patches, one padded) and
  one budget-1120 image (10080 patches), sampled rows of every image, the
  padding rows checked to be zero.
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


def run(q, k, v, pos2, lengths, theta=1e4, out_dtype=None):
    out = g4.vision_prefill(q, k, v, pos2, theta, lengths=lengths, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def ref_rows(q, k, v, pos2, lengths, theta=1e4, rows=None):
    return oracle.vision_prefill(to_oracle(q), to_oracle(k), to_oracle(v), pos2.cpu().numpy(),
                                 theta, None if lengths is None else lengths.cpu().numpy(),
                                 rows=rows)


SMALL = [  # B, S, Hq, Hkv, lengths
    (3, 300, 8, 8, [300, 177, 0]),
    (2, 300, 8, 4, [261, 33]),
    (2, 97, 8, 1, None),
    (1, 1100, 8, 8, [1100]),
    (2, 700, 16, 8, [700, 513]),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}-S{c[1]}-G{c[2] // c[3]}" for c in SMALL])
def test_vision_prefill_parity(case):
    B, S, Hq, Hkv, ln = case
    g = torch.Generator(device="cpu")
    g.manual_seed(S + Hkv)
    pos2 = torch.randint(0, 120, (B, S, 2), generator=g, dtype=torch.int32).to(DEV)
    q = inputs.randn((B, S, Hq, 256), 901 + S, torch.bfloat16, DEV)
    k = inputs.randn((B, S, Hkv, 256), 902 + S, torch.bfloat16, DEV)
    v = inputs.randn((B, S, Hkv, 256), 903 + S, torch.bfloat16, DEV)
    lengths = None if ln is None else torch.tensor(ln, dtype=torch.int32, device=DEV)
    print(f"vision B={B} S={S} Hq={Hq} Hkv={Hkv} lengths={ln}", flush=True)
    out = run(q, k, v, pos2, lengths)
    ref = ref_rows(q, k, v, pos2, lengths)
    assert torch.isfinite(out).all()
    assert_parity(out, ref, torch.bfloat16, f"vision {case}")
    if ln is not None:
        for b, n in enumerate(ln):
            assert (out[b, n:] == 0).all()


def test_vision_prefill_batch_of_eight_images():
    """8 images of up to 1024 patches, 8 heads (a grid of several whole
    rounds of workgroups); sampled rows of every image, one image padded."""
    layer = inputs.VisionLayer(((32, 32),) * 7 + ((30, 31),), Hq=8, Hkv=8)
    q, k, v, pos2, lengths = inputs.vision_inputs(layer, 92, torch.bfloat16, DEV)
    out = run(q, k, v, pos2, lengths)
    S = layer.S
    ids = []
    for b, (w, h) in enumerate(layer.grids):
        ids += [b * S + r for r in sample_rows(w * h, S, 90 + b)]
        assert (out[b, w * h:] == 0).all()
    ids = np.array(ids, np.int64)
    ref = ref_rows(q, k, v, pos2, lengths, rows=ids)
    got = out.view(layer.B * S, layer.Hq, layer.d)[torch.as_tensor(ids, device=DEV)]
    assert_parity(got, ref, torch.bfloat16, "vision batch of eight")


def test_vision_prefill_bf16_output_and_raster_grid():
    layer = inputs.VisionLayer(((20, 15), (17, 11)), Hq=8, Hkv=8)
    q, k, v, pos2, lengths = inputs.vision_inputs(layer, 91, torch.bfloat16, DEV)
    out = run(q, k, v, pos2, lengths, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ref = ref_rows(q, k, v, pos2, lengths)
    got = out.float().cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= 1e-2 + 2.0 ** -8 * np.abs(ref))


def test_vision_score_far_above_first_tile_takes_exact_path():
    B, S, H = 1, 300, 4
    q = torch.ones((B, S, H, 256), dtype=torch.bfloat16, device=DEV)
    k = inputs.randn((B, S, H, 256), 95, torch.bfloat16, DEV)
    v = inputs.randn((B, S, H, 256), 96, torch.bfloat16, DEV)
    k[:, :64] = 0      # every row's first tiles score exactly 0
    k[:, 150] = 8.0    # key 150 scores ~100 natural units above them
    pos2 = torch.zeros((B, S, 2), dtype=torch.int32, device=DEV)
    pos2[..., 0] = torch.arange(S, device=DEV) % 20
    pos2[..., 1] = torch.arange(S, device=DEV) // 20
    out = run(q, k, v, pos2, None)
    ref = ref_rows(q, k, v, pos2, None)
    assert_parity(out, ref, torch.bfloat16, "vision exact path")


def sample_rows(n, S, seed):
    rows = {0, 1, 31, 32, 255, 256, n // 2, n - 2, n - 1}
    rows |= set(np.random.default_rng(seed).choice(n, 12, replace=False).tolist())
    return sorted(r for r in rows if 0 <= r < min(n, S))


@pytest.mark.parametrize("layer", [inputs.VISION_280, inputs.VISION_1120],
                         ids=["budget280-b4", "budget1120-b1"])
def test_vision_full_size_sampled_rows(layer):
    q, k, v, pos2, lengths = inputs.vision_inputs(layer, 8, torch.bfloat16, DEV)
    print(f"vision full size {layer}", flush=True)
    out = run(q, k, v, pos2, lengths, layer.theta)
    assert torch.isfinite(out).all()
    S = layer.S
    ids = []
    for b, (w, h) in enumerate(layer.grids):
        ids += [b * S + r for r in sample_rows(w * h, S, 80 + b)]
        assert (out[b, w * h:] == 0).all()
    ids = np.array(ids, np.int64)
    ref = ref_rows(q, k, v, pos2, lengths, layer.theta, rows=ids)
    got = out.view(layer.B * S, layer.Hq, layer.d)[torch.as_tensor(ids, device=DEV)]
    mx, mean = assert_parity(got, ref, torch.bfloat16, f"vision {layer}")
    print(f"  rows {len(ids)}: max {mx:.2e} mean {mean:.2e}", flush=True)


@pytest.mark.parametrize("S,ln", [(1, None), (33, [1, 33]), (32, [32, 31])])
def test_vision_tiny_images(S, ln):
    """One patch, and images that end on or just past a 32-key tile edge."""
    B = 1 if ln is None else len(ln)
    g = torch.Generator(device="cpu")
    g.manual_seed(7 + S)
    pos2 = torch.randint(0, 50, (B, S, 2), generator=g, dtype=torch.int32).to(DEV)
    q = inputs.randn((B, S, 8, 256), 971 + S, torch.bfloat16, DEV)
    k = inputs.randn((B, S, 4, 256), 972 + S, torch.bfloat16, DEV)
    v = inputs.randn((B, S, 4, 256), 973 + S, torch.bfloat16, DEV)
    lengths = None if ln is None else torch.tensor(ln, dtype=torch.int32, device=DEV)
    out = run(q, k, v, pos2, lengths)
    ref = ref_rows(q, k, v, pos2, lengths)
    assert_parity(out, ref, torch.bfloat16, f"vision tiny S={S}")
