"""Shared test helpers: tensor -> oracle marshalling and the parity bar."""
import numpy as np
import torch

# Tolerances (measured on fp32 outputs): fp32 inputs max |err| <= 1e-4;
# bf16 N(0,1) inputs max |err| <= 1e-2 and mean |err| <= 1e-3.
TOL_F32_MAX = 1e-4
TOL_BF16_MAX = 1e-2
TOL_BF16_MEAN = 1e-3


def to_oracle(t):
    """Exact host copy for the oracle: float32, or bf16 as uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float32).numpy()


def errors(got, ref):
    g = got.detach().float().cpu().double().numpy()
    e = np.abs(g - ref)
    return float(e.max()), float(e.mean())


def assert_parity(got, ref, in_dtype, what=""):
    mx, mean = errors(got, ref)
    if in_dtype == torch.float32:
        assert mx <= TOL_F32_MAX, f"{what}: max |err| {mx:.3e} > {TOL_F32_MAX}"
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, \
            f"{what}: max |err| {mx:.3e}, mean {mean:.3e}"
    return mx, mean
