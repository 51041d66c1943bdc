"""Pins of the oracle's low-precision (FP8 E4M3) KV cache functions (CPU only).

- library routine: every code's value, and the code of every bf16 value below
  464 plus every midpoint between neighbouring values (and the floats just
  beside it), against torch's float8_e4m3fn conversion;
- closed forms: the largest value 448, the smallest subnormal 2^-9, the
  smallest normal 2^-6, ties to the even mantissa, saturation beyond 448,
  signed zero, NaN;
- invariants: every finite code survives value -> code; quantizing
  code value x 2^k with a head scale 2^k gives the code back, per KV head;
  decoding an fp8 cache equals decoding a float32 cache that holds
  code value x scale (exact in float32 for power-of-two scales);
- closed loop: for inputs already on the fp8 grid, prefill == fill the fp8
  cache + decode several query tokens, to rounding of the fp64 sums;
- mutants: plausible mistakes planted in a copy of oracle.c must fail a pin.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from tests import brute

F8 = torch.float8_e4m3fn


def torch_values():
    return torch.arange(256, dtype=torch.uint8).view(F8).to(torch.float64).numpy()


def torch_encode(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(F8).view(torch.uint8).numpy()


def same_or_both_nan(a, b):
    return np.array_equal(np.nan_to_num(a, nan=1e300), np.nan_to_num(b, nan=1e300))


def test_code_values_match_library_and_closed_forms():
    v = oracle.e4m3_values()
    assert same_or_both_nan(v, torch_values())
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x3C] == 1.5
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert [c for c in range(256) if np.isnan(v[c])] == [0x7F, 0xFF]
    assert np.all(np.diff(v[:0x7F]) > 0)  # increasing over the positive codes


def grid_and_midpoints():
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    xs = [x[np.isfinite(x) & (np.abs(x) < 464)]]
    v = torch_values()[:0x7F]
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)  # exact in float32
    xs += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    xs.append(np.random.default_rng(5).uniform(-460, 460, 20000).astype(np.float32))
    xs.append(np.random.default_rng(6).standard_normal(20000).astype(np.float32) * 0.01)
    x = np.concatenate(xs)
    return np.concatenate([x, -x])


def test_encode_matches_library_round_to_nearest_even():
    x = grid_and_midpoints()
    got = oracle.e4m3_encode(x)
    np.testing.assert_array_equal(got, torch_encode(x))


def test_encode_closed_forms():
    enc = lambda f: int(oracle.e4m3_encode(np.array([f], np.float32))[0])  # noqa: E731
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    for big in (449.0, 463.9, 464.0, 1e30, np.inf):  # saturation (the library gives NaN
        assert enc(big) == 0x7E and enc(-big) == 0xFE  # from 464 on)
    assert enc(np.nan) == 0x7F
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -10) == 0x00           # tie between 0 and 2^-9: even -> 0
    assert enc(3 * 2.0 ** -10) == 0x02       # tie between 2^-9 and 2^-8: even -> 2^-8
    assert enc(1.0 + 2.0 ** -4) == 0x38      # tie between 1 and 1.125: even -> 1
    assert enc(1.125 + 2.0 ** -4) == 0x3A    # tie between 1.125 and 1.25: even -> 1.25
    assert enc(1e-10) == 0x00 and enc(-1e-10) == 0x80


def test_every_finite_code_round_trips():
    v = oracle.e4m3_values()
    codes = np.array([c for c in range(256) if not np.isnan(v[c])])
    np.testing.assert_array_equal(oracle.e4m3_encode(v[codes].astype(np.float32)), codes)


def test_quantize_divides_by_the_scale_of_each_head():
    rng = np.random.default_rng(7)
    Hkv, d = 3, 16
    v = oracle.e4m3_values()
    codes = rng.integers(0, 0x7F, (5, Hkv, d)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    scale = np.array([2.0 ** -3, 1.0, 2.0 ** 5], np.float32)
    x = (v[codes] * scale[None, :, None]).astype(np.float32)  # exact
    np.testing.assert_array_equal(oracle.quantize_e4m3(x, scale), codes)
    # bf16 inputs (the values are exact in bf16: at most 4 significant bits)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(oracle.quantize_e4m3(xb, scale), codes)
    # a scale that is not a power of two: the quotient is rounded to float32 first
    s = np.array([0.37, 1.9, 3.3], np.float32)
    y = rng.standard_normal((5, Hkv, d)).astype(np.float32) * 50
    want = torch_encode(np.clip(y / s[None, :, None], -448, 448))  # float32 IEEE division
    np.testing.assert_array_equal(oracle.quantize_e4m3(y, s), want)


def _random_codes(shape, rng):
    c = rng.integers(0, 0x7F, shape).astype(np.uint8)  # finite codes, both signs
    return c | (rng.integers(0, 2, shape) << 7).astype(np.uint8)


@pytest.mark.parametrize("kv_shared", [False, True])
def test_decode_fp8_equals_decode_of_the_values(kv_shared):
    rng = np.random.default_rng(11)
    B, L, Hq, Hkv, d, C = 2, 3, 4, 2, 16, 12
    kc8 = _random_codes((B, Hkv, C, d), rng)
    vc8 = None if kv_shared else _random_codes((B, Hkv, C, d), rng)
    ks = np.array([2.0 ** -6, 2.0 ** -2], np.float32)
    vs = np.array([2.0 ** -1, 2.0 ** -7], np.float32)
    tv = torch_values()
    kf = (tv[kc8] * ks[None, :, None, None]).astype(np.float32)  # exact in float32
    vf = None if kv_shared else (tv[vc8] * vs[None, :, None, None]).astype(np.float32)
    q = rng.standard_normal((B, L, Hq, d)).astype(np.float32)
    for W, pos in ((C - L + 1, np.array([5, 30], np.int32)), (0, np.array([4, 11], np.int32))):
        got = oracle.decode_fp8(q, kc8, vc8, ks, None if kv_shared else vs, pos, W, 1e4, 1.0)
        want = oracle.decode_multi(q, kf, vf, pos, W, 1e4, 1.0)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("kind", ["ring", "linear-kv"])
def test_closed_loop_on_grid_inputs_equals_prefill(kind):
    """Keys and values already on the fp8 grid (code value x head scale, also
    exact in bf16) survive quantization, so fill + decode gives the prefill rows.
    The ring (separate values) uses p = 0, where turning the keys is the
    identity, so they stay on the grid; the turned fill is pinned below."""
    rng = np.random.default_rng(13)
    if kind == "ring":
        B, S, L, Hq, Hkv, d, W, C, theta, p, shared = 2, 29, 3, 4, 2, 16, 8, 10, 1e4, 0.0, False
    else:
        B, S, L, Hq, Hkv, d, W, C, theta, p, shared = 1, 21, 2, 8, 1, 32, 0, 24, 1e6, 0.25, True
    tv = torch_values()
    ks = np.array([2.0 ** -4, 2.0 ** -1][:Hkv], np.float32)
    vs = np.array([2.0 ** -2, 2.0 ** -5][:Hkv], np.float32)
    k = (tv[_random_codes((B, S, Hkv, d), rng)] * ks[None, None, :, None]).astype(np.float32)
    v = k if shared else (tv[_random_codes((B, S, Hkv, d), rng)]
                          * vs[None, None, :, None]).astype(np.float32)
    q = rng.standard_normal((B, S, Hq, d)).astype(np.float32)
    pos = np.arange(S, dtype=np.int32)[None].repeat(B, 0)
    pre = oracle.prefill(q, k, v, pos, W, theta, p)
    kc = np.full((B, Hkv, C, d), 0x7F, np.uint8)  # NaN codes where nothing is written
    vc = None if shared else kc.copy()
    kc, vc = oracle.fill_cache_fp8(k, None if shared else v, pos, kc, vc, W, ks,
                                   None if shared else vs, theta, p)
    got = oracle.decode_fp8(q[:, S - L:], kc, vc, ks, None if shared else vs,
                            np.full(B, S - 1, np.int32), W, theta, p)
    np.testing.assert_allclose(got, pre[:, S - L:], rtol=0, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fill_fp8_with_separate_values_turns_then_quantizes_the_keys(dtype):
    """Key codes are E4M3(float32(R(t) k_t) / scale): the brute-force rotation,
    rounded to float32, through the encoder pinned above; value codes are
    E4M3(v / scale) unturned."""
    rng = np.random.default_rng(21)
    B, S, Hkv, d, C, theta, p = 2, 11, 2, 16, 12, 1e4, 1.0
    k = rng.standard_normal((B, S, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, S, Hkv, d)).astype(np.float32)
    pos = (np.arange(S, dtype=np.int32) + 300)[None].repeat(B, 0)
    kin, vin = k, v
    kf = k.astype(np.float64)
    if dtype == "bf16":
        kin = (k.view(np.uint32) >> 16).astype(np.uint16)
        vin = (v.view(np.uint32) >> 16).astype(np.uint16)
        kf = oracle.bf16_bits_to_f64(kin)
        v = oracle.bf16_bits_to_f64(vin).astype(np.float32)
    ks = np.array([0.05, 0.2], np.float32)
    vs = np.array([0.1, 0.07], np.float32)
    kt = brute.rotate(kf, pos, theta, d // 2).astype(np.float32)
    want_k = torch_encode(kt / ks[None, None, :, None])
    want_v = torch_encode(v / vs[None, None, :, None])
    z = np.full((B, Hkv, C, d), 0x7F, np.uint8)
    kc, vc = oracle.fill_cache_fp8(kin, vin, pos, z, z, C, ks, vs, theta, p)
    for b in range(B):
        for i in range(S - C, S):
            s = pos[b, i] % C
            assert np.array_equal(kc[b, :, s], want_k[b, i])
            assert np.array_equal(vc[b, :, s], want_v[b, i])
    with pytest.raises(ValueError):
        oracle.fill_cache_fp8(kin, vin, pos, z, z, C, ks, vs)


# --- mutants ---------------------------------------------------------------------

MUTANTS = {
    "exponent_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                      "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "subnormal_scale": ("if (e == 0) v = ldexp((double)m, -9);",
                        "if (e == 0) v = ldexp((double)m, -10);"),
    "ties_away_from_zero": ("const double n = nearbyint(a / quantum);",
                            "const double n = round(a / quantum);"),
    "subnormal_spacing": ("if (E < -6) E = -6;", "if (E < -7) E = -7;"),
    "scale_of_head_zero": ("const float y = xf / scale[h];", "const float y = xf / scale[0];"),
    "scale_multiplies": ("const float y = xf / scale[h];", "const float y = xf * scale[h];"),
    "no_saturation": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 480.0) return sign | 0x7F;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("fp8_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = mutant_dir / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = mutant_dir / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", str(path), "-o", str(lib_path),
                    "-lm"], check=True)
    lib = oracle.load(str(lib_path))
    caught = not same_or_both_nan(oracle.e4m3_values(lib), torch_values())
    x = grid_and_midpoints()
    caught |= not np.array_equal(oracle.e4m3_encode(x, lib), torch_encode(x))
    caught |= int(oracle.e4m3_encode(np.array([1e30], np.float32), lib)[0]) != 0x7E
    s = np.array([0.5, 4.0], np.float32)
    y = np.random.default_rng(3).standard_normal((4, 2, 8)).astype(np.float32)
    caught |= not np.array_equal(oracle.quantize_e4m3(y, s, lib),
                                 torch_encode(np.clip(y / s[None, :, None], -448, 448)))
    assert caught, f"mutant {name} survived the pins"
