"""Pins of the fp64 oracle against things other than itself (CPU only).

- brute force: a dense numpy formulation (complex rotation, explicit mask matrix,
  repeated KV heads) on tiny inputs, atol 1e-12;
- closed forms: q = 0 gives the sliding-window mean of v; S = 1 gives v0;
  hand-derived rotation angles (tests/golden/rope_hand.json);
- library routine: p = 0 reduces to plain causal softmax attention, compared with
  torch's scaled_dot_product_attention in float64;
- invariants: W >= S equals W = 0; GQA equals MHA with repeated KV heads;
  K=V equals the standard path fed v := k; p = 1 rotates every pair; the
  rotation is orthogonal and additive in the position; outputs are invariant
  under a common position shift; probability rows equal the dense brute-force
  softmax weights, sum to 1 with exactly the window's keys non-zero, and times
  the values give the prefill's output row; decode equals the last prefill row; a ring cache
  equals a linear one; writing a prefill's rows into a cache (in two parts, as
  a prompt and then new tokens) and decoding the last L tokens at once
  reproduces those prefill rows; one query token equals ordinary decode;
- mutants: plausible mistakes planted in a copy of oracle.c must fail a pin.
"""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, dtype=np.float32):
    return np.random.default_rng(seed).standard_normal(shape).astype(dtype)


def to_bf16_bits(x):
    """Round-to-nearest-even float32 -> bf16 bit patterns (uint16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


CASES = [
    # B, S, Hq, Hkv, d, window, theta, p
    (1, 9, 2, 1, 8, 0, 1e4, 1.0),
    (2, 13, 4, 2, 16, 4, 1e4, 1.0),
    (1, 17, 8, 1, 32, 0, 1e6, 0.25),
    (2, 11, 4, 4, 8, 1, 1e4, 1.0),
    (1, 12, 8, 2, 16, 5, 1e6, 0.5),
    (1, 10, 2, 2, 8, 3, 1e4, 0.0),
    (1, 16, 8, 1, 64, 7, 1e6, 0.25),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("offset", [0, 1000])
def test_brute_force_prefill(case, offset):
    B, S, Hq, Hkv, d, W, theta, p = case
    q, k, v = rnd((B, S, Hq, d), 1), rnd((B, S, Hkv, d), 2), rnd((B, S, Hkv, d), 3)
    pos = (np.arange(S, dtype=np.int32) + offset)[None].repeat(B, 0)
    got = oracle.prefill(q, k, v, pos, W, theta, p)
    n_rot = int(math.floor(p * d / 2))
    want = brute.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                           pos, W, theta, n_rot)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_brute_force_bf16_inputs_and_random_positions():
    B, S, Hq, Hkv, d, W = 2, 15, 4, 2, 16, 6
    q, k, v = (to_bf16_bits(rnd(s, i)) for i, s in enumerate([(B, S, Hq, d), (B, S, Hkv, d),
                                                               (B, S, Hkv, d)]))
    pos = np.random.default_rng(5).integers(0, 262144, size=(B, S)).astype(np.int32)
    got = oracle.prefill(q, k, v, pos, W, 1e4, 1.0)
    want = brute.attention(bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v), pos, W, 1e4, d // 2)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


def test_row_subset_matches_full():
    B, S, Hq, Hkv, d, W = 2, 20, 4, 2, 16, 5
    q, k, v = rnd((B, S, Hq, d), 7), rnd((B, S, Hkv, d), 8), rnd((B, S, Hkv, d), 9)
    pos = np.arange(S, dtype=np.int32)[None].repeat(B, 0)
    full = oracle.prefill(q, k, v, pos, W, 1e4, 1.0)
    rows = np.array([0, 3, 19, 20, 27, 39])
    sub = oracle.prefill(q, k, v, pos, W, 1e4, 1.0, rows=rows)
    np.testing.assert_array_equal(sub, full.reshape(B * S, Hq, d)[rows])


@pytest.mark.parametrize("W", [1, 2, 5, 0])
def test_zero_query_gives_window_mean(W):
    """q = 0 makes every visible score 0, so each output is the plain mean of
    the visible values: a sliding-window mean, computed here with cumsum."""
    B, S, Hq, Hkv, d = 1, 23, 4, 2, 8
    q = np.zeros((B, S, Hq, d), np.float32)
    k, v = rnd((B, S, Hkv, d), 11), rnd((B, S, Hkv, d), 12)
    pos = np.arange(S, dtype=np.int32)[None]
    got = oracle.prefill(q, k, v, pos, W, 1e4, 1.0)
    c = np.concatenate([np.zeros((1, Hkv, d)), np.cumsum(v[0].astype(np.float64), axis=0)])
    for i in range(S):
        lo = 0 if W == 0 else max(0, i - W + 1)
        mean = (c[i + 1] - c[lo]) / (i + 1 - lo)
        for h in range(Hq):
            np.testing.assert_allclose(got[0, i, h], mean[h // (Hq // Hkv)], rtol=0, atol=1e-12)


def test_single_token_returns_v0():
    q, k, v = rnd((3, 1, 8, 32), 1), rnd((3, 1, 1, 32), 2), rnd((3, 1, 1, 32), 3)
    pos = np.array([[5], [0], [262143]], np.int32)
    got = oracle.prefill(q, k, v, pos, 0, 1e6, 0.25)
    np.testing.assert_array_equal(got, np.repeat(v.astype(np.float64), 8, axis=2))


def test_window_at_least_seq_equals_global():
    B, S, Hq, Hkv, d = 1, 19, 4, 2, 16
    q, k, v = rnd((B, S, Hq, d), 21), rnd((B, S, Hkv, d), 22), rnd((B, S, Hkv, d), 23)
    pos = np.arange(S, dtype=np.int32)[None]
    g = oracle.prefill(q, k, v, pos, 0, 1e4, 1.0)
    for W in (S, S + 1, 1000):
        np.testing.assert_array_equal(oracle.prefill(q, k, v, pos, W, 1e4, 1.0), g)
    assert not np.allclose(oracle.prefill(q, k, v, pos, S - 1, 1e4, 1.0), g)


def test_gqa_equals_mha_with_repeated_heads():
    B, S, Hq, Hkv, d, W = 2, 14, 8, 2, 16, 6
    q, k, v = rnd((B, S, Hq, d), 31), rnd((B, S, Hkv, d), 32), rnd((B, S, Hkv, d), 33)
    pos = np.arange(S, dtype=np.int32)[None].repeat(B, 0)
    gqa = oracle.prefill(q, k, v, pos, W, 1e4, 1.0)
    mha = oracle.prefill(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), pos, W, 1e4, 1.0)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-13)


def test_k_equals_v_is_standard_attention_fed_v_is_k():
    B, S, Hq, Hkv, d = 1, 16, 8, 1, 64
    q, kv = rnd((B, S, Hq, d), 41), rnd((B, S, Hkv, d), 42)
    pos = np.arange(S, dtype=np.int32)[None]
    got = oracle.prefill(q, kv, kv, pos, 0, 1e6, 0.25)
    want = brute.attention(q.astype(np.float64), kv.astype(np.float64), kv.astype(np.float64),
                           pos, 0, 1e6, 8)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # values are the raw tensor, not the rotated one
    rot_v = brute.rotate(kv.astype(np.float64), pos, 1e6, 8)
    wrong = brute.attention(q.astype(np.float64), kv.astype(np.float64), rot_v, pos, 0, 1e6, 8)
    assert np.abs(got - wrong).max() > 1e-3


@pytest.mark.parametrize("W", [0, 4])
def test_p0_is_plain_causal_attention_library_routine(W):
    torch = pytest.importorskip("torch")
    B, S, Hq, Hkv, d = 2, 12, 4, 4, 16
    q, k, v = rnd((B, S, Hq, d), 51), rnd((B, S, Hkv, d), 52), rnd((B, S, Hkv, d), 53)
    pos = np.arange(S, dtype=np.int32)[None].repeat(B, 0) + 777
    got = oracle.prefill(q, k, v, pos, W, 1e4, 0.0)
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)).transpose(1, 2) for x in (q, k, v))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    allowed = (j <= i) & (((i - j) < W) if W > 0 else torch.ones_like(j <= i))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed)
    np.testing.assert_allclose(got, ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("p,n_rot", [(1.0, 8), (0.25, 2), (0.5, 4)])
def test_p_rotates_exactly_the_first_pairs(p, n_rot):
    """attention(q, k; p) == attention(R_p q, R_p k; p = 0), where R_p rotates the
    first n_rot pairs in numpy: p = 1 is full RoPE, p = 0.25 the first quarter."""
    B, S, Hq, Hkv, d = 1, 10, 2, 1, 16
    q, k, v = rnd((B, S, Hq, d), 61), rnd((B, S, Hkv, d), 62), rnd((B, S, Hkv, d), 63)
    pos = np.arange(S, dtype=np.int32)[None] + 3
    got = oracle.prefill(q, k, v, pos, 0, 1e4, p)
    qr = brute.rotate(q.astype(np.float64), pos, 1e4, n_rot).astype(np.float32)
    kr = brute.rotate(k.astype(np.float64), pos, 1e4, n_rot).astype(np.float32)
    # fp32 storage of the pre-rotated operands costs ~1e-7
    np.testing.assert_allclose(got, oracle.prefill(qr, kr, v, pos, 0, 1e4, 0.0), atol=2e-6)
    assert oracle.nrot(d, p) == n_rot


def test_p0_is_identity_rotation():
    x = rnd(64, 70).astype(np.float64)
    np.testing.assert_array_equal(oracle.rope(x, 1e4, 0.0, 12345), x)


def test_rotation_orthogonal_norm_preserving_and_additive():
    d = 32
    for p, theta in ((1.0, 1e4), (0.25, 1e6)):
        R = np.stack([oracle.rope(np.eye(d)[c], theta, p, 977) for c in range(d)], axis=1)
        np.testing.assert_allclose(R.T @ R, np.eye(d), atol=1e-14)
        x = rnd(d, 71).astype(np.float64)
        np.testing.assert_allclose(np.linalg.norm(R @ x), np.linalg.norm(x), rtol=1e-14)
        # R(a) R(b) = R(a + b)
        y = oracle.rope(oracle.rope(x, theta, p, 1234), theta, p, 4321)
        np.testing.assert_allclose(y, oracle.rope(x, theta, p, 5555), atol=1e-11)


def test_hand_derived_angles():
    g = json.load(open(os.path.join(GOLDEN, "rope_hand.json")))
    for c in g["cases"]:
        d, t = c["d"], c["pair"]
        x = np.zeros(d)
        x[2 * t] = 1.0
        y = oracle.rope(x, c["theta"], c["p"], c["pos"])
        want = np.zeros(d)
        want[2 * t] = math.cos(c["angle"])
        want[2 * t + 1] = math.sin(c["angle"])
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-12, err_msg=str(c))
        x = np.zeros(d)
        x[2 * t + 1] = 1.0
        y = oracle.rope(x, c["theta"], c["p"], c["pos"])
        want = np.zeros(d)
        want[2 * t] = -math.sin(c["angle"])
        want[2 * t + 1] = math.cos(c["angle"])
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-12, err_msg=str(c))


def test_relative_position_invariance():
    B, S, Hq, Hkv, d, W = 1, 18, 4, 2, 32, 7
    q, k, v = rnd((B, S, Hq, d), 81), rnd((B, S, Hkv, d), 82), rnd((B, S, Hkv, d), 83)
    pos = np.arange(S, dtype=np.int32)[None]
    a = oracle.prefill(q, k, v, pos, W, 1e4, 1.0)
    b = oracle.prefill(q, k, v, pos + 200000, W, 1e4, 1.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)


PROB_CASES = [
    # B, S, Hq, Hkv, d, theta, p (G = 1, 2, 4, 8; full, partial and no rotation)
    (1, 30, 4, 2, 16, 1e4, 1.0),
    (2, 21, 8, 1, 32, 1e6, 0.25),
    (1, 19, 4, 1, 16, 1e4, 0.5),
    (1, 17, 3, 3, 8, 1e4, 0.0),
]


@pytest.mark.parametrize("case", PROB_CASES)
def test_probability_rows_are_the_weights_of_the_prefill(case):
    """g4o_probs against the dense brute-force softmax weights (value pin, so a
    dropped 1/sqrt(d), a wrong key rotation or a wrong GQA map fails it);
    every row sums to 1 with exactly the window's keys non-zero; and the row
    times the raw values reproduces g4o_prefill's output row, so the weights
    pinned here are the ones the prefill uses."""
    B, S, Hq, Hkv, d, theta, p = case
    q, k, v = rnd((B, S, Hq, d), 91), rnd((B, S, Hkv, d), 92), rnd((B, S, Hkv, d), 93)
    pos = (np.arange(S, dtype=np.int32) + 37)[None].repeat(B, 0)
    G = Hq // Hkv
    n_rot = int(math.floor(p * d / 2))
    for W in (0, 1, 4, S - 1):
        want = brute.probabilities(q.astype(np.float64), k.astype(np.float64), pos, W, theta,
                                   n_rot)
        out = oracle.prefill(q, k, v, pos, W, theta, p)
        for b in range(B):
            for i in (0, 3, 4, S // 2, S - 1):
                for h in sorted({0, G - 1, Hq - 1}):
                    pr = oracle.probs(q, k, pos, W, theta, p, b, i, h)
                    np.testing.assert_allclose(pr, want[b, h, i], rtol=0, atol=1e-12)
                    assert abs(pr.sum() - 1.0) < 1e-14
                    lo = 0 if W == 0 else max(0, i - W + 1)
                    nz = np.nonzero(pr)[0]
                    assert nz.min() == lo and nz.max() == i and nz.size == i - lo + 1
                    row = pr @ v[b, :, h // G].astype(np.float64)
                    np.testing.assert_allclose(row, out[b, i, h], rtol=0, atol=1e-12)


def _sequence(B, L, Hq, Hkv, d, seed):
    return rnd((B, L, Hq, d), seed), rnd((B, L, Hkv, d), seed + 1), rnd((B, L, Hkv, d), seed + 2)


def test_decode_linear_equals_last_prefill_row():
    B, L, Hq, Hkv, d, C = 2, 21, 8, 1, 32, 40
    q, k, _ = _sequence(B, L, Hq, Hkv, d, 100)
    pos = np.arange(L, dtype=np.int32)[None].repeat(B, 0)
    pre = oracle.prefill(q, k, k, pos, 0, 1e6, 0.25)
    cache = np.full((B, Hkv, C, d), np.nan, np.float32)  # unread rows stay NaN
    cache[:, :, :L] = k.transpose(0, 2, 1, 3)
    out = oracle.decode(q[:, L - 1], cache, None, np.full(B, L - 1, np.int32), 0, 1e6, 0.25)
    np.testing.assert_allclose(out, pre[:, L - 1], rtol=0, atol=1e-13)


def test_decode_ring_equals_linear_and_prefill():
    """Caches with separate values hold the keys turned at their positions
    (turned here by the independent brute-force rotation, kept in fp64)."""
    B, L, Hq, Hkv, d, W = 2, 29, 4, 2, 16, 8
    q, k, v = _sequence(B, L, Hq, Hkv, d, 200)
    pos = np.arange(L, dtype=np.int32)[None].repeat(B, 0)
    pre = oracle.prefill(q, k, v, pos, W, 1e4, 1.0)
    P = L - 1
    kt = brute.rotate(k.astype(np.float64), pos, 1e4, d // 2)
    ring_k = np.empty((B, Hkv, W, d), np.float64)
    ring_v = np.empty((B, Hkv, W, d), np.float64)
    for s in range(W):
        t = P - ((P - s) % W)  # the position slot s holds
        ring_k[:, :, s] = kt[:, t]
        ring_v[:, :, s] = v[:, t]
    lin_k = np.ascontiguousarray(kt.transpose(0, 2, 1, 3))
    lin_v = np.ascontiguousarray(v.astype(np.float64).transpose(0, 2, 1, 3))
    qP = q[:, P].astype(np.float64)
    ring = oracle.decode(qP, ring_k, ring_v, np.full(B, P, np.int32), W, 1e4, 1.0)
    np.testing.assert_allclose(ring, pre[:, P], rtol=0, atol=1e-13)
    # linear cache with no window sees everything: equals the global prefill row
    lin = oracle.decode(qP, lin_k, lin_v, np.full(B, P, np.int32), 0, 1e4, 1.0)
    glob = oracle.prefill(q, k, v, pos, 0, 1e4, 1.0)
    np.testing.assert_allclose(lin, glob[:, P], rtol=0, atol=1e-13)


def test_decode_bad_positions_give_nan_rows():
    B, Hq, Hkv, d, C = 3, 4, 2, 8, 10
    q = rnd((B, Hq, d), 1)
    kc = rnd((B, Hkv, C, d), 2)
    out = oracle.decode(q, kc, None, np.array([-1, 10, 9], np.int32), 0, 1e4, 1.0)
    assert np.isnan(out[0]).all() and np.isnan(out[1]).all() and np.isfinite(out[2]).all()


@pytest.mark.parametrize("theta,p,offset", [(1e4, 1.0, 0), (1e6, 0.25, 250000), (1e4, 0.5, 77)])
def test_rotate_rows_equals_brute_force_rotation(theta, p, offset):
    B, S, H, d = 2, 9, 3, 32
    x = rnd((B, S, H, d), 41)
    pos = (np.arange(S, dtype=np.int32) * 37 + offset)[None].repeat(B, 0)
    pos[1] = pos[1][::-1]
    got = oracle.rotate_rows(x, pos, theta, p)
    want = brute.rotate(x.astype(np.float64), pos, theta, int(p * d / 2))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)
    # bf16 inputs read exactly
    bits = to_bf16_bits(x)
    got16 = oracle.rotate_rows(bits, pos, theta, p)
    want16 = brute.rotate(bf16_to_f64(bits), pos, theta, int(p * d / 2))
    np.testing.assert_allclose(got16, want16, rtol=0, atol=1e-11)


def test_f64_to_bf16_bits_rounds_once_to_nearest_even():
    """Closed forms of rounding to bf16: a bf16 value maps to itself, the
    midpoint of two neighbours to the one with an even last bit, and points
    just off the midpoint to the nearer neighbour."""
    rng = np.random.default_rng(5)
    ra = rng.integers(0x3000, 0x4F00, 4000).astype(np.uint16)  # positive normal numbers
    rb = ra + np.uint16(1)                                        # their successors
    a, b = bf16_to_f64(ra), bf16_to_f64(rb)
    for sgn, sbit in ((1.0, np.uint16(0)), (-1.0, np.uint16(0x8000))):
        lo, hi = sgn * a, sgn * b
        assert np.array_equal(oracle.f64_to_bf16_bits(lo), ra | sbit)
        mid = (lo + hi) / 2.0
        even = np.where((ra & 1) == 0, ra, rb) | sbit
        assert np.array_equal(oracle.f64_to_bf16_bits(mid), even)
        eps = (hi - lo) * 1e-6
        assert np.array_equal(oracle.f64_to_bf16_bits(mid - eps), ra | sbit)
        assert np.array_equal(oracle.f64_to_bf16_bits(mid + eps), rb | sbit)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fill_with_separate_values_turns_the_keys(dtype):
    """Key slots hold R(t) k_t rounded once to the cache type (brute-force
    rotation), value slots the value bytes unchanged."""
    B, S, Hkv, d, C, theta, p = 2, 13, 2, 16, 16, 1e4, 1.0
    k, v = rnd((B, S, Hkv, d), 51), rnd((B, S, Hkv, d), 52)
    pos = (np.arange(S, dtype=np.int32) + 1000)[None].repeat(B, 0)
    kt = brute.rotate(k.astype(np.float64), pos, theta, d // 2)
    if dtype == "bf16":
        k, v = to_bf16_bits(k), to_bf16_bits(v)
        kt = brute.rotate(bf16_to_f64(k), pos, theta, d // 2)
        want_k = oracle.f64_to_bf16_bits(kt)
        z = np.zeros((B, Hkv, C, d), np.uint16)
    else:
        want_k = kt.astype(np.float32)
        z = np.zeros((B, Hkv, C, d), np.float32)
    kc, vc = oracle.fill_cache(k, v, pos, z, z, C, theta, p)
    for b in range(B):
        for i in range(S):
            s = pos[b, i] % C
            assert np.array_equal(kc[b, :, s], want_k[b, i])
            assert np.array_equal(vc[b, :, s], v[b, i])
    with pytest.raises(ValueError):
        oracle.fill_cache(k, v, pos, z, z, C)


# --- cache fill + decode of several query tokens ---------------------------------

def _closed_loop(B, S, L, Hq, Hkv, d, W, C, theta, p, kv_shared, seed, lib=None):
    """prefill rows S-L..S-1 and the same rows from fill_cache + decode_multi.
    With separate values the fill turns the keys and rounds them to float32,
    so the two agree to that rounding; K=V rows are copied and agree exactly."""
    q, k, v = _sequence(B, S, Hq, Hkv, d, seed)
    if kv_shared:
        v = k
    pos = np.arange(S, dtype=np.int32)[None].repeat(B, 0)
    pre = oracle.prefill(q, k, v, pos, W, theta, p, lib=lib)
    kc = np.full((B, Hkv, C, d), np.nan, np.float32)  # rows never written stay NaN
    vc = None if kv_shared else np.full((B, Hkv, C, d), np.nan, np.float32)
    # the prompt, then the L new tokens, as a decoding loop appends them
    kc, vc = oracle.fill_cache(k[:, :S - L], None if kv_shared else v[:, :S - L], pos[:, :S - L],
                               kc, vc, W, theta, p, lib=lib)
    kc, vc = oracle.fill_cache(k[:, S - L:], None if kv_shared else v[:, S - L:], pos[:, S - L:],
                               kc, vc, W, theta, p, lib=lib)
    got = oracle.decode_multi(q[:, S - L:], kc, vc, np.full(B, S - 1, np.int32), W, theta, p,
                              lib=lib)
    return got, pre[:, S - L:]


@pytest.mark.parametrize("L", [1, 3, 8])
@pytest.mark.parametrize("kind", ["ring-min", "ring-large", "linear-kv"])
def test_fill_cache_then_decode_several_tokens_equals_prefill_rows(L, kind):
    if kind == "ring-min":      # local layer, capacity exactly window + L - 1
        args = dict(B=2, S=37, Hq=4, Hkv=2, d=16, W=8, C=8 + L - 1, theta=1e4, p=1.0,
                    kv_shared=False)
    elif kind == "ring-large":  # a ring larger than needed
        args = dict(B=1, S=41, Hq=2, Hkv=1, d=8, W=6, C=20, theta=1e4, p=1.0, kv_shared=False)
    else:                       # global layer: linear K=V cache, p-RoPE
        args = dict(B=2, S=23, Hq=8, Hkv=1, d=32, W=0, C=30, theta=1e6, p=0.25, kv_shared=True)
    got, want = _closed_loop(L=L, seed=300 + L, **args)
    # float32 turned keys: scores off by about |q||k| 2^-24 per term
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13 if args["kv_shared"] else 2e-6)


def test_one_query_token_equals_decode():
    B, Hq, Hkv, d, C = 3, 4, 2, 16, 12
    q = rnd((B, 1, Hq, d), 5)
    kc, vc = rnd((B, Hkv, C, d), 6), rnd((B, Hkv, C, d), 7)
    for W, pos in ((C, np.array([3, 11, 40], np.int32)), (0, np.array([0, 5, 11], np.int32))):
        a = oracle.decode_multi(q, kc, vc, pos, W, 1e4, 1.0)
        b = oracle.decode(q[:, 0], kc, vc, pos, W, 1e4, 1.0)
        np.testing.assert_allclose(a[:, 0], b, rtol=0, atol=1e-13)


def test_fill_cache_ring_slots_hold_the_newest_tokens():
    """Slot s holds the newest token whose position is s mod C (searched per
    slot), as exact bf16 bytes; slots no token maps to keep their contents."""
    B, S, Hkv, d, C = 2, 23, 3, 8, 7
    k = to_bf16_bits(rnd((B, S, Hkv, d), 8))
    pos = (np.arange(S, dtype=np.int32) + 3)[None].repeat(B, 0)
    sentinel = np.full((B, Hkv, C, d), 0x7FC1, np.uint16)
    kc, vc = oracle.fill_cache(k, None, pos, sentinel, None, C)
    assert vc is None
    for b in range(B):
        for s_ in range(C):
            owners = [i for i in range(S) if pos[b, i] % C == s_]
            assert owners
            i = max(owners, key=lambda i: pos[b, i])
            assert np.array_equal(kc[b, :, s_], k[b, i]), (b, s_)
    # a short prefill leaves the other slots alone
    kc2, _ = oracle.fill_cache(k[:, :3], None, pos[:, :3], sentinel, None, C)
    touched = {int(x) % C for x in pos[0, :3]}
    for s_ in range(C):
        if s_ not in touched:
            assert (kc2[:, :, s_] == 0x7FC1).all()


def test_fill_cache_linear_skips_positions_outside_the_cache():
    B, S, Hkv, d, C = 1, 6, 1, 4, 5
    k = rnd((B, S, Hkv, d), 9)
    pos = np.array([[-2, 0, 1, 4, 5, 9]], np.int32)
    kc, _ = oracle.fill_cache(k, None, pos, np.zeros((B, Hkv, C, d), np.float32), None, 0)
    want = np.zeros((B, Hkv, C, d), np.float32)
    want[0, 0, 0], want[0, 0, 1], want[0, 0, 4] = k[0, 1, 0], k[0, 2, 0], k[0, 3, 0]
    np.testing.assert_array_equal(kc, want)


def test_decode_several_tokens_bad_positions_and_small_ring():
    B, L, Hq, Hkv, d, C = 3, 3, 2, 1, 8, 10
    q = rnd((B, L, Hq, d), 10)
    kc = rnd((B, Hkv, C, d), 11)
    out = oracle.decode_multi(q, kc, None, np.array([1, 10, 9], np.int32), 0, 1e4, 1.0)
    assert np.isnan(out[0, 0]).all() and np.isfinite(out[0, 1:]).all()  # query 0 at -1
    assert np.isnan(out[1]).all() and np.isfinite(out[2]).all()        # P beyond the cache
    with pytest.raises(ValueError):  # ring smaller than window + L - 1
        oracle.decode_multi(q, kc, None, np.array([20, 20, 20], np.int32), 9, 1e4, 1.0)


def test_invalid_arguments_rejected():
    q, k = rnd((1, 4, 3, 8), 1), rnd((1, 4, 2, 8), 2)
    pos = np.arange(4, dtype=np.int32)[None]
    with pytest.raises(ValueError):
        oracle.prefill(q, k, k, pos, 0, 1e4, 1.0)  # Hq % Hkv != 0
    q = rnd((1, 4, 2, 8), 1)
    for W, theta, p in ((-1, 1e4, 1.0), (0, 0.0, 1.0), (0, 1e4, 1.5), (0, 1e4, -0.1)):
        with pytest.raises(ValueError):
            oracle.prefill(q, k, k, pos, W, theta, p)


# --- mutants: plausible mistakes must fail a pin ---------------------------------

MUTANTS = {
    "rotation_sign": ("x[2 * t] = x0 * c - x1 * s;", "x[2 * t] = x0 * c + x1 * s;"),
    "dropped_scale": ("sc[(size_t)hh * nk + jj] = s * scale;", "sc[(size_t)hh * nk + jj] = s;"),
    "window_off_by_one": ("int64_t lo = i - window + 1;", "int64_t lo = i - window;"),
    "gqa_mapping": ("const int h = g * G + hh;\n          const size_t qoff",
                    "const int h = hh * Hkv + g;\n          const size_t qoff"),
    "freq_over_rotated_dims": ("return pos * pow(theta, -2.0 * (double)t / (double)d);",
                               "return pos * pow(theta, -2.0 * (double)t / (double)(d / 4));"),
    "key_rotated_with_table_sign": ("kr[2 * t + 1] = x0 * c[2 * t + 1] + x1 * c[2 * t];",
                                    "kr[2 * t + 1] = -x0 * c[2 * t + 1] + x1 * c[2 * t];"),
    "rotated_values": ("o[e] += w * g4o_in(v, dtype, voff + e);", "o[e] += w * kr[e];"),
    "probs_dropped_scale": ("probs[j] = s / sqrt((double)d);", "probs[j] = s;"),
    "probs_gqa_mapping": ("const int G = Hq / Hkv, g = h / G, n_rot = g4o_nrot(d, p);\n  double* qr",
                          "const int G = Hq / Hkv, g = h % Hkv, n_rot = g4o_nrot(d, p);\n  double* qr"),
    "probs_key_unrotated": ("g4o_rope(kr, d, n_rot, theta, (double)pos[(size_t)b * S + j]);\n    double s",
                            "double s"),
    "probs_window_off_by_one": ("if (j < j0 || j > i) { probs[j] = -INFINITY; continue; }",
                                "if (j <= j0 || j > i) { probs[j] = -INFINITY; continue; }"),
    "multi_query_position": ("Pj = P - L + 1 + j;", "Pj = P - L + j;"),
    "multi_ring_slot_by_window": ("const int64_t slot = window > 0 ? t % capacity : t;\n          const size_t koff",
                                  "const int64_t slot = window > 0 ? t % window : t;\n          const size_t koff"),
    "fill_ring_slot_by_window": ("const int64_t slot = window > 0 ? P % capacity : P;",
                                 "const int64_t slot = window > 0 ? P % window : P;"),
    "multi_turns_cached_keys_again": (
        "if (key_turn) g4o_rope(kr, d, n_rot, theta, (double)t);\n          double s = 0.0;",
        "g4o_rope(kr, d, n_rot, theta, (double)t);\n          double s = 0.0;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, name
    path = mutant_dir / f"{name}.c"
    path.write_text(src.replace(old, new, 1))
    lib_path = mutant_dir / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", str(path), "-o", str(lib_path),
                    "-lm"], check=True)
    lib = oracle.load(str(lib_path))
    # the brute-force pin over the prefill cases (one with G = 4, window, K=V)
    B, S, Hq, Hkv, d, W, theta, p = 1, 12, 8, 2, 16, 5, 1e4, 1.0
    q, k, v = rnd((B, S, Hq, d), 1), rnd((B, S, Hkv, d), 2), rnd((B, S, Hkv, d), 3)
    pos = np.arange(S, dtype=np.int32)[None] + 11
    got = oracle.prefill(q, k, v, pos, W, theta, p, lib=lib)
    want = brute.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                           pos, W, theta, d // 2)
    caught = not np.allclose(got, want, rtol=0, atol=1e-12)
    # rotation mistakes that only touch oracle.rope are caught by the hand angles
    x = np.zeros(8)
    x[2] = 1.0
    y = oracle.rope(x, 1e4, 1.0, 1, lib=lib)
    caught |= not np.allclose(y[2:4], [math.cos(0.1), math.sin(0.1)], atol=1e-12)
    x = np.zeros(8)
    x[3] = 1.0
    y = oracle.rope(x, 1e4, 1.0, 1, lib=lib)
    caught |= not np.allclose(y[2:4], [-math.sin(0.1), math.cos(0.1)], atol=1e-12)
    # cache fill + several query tokens: the closed loop against the prefill
    for L, C, W, S in ((3, 10, 8, 37), (2, 12, 6, 17)):
        got, want = _closed_loop(B=1, S=S, L=L, Hq=4, Hkv=2, d=16, W=W, C=C, theta=1e4, p=1.0,
                                 kv_shared=False, seed=77, lib=lib)
        caught |= not np.allclose(got, want, rtol=0, atol=2e-6, equal_nan=False)
    # the probability rows against the dense brute-force weights
    for W in (0, 5):
        want = brute.probabilities(q.astype(np.float64), k.astype(np.float64), pos, W, theta,
                                   d // 2)
        for i, h in ((11, 3), (7, 6)):
            pr = oracle.probs(q, k, pos, W, theta, p, 0, i, h, lib=lib)
            caught |= not np.allclose(pr, want[0, h, i], rtol=0, atol=1e-12)
    assert caught, f"mutant {name} survived the pins"
