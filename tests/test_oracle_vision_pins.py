"""Pins of the oracle's vision-encoder attention (2D RoPE, no causal mask), CPU only.

- brute force: a dense numpy formulation (complex rotation per half, explicit
  key mask) on tiny inputs, atol 1e-12;
- reduction to the pinned 1D oracle: with the h component 0, the first half
  is a 1D RoPE of dim d/2 (frequencies theta^(-4t/d) = (theta^2)^(-2t/d), the
  first d/4 pairs), so the last row equals the causal prefill's last row at
  base theta^2 and p = 0.5; with w = 0 the same holds for the second half once
  the halves of q and k are swapped;
- invariants: a common shift of (w, h) changes nothing; permuting the patches
  permutes the outputs (no causal order); padded patches do not change the
  valid rows (NaN in their q, k, v) and their own rows are zero; q = 0 gives
  the mean of the valid values;
- mutants: plausible mistakes planted in a copy of oracle.c must fail a pin.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import brute


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def grid_pos(B, S, seed, span=40):
    return np.random.default_rng(seed).integers(0, span, (B, S, 2)).astype(np.int32)


CASES = [  # B, S, Hq, Hkv, d, lengths
    (1, 9, 2, 1, 8, None),
    (2, 13, 4, 2, 16, [13, 7]),
    (2, 11, 4, 4, 32, [5, 0]),
    (1, 17, 8, 1, 16, [17]),
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force(case):
    B, S, Hq, Hkv, d, ln = case
    q, k, v = rnd((B, S, Hq, d), 1), rnd((B, S, Hkv, d), 2), rnd((B, S, Hkv, d), 3)
    pos2 = grid_pos(B, S, 4)
    got = oracle.vision_prefill(q, k, v, pos2, 1e4, lengths=ln)
    want = brute.vision_attention(q.astype(np.float64), k.astype(np.float64),
                                  v.astype(np.float64), pos2, 1e4, ln)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    B, S, Hq, Hkv, d = 2, 10, 4, 2, 16
    q, k, v = rnd((B, S, Hq, d), 5), rnd((B, S, Hkv, d), 6), rnd((B, S, Hkv, d), 7)
    pos2 = grid_pos(B, S, 8)
    full = oracle.vision_prefill(q, k, v, pos2, 1e4, lengths=[10, 6])
    ids = np.array([0, 5, 9, 10, 15, 17, 19])
    sub = oracle.vision_prefill(q, k, v, pos2, 1e4, lengths=[10, 6], rows=ids)
    np.testing.assert_array_equal(sub, full.reshape(B * S, Hq, d)[ids])


@pytest.mark.parametrize("component", [0, 1])
def test_one_axis_reduces_to_the_1d_oracle(component):
    B, S, Hq, Hkv, d, theta = 1, 12, 4, 2, 16, 1e4
    q, k, v = rnd((B, S, Hq, d), 9), rnd((B, S, Hkv, d), 10), rnd((B, S, Hkv, d), 11)
    pos = (np.arange(S, dtype=np.int32) * 3 + 2)[None]
    pos2 = np.zeros((B, S, 2), np.int32)
    pos2[..., component] = pos
    got = oracle.vision_prefill(q, k, v, pos2, theta)[:, S - 1]
    if component == 1:  # move the rotated half to the front for the 1D oracle
        q = np.concatenate([q[..., d // 2:], q[..., :d // 2]], axis=-1)
        k = np.concatenate([k[..., d // 2:], k[..., :d // 2]], axis=-1)
    want = oracle.prefill(q, k, v, pos, 0, theta ** 2, 0.5)[:, S - 1]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_common_shift_of_positions_changes_nothing():
    B, S, Hq, Hkv, d = 2, 9, 4, 2, 32
    q, k, v = rnd((B, S, Hq, d), 12), rnd((B, S, Hkv, d), 13), rnd((B, S, Hkv, d), 14)
    pos2 = grid_pos(B, S, 15)
    a = oracle.vision_prefill(q, k, v, pos2, 1e4)
    b = oracle.vision_prefill(q, k, v, pos2 + np.array([57, 1000], np.int32), 1e4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_permuting_patches_permutes_outputs():
    B, S, Hq, Hkv, d = 1, 11, 2, 1, 16
    q, k, v = rnd((B, S, Hq, d), 16), rnd((B, S, Hkv, d), 17), rnd((B, S, Hkv, d), 18)
    pos2 = grid_pos(B, S, 19)
    perm = np.random.default_rng(20).permutation(S)
    a = oracle.vision_prefill(q, k, v, pos2, 1e4)
    b = oracle.vision_prefill(q[:, perm], k[:, perm], v[:, perm], pos2[:, perm], 1e4)
    np.testing.assert_allclose(b, a[:, perm], rtol=0, atol=1e-12)


def test_padding_patches_are_ignored_and_zero():
    B, S, n, Hq, Hkv, d = 1, 12, 7, 4, 2, 16
    q, k, v = rnd((B, S, Hq, d), 21), rnd((B, S, Hkv, d), 22), rnd((B, S, Hkv, d), 23)
    pos2 = grid_pos(B, S, 24)
    short = oracle.vision_prefill(q[:, :n], k[:, :n], v[:, :n], pos2[:, :n], 1e4)
    q[:, n:], k[:, n:], v[:, n:] = np.nan, np.nan, np.nan
    got = oracle.vision_prefill(q, k, v, pos2, 1e4, lengths=[n])
    np.testing.assert_array_equal(got[:, :n], short)
    assert (got[:, n:] == 0).all()


def test_zero_query_gives_mean_of_valid_values():
    B, S, Hq, Hkv, d = 2, 10, 4, 2, 8
    q = np.zeros((B, S, Hq, d), np.float32)
    k, v = rnd((B, S, Hkv, d), 25), rnd((B, S, Hkv, d), 26)
    ln = [10, 4]
    got = oracle.vision_prefill(q, k, v, grid_pos(B, S, 27), 1e4, lengths=ln)
    for b in range(B):
        mean = v[b, :ln[b]].astype(np.float64).mean(axis=0)  # [Hkv, d]
        for h in range(Hq):
            np.testing.assert_allclose(got[b, :ln[b], h], np.broadcast_to(mean[h // 2], (ln[b], d)),
                                       rtol=0, atol=1e-12)


def test_invalid_arguments_rejected():
    q, k = rnd((1, 4, 2, 8), 1), rnd((1, 4, 1, 8), 2)
    with pytest.raises(ValueError):
        oracle.vision_prefill(q, k, k, grid_pos(1, 4, 3), 0.0)
    q6, k6 = rnd((1, 4, 2, 6), 1), rnd((1, 4, 1, 6), 2)  # d not a multiple of 4
    with pytest.raises(ValueError):
        oracle.vision_prefill(q6, k6, k6, grid_pos(1, 4, 3), 1e4)


# --- mutants ---------------------------------------------------------------------

MUTANTS = {
    "components_swapped": [
        ("g4o_rope(qr, half, half / 2, theta, (double)pos2[pq]);\n        g4o_rope(qr + half, half, half / 2, theta, (double)pos2[pq + 1]);",
         "g4o_rope(qr, half, half / 2, theta, (double)pos2[pq + 1]);\n        g4o_rope(qr + half, half, half / 2, theta, (double)pos2[pq]);"),
        ("g4o_rope(kr, half, half / 2, theta, (double)pos2[pk]);\n          g4o_rope(kr + half, half, half / 2, theta, (double)pos2[pk + 1]);",
         "g4o_rope(kr, half, half / 2, theta, (double)pos2[pk + 1]);\n          g4o_rope(kr + half, half, half / 2, theta, (double)pos2[pk]);"),
    ],
    "frequency_over_full_dim": [
        ("g4o_rope(qr, half, half / 2, theta, (double)pos2[pq]);",
         "g4o_rope(qr, d, half / 2, theta, (double)pos2[pq]);"),
        ("g4o_rope(kr, half, half / 2, theta, (double)pos2[pk]);",
         "g4o_rope(kr, d, half / 2, theta, (double)pos2[pk]);"),
    ],
    "causal_mask_kept": [
        ("for (int j = 0; j < n; ++j) {\n          const size_t koff",
         "for (int j = 0; j <= i; ++j) {\n          const size_t koff"),
        ("for (int j = 0; j < n; ++j) if (sc[j] > m) m = sc[j];",
         "for (int j = 0; j <= i; ++j) if (sc[j] > m) m = sc[j];"),
        ("for (int j = 0; j < n; ++j) { sc[j] = exp(sc[j] - m); l += sc[j]; }",
         "for (int j = 0; j <= i; ++j) { sc[j] = exp(sc[j] - m); l += sc[j]; }"),
        ("for (int j = 0; j < n; ++j) {\n          const size_t voff",
         "for (int j = 0; j <= i; ++j) {\n          const size_t voff"),
    ],
    "lengths_ignored": [("int n = lengths ? lengths[b] : S;", "int n = S;")],
    "padding_rows_attend": [("if (i >= n) {  /* padding patch */", "if (i >= S) {  /* padding patch */")],
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("vision_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    path = mutant_dir / f"{name}.c"
    path.write_text(src)
    lib_path = mutant_dir / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", str(path), "-o", str(lib_path),
                    "-lm"], check=True)
    lib = oracle.load(str(lib_path))
    caught = False
    for case in CASES:
        B, S, Hq, Hkv, d, ln = case
        q, k, v = rnd((B, S, Hq, d), 1), rnd((B, S, Hkv, d), 2), rnd((B, S, Hkv, d), 3)
        pos2 = grid_pos(B, S, 4)
        got = oracle.vision_prefill(q, k, v, pos2, 1e4, lengths=ln, lib=lib)
        want = brute.vision_attention(q.astype(np.float64), k.astype(np.float64),
                                      v.astype(np.float64), pos2, 1e4, ln)
        caught |= not np.allclose(got, want, rtol=0, atol=1e-12)
    # the one-axis reduction (catches a consistent swap of the components)
    S, d = 12, 16
    q, k, v = rnd((1, S, 4, d), 9), rnd((1, S, 2, d), 10), rnd((1, S, 2, d), 11)
    pos = (np.arange(S, dtype=np.int32) * 3 + 2)[None]
    pos2 = np.zeros((1, S, 2), np.int32)
    pos2[..., 0] = pos
    got = oracle.vision_prefill(q, k, v, pos2, 1e4, lib=lib)[:, S - 1]
    want = oracle.prefill(q, k, v, pos, 0, 1e8, 0.5)[:, S - 1]
    caught |= not np.allclose(got, want, rtol=0, atol=1e-12)
    assert caught, f"mutant {name} survived the pins"
