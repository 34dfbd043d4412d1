"""Pins for the oracle's scoring rule.

L2 mode stores ||k||_2 (L2Norm page, "How it works" step 1); projection mode
stores sign * (k . f) in float32 (Q-Filters page, "How it works" step 3).  The
oracle sums in fp64 and rounds once to float32.  Pinned by closed forms on
exactly representable inputs, by numpy's fp64 norm / dot as an independent
library route, and by the bf16 widening definition.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from kv_cache_token_amd import synth

D = 128


def _rows(vals, dtype):
    x = np.zeros((len(vals), D), dtype=np.float32)
    for i, v in enumerate(vals):
        x[i, :len(v)] = v
    return x if dtype == "f32" else synth.bf16_bits_from_f32_np(x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_l2_closed_forms(dtype):
    # Pythagorean quadruples: integer norms, exact in any sum order
    k = _rows([[3, 4], [1, 2, 2], [2, 3, 6], [1, 4, 8], [-2, -3, 6], [0]], dtype)
    assert oracle.score(k, "l2").tolist() == [5.0, 3.0, 7.0, 9.0, 7.0, 0.0]
    ones = np.ones((1, D), dtype=np.float32)
    ones = ones if dtype == "f32" else synth.bf16_bits_from_f32_np(ones)
    assert oracle.score(ones, "l2")[0] == np.float32(math.sqrt(128.0))


def test_l2_matches_numpy_fp64_norm():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((4000, D)) * rng.lognormal(0, 2, (4000, 1))).astype(np.float32)
    got = oracle.score(x, "l2")
    want = np.linalg.norm(x.astype(np.float64), axis=1).astype(np.float32)
    ulp = np.abs(got.view(np.int32) - want.view(np.int32))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.999


@pytest.mark.parametrize("sign", [1, -1])
def test_projection_exact_on_dyadic_inputs(sign):
    rng = np.random.default_rng(2)
    k = rng.integers(-8, 9, size=(64, D)).astype(np.float32)
    f = (rng.integers(-64, 65, size=D) / 64.0).astype(np.float32)
    got = oracle.score(synth.bf16_bits_from_f32_np(k), "proj", f, sign)
    for i in range(64):
        exact = sign * sum(Fraction(int(k[i, d])) * Fraction(float(f[d])) for d in range(D))
        assert got[i] == np.float32(float(exact))


def test_projection_matches_numpy_dot_and_sign_is_exact_negation():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((3000, D)).astype(np.float32)
    f = rng.standard_normal(D)
    f = (f / np.linalg.norm(f)).astype(np.float32)
    kb = synth.bf16_bits_from_f32_np(k)
    kw = synth.bf16_bits_to_f32(kb).astype(np.float64)
    pos = oracle.score(kb, "proj", f, 1)
    neg = oracle.score(kb, "proj", f, -1)
    want = (kw @ f.astype(np.float64)).astype(np.float32)
    ulp = np.abs(pos.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.999
    nz = pos != 0
    assert np.array_equal(neg[nz], -pos[nz])


def test_negative_zero_is_stored_as_positive_zero():
    k = np.zeros((2, D), dtype=np.float32)
    k[1, 0], k[1, 1] = 1.0, 1.0
    f = np.zeros(D, dtype=np.float32)
    f[0], f[1] = 1.0, -1.0
    for sign in (1, -1):
        s = oracle.score(k, "proj", f, sign)
        assert s.view(np.uint32).tolist() == [0, 0]


def test_bf16_widening_definition():
    bits = np.zeros((1, D), dtype=np.uint16)
    bits[0, :4] = [0x3F80, 0xC000, 0x4040, 0x0000]   # 1, -2, 3, 0 -> norm sqrt(14)
    assert oracle.score(bits, "l2")[0] == np.float32(math.sqrt(14.0))


def test_non_finite_keys_are_rejected():
    k = np.zeros((1, D), dtype=np.float32)
    k[0, 5] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.score(k, "l2")
    with pytest.raises(oracle.OracleError):
        oracle.score(k, "proj", np.zeros(D, np.float32), 2)


def test_bf16_rounding_helper_matches_numpy_definition():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(200000) * rng.lognormal(0, 3, 200000)).astype(np.float32)
    x[:6] = [0.0, -0.0, 1.0, 1.00390625, 1.005859375, -3.0e-39]   # ties and a subnormal
    assert np.array_equal(synth.bf16_bits_from_f32(x), synth.bf16_bits_from_f32_np(x))


def test_f16_widening_definition_and_numpy_route():
    bits = np.zeros((1, D), dtype=np.uint16)
    bits[0, :4] = [0x3C00, 0xC000, 0x4200, 0x0000]   # 1, -2, 3, 0 -> norm sqrt(14)
    assert oracle.score(bits, "l2", dtype="f16")[0] == np.float32(math.sqrt(14.0))
    # the largest normal, the smallest subnormal and a mid subnormal, against numpy's float16
    rng = np.random.default_rng(7)
    x64 = rng.standard_normal((500, D)) * rng.lognormal(0, 4, (500, 1))
    x64[np.abs(x64) > 65504.0] = 1.0          # keep every value finite in binary16
    x = x64.astype(np.float16)
    x[0, :3] = [65504.0, 2.0 ** -24, 3 * 2.0 ** -20]
    got = oracle.score(x.view(np.uint16), "l2", dtype="f16")
    want = np.linalg.norm(x.astype(np.float64), axis=1).astype(np.float32)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.99


@pytest.mark.parametrize("Dd", [64, 256])
def test_other_head_dims_match_numpy(Dd):
    rng = np.random.default_rng(Dd)
    k = rng.standard_normal((300, Dd)).astype(np.float32)
    f = rng.standard_normal(Dd).astype(np.float32)
    got = oracle.score(k, "proj", f, 1)
    want = (k.astype(np.float64) @ f.astype(np.float64)).astype(np.float32)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.99
    kb = synth.encode(k, "bf16")
    assert np.array_equal(oracle.score(kb, "l2"), oracle.score(synth.bits_to_f32(kb, "bf16"), "l2"))
