"""Pins for the oracle's 16-bit float handling and the comparison rule."""
import numpy as np
import pytest
import torch

import oracle
from oracle.numerics import bf16_to_f64, f64_to_bf16_rne, fp16_to_f64, bf16_bits_from_f64_rne


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # drop inf/nan
    ours = bf16_to_f64(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, t)


def test_fp16_widening_matches_numpy_half():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00]
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(fp16_to_f64(bits), ref)


def test_bf16_rne_hand_cases():
    # bf16 keeps 8 significant bits: the ulp of 1.0 is 2^-7.
    assert f64_to_bf16_rne(1.0 + 2.0 ** -8) == 1.0                    # tie -> even (1.0)
    assert f64_to_bf16_rne(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6    # tie -> even
    assert f64_to_bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7  # above the tie
    assert f64_to_bf16_rne(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    assert f64_to_bf16_rne(0.0) == 0.0
    assert f64_to_bf16_rne(3.0) == 3.0


def test_bf16_rne_matches_torch_on_fp32_values():
    # torch rounds fp32 -> bf16 to nearest even; on fp32-exact inputs there is
    # no double rounding, so the two must agree bit for bit.
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    ours = bf16_bits_from_f64_rne(v.astype(np.float64))
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, t)


def test_compare_rule_accepts_rounding_and_rejects_a_dropped_term():
    rng = np.random.default_rng(1)
    yo = rng.standard_normal(4096)
    ok, m = oracle.compare.check(f64_to_bf16_rne(yo), yo, "bf16")
    assert ok and m["rel_l2"] == 0.0
    assert m["literal_rel_l2"] > 1e-3  # why bf16 outputs compare against the rounded oracle
    ok, _ = oracle.compare.check(yo.astype(np.float32), yo, "f32")
    assert ok
    bad = yo.copy()
    bad[::7] = 0.0
    assert not oracle.compare.check(bad, yo, "f32")[0]
    assert not oracle.compare.check(yo * (1 + 2e-3), yo, "f32")[0]
