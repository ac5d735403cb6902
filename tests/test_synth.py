"""Pins for the seeded input generators (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from tests.conftest import GOLDEN


def test_splitmix64_known_answers():
    with open(os.path.join(GOLDEN, "splitmix64.json")) as f:
        ref = json.load(f)
    for s in ref["streams"]:
        if "outputs_hex" in s:
            expect = [int(h, 16) for h in s["outputs_hex"]]
        else:
            expect = [int(v) for v in s["outputs"]]
        got = synth.splitmix64(s["seed"], np.arange(len(expect), dtype=np.uint64))
        assert [int(v) for v in got] == expect


def test_random_words_are_low_halves():
    idx = np.arange(10, dtype=np.uint64)
    full = synth.splitmix64(12345, idx)
    assert np.array_equal(synth.random_words(12345, idx), (full & np.uint64(0xFFFFFFFF)).astype(np.uint32))


def test_random_words_balanced_signs():
    w = synth.random_words(synth.seed64("balance"), np.arange(1 << 16, dtype=np.uint64))
    ones = np.unpackbits(w.view(np.uint8)).mean()
    assert abs(ones - 0.5) < 0.005


def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(0)
    a = np.concatenate([g.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.0e38, 1e-40], np.float32)])
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_activation_outliers():
    x = synth.activations("t/outl", 3, 1000, "bf16", outlier_frac=0.01)
    for t in range(3):
        assert np.sum(np.abs(x[t]) == 20.0) == 10
    assert np.array_equal(synth.round_bf16(x), x)


def test_streams_are_reproducible_and_distinct():
    a = synth.normal_f32("a", 5)
    assert np.array_equal(a, synth.normal_f32("a", 5))
    assert not np.array_equal(a, synth.normal_f32("b", 5))
    assert synth.seed64("a") != synth.seed64("b")


def test_lognormal_parameters():
    s = synth.scales_lognormal("ln", 200000)
    ls = np.log(s.astype(np.float64))
    assert ls.mean() == pytest.approx(-4.0, abs=0.01)
    assert ls.std() == pytest.approx(0.5, abs=0.01)
