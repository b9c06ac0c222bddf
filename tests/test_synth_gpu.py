"""The device input generator reproduces the host generator bit for bit."""
import numpy as np
import pytest
import torch

import synth
import synth.gpu

pytestmark = pytest.mark.gpu


def test_planes_match_host():
    for (N, K) in [(77, 384), (64, 4096)]:
        got = synth.gpu.planes_shape(9, 3, 5, 1, N, K).cpu().numpy().view(np.uint32)
        assert np.array_equal(got, synth.gen_planes_shape(9, 3, 5, 1, N, K))


def test_parent_lut_matches_host():
    got = synth.gpu.parent_lut_shape(9, 2, 7, 0, 513).cpu().numpy()
    ref = synth.gen_parent_lut_shape(9, 2, 7, 0, 513)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_fp16_normal_matches_host():
    for std in (1.0, 0.02):
        got = synth.gpu.fp16_normal(4, 77, 100003, std).cpu().numpy()
        ref = synth.fp16_normal(4, 77, 100003, std)
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
