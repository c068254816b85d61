"""Seeded input generators: determinism and the recipe's shape facts."""

import numpy as np
import torch

import logmel_synth as S


def test_splitmix64_matches_reference():
    idx = torch.arange(-5, 1000, dtype=torch.int64)
    got = S.splitmix64(idx).tolist()
    ref = [S._s64(S.splitmix64_py(int(i) & ((1 << 64) - 1))) for i in idx.tolist()]
    assert got == ref


def test_gaussian_moments_and_determinism():
    g1 = S.gaussian(7, torch.arange(200000))
    g2 = S.gaussian(7, torch.arange(200000))
    assert torch.equal(g1, g2)
    assert abs(float(g1.mean())) < 0.01
    assert abs(float(g1.std()) - 1.0) < 0.01
    assert not torch.equal(g1, S.gaussian(8, torch.arange(200000)))


def test_three_tone():
    x, so = S.config0()
    assert x.dtype == torch.float32 and x.numel() == 16000
    assert float(x.abs().max()) <= 1.0
    assert so.tolist() == [0, 16000]


def test_speech_like_recipe():
    x = S.speech_like(1, 480000)
    assert x.dtype == torch.float32 and x.numel() == 480000
    assert abs(float(x.abs().max()) - 0.9) < 1e-6
    zero = float((x == 0).float().mean())
    assert 0.03 < zero < 0.07            # about 5 % exact silence
    assert torch.equal(x, S.speech_like(1, 480000))
    lay = S.speech_layout(1, 480000)
    L = lay.lengths
    assert L.min() >= 1600 and L.max() <= 6400
    assert np.all(np.diff(lay.starts) > 0)


def test_chunking_does_not_change_samples():
    a = S.speech_like(3, 100000, chunk=1 << 21)
    b = S.speech_like(3, 100000, chunk=7919)
    assert torch.equal(a, b)


def test_config4_lengths():
    lens = S.config4_lengths()
    assert lens.size == 200
    assert lens.min() >= 8000 and lens.max() <= 83_520_000
    assert int(lens.sum()) * 4 > 2**32      # byte offsets exceed 32 bits
