"""C-ABI library: loads, exports what include/logmel.h declares, and its host
logic (frame arithmetic, argument checks) behaves; no GPU needed."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from tests.libload import ROOT, load_binding


@pytest.fixture(scope="module")
def lm():
    return load_binding()


def _declared():
    text = open(os.path.join(ROOT, "include", "logmel.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(logmel_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lm):
    names = _declared()
    assert len(names) >= 15
    lib = ctypes.CDLL(lm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(lm.EXPORTED) == names


def test_abi_version(lm):
    assert lm.logmel_abi_version() == 1


def test_num_frames_matches_closed_form(lm):
    for n in list(range(0, 1200)) + [16000, 480000, 83_520_000, 2**40, -5]:
        assert lm.logmel_num_frames(n) == O.num_frames(max(n, 0))


def test_frame_offsets_int64(lm):
    rng = np.random.default_rng(0)
    lens = np.concatenate([[0, 399, 400, 401, 559, 560], rng.integers(0, 5000, 200),
                           [3_000_000_000, 83_520_000]])
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    fo = lm.logmel_frame_offsets(so)
    assert fo.dtype == np.int64
    assert np.array_equal(fo, O.frame_offsets(so))
    assert so[-1] > 2**31


def test_frame_offsets_rejects_bad_offsets(lm):
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_frame_offsets([0, 10, 5])
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
    with pytest.raises(lm.LogmelError):
        lm.logmel_frame_offsets([3, 10])


def test_status_strings(lm):
    for code in (0, -1, -2, -3, -4, -5):
        assert lm.logmel_status_string(code) not in ("", "unknown status")
    assert lm.logmel_status_string(7) == "unknown status"


def test_default_config_is_the_pages(lm):
    cfg = lm.logmel_default_config()
    assert (cfg.sample_rate, cfg.n_fft, cfg.hop, cfg.n_mels) == (16000, 400, 160, 128)
    assert (cfg.f_min, cfg.f_max, cfg.log_floor) == (0.0, 8000.0, 1e-10)


@pytest.mark.parametrize("field,value", [("sample_rate", 44100), ("n_fft", 512),
                                         ("hop", 256), ("n_mels", 80), ("f_max", 7600.0),
                                         ("log_floor", 1e-6)])
def test_unsupported_configs_rejected_before_device(lm, field, value):
    cfg = lm.logmel_default_config()
    setattr(cfg, field, value)
    with pytest.raises(lm.LogmelError) as e:
        lm.Plan(cfg)
    assert e.value.status == lm.LOGMEL_ERR_UNSUPPORTED


def test_null_arguments(lm):
    h = ctypes.c_void_p()
    assert lm._plan_create(None, ctypes.byref(h)) == lm.LOGMEL_ERR_INVALID_ARGUMENT
    assert lm._compute(None, None, None, None, 1, 1, None, None) == lm.LOGMEL_ERR_INVALID_ARGUMENT
    assert lm._stream_create(None, 1, 1, ctypes.byref(h)) == lm.LOGMEL_ERR_INVALID_ARGUMENT
    assert lm._stream_push(None, None, None, None, None, None) == lm.LOGMEL_ERR_INVALID_ARGUMENT


def test_chunk_offsets_and_frames_match_oracle(lm):
    rng = np.random.default_rng(3)
    lens = np.concatenate([[0, 399, 400, 480000, 480400, 960000, 480000 + 320],
                           rng.integers(0, 2_000_000, 100), [83_520_000, 3_000_000_000]])
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    co = lm.logmel_chunk_offsets(so)
    assert co.dtype == np.int64
    assert np.array_equal(co, O.chunk_offsets(so))
    cf = lm.logmel_chunk_frames(so, int(co[-1]))
    assert np.array_equal(cf, O.chunk_frames(so))
    assert lm.CHUNK_FRAMES == O.CHUNK_FRAMES


def test_chunk_helpers_reject_bad_input(lm):
    with pytest.raises(lm.LogmelError):
        lm.logmel_chunk_offsets([0, 10, 5])
    so = np.array([0, 480000], dtype=np.int64)
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_chunk_frames(so, 2)          # the batch has 1 chunk
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
    assert lm._compute_chunked(None, None, None, None, None, 1, 1, 1, None, None) == \
        lm.LOGMEL_ERR_INVALID_ARGUMENT


def test_compute_ex_null_arguments(lm):
    assert lm._compute_ex(None, None, lm.LOGMEL_F32, None, None, None, 1, 1, 0, None,
                          lm.LOGMEL_F32, None) == lm.LOGMEL_ERR_INVALID_ARGUMENT


def test_resample_lengths_and_offsets_match_oracle(lm):
    rng = np.random.default_rng(4)
    for rate in (8000, 11025, 16000, 22050, 44100, 48000, 96000, 192000, 7350, 1000, 384000):
        for n in list(range(0, 60)) + list(rng.integers(0, 10**9, 40)) + [2**40]:
            assert lm.logmel_resample_length(int(n), rate) == O.resample_length(int(n), rate)
        lens = rng.integers(0, 3 * rate, 50)
        so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        oo = lm.logmel_resample_offsets(so, rate)
        assert oo.dtype == np.int64 and np.array_equal(oo, O.resample_offsets(so, rate))


def test_resample_helpers_reject_bad_input(lm):
    assert lm.logmel_resample_length(-1, 44100) == -1
    assert lm.logmel_resample_length(100, 999) == -1
    assert lm.logmel_resample_length(100, 384001) == -1
    assert lm.logmel_resample_length(2**62, 44100) == -1
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_resample_offsets([0, 10, 5], 44100)
    assert e.value.status == lm.LOGMEL_ERR_INVALID_ARGUMENT
    with pytest.raises(lm.LogmelError) as e:
        lm.logmel_resample_offsets([0, 10], 500)
    assert e.value.status == lm.LOGMEL_ERR_UNSUPPORTED
    h = ctypes.c_void_p()
    assert lm._resampler_create(None, 44100, ctypes.byref(h)) == lm.LOGMEL_ERR_INVALID_ARGUMENT
    assert lm._resample(None, None, lm.LOGMEL_F32, None, None, 1, 1, None, None) == \
        lm.LOGMEL_ERR_INVALID_ARGUMENT
    assert lm._resampler_info(None, None, None) == lm.LOGMEL_ERR_INVALID_ARGUMENT
