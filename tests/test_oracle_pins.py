"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula and compares it with itself:
each check comes from a page value, a closed form, an invariant, a textbook
special case, or brute force written independently here. Each is chosen so
that a plausible slip in the oracle (a periodic instead of symmetric window,
a dropped 1/2, a wrong bin spacing, an off-by-one in framing, a log10 in
place of ln, unpinned end vertices) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- page facts

def test_page_parameters(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))
    assert O.SAMPLE_RATE == facts["sample_rate"]["value"]
    assert O.N_FFT == facts["n_fft"]["value"]
    assert O.HOP == facts["hop"]["value"]
    assert O.N_BINS == facts["rfft_bins"]["value"]
    assert O.N_MELS == facts["n_mels"]["value"]
    assert O.LOG_FLOOR == facts["log_floor"]["value"]
    assert len(O.hamming_window()) == facts["hamming_len"]["value"]
    # 25 ms and 10 ms at 16 kHz
    assert O.N_FFT == round(0.025 * O.SAMPLE_RATE)
    assert O.HOP == round(0.010 * O.SAMPLE_RATE)
    # mel formula constants (page 1, §2.3 step 4): evaluate at f = 700 Hz,
    # where it is a * log10(2)
    mf = facts["mel_formula"]
    assert O.hz_to_mel(mf["b"]) == pytest.approx(mf["a"] * math.log10(2.0), rel=1e-15)


def test_frame_count_page_example(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))
    ex = facts["frame_count_30s"]
    exact = (ex["n_samples"] - 400) / 160 + 1          # 2998.5 as printed
    F = O.num_frames(ex["n_samples"])
    assert F == math.floor(exact) == 2998
    assert abs(F - ex["page_value_approx"]) <= 2       # "≈ 3000"
    assert O.num_frames(facts["samples_1s"]["value"]) == 98


# ------------------------------------------------------------- framing pins

def _brute_frame_count(n):
    """Count starts s = 0, 160, 320, ... with a full 400-sample frame."""
    c, s = 0, 0
    while s + 400 <= n:
        c += 1
        s += 160
    return c


def test_frame_count_brute():
    for n in list(range(0, 2400)) + [16000, 176000, 480000, 83_520_000 // 100]:
        assert O.num_frames(n) == _brute_frame_count(n), n
    # closed values (C truncation would give 1 for 241..399)
    assert [O.num_frames(n) for n in (0, 241, 399, 400, 559, 560)] == [0, 0, 0, 1, 1, 2]
    assert O.num_frames(83_520_000) == 521_998
    assert O.num_frames(8000) == 48


def test_frame_offsets_int64():
    lens = [0, 399, 400, 401, 559, 560, 480000, 3_000_000_000]
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    fo = O.frame_offsets(so)
    assert fo.dtype == np.int64
    acc = [0]
    for n in lens:
        acc.append(acc[-1] + _brute_frame_count(n) if n < 10**6 else
                   acc[-1] + (n - 400) // 160 + 1)
    assert fo.tolist() == acc
    assert so[-1] > 2**31 and fo[-1] == acc[-1]


def test_frames_are_hop_strided():
    x = np.arange(1000, dtype=np.float64)
    fr = O.frames_of(x)
    assert fr.shape == (4, 400)
    for f in range(4):
        assert np.array_equal(fr[f], np.arange(160 * f, 160 * f + 400))


# -------------------------------------------------------------- window pins

def test_window_closed_forms():
    w = O.hamming_window()
    # sum_{n=0}^{399} cos(2 pi n / 399) = 1 (a full period of 399 plus n=399)
    assert w.sum() == pytest.approx(0.54 * 400 - 0.46 * 1.0, abs=1e-12)   # 215.54
    # sum cos^2 = 200.5 -> sum w^2 = 158.569
    assert (w ** 2).sum() == pytest.approx(
        0.54 ** 2 * 400 - 2 * 0.54 * 0.46 * 1.0 + 0.46 ** 2 * 200.5, abs=1e-11)
    assert np.allclose(w, w[::-1], atol=1e-15, rtol=0)          # symmetric
    assert w[0] == pytest.approx(0.08, abs=1e-15)
    assert w[399] == pytest.approx(0.08, abs=1e-15)
    assert w.argmax() in (199, 200)


def test_window_is_numpy_hamming():
    # page 1 §2.3 step 3 calls numpy's Hamming window of length 400
    assert np.max(np.abs(O.hamming_window() - np.hamming(400))) < 1e-15


# ---------------------------------------------------------- transform pins

def _brute_dft(y):
    N = len(y)
    n = np.arange(N)
    X = np.zeros(N, dtype=np.complex128)
    for k in range(N):
        X[k] = np.sum(y * np.exp(-2j * np.pi * k * n / N))
    return X


def test_power_spectrum_vs_brute_dft():
    rng = np.random.default_rng(1)
    fr = rng.uniform(-1, 1, (3, 400))
    P = O.power_spectrum(fr)
    w = np.array([0.54 - 0.46 * math.cos(2 * math.pi * n / 399) for n in range(400)])
    for i in range(3):
        X = _brute_dft(fr[i] * w)
        ref = np.abs(X[:201]) ** 2
        assert np.max(np.abs(P[i] - ref)) <= 1e-10 * np.max(ref)


def test_parseval():
    rng = np.random.default_rng(2)
    fr = rng.normal(size=(16, 400))
    P = O.power_spectrum(fr)
    w = O.hamming_window()
    lhs = np.sum((fr * w) ** 2, axis=1)
    rhs = (P[:, 0] + 2 * P[:, 1:200].sum(axis=1) + P[:, 200]) / 400
    assert np.allclose(lhs, rhs, rtol=1e-13, atol=0)


@pytest.mark.parametrize("k0", [1, 5, 25, 75, 150, 199])
def test_pure_tone(k0):
    """A sin(2 pi (40 k0) n / 16000) -> bin k0 with power
    (A/2)^2 |sum w - What(2 k0)|^2, What the window's DFT written as a sum;
    for k0 away from the ends that is (A sum w / 2)^2 to within 2e-3."""
    A = 0.3
    n = np.arange(400)
    x = A * np.sin(2 * np.pi * 40 * k0 * n / 16000)
    P = O.power_spectrum(x[None, :])[0]
    w = np.array([0.54 - 0.46 * math.cos(2 * math.pi * m / 399) for m in range(400)])
    What = np.sum(w * np.exp(-2j * np.pi * (2 * k0) * n / 400))
    exact = (A / 2) ** 2 * abs(w.sum() - What) ** 2
    assert P[k0] == pytest.approx(exact, rel=1e-12)
    assert int(np.argmax(P)) == k0
    if 2 <= k0 <= 198:
        assert P[k0] == pytest.approx((A * 215.54 / 2) ** 2, rel=2e-3)


# ----------------------------------------------------------------- mel pins

def test_mel_scale_values():
    assert O.hz_to_mel(0.0) == 0.0
    assert O.hz_to_mel(8000.0) == pytest.approx(2595 * math.log10(1 + 8000 / 700), rel=1e-15)
    assert O.hz_to_mel(8000.0) == pytest.approx(2840.023046708319, rel=1e-14)
    # natural-log form 1127 ln(1 + f/700) agrees to the constant's precision
    for f in (100.0, 1000.0, 4000.0):
        assert O.hz_to_mel(f) == pytest.approx(2595 / math.log(10) * math.log(1 + f / 700), rel=1e-15)
    for f in (1.0, 440.0, 7999.0):
        assert O.mel_to_hz(O.hz_to_mel(f)) == pytest.approx(f, rel=1e-12)


def test_mel_vertices():
    f = O.mel_vertices_hz()
    assert f.size == 130
    assert f[0] == 0.0 and f[-1] == 8000.0           # pinned exactly
    m = O.hz_to_mel(f)
    step = 2595 * math.log10(1 + 8000 / 700) / 129
    assert np.allclose(np.diff(m), step, rtol=0, atol=1e-9)   # even in mel
    assert np.all(np.diff(f) > 0) and np.all(np.diff(np.diff(f)) > 0)  # dense low


def _interp_weight(m, phi, f):
    """Triangle m as a piecewise-linear interpolation through its vertices."""
    return np.interp(phi, [f[m - 1], f[m], f[m + 1]], [0.0, 1.0, 0.0],
                     left=0.0, right=0.0)


def test_filterbank_vs_interpolation():
    W = O.mel_filterbank()
    f = O.mel_vertices_hz()
    phi = 40.0 * np.arange(201)
    for m in range(1, 129):
        assert np.allclose(W[m - 1], _interp_weight(m, phi, f), atol=1e-14, rtol=0)


def test_filterbank_invariants():
    W = O.mel_filterbank()
    f = O.mel_vertices_hz()
    assert W.shape == (128, 201)
    assert W.min() >= 0.0 and W.max() <= 1.0
    # bins 0 and 200 sit on the pinned end vertices: exactly zero weight
    assert np.all(W[:, 0] == 0.0) and np.all(W[:, 200] == 0.0)
    # each bin lies in at most two triangles
    assert ((W > 0).sum(axis=0)).max() == 2
    # partition of unity between the first and last peaks
    phi = 40.0 * np.arange(201)
    inner = (phi >= f[1]) & (phi <= f[128])
    assert np.allclose(W[:, inner].sum(axis=0), 1.0, atol=1e-13, rtol=0)
    # a filter is empty exactly when no bin falls strictly inside its support
    brute_empty = [m for m in range(1, 129)
                   if not np.any((phi > f[m - 1]) & (phi < f[m + 1]))]
    assert brute_empty == [1, 4, 7, 14]
    assert [m for m in range(1, 129) if not np.any(W[m - 1] > 0)] == brute_empty
    assert int((W > 0).sum()) == 394
    # no area normalisation: each non-empty filter's largest weight is the
    # interpolation at the bin nearest its peak, and the top one is < 1
    assert W.max() == pytest.approx(0.9972954518776668, abs=1e-12)


def test_whole_chain_brute_force():
    """Full chain on tiny inputs from independent pieces: the window written
    out, the DFT as a double sum, each triangle as a piecewise-linear
    interpolation through its vertices (vertices from the mel formula
    evaluated with math.log10), and ln(max(E, 1e-10))."""
    a = 2595.0 * math.log10(1.0 + 8000.0 / 700.0)
    f = [700.0 * (10.0 ** (a * i / 129 / 2595.0) - 1.0) for i in range(130)]
    f[0], f[129] = 0.0, 8000.0
    w = np.array([0.54 - 0.46 * math.cos(2 * math.pi * n / 399) for n in range(400)])
    rng = np.random.default_rng(8)
    n = np.arange(400)
    frames = [rng.uniform(-1, 1, 400),
              0.3 * np.sin(2 * np.pi * 200 * n / 16000),
              1e-4 * rng.normal(size=400)]
    for x in frames:
        X = _brute_dft(x * w)
        P = np.abs(X[:201]) ** 2
        phi = 40.0 * np.arange(201)
        E = np.array([np.sum(_interp_weight(m, phi, np.array(f)) * P)
                      for m in range(1, 129)])
        ref = np.log(np.maximum(E, 1e-10))
        L, Eo = O.logmel_frames(x[None, :])
        # fp64 rounding is relative to the frame's largest energy
        assert np.allclose(Eo[0], E, rtol=1e-9, atol=1e-13 * E.max())
        ok = E > 1e-6 * E.max()
        assert np.allclose(L[0][ok], ref[ok], rtol=0, atol=1e-9)
        assert np.array_equal(L[0][E == 0], ref[E == 0])


def test_white_noise_mel_expectation():
    """E[E_m] = sigma^2 * sum w^2 * sum_k W[m,k] for white noise."""
    rng = np.random.default_rng(3)
    sigma = 0.01
    x = rng.normal(0, sigma, 160 * 20000 + 240)
    L, E = O.logmel_clip(x)
    W = O.mel_filterbank()
    w2 = 0.54 ** 2 * 400 - 2 * 0.54 * 0.46 + 0.46 ** 2 * 200.5
    expect = sigma ** 2 * w2 * W.sum(axis=1)
    nz = expect > 0
    # bins 1..199 only: no DC / Nyquist weight, so no factor-2 bins involved
    assert np.allclose(E.mean(axis=0)[nz], expect[nz], rtol=0.05)


# ----------------------------------------------------------------- log pins

def test_silence():
    L, E = O.logmel_clip(np.zeros(16000))
    assert L.shape == (98, 128)
    assert np.all(E == 0.0)
    assert np.all(L == math.log(1e-10))
    assert L[0, 0] == -23.025850929940457


def test_empty_filters_floor():
    x = np.random.default_rng(4).uniform(-1, 1, 4000)
    L, E = O.logmel_clip(x)
    for m in (1, 4, 7, 14):
        assert np.all(L[:, m - 1] == math.log(1e-10))


def test_scale_invariance():
    rng = np.random.default_rng(5)
    x = rng.uniform(-0.5, 0.5, 4000)
    L1, E1 = O.logmel_clip(x)
    for c in (0.25, -3.0):
        L2, E2 = O.logmel_clip(c * x)
        ok = (E1 >= 1e-10) & (E2 >= 1e-10)
        assert np.allclose(L2[ok], L1[ok] + 2 * math.log(abs(c)), atol=1e-12)


def test_natural_log_not_log10():
    x = np.zeros(400)
    x[200] = 1.0                 # impulse: P[k] = w[200]^2 for every bin
    L, E = O.logmel_clip(x)
    W = O.mel_filterbank()
    w200 = 0.54 - 0.46 * math.cos(2 * math.pi * 200 / 399)
    m = 60
    assert L[0, m] == pytest.approx(math.log(w200 ** 2 * W[m].sum()), rel=1e-13)


def test_nan_propagates():
    x = np.zeros(400)
    x[10] = np.nan
    L, _ = O.logmel_clip(x)
    assert np.isnan(L[0, 60])


# ------------------------------------------------------- framing invariants

def test_shift_by_hop():
    rng = np.random.default_rng(6)
    x = rng.uniform(-1, 1, 5000)
    L1, _ = O.logmel_clip(x)
    L2, _ = O.logmel_clip(x[160:])
    assert np.array_equal(L1[1:], L2)


def test_periodic_signal_identical_frames():
    """200/1000/3000 Hz tones have a common period of 80 samples; the hop is
    160, so every frame of the noiseless signal is the same frame."""
    n = np.arange(16000)
    x = sum(0.3 * np.sin(2 * np.pi * f * n / 16000) for f in (200, 1000, 3000))
    L, E = O.logmel_clip(x)
    assert L.shape == (98, 128)
    # identical up to fp64 rounding, which is relative to the loudest band
    assert np.max(np.abs(E - E[0])) < 1e-12 * E.max()
    loud = E[0] > 1e-6 * E.max()
    assert np.max(np.abs(L[:, loud] - L[0, loud])) < 1e-9


def test_packed_equals_per_clip():
    rng = np.random.default_rng(7)
    lens = [0, 399, 400, 1000, 37, 2000]
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    s = rng.uniform(-1, 1, so[-1])
    L, E, fo = O.logmel_packed(s, so)
    for i, n in enumerate(lens):
        Li, _ = O.logmel_clip(s[so[i]:so[i + 1]])
        assert np.array_equal(L[fo[i]:fo[i + 1]], Li)
    rows = np.arange(fo[-1])
    Ls, _ = O.logmel_selected(s, so, rows)
    assert np.allclose(Ls, L, atol=1e-12, rtol=0)


# ------------------------------------------------------------ 30-s chunks

def _brute_chunk_count(F):
    """Count chunk starts 0, 3000, 6000, ... that hold at least one frame."""
    c, start = 0, 0
    while start < F:
        c += 1
        start += 3000
    return c


def test_chunk_page_facts(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))
    ch = facts["chunk_30s"]
    assert O.CHUNK_FRAMES == ch["frames"]
    # 3000 frames at the 10 ms hop are exactly the 30 s of the chunk
    assert O.CHUNK_FRAMES * O.HOP == ch["seconds"] * O.SAMPLE_RATE
    shape = facts["encoder_input_shape"]["shape"]
    assert shape[1:] == [O.CHUNK_FRAMES, O.N_MELS]


def test_chunk_counts_brute():
    for F in list(range(0, 7000)) + [521_998, 2_998_000]:
        assert O.num_chunks(F) == _brute_chunk_count(F), F
    # a 30 s clip has 2998 frames: one chunk, two rows of padding
    assert O.num_chunks(O.num_frames(480000)) == 1
    # 87 minutes (the longest input page 3 accepts) -> 174 chunks
    assert O.num_chunks(O.num_frames(87 * 60 * 16000)) == 174


def test_chunk_offsets_and_frames():
    lens = [0, 399, 400, 480000, 480160, 960000, 480000 + 160 * 2, 16000]
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    co = O.chunk_offsets(so)
    cf = O.chunk_frames(so)
    assert co.dtype == np.int64 and co[0] == 0
    F = [_brute_frame_count(n) for n in lens]
    assert F == [0, 0, 1, 2998, 2999, 5998, 3000, 98]
    assert list(np.diff(co)) == [_brute_chunk_count(f) for f in F]
    assert list(cf) == [1, 2998, 2999, 3000, 2998, 3000, 98]
    # the chunks of a clip hold its frames exactly once
    for i, f in enumerate(F):
        assert sum(cf[co[i]:co[i + 1]]) == f


def test_chunked_layout():
    rng = np.random.default_rng(5)
    lens = [0, 3000 * 160 + 240, 399, 3000 * 160 + 400, 6000 * 160 + 240 + 37, 12345]
    x = (0.3 * rng.standard_normal(sum(lens))).astype(np.float32)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    chunks, co = O.logmel_chunked(x, so)
    L, _, fo = O.logmel_packed(x, so)
    floor = math.log(1e-10)
    assert chunks.shape == (int(co[-1]), 3000, 128)
    for i in range(len(lens)):
        F = int(fo[i + 1] - fo[i])
        for j in range(int(co[i + 1] - co[i])):
            n = min(3000, F - 3000 * j)
            # frame 3000 j + r of clip i sits in row r of its chunk j
            np.testing.assert_array_equal(chunks[co[i] + j, :n], L[fo[i] + 3000 * j: fo[i] + 3000 * j + n])
            assert np.all(chunks[co[i] + j, n:] == floor)
    # a 3000-frame clip fills its chunk with no padding; one more frame opens
    # a second chunk holding a single frame
    assert [O.num_frames(n) for n in lens] == [0, 3000, 0, 3001, 6000, 75]
    assert list(np.diff(co)) == [0, 1, 0, 2, 2, 1]
    assert O.chunk_frames(so).tolist() == [3000, 3000, 1, 3000, 3000, 75]


# ------------------------------------------------------- streaming clocks

def test_stream_clocks_page_facts(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))
    cl = facts["stream_clocks_ms"]
    for ms, rate in zip(cl["value"], cl["decisions_per_s"]):
        assert 1000.0 / ms == pytest.approx(rate, abs=0.05)
    assert [ms * O.SAMPLE_RATE // 1000 for ms in cl["value"]] == [1280, 1920, 2560]
    assert facts["stream_push_80ms"]["value"] == 1280


@pytest.mark.parametrize("push,first,steady", [(1280, 6, 8), (1920, 10, 12), (2560, 14, 16)])
def test_stream_schedule_and_carry(push, first, steady):
    """Frames a push completes on the offline grid, and the carry left: by
    brute enumeration of frame starts over the concatenated stream."""
    emitted = 0
    for c in range(1, 200):
        n = c * push
        F = _brute_frame_count(n)
        per_push = F - emitted
        emitted = F
        assert per_push == (first if c == 1 else steady), (push, c)
        # the carry: samples from the next frame's start to the end
        carry = n - 160 * F
        assert carry == 320 == 240 + ((n - 400) % 160)
        assert O.num_frames(n) == F


# ------------------------------------------------------- resampling to 16 kHz
#
# The pages name no resampling method (the reading is in the oracle's
# docstring); these pin the oracle's resampler to what band-limited
# interpolation must do whatever its parameters: exact output counts, the
# time base (an output sample sits at n / 16000 s), passband tones kept,
# out-of-band tones removed, zero padding at clip edges, and the window.

RATES = [8000, 11025, 22050, 24000, 32000, 44100, 48000, 96000]


def _interior(rate, n_in, n_out):
    """Outputs whose kernel support lies inside the clip."""
    H = O.resample_halfwidth(rate)
    n = np.arange(n_out)
    p = n * rate / 16000
    return (p - H >= 0) & (p + H <= n_in - 1)


@pytest.mark.parametrize("rate", RATES)
def test_resample_length_brute(rate):
    rng = np.random.default_rng(rate)
    for N in list(range(0, 40)) + list(rng.integers(0, 100000, 30)):
        N = int(N)
        brute = 0
        while brute * rate < 16000 * N:     # output n exists iff its time n/16000 < N/rate
            brute += 1
        assert O.resample_length(N, rate) == brute, (rate, N)
    lens = rng.integers(0, 5000, 20)
    so = np.concatenate([[0], np.cumsum(lens)])
    oo = O.resample_offsets(so, rate)
    assert oo[0] == 0 and np.array_equal(np.diff(oo), [O.resample_length(int(n), rate) for n in lens])


def test_resample_16k_is_identity():
    x = np.random.default_rng(1).standard_normal(1234)
    y, a = O.resample_clip(x, 16000)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("rate", [8000, 22050, 32000, 44100, 48000, 96000])
def test_resample_passband_tones(rate):
    """A tone well inside the passband comes out as the same tone sampled at
    16 kHz (amplitude and phase), away from the clip edges."""
    n_in = rate // 2
    k = np.arange(n_in)
    top = 3000.0 if rate < 16000 else 6000.0
    for f in (300.0, 1000.0, top):
        th = 0.7
        x = np.sin(2 * np.pi * f * k / rate + th)
        y, _ = O.resample_clip(x, rate)
        n = np.arange(y.size)
        ref = np.sin(2 * np.pi * f * n / 16000 + th)
        m = _interior(rate, n_in, y.size)
        assert m.sum() > 1000
        assert np.abs(y - ref)[m].max() < 1e-3, (rate, f)


@pytest.mark.parametrize("rate,f", [(48000, 9000.0), (48000, 12000.0), (44100, 15000.0),
                                    (96000, 30000.0), (22050, 10000.0)])
def test_resample_stopband_tones(rate, f):
    """A tone above 8 kHz (which would alias into the 16 kHz band) is removed."""
    n_in = rate // 2
    x = np.sin(2 * np.pi * f * np.arange(n_in) / rate)
    y, _ = O.resample_clip(x, rate)
    m = _interior(rate, n_in, y.size)
    assert np.abs(y[m]).max() < 1e-4, (rate, f)


@pytest.mark.parametrize("rate", [8000, 44100, 48000])
def test_resample_dc_gain(rate):
    y, _ = O.resample_clip(np.ones(rate // 4), rate)
    m = _interior(rate, rate // 4, y.size)
    assert np.abs(y[m] - 1.0).max() < 1e-4


@pytest.mark.parametrize("rate,k0,n0", [(48000, 3 * 500, 500), (44100, 441 * 4, 160 * 4),
                                        (8000, 700, 1400), (22050, 441 * 2, 320 * 2)])
def test_resample_impulse_time_base(rate, k0, n0):
    """An impulse at input sample k0 whose time k0/R equals output time
    n0/16000 gives an output symmetric about n0 with its peak there (the
    kernel is even): pins the time base and the index arithmetic."""
    x = np.zeros(4 * k0)
    x[k0] = 1.0
    y, _ = O.resample_clip(x, rate)
    assert k0 * 16000 == n0 * rate
    assert int(np.argmax(y)) == n0
    d = np.arange(1, 200)
    np.testing.assert_allclose(y[n0 + d], y[n0 - d], rtol=0, atol=1e-15)
    # the peak is the kernel's centre value 2 fc / R (the window is 1 there)
    assert y[n0] == pytest.approx(2 * O.resample_cutoff(rate) / rate, rel=1e-14)


@pytest.mark.parametrize("rate", [11025, 44100, 48000, 24000])
def test_resample_shift_and_zero_edges(rate):
    """Delaying the input by M = R / gcd(R, 16000) samples delays the output
    by L = 16000 / gcd samples exactly; a clip's output equals the output of
    the same clip with zeros around it (samples outside a clip are zero)."""
    g = math.gcd(rate, 16000)
    M, L = rate // g, 16000 // g
    x = np.random.default_rng(rate).uniform(-1, 1, 3000 + rate // 50)
    y, _ = O.resample_clip(x, rate)
    P = 2 * (int(O.resample_halfwidth(rate)) // M + 2)
    xz = np.concatenate([np.zeros(P * M), x, np.zeros(P * M)])
    yz, _ = O.resample_clip(xz, rate)
    np.testing.assert_array_equal(yz[P * L: P * L + y.size], y)
    assert yz.size == y.size + 2 * P * L


def test_resample_kernel_against_library_window_and_sinc_zeros():
    """The window is numpy's Kaiser window sampled over the support; the
    kernel vanishes at the sinc's zero crossings and peaks at 2 fc / R."""
    for rate in (44100, 48000, 8000):
        fc = O.resample_cutoff(rate)
        H = O.resample_halfwidth(rate)
        K = 50
        r = (np.arange(2 * K + 1) - K) / K          # window positions in [-1, 1]
        d = r * H
        sinc = np.sinc(2 * fc * d / rate)
        with np.errstate(invalid="ignore", divide="ignore"):
            win = O.resample_kernel(d, rate) / ((2 * fc / rate) * sinc)
        ok = (np.abs(sinc) > 1e-6) & (np.abs(r) < 1)
        np.testing.assert_allclose(win[ok], np.kaiser(2 * K + 1, O.RESAMPLE_BETA)[ok], rtol=1e-12)
        m = np.arange(1, O.RESAMPLE_ZEROS)
        zeros = m * rate / (2 * fc)
        assert np.abs(O.resample_kernel(zeros, rate)).max() < 1e-15
        assert np.abs(O.resample_kernel(-zeros, rate)).max() < 1e-15
        assert O.resample_kernel(0.0, rate) == pytest.approx(2 * fc / rate, rel=1e-15)
        assert O.resample_kernel(H, rate) == 0.0 and O.resample_kernel(-H * 1.0001, rate) == 0.0


@pytest.mark.parametrize("rate", [8000, 44100, 48000])
def test_resample_half_gain_at_cutoff(rate):
    """A windowed sinc's transition is centred on its cutoff, where the gain
    is one half: pins the cutoff at 0.96 of the lower Nyquist frequency
    (7680 Hz into 16 kHz, 3840 Hz out of 8 kHz)."""
    f = 0.96 * min(rate, 16000) / 2
    n_in = rate
    x = np.sin(2 * np.pi * f * np.arange(n_in) / rate)
    y, _ = O.resample_clip(x, rate)
    m = _interior(rate, n_in, y.size)
    n = np.arange(y.size)[m]
    # amplitude by projection on the tone at 16 kHz
    c = np.cos(2 * np.pi * f * n / 16000)
    s = np.sin(2 * np.pi * f * n / 16000)
    A = np.hypot(np.dot(y[m], c), np.dot(y[m], s)) / (0.5 * n.size)
    assert A == pytest.approx(0.5, abs=0.01), (rate, A)


# ------------------------------------------ packed and selected resampling

RAGGED_RS = [0, 1, 37, 5000, 2, 12345, 0, 800]


@pytest.mark.parametrize("rate", [8000, 44100, 48000, 16000])
def test_resample_packed_equals_per_clip(rate):
    """Clip i of a packed batch is resample_clip of that clip alone, at the
    output rows the exclusive prefix sum of ceil(16000 N / R) gives; clips of
    0, 1 and 37 samples among them. Catches a misplaced output offset or a
    clip's window reading its neighbour's samples."""
    rng = np.random.default_rng(rate + 1)
    so = np.concatenate([[0], np.cumsum(RAGGED_RS)]).astype(np.int64)
    s = rng.uniform(-1, 1, so[-1])
    y, oo, a = O.resample_packed(s, so, rate)
    assert oo[0] == 0 and y.size == a.size == oo[-1]
    for i, n in enumerate(RAGGED_RS):
        assert oo[i + 1] - oo[i] == -(-n * 16000 // rate)
        yi, ai = O.resample_clip(s[so[i]:so[i + 1]], rate)
        assert np.array_equal(y[oo[i]:oo[i + 1]], yi)
        assert np.array_equal(a[oo[i]:oo[i + 1]], ai)


@pytest.mark.parametrize("rate", [8000, 44100, 48000, 16000])
def test_resample_selected_equals_packed(rate):
    """resample_selected, which forms each output from its own window, agrees
    with resample_packed at random rows, the first and last rows, and the
    rows on either side of every clip boundary. Catches an off-by-one in the
    row-to-clip lookup or in the window's clipping at a clip's ends."""
    rng = np.random.default_rng(rate + 2)
    so = np.concatenate([[0], np.cumsum(RAGGED_RS)]).astype(np.int64)
    s = rng.uniform(-1, 1, so[-1])
    y, oo, a = O.resample_packed(s, so, rate)
    total = int(oo[-1])
    rows = set(rng.integers(0, total, 60).tolist()) | {0, total - 1}
    for b in oo[1:-1]:
        rows |= {int(b) - 1, int(b)}
    rows = np.array(sorted(r for r in rows if 0 <= r < total), dtype=np.int64)
    ys, as_ = O.resample_selected(s, so, rate, rows)
    # the same terms summed in another order: equal to rounding
    assert np.allclose(ys, y[rows], rtol=0, atol=1e-13)
    assert np.allclose(as_, a[rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("rate", [11025, 44100, 48000])
def test_resample_error_scale_brute(rate):
    """The error scale a[n] = sum_k |x[k] h(p_n - k)| by a brute loop over
    every sample k of the clip (not only the window the oracle visits), with
    p_n = n R / 16000 from integer arithmetic. Catches a missing absolute
    value, a window narrower than the kernel's support, or a wrong position.
    Also a[n] >= |y[n]| (triangle inequality), with equality where every term
    has one sign."""
    rng = np.random.default_rng(rate + 3)
    N = 300
    x = rng.uniform(-1, 1, N)
    y, a = O.resample_clip(x, rate)
    for n in range(0, y.size, 7):
        p = n * rate / 16000.0
        acc = 0.0
        for k in range(N):
            acc += abs(x[k] * float(O.resample_kernel(p - k, rate)))
        assert a[n] == pytest.approx(acc, rel=1e-12, abs=1e-15)
    assert np.all(a >= np.abs(y) - 1e-15)
    # a single non-zero sample: one term per output, so a = |y| exactly
    x1 = np.zeros(N)
    x1[150] = -0.7
    y1, a1 = O.resample_clip(x1, rate)
    assert np.array_equal(a1, np.abs(y1))


def test_logmel_clip_multi_chunk():
    """logmel_clip works through a long clip in chunks of frames, each chunk's
    sample segment carrying the 240-sample halo its last frame needs. A clip
    of 65,600 frames (more than one default chunk of 65,536) gives the same
    frames with chunk 7 (thousands of boundaries), with the default chunk, and
    frame by frame from each frame's own 400 samples (logmel_selected).
    Catches a dropped halo (a short last frame) or a misplaced chunk start."""
    rng = np.random.default_rng(11)
    F = 65600
    x = rng.uniform(-1, 1, 160 * (F - 1) + 400 + 123)
    L1, E1 = O.logmel_clip(x)
    assert L1.shape == (F, 128)
    L7, E7 = O.logmel_clip(x, chunk=7)
    # the same per-frame arithmetic; only the batch size of the library calls differs
    assert np.allclose(E7, E1, rtol=1e-13, atol=0)
    assert np.allclose(L7, L1, rtol=0, atol=1e-12)
    rows = np.array([0, 6, 7, 65535, 65536, 65537, F - 1], dtype=np.int64)
    Ls, Es = O.logmel_selected(x, [0, x.size], rows)
    assert np.allclose(Es, E1[rows], rtol=1e-13, atol=0)
    assert np.allclose(Ls, L1[rows], rtol=0, atol=1e-12)


def test_nan_frame_is_nan_in_every_band():
    """A NaN sample reaches every bin of its frame's transform, and the
    filterbank sum of an empty filter (0 * NaN terms) is NaN too: the frames
    whose 400 samples hold the NaN are NaN in all 128 bands, the others are
    finite."""
    rng = np.random.default_rng(12)
    x = rng.uniform(-1, 1, 2000)
    x[700] = np.nan            # frames 2, 3 and 4 hold sample 700 (160 f <= 700 < 160 f + 400)
    L, _ = O.logmel_clip(x)
    bad = [f for f in range(L.shape[0]) if 160 * f <= 700 < 160 * f + 400]
    assert bad == [2, 3, 4]
    assert np.all(np.isnan(L[bad]))
    good = [f for f in range(L.shape[0]) if f not in bad]
    assert np.all(np.isfinite(L[good]))


def _library_audio_utils():
    return pytest.importorskip("transformers.audio_utils")


def test_filterbank_is_library_htk_bank():
    """The triangles as read (linear in Hz between vertices evenly spaced on
    the HTK mel scale, unnormalised; page 1, §2.3 step 4) are the bank that
    an independent library routine builds for mel_scale "htk", no norm:
    equal to fp64 rounding. The one cell whose support differs is filter
    128 at bin 200 (8000 Hz), where the oracle puts the end vertex exactly
    on 8000 Hz (weight 0) and the library's mel round trip lands a few ulps
    above it (weight ~1e-14). Both leave the same narrow low filters empty.
    Catches a triangle built in mel instead of Hz, a normalised bank, or
    vertices off by one."""
    au = _library_audio_utils()
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")   # the library warns about the empty filters
        T = au.mel_filter_bank(201, 128, 0.0, 8000.0, 16000, norm=None, mel_scale="htk").T
    W = O.mel_filterbank()
    assert T.shape == W.shape == (128, 201)
    assert np.max(np.abs(W - T)) < 1e-13
    differ = np.argwhere((W > 0) != (T > 0))
    assert [tuple(map(int, ij)) for ij in differ] == [(127, 200)]
    assert W[127, 200] == 0.0 and T[127, 200] < 1e-13
    assert np.array_equal(np.where(W.sum(1) == 0)[0], np.where(T.sum(1) == 0)[0])
    assert np.allclose(au.hertz_to_mel(np.array([0.0, 700.0, 8000.0]), mel_scale="htk"),
                       O.hz_to_mel(np.array([0.0, 700.0, 8000.0])), rtol=1e-15, atol=0)


@pytest.mark.parametrize("kind", ["noise", "tone_1k_full_scale", "dc", "silence_then_noise"])
def test_logmel_is_library_spectrogram(kind):
    """The whole chain (page 1, §2.3 steps 1-5: 400-sample frames at hop 160
    without centring, symmetric Hamming window, 400-point rFFT, power, HTK
    bank, ln of max(E, 1e-10)) against an independent library spectrogram
    routine given the same parameters and its own window and bank. The
    library keeps each frame's spectrum in complex64, so each bin's power
    carries a relative rounding of about 2**-23 and each band's log up to
    ~2.5e-7; 1e-6 is the bound. A wrong hop, a periodic window, a centred
    frame, a dropped partial frame kept, |X| instead of |X|^2 or log10 are
    all off by far more."""
    au = _library_audio_utils()
    import warnings
    rng = np.random.default_rng(21)
    n = 16000 + 123
    if kind == "noise":
        x = 0.3 * rng.standard_normal(n)
    elif kind == "tone_1k_full_scale":
        x = np.sin(2 * np.pi * 1000.0 * np.arange(n) / 16000.0)
    elif kind == "dc":
        x = np.full(n, 0.5)
    else:
        x = np.concatenate([np.zeros(4000), 0.1 * rng.standard_normal(n - 4000)])
    x32 = x.astype(np.float32)
    L, E, _ = O.logmel_packed(x32, np.array([0, n], dtype=np.int64))
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        T = au.mel_filter_bank(201, 128, 0.0, 8000.0, 16000, norm=None, mel_scale="htk")
    w = au.window_function(400, "hamming", periodic=False)
    S = au.spectrogram(x32.astype(np.float64), w, frame_length=400, hop_length=160,
                       fft_length=400, power=2.0, center=False, mel_filters=T, mel_floor=1e-10,
                       log_mel="log", dtype=np.float64).T
    assert S.shape == L.shape == (O.num_frames(n), 128)
    assert np.max(np.abs(S - L)) < 1e-6
