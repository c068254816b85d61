"""Seeded synthetic audio for the log-mel front end.

This module only makes input signals. It holds none of the front end's own
arithmetic (no framing, window, transform, filterbank or log) and is shared
by the tests, the benchmark and the smoke check, which feed the same fp32
buffer to the HIP library and to the fp64 oracle.

The workloads follow the shapes the pages give: 16 kHz mono float PCM in
[-1, 1], 1 s = 16000 samples and 30 s = 480000 samples (page 1, "从零理解
ASR…", §2.1); the 87-minute input limit of the transcribe.cpp Qwen3-ASR page
(§四); the 80 ms audio clock of the Audio8-ASR-Infinite page (1280 samples).
No dataset is used: every signal is synthetic and seeded.

Randomness:
* Small per-clip parameters (syllable lengths, pitches, phases, bursts, clip
  lengths) come from ``numpy.random.default_rng(seed)`` (PCG64).
* Per-sample Gaussian noise is counter based so that the same seed gives the
  same noise on the CPU and on a GPU: sample n of key k is Box-Muller of two
  uniforms taken from SplitMix64 (Steele, Lea & Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014) at counters 2n and 2n+1.

Sample synthesis runs in torch fp64 on any device and is cast once to fp32.
fp64 libm results may differ in the last bit between host and device, so a
test always generates its input once and hands that one buffer to both sides.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

FS = 16000

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """uint64 bit pattern -> the int64 with the same bits."""
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def splitmix64_py(x: int) -> int:
    """Reference SplitMix64 output for state ``x`` (pure Python, uint64)."""
    z = (x + _GOLDEN) & _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64(x: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output for int64 states ``x`` (bit patterns of uint64).

    int64 multiplication wraps modulo 2^64 in torch on CPU and GPU, which is
    the uint64 product's bit pattern.
    """
    z = x + _s64(_GOLDEN)
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def gaussian(key: int, idx: torch.Tensor) -> torch.Tensor:
    """Standard normal fp64 values for counters ``idx`` under ``key``."""
    base = _s64(splitmix64_py(key & _MASK64))
    h1 = splitmix64(base + 2 * idx)
    h2 = splitmix64(base + 2 * idx + 1)
    scale = 2.0 ** -53
    u1 = (_lsr(h1, 11).to(torch.float64) + 0.5) * scale
    u2 = (_lsr(h2, 11).to(torch.float64) + 0.5) * scale
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


# ---------------------------------------------------------------------------
# Config 0: three tones + light noise
# ---------------------------------------------------------------------------

def three_tone(seed: int = 0, n: int = 16000, device="cpu") -> torch.Tensor:
    """sum over f in {200, 1000, 3000} Hz of 0.3 sin(2 pi f n / 16000) plus
    0.01 N(0,1), clipped to [-1, 1]; fp32 [n].

    Time is n / 16000 exactly, so the tones sit on rFFT bins 5, 25 and 75.
    """
    idx = torch.arange(n, dtype=torch.int64, device=device)
    t = idx.to(torch.float64) / FS
    x = torch.zeros(n, dtype=torch.float64, device=device)
    for f in (200.0, 1000.0, 3000.0):
        x += 0.3 * torch.sin(2.0 * math.pi * f * t)
    x += 0.01 * gaussian(seed, idx)
    return x.clamp_(-1.0, 1.0).to(torch.float32)


# ---------------------------------------------------------------------------
# Speech-like clips
# ---------------------------------------------------------------------------

N_HARM = 20
_FIR_TAPS = 65


def _bandpass_fir(fs: int = FS) -> np.ndarray:
    """65-tap windowed-sinc band-pass, 2..6 kHz at fs (Hann taper)."""
    m = np.arange(_FIR_TAPS, dtype=np.float64) - (_FIR_TAPS - 1) / 2
    lo, hi = 2000.0 / fs, 6000.0 / fs
    h = 2 * hi * np.sinc(2 * hi * m) - 2 * lo * np.sinc(2 * lo * m)
    taper = 0.5 - 0.5 * np.cos(2 * np.pi * np.arange(_FIR_TAPS) / (_FIR_TAPS - 1))
    return h * taper


_FIR = _bandpass_fir()
_FIR_GAIN = float(np.sqrt(np.sum(_FIR ** 2)))


def _fir_at(fs: int):
    if fs == FS:
        return _FIR, _FIR_GAIN
    f = _bandpass_fir(fs)
    return f, float(np.sqrt(np.sum(f ** 2)))


@dataclass
class SpeechLayout:
    starts: np.ndarray      # int64 syllable start samples
    lengths: np.ndarray     # int64 syllable lengths
    f0: np.ndarray          # fp64 pitch per syllable (Hz)
    phases: np.ndarray      # fp64 [S, 20]
    burst_len: np.ndarray   # int64, 0 = no burst
    burst_off: np.ndarray   # int64 offset of the burst inside its syllable


def speech_layout(seed: int, n: int, fs: int = FS) -> SpeechLayout:
    """Syllable plan of G(seed, n).

    Syllables of U(100, 400) ms, each followed by an exact-zero gap of
    round(0.0526 * length) samples (about 5 % silence overall); pitch
    U(80, 300) Hz per syllable; 20 harmonic phases U(0, 2 pi); with
    probability 0.5 a noise burst of U(20, 80) ms placed uniformly inside the
    syllable.
    """
    rng = np.random.default_rng(seed)
    starts, lengths = [], []
    pos = 0
    while pos < n:
        L = int(round(rng.uniform(0.100, 0.400) * fs))
        starts.append(pos)
        lengths.append(L)
        pos += L + int(round(0.0526 * L))
    S = len(starts)
    starts = np.asarray(starts, dtype=np.int64)
    lengths = np.asarray(lengths, dtype=np.int64)
    f0 = rng.uniform(80.0, 300.0, S)
    phases = rng.uniform(0.0, 2 * np.pi, (S, N_HARM))
    has = rng.uniform(size=S) < 0.5
    blen = np.rint(rng.uniform(0.020, 0.080, S) * fs).astype(np.int64)
    boff = np.floor(rng.uniform(size=S) * (lengths - blen + 1)).astype(np.int64)
    blen = np.where(has, blen, 0)
    return SpeechLayout(starts, lengths, f0, phases, blen, boff)


def _speech_chunk(lay_t, key: int, a: int, b: int, device, fs: int = FS) -> torch.Tensor:
    starts, lengths, f0, phases, blen, boff = lay_t
    n = torch.arange(a, b, dtype=torch.int64, device=device)
    s = torch.searchsorted(starts, n, right=True) - 1
    t = n - starts[s]
    L = lengths[s]
    inside = t < L
    tf = t.to(torch.float64)
    env = 0.5 - 0.5 * torch.cos((2 * math.pi) * tf / L.to(torch.float64))
    w = (2 * math.pi / fs) * f0[s] * tf
    harm = torch.zeros(b - a, dtype=torch.float64, device=device)
    ph = phases[s]
    for h in range(1, N_HARM + 1):
        harm += torch.sin(h * w + ph[:, h - 1]) / h
    harm /= sum(1.0 / h for h in range(1, N_HARM + 1))
    x = torch.where(inside, env * harm, torch.zeros_like(harm))
    # band-limited noise bursts
    nb = t - boff[s]
    bl = blen[s]
    in_burst = inside & (bl > 0) & (nb >= 0) & (nb < bl)
    if bool(in_burst.any()):
        half = (_FIR_TAPS - 1) // 2
        idx = torch.arange(a - half, b + half, dtype=torch.int64, device=device)
        g = gaussian(key, idx)
        fir, fir_gain = _fir_at(fs)
        filt = torch.zeros(b - a, dtype=torch.float64, device=device)
        for j in range(_FIR_TAPS):
            filt += float(fir[j]) * g[j:j + (b - a)]
        taper = 0.5 - 0.5 * torch.cos((2 * math.pi) * nb.to(torch.float64)
                                      / bl.clamp(min=1).to(torch.float64))
        x = x + torch.where(in_burst, (0.1 / fir_gain) * filt * taper,
                            torch.zeros_like(filt))
    return x


def speech_like(seed: int, n: int, device="cpu", out: torch.Tensor | None = None,
                chunk: int = 1 << 21, fs: int = FS) -> torch.Tensor:
    """G(seed, n): fp32 [n] speech-like clip, peak-normalised to 0.9.

    Harmonic series (20 harmonics, amplitude 1/h) at a per-syllable pitch
    under a raised-cosine syllable envelope, plus 2..6 kHz noise bursts of
    RMS 0.1 under a raised-cosine taper, separated by exact-zero gaps.
    ``out`` may be a preallocated fp32 view of length n on ``device``. ``fs``
    is the sample rate the clip is made at (16 kHz unless another is asked
    for, as input for resampling); durations and pitches are in seconds and
    Hz, so a clip at another rate has the same structure.
    """
    lay = speech_layout(seed, n, fs)
    lay_t = tuple(torch.as_tensor(v, device=device) for v in
                  (lay.starts, lay.lengths, lay.f0, lay.phases, lay.burst_len,
                   lay.burst_off))
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    peak = 0.0
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        xc = _speech_chunk(lay_t, seed, a, b, device, fs)
        peak = max(peak, float(xc.abs().max()))
        out[a:b] = xc.to(torch.float32)
    if peak > 0:
        g = 0.9 / peak
        for a in range(0, n, chunk):
            b = min(n, a + chunk)
            out[a:b] = (out[a:b].to(torch.float64) * g).to(torch.float32)
    return out


# ---------------------------------------------------------------------------
# Packed batches
# ---------------------------------------------------------------------------

def pack(lengths, make, device="cpu"):
    """Pack clips of ``lengths`` contiguously. ``make(i, view)`` fills clip i.

    Returns (samples fp32 [sum], sample_offsets int64 numpy [n+1]).
    """
    lengths = [int(v) for v in lengths]
    so = np.zeros(len(lengths) + 1, dtype=np.int64)
    so[1:] = np.cumsum(lengths)
    samples = torch.empty(int(so[-1]), dtype=torch.float32, device=device)
    for i, L in enumerate(lengths):
        make(i, samples[so[i]:so[i + 1]])
    return samples, so


def config0(device="cpu"):
    """1 clip, 16000 samples: three tones + noise (seed 0)."""
    x = three_tone(0, 16000, device)
    return x, np.array([0, 16000], dtype=np.int64)


def config1(device="cpu"):
    """1 clip, 480000 samples (30 s): G(1, 480000)."""
    x = speech_like(1, 480000, device)
    return x, np.array([0, 480000], dtype=np.int64)


def config2(device="cpu", n_clips: int = 64):
    """64 clips of 480000 samples, clip i = G(100 + i, 480000), packed."""
    return pack([480000] * n_clips,
                lambda i, v: speech_like(100 + i, 480000, device, out=v), device)


def config2_at(rate: int, device="cpu", n_clips: int = 64, seconds: int = 30):
    """Config 2's clips made at another sample rate (input for resampling):
    clip i = G(100 + i, seconds * rate) at ``rate``, packed."""
    n = int(seconds) * int(rate)
    return pack([n] * n_clips,
                lambda i, v: speech_like(100 + i, n, device, out=v, fs=int(rate)), device)


def config3_streams(device="cpu", n_streams: int = 512, n_samples: int = 480000):
    """Stream j = G(10000 + j, 480000); fp32 [n_streams, n_samples]."""
    x = torch.empty((n_streams, n_samples), dtype=torch.float32, device=device)
    for j in range(n_streams):
        speech_like(10000 + j, n_samples, device, out=x[j])
    return x


def config3_streams_at(rate: int, device="cpu", n_streams: int = 512, seconds: int = 30):
    """Config 3's streams made at another sample rate (input for resampling
    streams): stream j = G(10000 + j, seconds * rate) at ``rate``; fp32
    [n_streams, seconds * rate]."""
    n = int(seconds) * int(rate)
    x = torch.empty((n_streams, n), dtype=torch.float32, device=device)
    for j in range(n_streams):
        speech_like(10000 + j, n, device, out=x[j], fs=int(rate))
    return x


C4_MIN_LEN = 8000
C4_MAX_LEN = 83_520_000


def config4_lengths(seed: int = 20000, n_clips: int = 200) -> np.ndarray:
    """Log-uniform clip lengths floor(exp(U(ln 8000, ln 83520000)))."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(C4_MIN_LEN), math.log(C4_MAX_LEN), n_clips)
    return np.floor(np.exp(u)).astype(np.int64)


def config4(device="cpu", seed: int = 20000, n_clips: int = 200):
    """200 ragged clips, clip i = G(seed + 1 + i, L_i), packed."""
    lens = config4_lengths(seed, n_clips)
    return pack(lens, lambda i, v: speech_like(seed + 1 + i, int(lens[i]),
                                               device, out=v), device)
