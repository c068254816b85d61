"""Plain fp64 CPU oracle for the 128-bin log-mel front end.

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product path.

What it computes, step by step, with the passage each step follows. "Page 1"
is the tutorial "从零理解 ASR：音频基础、Qwen3-ASR 架构，以及离线 vs 流式推理原理"
(marsggbo blog); its section 2.3 "Log-Mel Spectrogram 提取流水线" lists five
steps, quoted here by number.

1. Framing (page 1, §2.3 step 1 "分帧"): 400-sample frames (25 ms at 16 kHz)
   every 160 samples (10 ms), no centring or padding. The page writes the
   count for 30 s as (480000-400)/160+1; read as floor, and 0 frames for
   fewer than 400 samples.
2. Window (page 1, §2.3 step 2 "加窗", and the code of step 3, which calls
   numpy's 400-point Hamming window): symmetric Hamming,
   w[n] = 0.54 - 0.46 cos(2 pi n / 399), written out here rather than called.
3. rFFT and power (page 1, §2.3 step 3 "FFT → 功率谱"): 400-point real FFT to
   201 bins (0..8 kHz), power |X|^2 with no scaling. ``numpy.fft.rfft`` is
   the library primitive for the transform; the tests pin it against a
   brute-force DFT written as a double sum.
4. Mel filterbank (page 1, §2.3 step 4 "Mel 滤波器组"): mel = 2595 log10(1 +
   f/700); 128 triangular filters evenly spaced on the mel scale over
   0..8000 Hz. Readings where the page is silent: the 130 triangle vertices
   are evenly spaced in mel with the end vertices pinned to exactly 0 Hz and
   8000 Hz; each triangle is linear in Hz between its vertices with peak 1
   and no area normalisation. (The Hz-linear shape is a reading; the page
   does not fix it.)
5. Log (page 1, §2.3 step 5 "取对数"): natural log of max(mel energy, 1e-10),
   numpy's maximum semantics (a NaN propagates).

The output layout is frame-major [frames, 128] (page 1, the shape table after
step 5). The streaming result is, by definition, this offline result on the
concatenated stream.

30-s chunks for the encoder (page 1, the preprocessor-config list after
§2.3: chunk_length 30 s gives 3000 frames; page 1, §4 point 1: the encoder
input has the fixed shape [B, 3000, 128], and point 4: every input is padded
to 3000 frames; page 3, §二 stage 1: the front end cuts at 30 s). The pages do
not say which frames fall into which chunk, nor the pad value. Reading: chunk
j of a clip holds the clip's own frames 3000 j .. 3000 j + 2999 (the frames
that start in seconds 30 j .. 30 j + 30), so chunking never changes a frame;
the rows of the last chunk past the clip's last frame hold ln(1e-10), the
value the recipe gives silence; a clip with no frame has no chunk.

Resampling to 16 kHz (page 1, §6, the offline example in "可运行代码示例":
the processor takes 16 kHz input only and the example refuses other rates,
noting that a library resampler would be used in practice; page 1, §2.1:
speech content of interest lies below 8 kHz, hence 16 kHz). The pages name
no method. Reading: band-limited interpolation with a Kaiser-windowed sinc
(the textbook method of J. O. Smith's bandlimited interpolation). Output
sample n sits at time n / 16000 s, that is at input position
p = n R / 16000 for input rate R, and
    y[n] = sum_k x[k] h(p - k),   over the clip's samples k (zero outside),
    h(d) = (2 fc / R) sinc(2 fc d / R) kaiser(d / H),  |d| < H,  else 0,
with cutoff fc = 0.96 min(R, 16000) / 2, half-width H = 24 R / (2 fc) input
samples (24 zero crossings of the sinc on each side), kaiser(r) =
I0(9 sqrt(1 - r^2)) / I0(9). A clip of N samples gives ceil(16000 N / R)
output samples (those with p < N). At R = 16000 nothing is resampled: the
output is the input. These parameters are a reading; nothing in the pages
fixes them.

Everything here is fp64. The fp32 samples are upcast exactly.
"""

from __future__ import annotations

import numpy as np

SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160
N_BINS = N_FFT // 2 + 1
N_MELS = 128
F_MIN = 0.0
F_MAX = 8000.0
LOG_FLOOR = 1e-10
CHUNK_FRAMES = 3000   # page 1, preprocessor-config list: 30 s -> 3000 frames


def num_frames(n_samples: int) -> int:
    """Frame count of a clip of ``n_samples`` (page 1, §2.3 step 1).

    floor((N - 400) / 160) + 1 for N >= 400, else 0. Exact integer arithmetic.
    """
    n = int(n_samples)
    if n < N_FFT:
        return 0
    return (n - N_FFT) // HOP + 1


def frame_offsets(sample_offsets) -> np.ndarray:
    """Exclusive prefix sum of per-clip frame counts, int64, length n_clips+1.

    Clip i holds samples [sample_offsets[i], sample_offsets[i+1]); its frames
    are rows [result[i], result[i+1]) of the packed output.
    """
    so = [int(v) for v in np.asarray(sample_offsets).reshape(-1)]
    out = [0]
    for i in range(len(so) - 1):
        out.append(out[-1] + num_frames(so[i + 1] - so[i]))
    return np.asarray(out, dtype=np.int64)


def hamming_window() -> np.ndarray:
    """Symmetric 400-point Hamming window (page 1, §2.3 steps 2-3), fp64."""
    n = np.arange(N_FFT, dtype=np.float64)
    return 0.54 - 0.46 * np.cos(2.0 * np.pi * n / (N_FFT - 1))


def hz_to_mel(f):
    """HTK mel scale as printed in page 1, §2.3 step 4."""
    return 2595.0 * np.log10(1.0 + np.asarray(f, dtype=np.float64) / 700.0)


def mel_to_hz(m):
    """Inverse of :func:`hz_to_mel`."""
    return 700.0 * (10.0 ** (np.asarray(m, dtype=np.float64) / 2595.0) - 1.0)


def mel_vertices_hz() -> np.ndarray:
    """The 130 triangle vertices in Hz, evenly spaced in mel over 0..8000 Hz.

    The end vertices are set to exactly F_MIN and F_MAX (the mel round trip
    of 8000 Hz is 8000.000000000002 in fp64).
    """
    m = np.linspace(hz_to_mel(F_MIN), hz_to_mel(F_MAX), N_MELS + 2)
    f = mel_to_hz(m)
    f[0] = F_MIN
    f[-1] = F_MAX
    return f


def mel_filterbank() -> np.ndarray:
    """Dense [128, 201] fp64 filterbank (page 1, §2.3 step 4).

    W[m, k] = max(0, min((phi_k - f_{m-1}) / (f_m - f_{m-1}),
                         (f_{m+1} - phi_k) / (f_{m+1} - f_m)))
    for filter m = 1..128 (row m-1), bin frequency phi_k = k * 16000 / 400.
    """
    f = mel_vertices_hz()
    phi = np.arange(N_BINS, dtype=np.float64) * (SAMPLE_RATE / N_FFT)
    W = np.zeros((N_MELS, N_BINS), dtype=np.float64)
    for m in range(1, N_MELS + 1):
        lo, mid, hi = f[m - 1], f[m], f[m + 1]
        rise = (phi - lo) / (mid - lo)
        fall = (hi - phi) / (hi - mid)
        W[m - 1] = np.maximum(0.0, np.minimum(rise, fall))
    return W


_WINDOW = hamming_window()
_FILTERBANK = mel_filterbank()


def frames_of(x: np.ndarray) -> np.ndarray:
    """[F, 400] fp64 frames of one clip (page 1, §2.3 step 1); frame f is
    x[160 f : 160 f + 400]."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    F = num_frames(x.size)
    if F == 0:
        return np.zeros((0, N_FFT), dtype=np.float64)
    idx = HOP * np.arange(F)[:, None] + np.arange(N_FFT)[None, :]
    return x[idx]


def power_spectrum(frames: np.ndarray) -> np.ndarray:
    """|rFFT(w * frame)|^2, [F, 201] fp64 (page 1, §2.3 steps 2-3)."""
    spec = np.fft.rfft(frames * _WINDOW[None, :], n=N_FFT, axis=1)
    return spec.real ** 2 + spec.imag ** 2


def mel_energy(power: np.ndarray) -> np.ndarray:
    """E[f, m] = sum_k W[m, k] P[f, k], [F, 128] fp64 (page 1, §2.3 step 4)."""
    return power @ _FILTERBANK.T


def log_compress(energy: np.ndarray) -> np.ndarray:
    """ln(max(E, 1e-10)) with numpy maximum semantics (page 1, §2.3 step 5)."""
    return np.log(np.maximum(energy, LOG_FLOOR))


def logmel_frames(frames: np.ndarray):
    """Whole chain on given [F, 400] frames. Returns (logmel, mel_energy)."""
    E = mel_energy(power_spectrum(frames))
    return log_compress(E), E


def logmel_clip(x: np.ndarray, chunk: int = 65536):
    """Log-mel of one clip: ([F, 128] fp64 log-mel, [F, 128] fp64 energy)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    F = num_frames(x.size)
    L = np.empty((F, N_MELS), dtype=np.float64)
    E = np.empty((F, N_MELS), dtype=np.float64)
    for f0 in range(0, F, chunk):
        f1 = min(F, f0 + chunk)
        seg = x[HOP * f0: HOP * (f1 - 1) + N_FFT]
        Lc, Ec = logmel_frames(frames_of(seg))
        L[f0:f1] = Lc
        E[f0:f1] = Ec
    return L, E


def logmel_packed(samples: np.ndarray, sample_offsets):
    """Packed ragged batch: clip i is samples[so[i]:so[i+1]].

    Returns (logmel [sum F, 128], energy [sum F, 128], frame_offsets).
    """
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    fo = frame_offsets(so)
    total = int(fo[-1])
    L = np.empty((total, N_MELS), dtype=np.float64)
    E = np.empty((total, N_MELS), dtype=np.float64)
    for i in range(so.size - 1):
        if fo[i + 1] == fo[i]:
            continue
        Li, Ei = logmel_clip(samples[so[i]:so[i + 1]])
        L[fo[i]:fo[i + 1]] = Li
        E[fo[i]:fo[i + 1]] = Ei
    return L, E, fo


def logmel_selected(samples: np.ndarray, sample_offsets, rows):
    """Log-mel of selected output rows of a packed batch, one frame at a time
    from its own 400 samples. Returns (logmel [R, 128], energy [R, 128])."""
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    fo = frame_offsets(so)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    clip = np.searchsorted(fo, rows, side="right") - 1
    start = so[clip] + HOP * (rows - fo[clip])
    frames = np.stack([np.asarray(samples[s:s + N_FFT], dtype=np.float64)
                       for s in start]) if rows.size else np.zeros((0, N_FFT))
    return logmel_frames(frames)


def num_chunks(n_frames: int) -> int:
    """30-s chunks of a clip with ``n_frames`` frames: ceil(F / 3000) (see the
    chunking reading in the module docstring)."""
    return -(-int(n_frames) // CHUNK_FRAMES)


def chunk_offsets(sample_offsets) -> np.ndarray:
    """Exclusive prefix sum of per-clip chunk counts, int64, length n_clips+1."""
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    counts = [num_chunks(num_frames(int(so[i + 1] - so[i]))) for i in range(so.size - 1)]
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int64)


def chunk_frames(sample_offsets) -> np.ndarray:
    """Frames of the clip held by each chunk (the rest of its 3000 rows are
    padding), int64, one entry per chunk in order."""
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    out = []
    for i in range(so.size - 1):
        F = num_frames(int(so[i + 1] - so[i]))
        for j in range(num_chunks(F)):
            out.append(min(CHUNK_FRAMES, F - CHUNK_FRAMES * j))
    return np.asarray(out, dtype=np.int64)


def logmel_chunked(samples: np.ndarray, sample_offsets):
    """Encoder input [chunks, 3000, 128] fp64 of a packed batch: each clip's
    frames in order, cut every 3000 frames, the last chunk padded with
    ln(1e-10). Returns (chunks, chunk_offsets)."""
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    co = chunk_offsets(so)
    out = np.full((int(co[-1]), CHUNK_FRAMES, N_MELS), np.log(LOG_FLOOR), dtype=np.float64)
    for i in range(so.size - 1):
        F = num_frames(int(so[i + 1] - so[i]))
        if F == 0:
            continue
        Li, _ = logmel_clip(samples[so[i]:so[i + 1]])
        for j in range(int(co[i + 1] - co[i])):
            rows = Li[CHUNK_FRAMES * j:CHUNK_FRAMES * (j + 1)]
            out[co[i] + j, :rows.shape[0]] = rows
    return out, co


# ---------------------------------------------------------------------------
# Resampling to 16 kHz (see the reading in the module docstring)
# ---------------------------------------------------------------------------

RESAMPLE_ZEROS = 24        # zero crossings of the sinc on each side
RESAMPLE_ROLLOFF = 0.96    # cutoff as a fraction of the lower Nyquist frequency
RESAMPLE_BETA = 9.0        # Kaiser window shape


def resample_length(n_samples: int, rate: int) -> int:
    """Output samples of a clip of ``n_samples`` at ``rate`` Hz: the n >= 0
    with n rate < 16000 n_samples, i.e. ceil(16000 N / R)."""
    return -(-int(n_samples) * SAMPLE_RATE // int(rate))


def resample_offsets(sample_offsets, rate: int) -> np.ndarray:
    """Exclusive prefix sum of per-clip output lengths, int64."""
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    n = [resample_length(int(so[i + 1] - so[i]), rate) for i in range(so.size - 1)]
    return np.concatenate([[0], np.cumsum(np.asarray(n, dtype=np.int64))]).astype(np.int64)


def resample_cutoff(rate: int) -> float:
    """Cutoff fc in Hz."""
    return RESAMPLE_ROLLOFF * min(int(rate), SAMPLE_RATE) / 2.0


def resample_halfwidth(rate: int) -> float:
    """Half-width H of the kernel in input samples."""
    return RESAMPLE_ZEROS * int(rate) / (2.0 * resample_cutoff(rate))


def resample_kernel(d, rate: int) -> np.ndarray:
    """h(d) for offsets d (input samples, fp64): the windowed sinc above.
    ``numpy.sinc`` and ``numpy.i0`` are the library primitives."""
    d = np.asarray(d, dtype=np.float64)
    fc = resample_cutoff(rate)
    H = resample_halfwidth(rate)
    r = d / H
    inside = np.abs(r) < 1.0
    win = np.i0(RESAMPLE_BETA * np.sqrt(np.where(inside, 1.0 - r * r, 0.0))) / np.i0(RESAMPLE_BETA)
    return np.where(inside, (2.0 * fc / rate) * np.sinc(2.0 * fc * d / rate) * win, 0.0)


def resample_clip(x: np.ndarray, rate: int):
    """One clip resampled to 16 kHz: (y fp64 [ceil(16000 N / R)], a) where
    a[n] = sum_k |x[k] h(p - k)| (the scale of output n's rounding).

    The position of output n is p = n R / 16000, kept exact as the integer
    part q = floor(n R / 16000) and the remainder n R mod 16000."""
    x = np.asarray(x, dtype=np.float64)
    N = x.size
    rate = int(rate)
    n_out = resample_length(N, rate)
    if rate == SAMPLE_RATE:
        return x.copy(), np.abs(x)
    n = np.arange(n_out, dtype=np.int64)
    q = (n * rate) // SAMPLE_RATE
    frac = ((n * rate) % SAMPLE_RATE) / SAMPLE_RATE
    J = int(np.ceil(resample_halfwidth(rate)))
    y = np.zeros(n_out)
    a = np.zeros(n_out)
    for j in range(-J, J + 1):
        k = q + j
        ok = (k >= 0) & (k < N)
        h = resample_kernel(frac - j, rate)
        t = np.where(ok, x[np.clip(k, 0, max(N - 1, 0))] if N else 0.0, 0.0) * h
        y += t
        a += np.abs(t)
    return y, a


def resample_packed(samples: np.ndarray, sample_offsets, rate: int):
    """A packed batch resampled clip by clip: (y fp64, out_offsets, a)."""
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    oo = resample_offsets(so, rate)
    y = np.zeros(int(oo[-1]))
    a = np.zeros(int(oo[-1]))
    for i in range(so.size - 1):
        yi, ai = resample_clip(samples[so[i]:so[i + 1]], rate)
        y[oo[i]:oo[i + 1]] = yi
        a[oo[i]:oo[i + 1]] = ai
    return y, oo, a


def resample_selected(samples: np.ndarray, sample_offsets, rate: int, rows):
    """Chosen outputs of resample_packed, each from its definition (for
    batches too large to resample whole): (y fp64, a) at flat output rows."""
    so = np.asarray(sample_offsets, dtype=np.int64).reshape(-1)
    oo = resample_offsets(so, rate)
    rows = np.asarray(rows, dtype=np.int64)
    clip = np.searchsorted(oo, rows, side="right") - 1
    y = np.zeros(rows.size)
    a = np.zeros(rows.size)
    J = int(np.ceil(resample_halfwidth(rate)))
    for t, (g, c) in enumerate(zip(rows, clip)):
        n = int(g - oo[c])
        N = int(so[c + 1] - so[c])
        if int(rate) == SAMPLE_RATE:
            y[t] = samples[so[c] + n]
            a[t] = abs(y[t])
            continue
        q = (n * int(rate)) // SAMPLE_RATE
        frac = ((n * int(rate)) % SAMPLE_RATE) / SAMPLE_RATE
        j = np.arange(-J, J + 1)
        k = q + j
        ok = (k >= 0) & (k < N)
        xs = np.asarray(samples[so[c] + k[ok]], dtype=np.float64)
        terms = xs * resample_kernel(frac - j[ok], rate)
        y[t] = terms.sum()
        a[t] = np.abs(terms).sum()
    return y, a
