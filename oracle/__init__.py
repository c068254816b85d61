"""fp64 CPU oracle for the log-mel front end.

TEST INFRASTRUCTURE: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library under ``log_mel_spectrogram_amd/`` and imports nothing from it.
"""

from .logmel_oracle import (  # noqa: F401
    SAMPLE_RATE, N_FFT, HOP, N_BINS, N_MELS, F_MIN, F_MAX, LOG_FLOOR, CHUNK_FRAMES,
    num_frames, frame_offsets, hamming_window, hz_to_mel, mel_to_hz,
    mel_vertices_hz, mel_filterbank, frames_of, power_spectrum, mel_energy,
    log_compress, logmel_frames, logmel_clip, logmel_packed, logmel_selected,
    num_chunks, chunk_offsets, chunk_frames, logmel_chunked,
    RESAMPLE_ZEROS, RESAMPLE_ROLLOFF, RESAMPLE_BETA, resample_length, resample_offsets,
    resample_cutoff, resample_halfwidth, resample_kernel, resample_clip, resample_packed,
    resample_selected,
)
