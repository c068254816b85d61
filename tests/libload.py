"""Loads the built HIP library for tests, building it first only if it is
missing (build() is what normally produces it)."""

import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "log_mel_spectrogram_amd", "liblogmel.so")


def load_binding():
    if not os.path.exists(LIB):
        from log_mel_spectrogram_amd.build import build
        build()
    import log_mel_spectrogram_amd as lm
    return lm
