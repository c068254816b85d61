"""Loads the built HIP library for tests, building it first only if it is
missing (build() is what normally produces it)."""

import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "log_mel_spectrogram_amd", "liblogmel.so")


def load_binding():
    if not os.path.exists(LIB):
        # build.py by path: importing the package itself needs the library
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "logmel_build", os.path.join(ROOT, "log_mel_spectrogram_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import log_mel_spectrogram_amd as lm
    return lm
