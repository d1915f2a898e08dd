"""Fused STFT -> mel-spectrogram forward pass for AMD MI355X (gfx950).

The compute lives in libfm.so (C ABI in include/fm.h); `MelSpectrogram` is a
thin torch-facing caller of it.  Importing the package does not load the
library; touching `MelSpectrogram` does, and fails loudly if it is missing.
"""

__all__ = ["MelSpectrogram"]


def __getattr__(name):
    if name == "MelSpectrogram":
        from .melspec import MelSpectrogram
        return MelSpectrogram
    raise AttributeError(name)
