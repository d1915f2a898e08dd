"""Seeded synthetic inputs and the workload parameter sets.

This module holds no step of the mel-spectrogram computation: it only names
parameter sets and draws input signals.  Both the HIP path's tests/bench and
the oracle's tests take their inputs from here, so the two sides always see
the very same cast array (f32, or int16 PCM).

Signal recipes (random numbers drawn with numpy.random.default_rng(seed) in
float64, then cast once to the device dtype):

* ``noise``   : N(0, sigma^2) white noise.
* ``sines``   : noise sigma=0.1 plus, per signal, 3 sines of amplitude 0.3 with
                frequencies ~ U(50, 7000) Hz and phases ~ U(0, 2*pi).
* ``pcm16``   : int16 drawn uniformly over [-32768, 32767].
* ``chirp``   : noise sigma=0.1 plus 0.3*sin(phi(t)), a linear chirp from
                100 Hz to 10 kHz over the signal, identical on every row.
"""
from __future__ import annotations

import numpy as np

# Parameter sets of the five workloads (torchaudio MelSpectrogram arguments
# plus the input shape and dtype).  All use a periodic Hann window, centre
# reflect padding, the HTK mel scale, no filter norm and f_min = 0.
WORKLOADS = {
    "tiny": dict(batch=1, length=16000, dtype="f32", signal="noise", sigma=0.1, seed=1,
                 sample_rate=16000, n_fft=400, win_length=400, hop_length=160,
                 n_mels=80, f_min=0.0, f_max=8000.0, power=2.0),
    "whisper": dict(batch=8, length=480000, dtype="f32", signal="sines", sigma=0.1, seed=2,
                    sample_rate=16000, n_fft=400, win_length=400, hop_length=160,
                    n_mels=128, f_min=0.0, f_max=8000.0, power=2.0),
    "int16": dict(batch=8, length=480000, dtype="i16", signal="pcm16", seed=3,
                  sample_rate=16000, n_fft=400, win_length=400, hop_length=160,
                  n_mels=128, f_min=0.0, f_max=8000.0, power=2.0),
    "pow2": dict(batch=8, length=32768, dtype="f32", signal="noise", sigma=1.0, seed=4,
                 sample_rate=16000, n_fft=1024, win_length=1024, hop_length=256,
                 n_mels=80, f_min=0.0, f_max=8000.0, power=2.0),
    "large": dict(batch=64, length=220500, dtype="f32", signal="chirp", sigma=0.1, seed=5,
                  sample_rate=22050, n_fft=2048, win_length=2048, hop_length=512,
                  n_mels=128, f_min=0.0, f_max=11025.0, power=1.0),
    # measurement and parity cases for the other FFT sizes (not in the pages'
    # benchmark table; shapes of common speech and music front ends)
    "asr512": dict(batch=8, length=480000, dtype="f32", signal="sines", sigma=0.1, seed=6,
                   sample_rate=16000, n_fft=512, win_length=400, hop_length=160,
                   n_mels=80, f_min=0.0, f_max=8000.0, power=2.0),
    "music4096": dict(batch=4, length=1323000, dtype="f32", signal="chirp", sigma=0.1, seed=7,
                      sample_rate=44100, n_fft=4096, win_length=4096, hop_length=1024,
                      n_mels=128, f_min=0.0, f_max=22050.0, power=2.0),
    "fft256": dict(batch=8, length=480000, dtype="f32", signal="noise", sigma=0.1, seed=8,
                   sample_rate=16000, n_fft=256, win_length=256, hop_length=64,
                   n_mels=64, f_min=0.0, f_max=8000.0, power=2.0),
    "fft128": dict(batch=8, length=480000, dtype="f32", signal="noise", sigma=0.1, seed=9,
                   sample_rate=16000, n_fft=128, win_length=128, hop_length=32,
                   n_mels=40, f_min=0.0, f_max=8000.0, power=2.0),
    "fft64": dict(batch=8, length=480000, dtype="f32", signal="noise", sigma=0.1, seed=10,
                  sample_rate=16000, n_fft=64, win_length=64, hop_length=16,
                  n_mels=24, f_min=0.0, f_max=8000.0, power=2.0),
    # the pages' "huge" case (16384/4096, 256 mels, 44.1 kHz, batch 16; 10 s
    # signals, the length its input + output bytes and time imply), and the
    # same shape at n_fft 8192
    "huge": dict(batch=16, length=441000, dtype="f32", signal="chirp", sigma=0.1, seed=11,
                 sample_rate=44100, n_fft=16384, win_length=16384, hop_length=4096,
                 n_mels=256, f_min=0.0, f_max=22050.0, power=2.0),
    "fft8192": dict(batch=16, length=441000, dtype="f32", signal="chirp", sigma=0.1, seed=12,
                    sample_rate=44100, n_fft=8192, win_length=8192, hop_length=2048,
                    n_mels=256, f_min=0.0, f_max=22050.0, power=2.0),
}

# The arguments that define the transform (everything but the input recipe).
TRANSFORM_KEYS = ("sample_rate", "n_fft", "win_length", "hop_length", "n_mels",
                  "f_min", "f_max", "power")


def transform_args(cfg: dict) -> dict:
    """The MelSpectrogram keyword arguments of a workload (defaults for the
    rest: centre reflect padding, HTK, no norm)."""
    out = {k: cfg[k] for k in TRANSFORM_KEYS}
    for k in ("center", "pad_mode", "mel_scale", "norm", "normalized", "pad"):
        if k in cfg:
            out[k] = cfg[k]
    return out


def workload(name: str, **overrides) -> dict:
    """A copy of a named workload with fields replaced (e.g. a smaller batch)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def make_signal(cfg: dict) -> np.ndarray:
    """Draw the input of `cfg` as the exact array handed to the GPU.

    Returns float32 [batch, length] or int16 [batch, length].
    """
    rng = np.random.default_rng(cfg["seed"])
    b, n = int(cfg["batch"]), int(cfg["length"])
    sr = float(cfg.get("sample_rate", 16000))
    kind = cfg["signal"]
    if kind == "pcm16":
        return rng.integers(-32768, 32768, size=(b, n), dtype=np.int64).astype(np.int16)
    x = rng.standard_normal((b, n)) * float(cfg.get("sigma", 0.1))
    t = np.arange(n, dtype=np.float64) / sr
    if kind == "sines":
        f = rng.uniform(50.0, 7000.0, size=(b, 3))
        ph = rng.uniform(0.0, 2.0 * np.pi, size=(b, 3))
        for j in range(3):
            x += 0.3 * np.sin(2.0 * np.pi * f[:, j:j + 1] * t[None, :] + ph[:, j:j + 1])
    elif kind == "chirp":
        dur = n / sr
        f0, f1 = 100.0, 10000.0
        phase = 2.0 * np.pi * (f0 * t + (f1 - f0) * t * t / (2.0 * dur))
        x += 0.3 * np.sin(phase)[None, :]
    elif kind != "noise":
        raise ValueError(f"unknown signal recipe {kind!r}")
    if cfg.get("dtype", "f32") == "i16":
        raise ValueError("int16 workloads use the pcm16 recipe")
    return x.astype(np.float32)
