"""torchaudio-style callable over the HIP library.

flashmel 0.1.0 page, README "Usage": MelSpectrogram takes torchaudio's
arguments (plus out_dtype), accepts float32 or int16 input of shape
(..., time) on the GPU and returns (..., n_mels, n_frames) in float32 or
float16.  PyTorch only supplies device memory and the
current stream here; the whole forward pass is one fm_forward launch.
"""
from __future__ import annotations

import math

import torch

from . import _native as N


class MelSpectrogram:
    def __init__(self, sample_rate: int = 16000, n_fft: int = 400, win_length=None,
                 hop_length=None, f_min: float = 0.0, f_max=None, n_mels: int = 128,
                 pad: int = 0, power: float = 2.0, normalized=False, center: bool = True,
                 pad_mode: str = "reflect", mel_scale: str = "htk", norm=None,
                 out_dtype=torch.float32, device=None):
        if not torch.cuda.is_available():
            raise RuntimeError("MelSpectrogram needs a ROCm GPU (there is no CPU path)")
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        if out_dtype not in (torch.float32, torch.float16):
            raise TypeError(f"out_dtype must be torch.float32 or torch.float16, got {out_dtype}")
        self.out_dtype = out_dtype
        with torch.cuda.device(self.device):
            self.plan = N.Plan(sample_rate=sample_rate, n_fft=n_fft, win_length=win_length,
                               hop_length=hop_length, n_mels=n_mels, f_min=f_min, f_max=f_max,
                               power=power, center=center, pad_mode=pad_mode,
                               mel_scale=mel_scale, norm=norm, pad=pad, normalized=normalized,
                               out_dtype="f16" if out_dtype == torch.float16 else "f32",
                               device=True)
        self.n_mels = n_mels
        self._frames = {}

    def out_frames(self, length: int) -> int:
        T = self._frames.get(length)
        if T is None:
            T = self._frames[length] = self.plan.out_frames(length)
        return T

    def __call__(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        if not isinstance(x, torch.Tensor) or x.device != self.device:
            raise ValueError(f"input must be a tensor on {self.device}")
        if x.dtype == torch.float32:
            dt = N.FM_F32
        elif x.dtype == torch.int16:
            dt = N.FM_I16
        else:
            raise TypeError(f"input dtype must be float32 or int16, got {x.dtype}")
        if x.requires_grad and torch.is_grad_enabled():
            raise RuntimeError("inference only: input requires grad (no backward is implemented)")
        if not x.is_contiguous():
            raise ValueError("input must be contiguous")
        if x.dim() < 1:
            raise ValueError("input must have a time axis")
        lead = tuple(x.shape[:-1])
        length = int(x.shape[-1])
        batch = math.prod(lead) if lead else 1
        T = self.out_frames(length)
        shape = lead + (self.n_mels, T)
        if out is None:
            out = torch.empty(shape, dtype=self.out_dtype, device=self.device)
        elif (tuple(out.shape) != shape or out.dtype != self.out_dtype or out.device != self.device
              or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous {self.out_dtype} tensor of shape {shape} "
                             f"on {self.device}")
        stream = torch.cuda.current_stream(self.device).cuda_stream
        if torch.cuda.current_device() == self.device.index:
            self.plan.forward_ptr(x.data_ptr(), dt, batch, length, out.data_ptr(), stream)
        else:
            with torch.cuda.device(self.device):
                self.plan.forward_ptr(x.data_ptr(), dt, batch, length, out.data_ptr(), stream)
        return out
