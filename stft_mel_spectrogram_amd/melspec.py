"""torchaudio-style callable over the HIP library.

flashmel 0.1.0 page, README "Usage": MelSpectrogram takes torchaudio's
arguments (plus out_dtype), accepts float32 or int16 input of shape
(..., time) on the GPU and returns (..., n_mels, n_frames) in float32 or
float16.  PyTorch only supplies device memory and the current stream here;
the whole forward pass is one fm_forward launch.

Float32 inputs that require grad are differentiable (specux "Backends"
page, section "Gradients": the backward is the analytic adjoint in kernels
of the forward's family): the autograd node's backward is one fm_backward
launch, which recomputes the spectrum from the saved input.
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

    def _check_input(self, x: torch.Tensor) -> int:
        if not isinstance(x, torch.Tensor) or x.device != self.device:
            raise ValueError(f"input must be a tensor on {self.device}")
        if x.dtype == torch.float32:
            dt = N.FM_F32
        elif x.dtype == torch.int16:
            dt = N.FM_I16
        else:
            raise TypeError(f"input dtype must be float32 or int16, got {x.dtype}")
        if not x.is_contiguous():
            raise ValueError("input must be contiguous")
        if x.dim() < 1:
            raise ValueError("input must have a time axis")
        return dt

    def _launch(self, fn, *args) -> None:
        if torch.cuda.current_device() == self.device.index:
            fn(*args)
        else:
            with torch.cuda.device(self.device):
                fn(*args)

    def __call__(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        dt = self._check_input(x)
        if x.requires_grad and torch.is_grad_enabled():
            if out is not None:
                raise ValueError("out= is not supported for inputs that require grad")
            return _MelFunction.apply(x, self)
        return self._forward(x, dt, out)

    def _forward(self, x: torch.Tensor, dt: int, out: torch.Tensor | None = None) -> torch.Tensor:
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
        self._launch(self.plan.forward_ptr, x.data_ptr(), dt, batch, length, out.data_ptr(), stream)
        return out

    def backward(self, x: torch.Tensor, grad_out: torch.Tensor,
                 out: torch.Tensor | None = None) -> torch.Tensor:
        """Gradient of sum(grad_out * self(x)) with respect to the float32
        signal x (same shape as x), from one fm_backward launch."""
        if self._check_input(x) != N.FM_F32:
            raise TypeError("the gradient is defined for float32 input only")
        lead = tuple(x.shape[:-1])
        length = int(x.shape[-1])
        batch = math.prod(lead) if lead else 1
        shape = lead + (self.n_mels, self.out_frames(length))
        if (not isinstance(grad_out, torch.Tensor) or tuple(grad_out.shape) != shape
                or grad_out.dtype != torch.float32 or grad_out.device != self.device
                or not grad_out.is_contiguous()):
            raise ValueError(f"grad_out must be a contiguous float32 tensor of shape {shape} "
                             f"on {self.device}")
        if out is None:
            out = torch.empty(x.shape, dtype=torch.float32, device=self.device)
        elif (tuple(out.shape) != tuple(x.shape) or out.dtype != torch.float32
              or out.device != self.device or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous float32 tensor of shape {tuple(x.shape)} "
                             f"on {self.device}")
        stream = torch.cuda.current_stream(self.device).cuda_stream
        self._launch(self.plan.backward_ptr, x.data_ptr(), batch, length, grad_out.data_ptr(),
                     out.data_ptr(), stream)
        return out


class _MelFunction(torch.autograd.Function):
    """Autograd node: forward = fm_forward, backward = fm_backward (the
    spectrum is recomputed from the saved input)."""

    @staticmethod
    def forward(ctx, x, mel):
        if x.dtype != torch.float32:
            raise TypeError("the gradient is defined for float32 input only")
        ctx.mel = mel
        ctx.save_for_backward(x)
        return mel._forward(x, N.FM_F32)

    @staticmethod
    def backward(ctx, grad_y):
        (x,) = ctx.saved_tensors
        # a float16 output's gradient arrives in float16: the kernel reads float32
        g = grad_y if grad_y.dtype == torch.float32 else grad_y.float()
        return ctx.mel.backward(x, g.contiguous()), None
