"""ctypes binding of libfm.so (the C ABI declared in include/fm.h).

Argument marshalling only: every step of the forward pass runs in the HIP
library.  Importing this module fails loudly if the library has not been
built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfm.so")

FM_OK = 0
FM_E_INVAL = -1
FM_E_UNSUPPORTED = -2
FM_E_HIP = -3
FM_E_NOMEM = -4
FM_E_NODEVICE = -5

FM_PAD = {"reflect": 0, "constant": 1, "replicate": 2, "circular": 3}
FM_MEL = {"htk": 0, "slaney": 1}
FM_NORM = {None: 0, "slaney": 1}
FM_F32 = 0
FM_I16 = 1
FM_F16 = 2
FM_FWD_SPLIT = 0
FM_FWD_PAIRED = 1
FM_FWD_LARGE = 2
FM_FWD_ROWS = 3
FM_FWD_AUTO = 4
FM_NORMALIZED = {False: 0, None: 0, True: 1, "window": 1, "frame_length": 2}
FM_OUT = {"f32": FM_F32, "f16": FM_F16}


class FmError(RuntimeError):
    """A negative status returned by the library, with its message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"fm error {status}: {message}")
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_fft", "win_length", "hop_length", "n_mels", "n_freqs", "pad", "normalized",
        "out_dtype", "nnz", "w_max", "fft_n1", "fft_n2", "tile_frames", "threads", "lds_bytes",
        "has_device", "forward_variant", "fft_n3")]


class Args(ctypes.Structure):
    """fm_args of include/fm.h."""
    _fields_ = ([(n, ctypes.c_int) for n in ("sample_rate", "n_fft", "win_length", "hop_length",
                                              "n_mels")] +
                [(n, ctypes.c_double) for n in ("f_min", "f_max", "power")] +
                [(n, ctypes.c_int) for n in ("center", "pad_mode", "mel_scale", "norm", "pad",
                                              "normalized", "out_dtype")])


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m stft_mel_spectrogram_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    I64 = ctypes.c_int64
    create_args = [ctypes.POINTER(P), I, I, I, I, I, D, D, D, I, I, I, I]
    sigs = {
        "fm_plan_create": (I, create_args),
        "fm_plan_create_host": (I, create_args),
        "fm_args_default": (I, [ctypes.POINTER(Args)]),
        "fm_plan_create_args": (I, [ctypes.POINTER(P), ctypes.POINTER(Args)]),
        "fm_plan_create_args_host": (I, [ctypes.POINTER(P), ctypes.POINTER(Args)]),
        "fm_forward": (I, [P, P, I, I64, I64, P, P]),
        "fm_backward": (I, [P, P, I64, I64, P, P, P]),
        "fm_out_frames": (I64, [P, I64]),
        "fm_forward_config": (I, [P, I64, I64, ctypes.POINTER(I), ctypes.POINTER(I),
                                  ctypes.POINTER(I64)]),
        "fm_plan_destroy": (I, [P]),
        "fm_strerror": (ctypes.c_char_p, [I]),
        "fm_last_error": (ctypes.c_char_p, []),
        "fm_plan_info_get": (I, [P, ctypes.POINTER(PlanInfo)]),
        "fm_plan_tables": (I, [P, P, P, P, P, P, P, P]),
        "fm_plan_mel_blocks": (I, [P, P, P, P, P, P]),
        "fm_plan_mel_quads": (I, [P, P, P, P, P, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def check(status: int) -> int:
    if status < 0:
        raise FmError(status, (lib.fm_last_error() or b"").decode() or
                      lib.fm_strerror(status).decode())
    return status


class Plan:
    """Owns an fm_plan*.  `device=True` builds and uploads on the current HIP
    device; `device=False` builds the host tables only (no GPU needed)."""

    def __init__(self, *, sample_rate=16000, n_fft=400, win_length=None, hop_length=None,
                 n_mels=128, f_min=0.0, f_max=None, power=2.0, center=True,
                 pad_mode="reflect", mel_scale="htk", norm=None, pad=0, normalized=False,
                 out_dtype="f32", device=True):
        win_length = n_fft if win_length is None else int(win_length)
        hop_length = win_length // 2 if hop_length is None else int(hop_length)
        f_max = float(sample_rate // 2) if f_max is None else float(f_max)
        if pad_mode not in FM_PAD:
            raise ValueError(f"unknown pad_mode {pad_mode!r}")
        if mel_scale not in FM_MEL:
            raise ValueError(f"unknown mel_scale {mel_scale!r}")
        if norm not in FM_NORM:
            raise ValueError(f"unknown norm {norm!r}")
        if not any(normalized is k or (isinstance(k, str) and normalized == k)
                   for k in FM_NORMALIZED):
            raise ValueError(f"unknown normalized {normalized!r}")
        if out_dtype not in FM_OUT:
            raise ValueError(f"out_dtype must be 'f32' or 'f16', got {out_dtype!r}")
        a = Args()
        check(lib.fm_args_default(ctypes.byref(a)))
        a.sample_rate, a.n_fft, a.win_length, a.hop_length = (int(sample_rate), int(n_fft),
                                                                win_length, hop_length)
        a.n_mels, a.f_min, a.f_max, a.power = int(n_mels), float(f_min), f_max, float(power)
        a.center, a.pad_mode = int(bool(center)), FM_PAD[pad_mode]
        a.mel_scale, a.norm = FM_MEL[mel_scale], FM_NORM[norm]
        a.pad = int(pad)
        a.normalized = FM_NORMALIZED[normalized if not isinstance(normalized, bool) else bool(normalized)]
        a.out_dtype = FM_OUT[out_dtype]
        self._h = ctypes.c_void_p()
        fn = lib.fm_plan_create_args if device else lib.fm_plan_create_args_host
        check(fn(ctypes.byref(self._h), ctypes.byref(a)))
        self.args = dict(sample_rate=sample_rate, n_fft=n_fft, win_length=win_length,
                         hop_length=hop_length, n_mels=n_mels, f_min=f_min, f_max=f_max,
                         power=power, center=center, pad_mode=pad_mode, mel_scale=mel_scale,
                         norm=norm, pad=pad, normalized=normalized, out_dtype=out_dtype)

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise RuntimeError("plan already destroyed")
        return self._h

    def info(self) -> PlanInfo:
        out = PlanInfo()
        check(lib.fm_plan_info_get(self.handle, ctypes.byref(out)))
        return out

    def out_frames(self, length: int) -> int:
        return check(lib.fm_out_frames(self.handle, int(length)))

    def forward_config(self, batch: int, length: int):
        """(variant, tile_frames, workgroups) that fm_forward takes for this call."""
        v, t, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
        check(lib.fm_forward_config(self.handle, int(batch), int(length), ctypes.byref(v),
                                    ctypes.byref(t), ctypes.byref(w)))
        return v.value, t.value, w.value

    def tables(self):
        """Host tables as numpy arrays (window, first, len, off, weights, tw_m, tw_n)."""
        import numpy as np
        inf = self.info()
        m = inf.n_fft // 2
        win = np.zeros(inf.n_fft, np.float32)
        first = np.zeros(inf.n_mels, np.int32)
        ln = np.zeros(inf.n_mels, np.int32)
        off = np.zeros(inf.n_mels, np.int32)
        w = np.zeros(max(inf.nnz, 1), np.float32)
        twm = np.zeros(2 * m, np.float32)
        twn = np.zeros(2 * m, np.float32)
        ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        check(lib.fm_plan_tables(self.handle, ptr(win), ptr(first), ptr(ln), ptr(off), ptr(w),
                                 ptr(twm), ptr(twn)))
        return dict(window=win, first=first, len=ln, off=off, weights=w[:inf.nnz],
                    tw_m=twm[0::2] + 1j * twm[1::2], tw_n=twn[0::2] + 1j * twn[1::2])

    def mel_blocks(self):
        """The mel stage's block layout: (blocks[n,4] = kb, ksteps, w_off,
        mel0 + 65536 * filters; wave_beg[5]; weights)."""
        import numpy as np
        nb = ctypes.c_int32()
        nw = ctypes.c_int64()
        check(lib.fm_plan_mel_blocks(self.handle, None, None, None, ctypes.byref(nb), ctypes.byref(nw)))
        blocks = np.zeros(max(nb.value, 1) * 4, np.int32)
        wave_beg = np.zeros(5, np.int32)
        w = np.zeros(max(nw.value, 1), np.float32)
        ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        check(lib.fm_plan_mel_blocks(self.handle, ptr(blocks), ptr(wave_beg), ptr(w), None, None))
        return blocks[:4 * nb.value].reshape(-1, 4), wave_beg, w[:nw.value]

    def mel_quads(self):
        """The vector-unit mel stage's layout: (headers[n,6] = start_0..3, L,
        off; share_beg[9]; weights, 4 per step)."""
        import numpy as np
        nq = ctypes.c_int32()
        nw = ctypes.c_int64()
        check(lib.fm_plan_mel_quads(self.handle, None, None, None, ctypes.byref(nq), ctypes.byref(nw)))
        hdr = np.zeros(max(nq.value, 1) * 6, np.int32)
        share = np.zeros(9, np.int32)
        w = np.zeros(max(nw.value, 1), np.float32)
        ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        check(lib.fm_plan_mel_quads(self.handle, ptr(hdr), ptr(share), ptr(w), None, None))
        return hdr[:6 * nq.value].reshape(-1, 6), share, w[:nw.value]

    def forward_ptr(self, in_ptr: int, in_dtype: int, batch: int, length: int, out_ptr: int,
                    stream: int = 0) -> None:
        """Raw device-pointer entry (fm_forward)."""
        check(lib.fm_forward(self.handle, ctypes.c_void_p(in_ptr), int(in_dtype), int(batch),
                             int(length), ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream)))

    def backward_ptr(self, in_ptr: int, batch: int, length: int, grad_out_ptr: int,
                     grad_in_ptr: int, stream: int = 0) -> None:
        """Raw device-pointer entry (fm_backward): float32 signal, float32
        output gradient [batch, n_mels, T] -> float32 signal gradient."""
        check(lib.fm_backward(self.handle, ctypes.c_void_p(in_ptr), int(batch), int(length),
                              ctypes.c_void_p(grad_out_ptr), ctypes.c_void_p(grad_in_ptr),
                              ctypes.c_void_p(stream)))

    def close(self) -> None:
        if self._h:
            lib.fm_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
