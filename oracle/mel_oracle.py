"""Plain f64 CPU oracle for the fused mel-spectrogram forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or calls
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, tables or
constants with the HIP path under ``stft_mel_spectrogram_amd/``.

What it computes is the definition the flashmel 0.1.0 page (PyPI sdist diff
view, README "Usage" and "How it works", and ``flashmel/filters.py``) states
for a torchaudio-``MelSpectrogram``-compatible forward pass:

  optional constant ``pad`` -> centre padding by n_fft//2 in ``pad_mode``
  -> frames every ``hop_length`` samples -> periodic Hann window (win_length
  centred inside n_fft, STFT ``normalized`` folded into it) -> one-sided DFT
  of size n_fft -> |X|**power -> triangular mel filterbank (HTK or Slaney
  scale, optional Slaney area norm) -> output [..., n_mels, n_frames].

Every step is written out in the plainest form, in float64: explicit index
maps for padding, a dense O(N^2) DFT whose angles are reduced on integers
(2*pi*((n*k) mod N)/N) before any rounding, and the filterbank triangles
evaluated directly from their corner frequencies.  Library calls are used
only as single steps (a matmul, a log10).

Where the page leaves a step open (it delegates the definitions to
torchaudio), the reading taken is stated in the docstring of the function
that implements that step.
"""
from __future__ import annotations

from functools import lru_cache

import numpy as np

PAD_MODES = ("reflect", "constant", "replicate", "circular")

# ---------------------------------------------------------------------------
# Input conversion
# ---------------------------------------------------------------------------


def to_float64(x: np.ndarray) -> np.ndarray:
    """Integer PCM is scaled by 1/32768 on load; floats are upcast as-is.

    flashmel page, README "Usage": int16 raw PCM input is scaled by 1/32768.
    The oracle takes exactly the array the GPU is handed (f32 or i16), so no
    information is lost or added before the comparison.
    """
    x = np.asarray(x)
    if x.dtype == np.int16:
        return x.astype(np.float64) / 32768.0
    if x.dtype.kind != "f":
        raise TypeError(f"unsupported input dtype {x.dtype}")
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# Padding and framing
# ---------------------------------------------------------------------------


def padded_index(i: np.ndarray, length: int, mode: str) -> np.ndarray:
    """Map positions i of the padded signal (relative to sample 0) to source
    sample indices, or -1 where the padded value is a constant zero.

    flashmel page, README "How it works": padding ("pad", "center", the four
    pad modes) is index arithmetic on the unpadded signal.  The modes follow
    torch's definitions: reflect does not repeat the edge sample
    ([x2 x1 | x0 .. x4 | x3 x2]), replicate repeats it, circular wraps,
    constant pads with zeros.
    """
    i = np.asarray(i, dtype=np.int64)
    if mode == "reflect":
        if length < 2:
            raise ValueError("reflect padding needs at least 2 samples")
        period = 2 * (length - 1)
        j = np.mod(i, period)
        return np.where(j < length, j, period - j)
    if mode == "replicate":
        return np.clip(i, 0, length - 1)
    if mode == "circular":
        return np.mod(i, length)
    if mode == "constant":
        return np.where((i >= 0) & (i < length), i, -1)
    raise ValueError(f"unknown pad mode {mode!r}")


def pad_signal(x: np.ndarray, left: int, right: int, mode: str) -> np.ndarray:
    """Pad the last axis of x by `left`/`right` samples in `mode`.

    torch's own reflect pad only reflects once (it requires pad < length);
    the caller checks that bound, this function just evaluates the index map.
    """
    length = x.shape[-1]
    idx = padded_index(np.arange(-left, length + right), length, mode)
    out = x[..., np.maximum(idx, 0)]
    if mode == "constant":
        out = np.where(idx >= 0, out, 0.0)
    return out


def frame_count(length: int, n_fft: int, hop: int, center: bool, pad: int = 0) -> int:
    """Number of STFT frames: 1 + floor((L_padded - n_fft) / hop).

    With centre padding L_padded = L + 2*pad + 2*(n_fft//2); for even n_fft this
    is 1 + floor((L + 2*pad)/hop).  flashmel page, README "Usage": 480000
    samples at hop 160 give 3001 frames.
    """
    lp = length + 2 * pad + (2 * (n_fft // 2) if center else 0)
    if lp < n_fft:
        raise ValueError("signal shorter than one frame")
    return 1 + (lp - n_fft) // hop


def frame_signal(xp: np.ndarray, n_fft: int, hop: int) -> np.ndarray:
    """Gather frames f_t[n] = xp[t*hop + n] from an already padded signal."""
    n_frames = 1 + (xp.shape[-1] - n_fft) // hop
    idx = np.arange(n_frames)[:, None] * hop + np.arange(n_fft)[None, :]
    return xp[..., idx]


# ---------------------------------------------------------------------------
# Window
# ---------------------------------------------------------------------------


def hann_window(win_length: int) -> np.ndarray:
    """Periodic Hann window w[n] = 0.5 - 0.5*cos(2*pi*n/win), n < win.

    flashmel page, ``flashmel/filters.py`` (window construction): a periodic
    Hann window of length win_length.  The angle is reduced on integers
    (n mod win) before the cosine.
    """
    n = np.arange(win_length, dtype=np.int64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * (n % win_length) / win_length)


def window_scale(hann: np.ndarray, normalized) -> float:
    """Factor the STFT normalisation multiplies the window by.

    flashmel page, ``flashmel/filters.py`` (window construction): the
    normalisation is folded into the window.  ``True`` or ``"window"`` makes
    the window's energy 1 (divide by its Euclidean norm); ``"frame_length"``
    divides by the square root of the window length; ``False``/``None``
    leaves it unscaled.
    """
    if normalized is None or normalized is False:
        return 1.0
    if normalized is True or (isinstance(normalized, str) and normalized == "window"):
        return 1.0 / float(np.sqrt(np.dot(hann, hann)))
    if isinstance(normalized, str) and normalized == "frame_length":
        return 1.0 / float(np.sqrt(len(hann)))
    raise ValueError(f"unknown normalized={normalized!r}")


def analysis_window(n_fft: int, win_length: int, normalized) -> np.ndarray:
    """The length-n_fft analysis window, evaluated position by position.

    flashmel page, ``flashmel/filters.py`` (window construction): a periodic
    Hann window of win_length samples sits centred in the n_fft-sample frame,
    its first sample at offset (n_fft - win_length) // 2, and is zero
    elsewhere; the STFT normalisation (window_scale) is a constant factor.
    """
    if win_length > n_fft or win_length < 1:
        raise ValueError("need 1 <= win_length <= n_fft")
    hann = hann_window(win_length)
    scale = window_scale(hann, normalized)
    offset = (n_fft - win_length) // 2
    w = np.empty(n_fft)
    for n in range(n_fft):
        j = n - offset                      # index into the Hann window
        w[n] = hann[j] * scale if 0 <= j < win_length else 0.0
    return w


# ---------------------------------------------------------------------------
# DFT and power
# ---------------------------------------------------------------------------


@lru_cache(maxsize=8)
def _dft_basis(n_fft: int):
    """cos/sin of theta[n,k] = 2*pi*((n*k) mod N)/N for k = 0..N/2.

    The product n*k is reduced modulo N in exact integer arithmetic first, so
    each f64 angle is within one rounding of its true value.
    """
    k = np.arange(n_fft // 2 + 1, dtype=np.int64)[None, :]
    # only N distinct angles occur: evaluate each once and index by (n*k) mod N
    # (the same f64 value per entry as evaluating the entry's own angle),
    # filling the matrices a block of rows at a time
    theta = 2.0 * np.pi * np.arange(n_fft, dtype=np.int64) / n_fft
    cos_t, sin_t = np.cos(theta), np.sin(theta)
    c = np.empty((n_fft, n_fft // 2 + 1))
    s = np.empty_like(c)
    for n0 in range(0, n_fft, 256):
        n = np.arange(n0, min(n_fft, n0 + 256), dtype=np.int64)[:, None]
        j = (n * k) % n_fft
        c[n0:n0 + n.shape[0]] = cos_t[j]
        s[n0:n0 + n.shape[0]] = sin_t[j]
    return c, s


def dft_onesided(frames: np.ndarray) -> np.ndarray:
    """One-sided DFT X[k] = sum_n f[n] exp(-2*pi*i*n*k/N), k = 0..N/2.

    flashmel page, README "How it works": the kernel computes a real-to-
    complex FFT of size n_fft; onesided=True only (README "Usage").  Here it
    is the dense O(N^2) definition as two real matmuls.
    """
    n_fft = frames.shape[-1]
    c, s = _dft_basis(n_fft)
    # (contiguous rows, so that the products run as BLAS matrix products)
    frames = np.ascontiguousarray(frames)
    return frames @ c - 1j * (frames @ s)


def power_spectrum(X: np.ndarray, power: float) -> np.ndarray:
    """|X|**power; for power 2 the sum of squares is used directly, for
    power 1 the modulus.  flashmel page, README "Usage" (torchaudio args)."""
    if power == 2.0:
        return X.real * X.real + X.imag * X.imag
    if power == 1.0:
        return np.abs(X)
    if power <= 0:
        raise ValueError("power must be positive")
    return np.abs(X) ** power


# ---------------------------------------------------------------------------
# Mel filterbank
# ---------------------------------------------------------------------------


def hz_to_mel(f, mel_scale: str = "htk"):
    """HTK: 2595*log10(1 + f/700).  Slaney: linear 3 mel per 200 Hz below
    1 kHz, logarithmic (27 steps per factor 6.4) above."""
    f = np.asarray(f, dtype=np.float64)
    if mel_scale == "htk":
        return 2595.0 * np.log10(1.0 + f / 700.0)
    if mel_scale == "slaney":
        f_sp = 200.0 / 3.0
        min_log_hz = 1000.0
        min_log_mel = min_log_hz / f_sp
        logstep = np.log(6.4) / 27.0
        lin = f / f_sp
        logpart = min_log_mel + np.log(np.maximum(f, min_log_hz) / min_log_hz) / logstep
        return np.where(f >= min_log_hz, logpart, lin)
    raise ValueError(f"unknown mel_scale {mel_scale!r}")


def mel_to_hz(m, mel_scale: str = "htk"):
    """Inverse of hz_to_mel."""
    m = np.asarray(m, dtype=np.float64)
    if mel_scale == "htk":
        return 700.0 * (10.0 ** (m / 2595.0) - 1.0)
    if mel_scale == "slaney":
        f_sp = 200.0 / 3.0
        min_log_hz = 1000.0
        min_log_mel = min_log_hz / f_sp
        logstep = np.log(6.4) / 27.0
        return np.where(m >= min_log_mel,
                        min_log_hz * np.exp(logstep * (m - min_log_mel)),
                        f_sp * m)
    raise ValueError(f"unknown mel_scale {mel_scale!r}")


def fft_bin_frequencies(n_freqs: int, sample_rate: int) -> np.ndarray:
    """Centre frequency of each one-sided bin: f_k = k*(sr//2)/(n_freqs-1),
    i.e. n_freqs points evenly spaced from 0 to sr//2 (torchaudio's grid)."""
    k = np.arange(n_freqs, dtype=np.float64)
    return k * float(sample_rate // 2) / float(n_freqs - 1)


def mel_corner_frequencies(f_min: float, f_max: float, n_mels: int,
                           mel_scale: str = "htk") -> np.ndarray:
    """n_mels+2 corner frequencies evenly spaced on the mel scale."""
    m_min = hz_to_mel(f_min, mel_scale)
    m_max = hz_to_mel(f_max, mel_scale)
    i = np.arange(n_mels + 2, dtype=np.float64)
    return mel_to_hz(m_min + i * (m_max - m_min) / (n_mels + 1), mel_scale)


def triangles(freqs: np.ndarray, f_pts: np.ndarray) -> np.ndarray:
    """W[k, m] = max(0, min(rising, falling)) with
    rising  = (f_k - f_pts[m])   / (f_pts[m+1] - f_pts[m]),
    falling = (f_pts[m+2] - f_k) / (f_pts[m+2] - f_pts[m+1]).
    Filter m rises from its left corner to 1 at its centre f_pts[m+1] and
    falls to 0 at its right corner."""
    f = np.asarray(freqs, dtype=np.float64)[:, None]
    lo, mid, hi = f_pts[None, :-2], f_pts[None, 1:-1], f_pts[None, 2:]
    rising = (f - lo) / (mid - lo)
    falling = (hi - f) / (hi - mid)
    return np.maximum(0.0, np.minimum(rising, falling))


def mel_filterbank(n_freqs: int, f_min: float, f_max: float, n_mels: int,
                   sample_rate: int, norm=None, mel_scale: str = "htk") -> np.ndarray:
    """Dense f64 filterbank [n_freqs, n_mels].

    flashmel page, ``flashmel/filters.py`` pack_fbank: the filterbank is the
    torchaudio triangular one for (n_freqs, f_min, f_max, n_mels, sample_rate,
    norm, mel_scale); its rows have contiguous support.  norm="slaney" scales
    filter m by 2/(f_pts[m+2] - f_pts[m]) (unit area).
    """
    f_pts = mel_corner_frequencies(f_min, f_max, n_mels, mel_scale)
    fb = triangles(fft_bin_frequencies(n_freqs, sample_rate), f_pts)
    if norm == "slaney":
        fb = fb * (2.0 / (f_pts[2:] - f_pts[:-2]))[None, :]
    elif norm is not None:
        raise ValueError(f"unknown norm {norm!r}")
    return fb


# ---------------------------------------------------------------------------
# Whole forward pass
# ---------------------------------------------------------------------------


def mel_spectrogram(x, *, sample_rate: int = 16000, n_fft: int = 400,
                    win_length: int | None = None, hop_length: int | None = None,
                    f_min: float = 0.0, f_max: float | None = None, pad: int = 0,
                    n_mels: int = 128, power: float = 2.0, normalized=False,
                    center: bool = True, pad_mode: str = "reflect", norm=None,
                    mel_scale: str = "htk", chunk: int = 1) -> np.ndarray:
    """f64 mel spectrogram of x with shape (..., time) -> (..., n_mels, T).

    flashmel page, README "Usage": torchaudio MelSpectrogram arguments, input
    (..., time), output (..., n_mels, n_frames).  Defaults follow torchaudio:
    win_length = n_fft, hop = win_length // 2, f_max = sr // 2.
    `chunk` signals are processed at a time to bound memory; it does not
    change the arithmetic.
    """
    win_length = n_fft if win_length is None else win_length
    hop_length = win_length // 2 if hop_length is None else hop_length
    f_max = float(sample_rate // 2) if f_max is None else float(f_max)
    if pad_mode not in PAD_MODES:
        raise ValueError(f"unknown pad_mode {pad_mode!r}")
    xf = to_float64(x)
    lead = xf.shape[:-1]
    xf = xf.reshape(-1, xf.shape[-1])
    window = analysis_window(n_fft, win_length, normalized)
    fb = mel_filterbank(n_fft // 2 + 1, f_min, f_max, n_mels, sample_rate, norm, mel_scale)
    outs = []
    for s in range(0, xf.shape[0], max(1, chunk)):
        sig = xf[s:s + max(1, chunk)]
        if pad > 0:
            sig = pad_signal(sig, pad, pad, "constant")
        if center:
            p = n_fft // 2
            if pad_mode == "reflect" and p >= sig.shape[-1]:
                raise ValueError("reflect padding needs n_fft//2 < signal length")
            sig = pad_signal(sig, p, p, pad_mode)
        fr = frame_signal(sig, n_fft, hop_length) * window   # [b, T, N]
        P = power_spectrum(dft_onesided(fr), power)          # [b, T, K]
        outs.append(np.swapaxes(P @ fb, -1, -2))             # [b, n_mels, T]
    out = np.concatenate(outs, axis=0)
    return out.reshape(lead + out.shape[-2:])


# ---------------------------------------------------------------------------
# Backward: vector-Jacobian product with respect to the input signal
# ---------------------------------------------------------------------------


def power_gradient(X: np.ndarray, dP: np.ndarray, power: float) -> np.ndarray:
    """Gradient of sum(dP * |X|**power) with respect to (Re X, Im X), packed
    as the complex number dRe + i*dIm.

    d|X|^p / dRe = p*|X|^(p-2)*Re X (and likewise for Im), so the gradient is
    p*dP*|X|^(p-2)*X; for power 2 that is 2*dP*X.  Reading (the page is
    silent on it): where X = 0 and power != 2 the gradient is taken as 0, the
    value torch's abs() backward gives there (sgn(0) = 0).
    """
    if power == 2.0:
        return 2.0 * dP * X
    mag = np.abs(X)
    safe = np.where(mag > 0.0, mag, 1.0)
    return np.where(mag > 0.0, power * dP * safe ** (power - 2.0) * X, 0.0)


def dft_onesided_adjoint(dX: np.ndarray, n_fft: int) -> np.ndarray:
    """Adjoint of dft_onesided as a real-linear map: given the gradient
    dX = dRe + i*dIm of the K one-sided bins, the gradient of each real frame
    sample is  sum_k dRe[k]*cos(theta_nk) - dIm[k]*sin(theta_nk),
    since Re X[k] = sum_n f[n] cos(theta_nk) and Im X[k] = -sum_n f[n] sin(theta_nk).
    """
    c, s = _dft_basis(n_fft)
    return dX.real @ c.T - dX.imag @ s.T


def pad_signal_adjoint(g: np.ndarray, length: int, left: int, right: int, mode: str) -> np.ndarray:
    """Adjoint of pad_signal: every padded position hands its gradient to the
    source sample it was copied from; constant-zero positions drop theirs."""
    idx = padded_index(np.arange(-left, length + right), length, mode)
    keep = idx >= 0
    out = np.zeros(g.shape[:-1] + (length,))
    flat_out = out.reshape(-1, length)
    flat_g = g.reshape(-1, g.shape[-1])
    for r in range(flat_g.shape[0]):
        np.add.at(flat_out[r], idx[keep], flat_g[r][keep])
    return out


def mel_spectrogram_vjp(x, grad_out, *, sample_rate: int = 16000, n_fft: int = 400,
                        win_length: int | None = None, hop_length: int | None = None,
                        f_min: float = 0.0, f_max: float | None = None, pad: int = 0,
                        n_mels: int = 128, power: float = 2.0, normalized=False,
                        center: bool = True, pad_mode: str = "reflect", norm=None,
                        mel_scale: str = "htk", chunk: int = 1) -> np.ndarray:
    """f64 gradient of sum(grad_out * mel_spectrogram(x)) with respect to x.

    specux "Backends" page, section "Gradients": a spectrogram's gradient is
    the analytic adjoint of the transform (checked there against float64
    gradcheck); the flashmel 0.1.0 page itself is inference-only.  The forward chain (padding, framing, window, one-sided DFT, |X|**power,
    mel projection) is run again and each step is replaced by its adjoint, in
    reverse order: the transposed filterbank, power_gradient,
    dft_onesided_adjoint, the window, overlap-add of the frames, and the
    adjoint of the padding maps.  x is a float array (..., time); grad_out has
    the forward output's shape (..., n_mels, T).  The derivative is with
    respect to the float signal; integer PCM has no gradient.
    """
    win_length = n_fft if win_length is None else win_length
    hop_length = win_length // 2 if hop_length is None else hop_length
    f_max = float(sample_rate // 2) if f_max is None else float(f_max)
    if pad_mode not in PAD_MODES:
        raise ValueError(f"unknown pad_mode {pad_mode!r}")
    xf = np.asarray(x)
    if xf.dtype.kind != "f":
        raise TypeError("the gradient is defined for floating-point input only")
    xf = xf.astype(np.float64)
    lead = xf.shape[:-1]
    L = xf.shape[-1]
    xf = xf.reshape(-1, L)
    g = np.asarray(grad_out, dtype=np.float64).reshape((xf.shape[0],) + np.shape(grad_out)[-2:])
    window = analysis_window(n_fft, win_length, normalized)
    fb = mel_filterbank(n_fft // 2 + 1, f_min, f_max, n_mels, sample_rate, norm, mel_scale)
    outs = []
    for s in range(0, xf.shape[0], max(1, chunk)):
        sig = xf[s:s + max(1, chunk)]
        if pad > 0:
            sig = pad_signal(sig, pad, pad, "constant")
        lz = sig.shape[-1]
        p = n_fft // 2 if center else 0
        if center:
            if pad_mode == "reflect" and p >= lz:
                raise ValueError("reflect padding needs n_fft//2 < signal length")
            sig = pad_signal(sig, p, p, pad_mode)
        fr = frame_signal(sig, n_fft, hop_length)                  # [b, T, N]
        T = fr.shape[-2]
        X = dft_onesided(fr * window)                               # [b, T, K]
        gs = g[s:s + max(1, chunk)]
        if gs.shape[-1] != T or gs.shape[-2] != n_mels:
            raise ValueError("grad_out must have the forward output's shape")
        dP = np.swapaxes(gs, -1, -2) @ fb.T                         # [b, T, K]
        dfr = dft_onesided_adjoint(power_gradient(X, dP, power), n_fft) * window
        dsig = np.zeros(sig.shape)                                  # overlap-add
        for t in range(T):
            dsig[..., t * hop_length:t * hop_length + n_fft] += dfr[..., t, :]
        if center:
            dsig = pad_signal_adjoint(dsig, lz, p, p, pad_mode)
        if pad > 0:
            dsig = dsig[..., pad:pad + L]
        outs.append(dsig)
    out = np.concatenate(outs, axis=0)
    return out.reshape(lead + (L,))
