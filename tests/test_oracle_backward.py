"""Pins of the oracle's backward (vector-Jacobian product w.r.t. the signal).

The backward is pinned against routes that share none of its code:
central finite differences of the (separately pinned) forward oracle, torch's
own autograd through torch.stft in float64 on the CPU, and Euler's identity
for functions that are positively homogeneous of degree `power` in x.
"""
import numpy as np
import pytest
import scipy.signal
import torch

from oracle import mel_oracle as O


def _fd_grad(x, u, kw, eps=1e-6):
    """Central differences of sum(u * F(x)) in every sample of x."""
    F = lambda z: float(np.sum(u * O.mel_spectrogram(z, **kw)))  # noqa: E731
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        e = np.zeros_like(x)
        e[idx] = eps
        g[idx] = (F(x + e) - F(x - e)) / (2 * eps)
    return g


FD_CASES = [
    dict(n_fft=16, hop_length=4),
    dict(n_fft=16, hop_length=5),                       # ragged hop
    dict(n_fft=16, hop_length=4, pad_mode="constant"),
    dict(n_fft=16, hop_length=4, pad_mode="replicate"),
    dict(n_fft=16, hop_length=4, pad_mode="circular"),
    dict(n_fft=16, hop_length=3, center=False),
    dict(n_fft=16, hop_length=4, power=1.0),
    dict(n_fft=16, hop_length=4, power=1.5),
    dict(n_fft=16, hop_length=4, power=0.7, pad_mode="replicate"),
    dict(n_fft=16, hop_length=4, win_length=10, normalized=True),
    dict(n_fft=16, hop_length=4, normalized="frame_length", pad=3),
    dict(n_fft=16, hop_length=4, pad=5, pad_mode="reflect"),
    dict(n_fft=12, hop_length=4, norm="slaney", mel_scale="slaney"),
]


@pytest.mark.parametrize("case", FD_CASES, ids=[str(i) for i in range(len(FD_CASES))])
def test_vjp_matches_central_differences(case):
    rng = np.random.default_rng(11)
    kw = dict(sample_rate=16000, n_mels=5, **case)
    x = rng.standard_normal((2, 37))
    T = O.mel_spectrogram(x, **kw).shape[-1]
    u = rng.standard_normal((2, 5, T))
    dx = O.mel_spectrogram_vjp(x, u, **kw)
    fd = _fd_grad(x, u, kw)
    assert dx.shape == x.shape
    assert np.max(np.abs(dx - fd)) <= 1e-7 * np.max(np.abs(dx))


@pytest.mark.parametrize("power", [2.0, 1.0, 1.5])
@pytest.mark.parametrize("mode", ["reflect", "constant", "replicate", "circular"])
def test_euler_identity(power, mode):
    # mel(c*x) = c^p mel(x) for c > 0, so <grad_x <u, mel(x)>, x> = p <u, mel(x)>
    rng = np.random.default_rng(12)
    kw = dict(sample_rate=16000, n_fft=64, hop_length=16, n_mels=12, power=power,
              pad_mode=mode, pad=2)
    x = rng.standard_normal((3, 300))
    y = O.mel_spectrogram(x, **kw)
    u = rng.standard_normal(y.shape)
    dx = O.mel_spectrogram_vjp(x, u, **kw)
    lhs, rhs = float(np.sum(dx * x)), power * float(np.sum(u * y))
    assert abs(lhs - rhs) <= 1e-11 * (abs(rhs) + float(np.sum(np.abs(u * y))))


def _torch_vjp(x, u, n_fft, hop, win_length, power, center, pad_mode, fb):
    """The same gradient through torch.stft's autograd in float64 (CPU)."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    # scipy's periodic Hann placed in the middle of an all-zero n_fft frame
    w = torch.zeros(n_fft, dtype=torch.float64)
    start = (n_fft - win_length) // 2
    w[start:start + win_length] = torch.from_numpy(scipy.signal.get_window("hann", win_length))
    S = torch.stft(xt, n_fft, hop_length=hop, win_length=n_fft, window=w, center=center,
                   pad_mode=pad_mode, normalized=False, onesided=True, return_complex=True)
    P = S.abs() ** power                                       # [b, K, T]
    mel = torch.matmul(torch.tensor(fb.T), P)                  # [b, n_mels, T]
    (mel * torch.tensor(u)).sum().backward()
    return xt.grad.numpy()


@pytest.mark.parametrize("mode", ["reflect", "constant", "replicate", "circular"])
@pytest.mark.parametrize("power,center,win", [(2.0, True, 400), (1.0, True, 300), (2.0, False, 400)])
def test_vjp_matches_torch_autograd(mode, power, center, win):
    rng = np.random.default_rng(13)
    n_fft, hop, n_mels, sr = 400, 160, 40, 16000
    x = rng.standard_normal((2, 3000))
    kw = dict(sample_rate=sr, n_fft=n_fft, hop_length=hop, win_length=win, n_mels=n_mels,
              power=power, center=center, pad_mode=mode)
    y = O.mel_spectrogram(x, **kw)
    u = rng.standard_normal(y.shape)
    fb = O.mel_filterbank(n_fft // 2 + 1, 0.0, sr / 2, n_mels, sr)
    ref = _torch_vjp(x, u, n_fft, hop, win, power, center, mode, fb)
    got = O.mel_spectrogram_vjp(x, u, **kw)
    assert np.max(np.abs(got - ref)) <= 1e-10 * np.max(np.abs(ref))


def test_vjp_linear_in_grad_out_and_zero_signal():
    rng = np.random.default_rng(14)
    kw = dict(sample_rate=16000, n_fft=32, hop_length=8, n_mels=6)
    x = rng.standard_normal((1, 200))
    T = O.mel_spectrogram(x, **kw).shape[-1]
    u1, u2 = rng.standard_normal((2, 1, 6, T))
    a = O.mel_spectrogram_vjp(x, 2.0 * u1 - 3.0 * u2, **kw)
    b = 2.0 * O.mel_spectrogram_vjp(x, u1, **kw) - 3.0 * O.mel_spectrogram_vjp(x, u2, **kw)
    assert np.allclose(a, b, rtol=0, atol=1e-12 * np.max(np.abs(a)))
    # |X|^p has a zero gradient at X = 0 (power 1 by the stated reading)
    for p in (2.0, 1.0):
        z = O.mel_spectrogram_vjp(np.zeros((1, 200)), u1, power=p, **kw)
        assert np.all(z == 0.0)


def test_vjp_rejects_integer_pcm():
    with pytest.raises(TypeError):
        O.mel_spectrogram_vjp(np.zeros((1, 1000), np.int16), np.zeros((1, 128, 7)))
