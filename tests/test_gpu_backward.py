"""GPU parity of the backward (fm_backward through the C ABI) against the
f64 oracle's vector-Jacobian product.

Bar: |gpu - ref| <= 1e-4 * (rms_b + |ref|) elementwise, rms_b the RMS of the
reference gradient over the signal b.  The float32 error of an FFT-based
adjoint is a few ulp times log2(n_fft) times the frame gradient's norm, not
the sample's own value (a sample's gradient can cancel to near zero), so
the absolute part scales with the signal's RMS; 1e-4 leaves two orders of
magnitude over that estimate.
"""
import numpy as np
import pytest

from oracle import mel_oracle as O
from stft_mel_spectrogram_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-4


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(batch, length, n_mels, targs, seed):
    rng = np.random.default_rng(seed)
    x = (0.1 * rng.standard_normal((batch, length))
         + 0.3 * np.sin(2 * np.pi * 440.0 * np.arange(length) / 16000.0)).astype(np.float32)
    T = O.mel_spectrogram(x[:1, :], **targs).shape[-1]
    u = rng.standard_normal((batch, n_mels, T)).astype(np.float32)
    return x, u


def gpu_backward(x, u, **targs):
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    mel = MelSpectrogram(**targs)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    ud = torch.from_numpy(np.ascontiguousarray(u)).cuda()
    # NaN-poisoned output: an element the kernel leaves unwritten fails the check
    g = torch.full(xd.shape, float("nan"), device="cuda")
    mel.backward(xd, ud, out=g)
    torch.cuda.synchronize()
    return g.cpu().numpy()


def assert_grad_parity(got, ref, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1])
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    err = np.abs(got - ref)
    bound = TOL * (rms + np.abs(ref))
    ratio = err / np.where(bound > 0, bound, 1.0)
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    r = float(ratio[worst])
    print(f"[grad parity] {what}: max err/bound = {r:.3g} at {worst} (gpu {got[worst]:.6g}, "
          f"ref {ref[worst]:.6g}, rms {float(rms[worst[0], 0]):.3g})", flush=True)
    assert r <= 1.0, what
    # exact zeros stay exact where the reference gradient is exactly zero
    assert np.all(got[ref == 0.0] == 0.0), what


CASES = [
    # (id, batch, length, transform args)
    ("whisper_3tiles", 2, 16000, dict(n_fft=400, hop_length=160, n_mels=128)),
    ("constant", 2, 16000, dict(n_fft=400, hop_length=160, n_mels=80, pad_mode="constant")),
    ("replicate", 2, 16000, dict(n_fft=400, hop_length=160, n_mels=80, pad_mode="replicate")),
    ("circular", 2, 16000, dict(n_fft=400, hop_length=160, n_mels=80, pad_mode="circular")),
    ("no_center", 2, 16001, dict(n_fft=400, hop_length=160, n_mels=80, center=False)),
    ("power1", 1, 16000, dict(n_fft=400, hop_length=160, n_mels=80, power=1.0)),
    ("power1.5", 1, 16000, dict(n_fft=400, hop_length=160, n_mels=80, power=1.5)),
    ("zpad_norm_win", 2, 9999, dict(n_fft=400, win_length=300, hop_length=100, n_mels=64,
                                    pad=37, normalized=True)),
    ("zpad_replicate", 1, 8000, dict(n_fft=400, hop_length=160, n_mels=64, pad=50,
                                     pad_mode="replicate")),
    ("slaney_odd_hop", 2, 12345, dict(n_fft=400, hop_length=157, n_mels=40, mel_scale="slaney",
                                      norm="slaney")),
    ("short_whole", 3, 333, dict(n_fft=400, hop_length=160, n_mels=40)),
    ("short_circular", 2, 250, dict(n_fft=400, hop_length=100, n_mels=40, pad_mode="circular")),
    ("nfft64", 2, 4000, dict(n_fft=64, hop_length=16, n_mels=24)),
    ("nfft128", 2, 4000, dict(n_fft=128, hop_length=32, n_mels=40)),
    ("nfft256", 2, 8000, dict(n_fft=256, hop_length=64, n_mels=64)),
    ("nfft512", 2, 8000, dict(n_fft=512, hop_length=128, n_mels=80, win_length=400)),
    ("nfft1024", 2, 16384, dict(n_fft=1024, hop_length=256, n_mels=80)),
    ("nfft2048_p1", 2, 22050, dict(sample_rate=22050, n_fft=2048, hop_length=512, n_mels=128,
                                   power=1.0)),
    ("nfft4096", 1, 44100, dict(sample_rate=44100, n_fft=4096, hop_length=1024, n_mels=128)),
    # small hops: more frames overlap a sample than one pass holds (several passes)
    ("hop8_nfft400", 2, 3000, dict(n_fft=400, hop_length=8, n_mels=40)),
    ("hop32_nfft1024_p1", 1, 8000, dict(n_fft=1024, hop_length=32, n_mels=64, power=1.0)),
    ("hop100_nfft2048_circ", 2, 9000, dict(sample_rate=22050, n_fft=2048, hop_length=100,
                                           n_mels=80, pad_mode="circular")),
    ("hop64_nfft4096", 1, 8192, dict(sample_rate=44100, n_fft=4096, hop_length=64, n_mels=128)),
    # frames that do not overlap: samples between frames get a zero gradient
    ("hop400_nfft400", 2, 9001, dict(n_fft=400, hop_length=400, n_mels=40)),
    ("hop500_gaps", 2, 9001, dict(n_fft=400, hop_length=500, n_mels=40)),
    ("hop1000_gaps_constant", 1, 9001, dict(n_fft=400, hop_length=1000, n_mels=40,
                                            pad_mode="constant")),
    ("hop1_nfft64", 1, 300, dict(n_fft=64, hop_length=1, n_mels=16)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(case):
    name, batch, length, targs = case
    targs = dict(targs)
    targs.setdefault("sample_rate", 16000)
    x, u = _inputs(batch, length, targs["n_mels"], targs, seed=sum(map(ord, name)))
    print(f"[case] backward {name} {x.shape} {targs}", flush=True)
    got = gpu_backward(x, u, **targs)
    ref = O.mel_spectrogram_vjp(x, u, chunk=4, **targs)
    assert_grad_parity(got, ref, name)


def test_backward_full_whisper_shape():
    """8 x 480000 at the whisper transform: every gradient sample."""
    cfg = W.workload("whisper")
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    T = O.frame_count(x.shape[-1], targs["n_fft"], targs["hop_length"], center=True)
    u = np.random.default_rng(21).standard_normal((x.shape[0], targs["n_mels"], T)).astype(np.float32)
    print(f"[case] backward full whisper {x.shape}", flush=True)
    got = gpu_backward(x, u, **targs)
    ref = O.mel_spectrogram_vjp(x, u, chunk=2, **targs)
    assert_grad_parity(got, ref, "full whisper")


@pytest.mark.parametrize("name,rows", [("large", [0, 37, 63]), ("pow2", None)])
def test_backward_full_other_workloads(name, rows):
    """64 x 220500 (n_fft 2048, power 1) on sampled rows of the full launch;
    8 x 32768 (n_fft 1024) on every row."""
    cfg = W.workload(name)
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    T = O.frame_count(x.shape[-1], targs["n_fft"], targs["hop_length"], center=True)
    u = np.random.default_rng(22).standard_normal((x.shape[0], targs["n_mels"], T)).astype(np.float32)
    print(f"[case] backward full {name} {x.shape} rows {rows}", flush=True)
    got = gpu_backward(x, u, **targs)
    sel = slice(None) if rows is None else rows
    ref = O.mel_spectrogram_vjp(x[sel], u[sel], chunk=2, **targs)
    assert_grad_parity(got[sel], ref, f"full {name}")


def test_backward_is_deterministic_and_autograd_matches():
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    targs = dict(n_fft=400, hop_length=160, n_mels=80)
    x, u = _inputs(3, 20000, 80, dict(sample_rate=16000, **targs), seed=5)
    mel = MelSpectrogram(**targs)
    xd = torch.from_numpy(x).cuda()
    ud = torch.from_numpy(u).cuda()
    g1 = mel.backward(xd, ud)
    g2 = mel.backward(xd, ud)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    xr = xd.clone().requires_grad_(True)
    y = mel(xr)
    assert y.requires_grad
    assert torch.equal(y.detach(), mel(xd))
    (y * ud).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(xr.grad, g1)


def test_backward_through_float16_output():
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    targs = dict(n_fft=400, hop_length=160, n_mels=80)
    x, u = _inputs(1, 8000, 80, dict(sample_rate=16000, **targs), seed=6)
    mel16 = MelSpectrogram(out_dtype=torch.float16, **targs)
    xr = torch.from_numpy(x).cuda().requires_grad_(True)
    y = mel16(xr)
    assert y.dtype == torch.float16
    ud = torch.from_numpy(u).cuda()
    y.backward(ud.half())
    torch.cuda.synchronize()
    ref = O.mel_spectrogram_vjp(x, u.astype(np.float16).astype(np.float64), **targs,
                                sample_rate=16000)
    assert_grad_parity(xr.grad.cpu().numpy(), ref, "f16 output")


def test_backward_errors_and_empty_batch():
    from stft_mel_spectrogram_amd import MelSpectrogram
    from stft_mel_spectrogram_amd._native import FM_E_UNSUPPORTED, FmError
    _require_gpu()
    mel = MelSpectrogram(n_fft=400, hop_length=160, n_mels=40)
    with pytest.raises(TypeError):
        mel.backward(torch.zeros(4000, dtype=torch.int16, device="cuda"),
                     torch.zeros(40, 26, device="cuda"))
    with pytest.raises(ValueError):
        mel.backward(torch.zeros(4000, device="cuda"), torch.zeros(40, 25, device="cuda"))
    z = mel.backward(torch.empty((0, 4000), device="cuda"), torch.empty((0, 40, 26), device="cuda"))
    assert tuple(z.shape) == (0, 4000)
    # a zero padding so wide that one workgroup's samples cannot fit its LDS
    wide = MelSpectrogram(sample_rate=44100, n_fft=4096, hop_length=64, n_mels=128, pad=40000)
    T = wide.out_frames(8192)
    with pytest.raises(FmError) as e:
        wide.backward(torch.zeros(1, 8192, device="cuda"), torch.zeros(1, 128, T, device="cuda"))
    assert e.value.status == FM_E_UNSUPPORTED
