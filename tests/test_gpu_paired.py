"""GPU parity of the opt-in paired-frame forward kernel (two real frames per
complex FFT of n_fft points, n_fft 400), selected with FM_FORWARD=paired at
plan creation, against the f64 oracle at the bar of the other parity tests:
max |gpu - ref| <= 1e-4 * (1 + |ref|) elementwise (fp16 output: the fp16
tests' bar).  The flashmel 0.1.0 page names the packing (README "How it
works") and measured its own paired variant slower ("Where each case
actually sits"); so does this build, which keeps it as an A/B variant."""
import numpy as np
import pytest

from stft_mel_spectrogram_amd import workloads as W
from test_gpu_parity import assert_parity, assert_parity_f16, oracle, torch  # noqa: F401

pytestmark = pytest.mark.gpu


def run_paired(x_np, out_dtype=None, **targs):
    """The forward pass with the paired kernel (checked), into a NaN-filled
    output."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    from stft_mel_spectrogram_amd._native import FM_FWD_PAIRED
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kw = {} if out_dtype is None else dict(out_dtype=out_dtype)
    mel = MelSpectrogram(**targs, **kw)
    assert mel.plan.info().forward_variant == FM_FWD_PAIRED
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to("cuda")
    shape = tuple(x.shape[:-1]) + (mel.n_mels, mel.out_frames(x.shape[-1]))
    out = torch.full(shape, float("nan"), dtype=mel.out_dtype, device="cuda")
    mel(x, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.fixture(autouse=True)
def paired_env(monkeypatch):
    monkeypatch.setenv("FM_FORWARD", "paired")


CASES = [
    ("tiny", dict()),
    ("whisper", dict(batch=3, length=48_000)),
    ("int16", dict(batch=2, length=48_000)),
    ("whisper", dict(batch=2, length=16_001)),     # odd length: unpaired loads
]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_paired_parity(name, over):
    cfg = W.workload(name, **over)
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    print(f"[case] paired {name} {x.shape} {x.dtype}", flush=True)
    assert_parity(run_paired(x, **targs), oracle(x, **targs), f"paired {name}")


@pytest.mark.parametrize("L", [201, 400, 1000, 5121])
@pytest.mark.parametrize("pad_mode", ["reflect", "constant", "circular"])
def test_paired_short_signals_and_pad_modes(L, pad_mode):
    if pad_mode == "circular" and L < 200:
        pytest.skip("circular padding needs length >= n_fft/2")
    x = np.random.default_rng(L).standard_normal((3, L)).astype(np.float32) * 0.3
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=80, pad_mode=pad_mode)
    print(f"[case] paired L={L} {pad_mode}", flush=True)
    assert_parity(run_paired(x, **targs), oracle(x, **targs), f"paired L={L} {pad_mode}")


def test_paired_arguments_and_f16():
    x = np.random.default_rng(5).standard_normal((2, 9001)).astype(np.float32) * 0.3
    for targs in (dict(n_fft=400, hop_length=100, n_mels=64, power=1.0),
                  dict(n_fft=400, hop_length=160, n_mels=40, mel_scale="slaney", norm="slaney"),
                  dict(n_fft=400, win_length=320, hop_length=160, n_mels=60, pad=37),
                  dict(n_fft=400, hop_length=160, n_mels=16, f_max=8000.0)):
        print(f"[case] paired {targs}", flush=True)
        assert_parity(run_paired(x, sample_rate=16000, **targs),
                      oracle(x, sample_rate=16000, **targs), f"paired {targs}")
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    assert_parity_f16(run_paired(x, out_dtype=torch.float16, **targs), oracle(x, **targs),
                      "paired f16")


def test_paired_full_whisper_sampled_rows():
    cfg = W.workload("whisper")
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    got = run_paired(x, **targs)
    assert got.shape == (8, 128, 3001) and np.all(np.isfinite(got))
    assert_parity(got[[0, 7]], oracle(x[[0, 7]], **targs), "paired full whisper rows 0, 7")
