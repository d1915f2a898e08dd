"""The GPU parity suite of test_gpu_parity.py run again with the second FFT
pass's row layout forced at plan creation (FM_FORWARD=rows: one thread per
row of a frame, 512 threads per workgroup; built for n_fft 64 ... 2048, while
n_fft 4096 and the three-pass sizes keep their kernel), against the same f64
oracle at the same bar, max |gpu - ref| <= 1e-4 * (1 + |ref|); and, per FFT
size, the row layout's output equal bit for bit to the pair layout's (both
run the same operations in the same order)."""
import numpy as np
import pytest

from test_gpu_parity import *  # noqa: F401,F403  (its tests, collected again under this module's fixture)
from test_gpu_parity import torch


@pytest.fixture(autouse=True)
def row_layout(monkeypatch):
    monkeypatch.setenv("FM_FORWARD", "rows")


@pytest.mark.parametrize("n_fft", [64, 128, 256, 400, 512, 1024, 2048])
@pytest.mark.parametrize("dtype", ["f32", "i16"])
def test_row_layout_equals_pair_layout(n_fft, dtype, monkeypatch):
    from stft_mel_spectrogram_amd import MelSpectrogram
    from stft_mel_spectrogram_amd._native import FM_FWD_ROWS, FM_FWD_SPLIT
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(n_fft)
    L = 40 * n_fft + 123
    if dtype == "f32":
        x = torch.from_numpy(rng.standard_normal((3, L)).astype(np.float32) * 0.3).to("cuda")
    else:
        x = torch.from_numpy(rng.integers(-32768, 32768, size=(3, L)).astype(np.int16)).to("cuda")
    targs = dict(sample_rate=16000, n_fft=n_fft, hop_length=max(1, n_fft // 4), n_mels=64)
    outs = {}
    for name, want in (("rows", FM_FWD_ROWS), ("split", FM_FWD_SPLIT)):
        monkeypatch.setenv("FM_FORWARD", name)
        mel = MelSpectrogram(**targs)
        assert mel.plan.info().forward_variant == want
        outs[name] = mel(x)
    torch.cuda.synchronize()
    print(f"[case] n_fft={n_fft} {dtype}: rows vs split", flush=True)
    assert torch.equal(outs["rows"], outs["split"])
