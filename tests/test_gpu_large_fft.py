"""GPU parity of the three-pass kernel (n_fft 8192 and 16384) against the
f64 oracle, at the bar of the other parity tests: max |gpu - ref| <=
1e-4 * (1 + |ref|) elementwise.

The flashmel 0.1.0 page allows n_fft up to 16384 (README "Usage") and
measures a "huge" case at 16384/4096 with 256 mels (README "Performance").
"""
import numpy as np
import pytest

from stft_mel_spectrogram_amd import workloads as W
from test_gpu_parity import assert_parity, assert_parity_f16, oracle, run_gpu, torch  # noqa: F401

pytestmark = pytest.mark.gpu

# (n_fft, hop, n_mels, length, extra transform arguments)
CASES = [
    (8192, 2048, 128, 60001, dict()),                                  # ragged last tile
    (16384, 4096, 256, 60001, dict()),
    (8192, 1000, 64, 30000, dict(power=1.0)),                         # hop not dividing n_fft
    (16384, 333, 40, 20000, dict(power=1.5)),                         # odd hop: unpaired loads
    (16384, 16384, 256, 70000, dict()),                               # frames do not overlap
    (8192, 4096, 1, 9000, dict(f_max=22050.0)),                       # one filter
    (16384, 4096, 8, 8193, dict()),                                   # shortest reflect signal
    (8192, 2048, 96, 25000, dict(center=False)),
    (16384, 2048, 128, 40000, dict(win_length=12000, normalized=True)),
    (8192, 2048, 80, 30000, dict(mel_scale="slaney", norm="slaney", f_min=50.0)),
    (16384, 4096, 128, 30000, dict(pad_mode="constant", pad=777)),
    (8192, 2048, 128, 30000, dict(pad_mode="replicate")),
    (16384, 4096, 128, 30000, dict(pad_mode="circular", pad=5)),
]


@pytest.mark.parametrize("n_fft,hop,mels,L,extra", CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}-{'-'.join(c[4])}" for c in CASES])
def test_large_fft_parity(n_fft, hop, mels, L, extra):
    x = np.random.default_rng(n_fft + hop + L).standard_normal((2, L)).astype(np.float32) * 0.3
    targs = dict(sample_rate=44100, n_fft=n_fft, hop_length=hop, n_mels=mels, **extra)
    print(f"[case] n_fft {n_fft} hop {hop} mels {mels} L {L} {extra}", flush=True)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"{n_fft}/{hop} {extra}")


@pytest.mark.parametrize("n_fft", [8192, 16384])
def test_large_fft_int16_and_f16_output(n_fft):
    q = np.random.default_rng(n_fft).integers(-32768, 32768, size=(3, 50001)).astype(np.int16)
    targs = dict(sample_rate=44100, n_fft=n_fft, hop_length=n_fft // 4, n_mels=256)
    print(f"[case] int16 n_fft {n_fft}", flush=True)
    ref = oracle(q, **targs)
    assert_parity(run_gpu(q, **targs), ref, f"i16 {n_fft}")
    # float16 output: the f32 result rounded once (values past the float16
    # range may come out as inf)
    assert_parity_f16(run_gpu(q, out_dtype=torch.float16, **targs), ref, f"i16 -> f16 {n_fft}")


@pytest.mark.parametrize("tile", [1, 3, 7, 40])
def test_large_fft_forced_tiles(monkeypatch, tile):
    """Workgroups that walk 1, 3, 7 or 40 frames (the last tile ragged)."""
    monkeypatch.setenv("FM_TILE_FRAMES", str(tile))
    x = np.random.default_rng(tile).standard_normal((2, 100000)).astype(np.float32)
    targs = dict(sample_rate=44100, n_fft=8192, hop_length=2048, n_mels=128)
    print(f"[case] forced tile {tile}", flush=True)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"tile {tile}")


@pytest.mark.parametrize("name", ["huge", "fft8192"])
def test_large_fft_full_workloads(name):
    """Full size (16 x 441000 samples): every output finite, non-negative and
    identical on a second launch; the first and last signals against the
    oracle."""
    cfg = W.workload(name)
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    print(f"[case] full {name} {x.shape}", flush=True)
    got = run_gpu(x, **targs)
    assert np.all(np.isfinite(got)) and np.all(got >= 0)
    assert np.array_equal(got, run_gpu(x, **targs))
    rows = [0, cfg["batch"] - 1]
    assert_parity(got[rows], oracle(x[rows], **targs), f"full {name} (rows {rows})")


# n_fft 4096 runs on the three-pass kernel (16 x 16 x 8) in calls where the
# two-pass kernel's tiles would take more than one round; FM_FORWARD=large
# forces it for the small cases here.
CASES_4096 = [
    (4096, 1024, 128, 60001, dict()),                                 # ragged last tile
    (4096, 1000, 64, 30000, dict(power=1.0)),                         # hop not dividing n_fft
    (4096, 333, 40, 20000, dict(power=1.5)),                          # odd hop: unpaired loads
    (4096, 4096, 128, 40000, dict()),                                 # frames do not overlap
    (4096, 1024, 1, 9000, dict(f_max=22050.0)),                       # one filter
    (4096, 1024, 8, 4097, dict()),                                    # shortest reflect signal
    (4096, 1024, 96, 25000, dict(center=False)),
    (4096, 512, 128, 40000, dict(win_length=3000, normalized=True)),
    (4096, 1024, 80, 30000, dict(mel_scale="slaney", norm="slaney", f_min=50.0)),
    (4096, 1024, 128, 30000, dict(pad_mode="constant", pad=777)),
    (4096, 1024, 128, 30000, dict(pad_mode="replicate")),
    (4096, 1024, 128, 30000, dict(pad_mode="circular", pad=5)),
    (4096, 1024, 256, 30000, dict()),                                 # two filters per thread
    (4096, 1024, 129, 30000, dict(power=1.0)),                        # one thread takes a second
]


@pytest.mark.parametrize("n_fft,hop,mels,L,extra", CASES_4096,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}-{'-'.join(c[4])}" for c in CASES_4096])
def test_three_pass_4096_parity(monkeypatch, n_fft, hop, mels, L, extra):
    monkeypatch.setenv("FM_FORWARD", "large")
    x = np.random.default_rng(n_fft + hop + L + 1).standard_normal((2, L)).astype(np.float32) * 0.3
    targs = dict(sample_rate=44100, n_fft=n_fft, hop_length=hop, n_mels=mels, **extra)
    print(f"[case] three-pass n_fft {n_fft} hop {hop} mels {mels} L {L} {extra}", flush=True)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"three-pass {n_fft}/{hop} {extra}")


def test_three_pass_4096_int16_f16_and_tiles(monkeypatch):
    monkeypatch.setenv("FM_FORWARD", "large")
    q = np.random.default_rng(4096).integers(-32768, 32768, size=(3, 50001)).astype(np.int16)
    targs = dict(sample_rate=44100, n_fft=4096, hop_length=1024, n_mels=128)
    print("[case] three-pass int16 n_fft 4096", flush=True)
    ref = oracle(q, **targs)
    assert_parity(run_gpu(q, **targs), ref, "three-pass i16 4096")
    assert_parity_f16(run_gpu(q, out_dtype=torch.float16, **targs), ref, "three-pass i16 -> f16 4096")
    for tile in (1, 3, 5):
        monkeypatch.setenv("FM_TILE_FRAMES", str(tile))
        print(f"[case] three-pass n_fft 4096 tile {tile}", flush=True)
        assert_parity(run_gpu(q, **targs), ref, f"three-pass 4096 tile {tile}")


def test_music4096_full_workload_takes_three_pass():
    """Full size (4 x 1323000 samples, 128 mels): the call takes the
    three-pass kernel; every output finite, non-negative and identical on a
    second launch; the first and last signals against the oracle."""
    from stft_mel_spectrogram_amd import _native as N
    cfg = W.workload("music4096")
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    p = N.Plan(**targs)
    assert p.forward_config(cfg["batch"], x.shape[1])[0] == N.FM_FWD_LARGE
    p.close()
    print(f"[case] full music4096 {x.shape}", flush=True)
    got = run_gpu(x, **targs)
    assert np.all(np.isfinite(got)) and np.all(got >= 0)
    assert np.array_equal(got, run_gpu(x, **targs))
    rows = [0, cfg["batch"] - 1]
    assert_parity(got[rows], oracle(x[rows], **targs), f"full music4096 (rows {rows})")
