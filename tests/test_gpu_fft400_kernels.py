"""GPU parity of the two n_fft-400 forward kernels, each forced at plan
creation (FM_FORWARD=rows: 512-thread workgroups, one second-pass thread per
row of 25 points, the mirrored row exchanged between lanes; FM_FORWARD=split:
256 threads, one per pair of mirrored rows), against the f64 oracle at the bar
of the other parity tests: max |gpu - ref| <= 1e-4 * (1 + |ref|) elementwise
(fp16 output: the fp16 tests' bar); and the default per-call choice between
them, whose output must equal both bit for bit (the two kernels compute the
same operations in the same order; the transform is the torchaudio
MelSpectrogram page's definition)."""
import numpy as np
import pytest

from stft_mel_spectrogram_amd import workloads as W
from test_gpu_parity import assert_parity, assert_parity_f16, oracle, torch  # noqa: F401

pytestmark = pytest.mark.gpu


VARIANT = {"rows": (3, 512), "split": (0, 256)}  # FM_FWD_ROWS / FM_FWD_SPLIT, threads


def run_forced(x_np, out_dtype=None, **targs):
    """The forward pass with the kernel FM_FORWARD names (checked), into a
    NaN-filled output."""
    import os
    from stft_mel_spectrogram_amd import MelSpectrogram
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kw = {} if out_dtype is None else dict(out_dtype=out_dtype)
    mel = MelSpectrogram(**targs, **kw)
    info = mel.plan.info()
    assert (info.forward_variant, info.threads) == VARIANT[os.environ["FM_FORWARD"]]
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to("cuda")
    shape = tuple(x.shape[:-1]) + (mel.n_mels, mel.out_frames(x.shape[-1]))
    out = torch.full(shape, float("nan"), dtype=mel.out_dtype, device="cuda")
    mel(x, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.fixture(params=["rows", "split"])
def variant(request, monkeypatch):
    monkeypatch.setenv("FM_FORWARD", request.param)
    return request.param


CASES = [
    ("tiny", dict()),
    ("whisper", dict(batch=3, length=48_000)),
    ("int16", dict(batch=2, length=48_000)),
    ("whisper", dict(batch=2, length=16_001)),     # odd length: unpaired loads
]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_rows_parity(name, over, variant):
    cfg = W.workload(name, **over)
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    print(f"[case] {variant} {name} {x.shape} {x.dtype}", flush=True)
    assert_parity(run_forced(x, **targs), oracle(x, **targs), f"{variant} {name}")


@pytest.mark.parametrize("tile", [1, 16, 17, 33, 47, 64])
def test_rows_tile_sizes(tile, variant, monkeypatch):
    """Every column-group count of the mel stage (1..4, staged or not), a
    ragged last tile, and the full 64-frame tile (all 512 threads in the
    second pass)."""
    monkeypatch.setenv("FM_TILE_FRAMES", str(tile))
    x = np.random.default_rng(100 + tile).standard_normal((2, 33_123)).astype(np.float32) * 0.3
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    print(f"[case] {variant} tile={tile}", flush=True)
    assert_parity(run_forced(x, **targs), oracle(x, **targs), f"{variant} tile={tile}")


@pytest.mark.parametrize("L", [201, 400, 1000, 5121])
@pytest.mark.parametrize("pad_mode", ["reflect", "constant", "circular"])
def test_rows_short_signals_and_pad_modes(L, pad_mode, variant):
    if pad_mode == "circular" and L < 200:
        pytest.skip("circular padding needs length >= n_fft/2")
    x = np.random.default_rng(L).standard_normal((3, L)).astype(np.float32) * 0.3
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=80, pad_mode=pad_mode)
    print(f"[case] {variant} L={L} {pad_mode}", flush=True)
    assert_parity(run_forced(x, **targs), oracle(x, **targs), f"{variant} L={L} {pad_mode}")


def test_rows_arguments_and_f16(variant):
    x = np.random.default_rng(5).standard_normal((2, 9001)).astype(np.float32) * 0.3
    for targs in (dict(n_fft=400, hop_length=100, n_mels=64, power=1.0),
                  dict(n_fft=400, hop_length=160, n_mels=40, power=0.7),
                  dict(n_fft=400, hop_length=160, n_mels=40, mel_scale="slaney", norm="slaney"),
                  dict(n_fft=400, win_length=320, hop_length=160, n_mels=60, pad=37),
                  dict(n_fft=400, hop_length=160, n_mels=16, f_max=8000.0)):
        print(f"[case] {variant} {targs}", flush=True)
        assert_parity(run_forced(x, sample_rate=16000, **targs),
                      oracle(x, sample_rate=16000, **targs), f"rows {targs}")
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    assert_parity_f16(run_forced(x, out_dtype=torch.float16, **targs), oracle(x, **targs),
                      "rows f16")


def test_rows_full_whisper_sampled_rows(variant):
    cfg = W.workload("whisper")
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    got = run_forced(x, **targs)
    assert got.shape == (8, 128, 3001) and np.all(np.isfinite(got))
    assert_parity(got[[0, 7]], oracle(x[[0, 7]], **targs), "rows full whisper rows 0, 7")


@pytest.mark.parametrize("batch,L", [(1, 16000), (3, 48000), (4, 480000), (8, 480000), (2, 16001)])
def test_auto_choice_equals_both_kernels(batch, L, monkeypatch):
    """The default plan picks a kernel per call; its output equals the forced
    split and row kernels' outputs exactly."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    from stft_mel_spectrogram_amd._native import FM_FWD_AUTO, FM_FWD_ROWS, FM_FWD_SPLIT
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    x = torch.from_numpy(np.random.default_rng(batch * 7 + L).standard_normal((batch, L))
                         .astype(np.float32) * 0.3).to("cuda")
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    monkeypatch.delenv("FM_FORWARD", raising=False)
    auto = MelSpectrogram(**targs)
    assert auto.plan.info().forward_variant == FM_FWD_AUTO
    v, g, wg = auto.plan.forward_config(batch, L)
    assert v in (FM_FWD_ROWS, FM_FWD_SPLIT)
    print(f"[case] auto batch={batch} L={L}: variant {v}, tile {g}, workgroups {wg}", flush=True)
    outs = {"auto": auto(x)}
    for name in ("rows", "split"):
        monkeypatch.setenv("FM_FORWARD", name)
        outs[name] = MelSpectrogram(**targs)(x)
    torch.cuda.synchronize()
    assert torch.equal(outs["auto"], outs["rows"]) and torch.equal(outs["auto"], outs["split"])


def test_auto_choice_on_the_device():
    """On the device (256 compute units) every n_fft-400 call takes the row
    layout: 8 x 480000 in 47-frame tiles, two per compute unit."""
    import os
    from stft_mel_spectrogram_amd import MelSpectrogram
    from stft_mel_spectrogram_amd._native import FM_FWD_ROWS
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if "FM_FORWARD" in os.environ or "FM_TILE_FRAMES" in os.environ:
        pytest.skip("variant or tile forced by the environment")
    mel = MelSpectrogram(sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    if n_cu != 256:
        pytest.skip(f"device with {n_cu} compute units")
    assert mel.plan.forward_config(8, 480000) == (FM_FWD_ROWS, 47, 512)
    assert mel.plan.forward_config(1, 16000)[0] == FM_FWD_ROWS
    assert mel.plan.forward_config(16, 480000)[0] == FM_FWD_ROWS


@pytest.mark.parametrize("n_fft,tiles", [(400, [17, 24, 32, 33, 47, 48, 49, 64]), (128, [17, 40, 64]),
                                         (256, [20, 64])])
@pytest.mark.parametrize("dtype", ["f32", "i16"])
def test_vector_mel_equals_matrix_mel(n_fft, tiles, dtype, monkeypatch):
    """Tiles of 17 frames or more project on the vector units (quads of 4
    filters, one frame per lane); FM_MEL=mfma forces the matrix-core blocks.
    Both add each filter's nonzero products in increasing bin order with one
    rounding per multiply-add (the padding adds exact zeros), so the outputs
    are equal bit for bit, in both second-pass layouts; 80 filters, and 81
    (a last quad of one filter)."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(n_fft + len(tiles))
    L = 70 * (n_fft // 4) + 77
    if dtype == "f32":
        x = torch.from_numpy(rng.standard_normal((2, L)).astype(np.float32)).to("cuda")
    else:
        x = torch.from_numpy(rng.integers(-32768, 32768, size=(2, L)).astype(np.int16)).to("cuda")
    for n_mels in (80, 81):
        for layout in ("rows", "split"):
            for g in tiles:
                outs = {}
                for mel in ("valu", "mfma"):
                    monkeypatch.setenv("FM_FORWARD", layout)
                    monkeypatch.setenv("FM_TILE_FRAMES", str(g))
                    monkeypatch.setenv("FM_MEL", mel)
                    m = MelSpectrogram(sample_rate=16000, n_fft=n_fft, hop_length=n_fft // 4,
                                       n_mels=n_mels)
                    outs[mel] = m(x)
                torch.cuda.synchronize()
                print(f"[case] n_fft={n_fft} {dtype} mels={n_mels} {layout} tile={g}", flush=True)
                assert torch.equal(outs["valu"], outs["mfma"]), (n_fft, dtype, n_mels, layout, g)


@pytest.mark.parametrize("n_fft,hop", [(400, 160), (512, 160), (1024, 256)])
def test_phase_priority_variant_equals_plain(n_fft, hop, monkeypatch):
    """The phase-priority kernels (each wave lowering its issue priority
    phase by phase; chosen for calls of one round with two or more
    workgroups on a CU, FM_PRIO=1 forces them) only reorder issue: outputs
    equal the plain kernels' bit for bit, in both second-pass layouts."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(n_fft + hop)
    x = torch.from_numpy(rng.standard_normal((4, 60 * hop + 311)).astype(np.float32)).to("cuda")
    for layout in ("rows", "split"):
        outs = {}
        for prio in ("0", "1"):
            monkeypatch.setenv("FM_FORWARD", layout)
            monkeypatch.setenv("FM_PRIO", prio)
            outs[prio] = MelSpectrogram(sample_rate=16000, n_fft=n_fft, hop_length=hop, n_mels=64)(x)
        torch.cuda.synchronize()
        print(f"[case] n_fft={n_fft} hop={hop} {layout}: FM_PRIO 0 vs 1", flush=True)
        assert torch.equal(outs["0"], outs["1"]), (n_fft, layout)
