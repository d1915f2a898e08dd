"""GPU parity: the HIP path (through the C ABI) against the f64 oracle.

Bar: max |gpu - ref| <= 1e-4 * (1 + |ref|) elementwise (the fp32 tolerance
atol = rtol = 1e-4 the flashmel page states against torchaudio, README
"Development", here against the f64 definition).
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


def run_gpu(x_np, **targs):
    """The HIP forward pass through the C ABI, written into an output
    tensor filled with NaN first, so an element the kernel fails to write
    cannot pass on a previous call's value left in reused memory."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    mel = MelSpectrogram(**targs)
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to("cuda")
    shape = tuple(x.shape[:-1]) + (mel.n_mels, mel.out_frames(x.shape[-1]))
    out = torch.full(shape, float("nan"), dtype=mel.out_dtype, device="cuda")
    y = mel(x, out=out)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    return y.cpu().numpy()


def oracle(x_np, **targs):
    return O.mel_spectrogram(x_np, chunk=4, **targs)


def assert_parity(got, ref, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got.astype(np.float64) - ref)
    bound = TOL * (1.0 + np.abs(ref))
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    ratio = float((err / bound)[worst])
    print(f"[parity] {what}: max err/bound = {ratio:.3g} at {worst} "
          f"(gpu {got[worst]:.6g}, ref {ref[worst]:.6g}), max abs err {err.max():.3g}", flush=True)
    assert ratio <= 1.0, what


# ------------------------------------------------------------------ small cases: every output

SMALL = [
    ("tiny", dict()),                                     # 1 x 16000, 101 frames (4 tiles, ragged)
    ("whisper", dict(batch=3, length=48_000)),           # 301 frames per signal
    ("int16", dict(batch=2, length=48_000)),
    ("pow2", dict()),                                     # full size: 8 x 32768
    ("large", dict(batch=3)),                             # 3 x 220500, n_fft 2048, power 1
]


@pytest.mark.parametrize("name,over", SMALL, ids=[s[0] for s in SMALL])
def test_parity_small(name, over):
    cfg = W.workload(name, **over)
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    print(f"[case] {name} {x.shape} {x.dtype}", flush=True)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), name)


# ------------------------------------------------------------------ full workloads

@pytest.mark.parametrize("name", ["whisper", "int16"])
def test_parity_full_whisper_shape(name):
    cfg = W.workload(name)
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    print(f"[case] full {name} {x.shape}", flush=True)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"full {name}")


def test_parity_full_large_sampled_rows():
    """64 x 220500: every output is checked for finiteness and sign; the
    oracle recomputes 6 whole rows (first, last and four inside)."""
    cfg = W.workload("large")
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    got = run_gpu(x, **targs)
    assert got.shape == (64, 128, 431)
    assert np.all(np.isfinite(got)) and np.all(got >= 0)
    rows = [0, 1, 17, 31, 50, 63]
    assert_parity(got[rows], oracle(x[rows], **targs), "full large (sampled rows)")


# ------------------------------------------------------------------ edge cases

EDGE_LENGTHS = [201, 202, 399, 400, 401, 1000, 5119, 5121, 16001]


@pytest.mark.parametrize("L", EDGE_LENGTHS)
def test_short_and_ragged_lengths(L):
    """Lengths just above n_fft/2, not multiples of hop, one tile straddling
    both signal edges, odd lengths (unpaired-load path)."""
    x = np.random.default_rng(L).standard_normal((2, L)).astype(np.float32) * 0.3
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=80, f_max=8000.0)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"L={L}")


@pytest.mark.parametrize("n_fft,hop", [(1024, 256), (2048, 512), (1024, 100)])
def test_ragged_large_fft(n_fft, hop):
    x = np.random.default_rng(n_fft).standard_normal((2, 9001)).astype(np.float32)
    targs = dict(sample_rate=22050, n_fft=n_fft, hop_length=hop, n_mels=96)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"{n_fft}/{hop}")


@pytest.mark.parametrize("n_fft,hop,L,pad_mode,center", [
    (400, 400, 9001, "reflect", True), (400, 500, 9001, "reflect", True),
    (400, 1000, 9001, "constant", True), (400, 777, 9001, "reflect", False),
    (64, 1, 300, "reflect", True), (128, 1, 257, "circular", True)])
def test_hop_extremes(n_fft, hop, L, pad_mode, center):
    """Frames that do not overlap (hop >= n_fft: samples between frames are
    never read) and hop = 1 (every sample starts a frame)."""
    x = np.random.default_rng(hop + L).standard_normal((2, L)).astype(np.float32)
    targs = dict(sample_rate=16000, n_fft=n_fft, hop_length=hop, n_mels=24, pad_mode=pad_mode,
                 center=center)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"n_fft={n_fft} hop={hop}")


OTHER_FFT = [(64, 16, 40), (64, 20, 8), (128, 32, 40), (256, 64, 64), (256, 100, 128),
             (512, 128, 80), (512, 100, 256), (4096, 1024, 128), (4096, 512, 40)]


@pytest.mark.parametrize("n_fft,hop,mels", OTHER_FFT)
def test_other_fft_sizes(n_fft, hop, mels):
    """Powers of two 64..4096 besides 1024/2048 (ragged signal lengths)."""
    x = np.random.default_rng(n_fft + hop).standard_normal((2, 9001)).astype(np.float32)
    targs = dict(sample_rate=16000, n_fft=n_fft, hop_length=hop, n_mels=mels)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"n_fft={n_fft} hop={hop} mels={mels}")


@pytest.mark.parametrize("name", ["asr512", "music4096", "fft256", "fft128", "fft64"])
def test_parity_full_other_fft_workloads(name):
    """Full-size measurement workloads of the other FFT sizes: every output
    finite and non-negative; first and last signals against the oracle."""
    cfg = W.workload(name)
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    got = run_gpu(x, **targs)
    assert np.all(np.isfinite(got)) and np.all(got >= 0)
    rows = [0, cfg["batch"] - 1]
    assert_parity(got[rows], oracle(x[rows], **targs), f"full {name} (rows {rows})")


def test_other_fft_sizes_mixed_arguments():
    q = np.random.default_rng(21).integers(-32768, 32768, size=(3, 7777)).astype(np.int16)
    for targs in (dict(n_fft=64, hop_length=32, n_mels=24, power=1.0, center=False),
                  dict(n_fft=256, win_length=200, hop_length=80, n_mels=64, pad_mode="constant"),
                  dict(n_fft=512, hop_length=160, n_mels=96, power=1.5, normalized=True),
                  dict(n_fft=128, hop_length=64, n_mels=32, mel_scale="slaney", norm="slaney"),
                  dict(n_fft=4096, win_length=3000, hop_length=700, n_mels=64, pad=123)):
        assert_parity(run_gpu(q, sample_rate=22050, **targs), oracle(q, sample_rate=22050, **targs),
                      f"i16 {targs}")


@pytest.mark.parametrize("pad_mode", ["constant", "replicate", "circular"])
def test_other_pad_modes(pad_mode):
    x = np.random.default_rng(3).standard_normal((2, 5000)).astype(np.float32)
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=64, pad_mode=pad_mode)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), pad_mode)


def test_center_false_and_general_power_and_slaney():
    x = np.random.default_rng(4).standard_normal((3, 7000)).astype(np.float32)
    for targs in (dict(n_fft=400, hop_length=100, n_mels=64, center=False),
                  dict(n_fft=1024, hop_length=256, n_mels=80, power=1.5),
                  dict(n_fft=400, hop_length=160, n_mels=40, mel_scale="slaney", norm="slaney"),
                  dict(n_fft=400, hop_length=160, n_mels=60, f_min=125.0, f_max=7000.0),
                  dict(n_fft=400, win_length=320, hop_length=160, n_mels=60),
                  dict(n_fft=2048, hop_length=512, n_mels=8),        # rows wider than 64 bins
                  dict(n_fft=400, hop_length=160, n_mels=256)):
        assert_parity(run_gpu(x, sample_rate=16000, **targs), oracle(x, sample_rate=16000, **targs),
                      str(targs))


@pytest.mark.parametrize("pad", [1, 3, 160, 999])
@pytest.mark.parametrize("pad_mode", ["reflect", "constant", "replicate", "circular"])
def test_zero_pad_argument(pad, pad_mode):
    """`pad` zeros on both sides, then centre padding of the zero-extended
    signal (odd pads take the unpaired-load path)."""
    x = np.random.default_rng(pad).standard_normal((2, 4321)).astype(np.float32)
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=64, pad=pad, pad_mode=pad_mode)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"pad={pad} {pad_mode}")


def test_zero_pad_short_signal_and_no_centring():
    x = np.random.default_rng(11).standard_normal((3, 150)).astype(np.float32)
    for targs in (dict(n_fft=400, hop_length=160, n_mels=40, pad=60),     # 150 < 200 < 270
                  dict(n_fft=400, hop_length=100, n_mels=40, pad=200, center=False),
                  dict(n_fft=1024, hop_length=256, n_mels=80, pad=700)):
        assert_parity(run_gpu(x, sample_rate=16000, **targs), oracle(x, sample_rate=16000, **targs),
                      str(targs))


@pytest.mark.parametrize("normalized", [True, "frame_length"])
@pytest.mark.parametrize("n_fft,win", [(400, 400), (400, 320), (1024, 1000)])
def test_normalized_window(normalized, n_fft, win):
    x = np.random.default_rng(win).standard_normal((2, 8000)).astype(np.float32)
    targs = dict(sample_rate=16000, n_fft=n_fft, win_length=win, hop_length=n_fft // 4, n_mels=64,
                 normalized=normalized)
    assert_parity(run_gpu(x, **targs), oracle(x, **targs), f"normalized={normalized} {n_fft}/{win}")


TOL16 = 1e-2


def assert_parity_f16(got, ref64, what=""):
    """fp16 output: against the f64 oracle rounded to fp16, |gpu - ref16| <=
    1e-2 * (1 + |ref16|); values beyond the fp16 range may come out as inf."""
    assert got.dtype == np.float16 and got.shape == ref64.shape, what
    with np.errstate(over="ignore", invalid="ignore"):   # fp16 overflow is part of the contract
        ref16 = ref64.astype(np.float16).astype(np.float64)
        g = got.astype(np.float64)
        big = np.abs(ref64) >= 65504.0 * (1 - TOL16)
        assert np.all(np.isinf(g[big]) | (np.abs(g[big] - ref16[big]) <= TOL16 * (1 + np.abs(ref16[big])))), what
    assert np.all(np.isfinite(g[~big])), what
    err = np.abs(g[~big] - ref16[~big])
    ratio = float(np.max(err / (TOL16 * (1 + np.abs(ref16[~big]))))) if err.size else 0.0
    print(f"[parity f16] {what}: max err/bound {ratio:.3g}, {int(big.sum())} values past fp16 range",
          flush=True)
    assert ratio <= 1.0, what


@pytest.mark.parametrize("name,over,scale", [("whisper", dict(batch=2, length=48_000), 1.0),
                                             ("int16", dict(batch=2, length=48_000), 1.0),
                                             ("pow2", dict(batch=3), 1.0),
                                             ("tiny", dict(), 80.0),
                                             ("large", dict(batch=2), 1.0)])
def test_f16_output(name, over, scale):
    cfg = W.workload(name, **over)
    x = W.make_signal(cfg)
    if scale != 1.0:
        x = (x * scale).astype(x.dtype)       # pushes some powers past 65504
    targs = W.transform_args(cfg)
    got = run_gpu(x, out_dtype=torch.float16, **targs)
    assert_parity_f16(got, oracle(x, **targs), f"f16 {name} x{scale}")


def test_f16_full_whisper_sampled_rows():
    cfg = W.workload("whisper")
    x = W.make_signal(cfg)
    targs = W.transform_args(cfg)
    got = run_gpu(x, out_dtype=torch.float16, **targs)
    assert got.shape == (8, 128, 3001)
    assert_parity_f16(got[[0, 7]], oracle(x[[0, 7]], **targs), "f16 full whisper rows 0, 7")


@pytest.mark.parametrize("n_fft,hop,tile", [(128, 32, 0), (256, 64, 0), (400, 100, 0), (400, 160, 40),
                                            (512, 128, 0), (1024, 256, 0), (2048, 512, 0), (4096, 1024, 0)])
@pytest.mark.parametrize("dtype", ["f32", "i16"])
def test_tile_copy_path(n_fft, hop, tile, dtype, monkeypatch):
    """Interior tiles copy their sample span into LDS (edge tiles, and inputs
    not aligned for it, gather): at hop = n_fft/4 in both layouts of the
    second pass, at n_fft 400, hop 160 in the row layout's tiles of 32
    frames or more (forced here to 40), and for n_fft 512 ... 4096 (one frame
    per pass-1 thread), whose calls copy only when they have more workgroups
    than compute units (forced here with FM_TILE_COPY=1); also from an input
    that starts 4 (f32) or 2 (int16) bytes into its allocation."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    if tile:
        monkeypatch.setenv("FM_TILE_FRAMES", str(tile))
    if n_fft >= 512:
        monkeypatch.setenv("FM_TILE_COPY", "1")
    rng = np.random.default_rng(n_fft)
    n = 20_011
    if dtype == "f32":
        x = rng.standard_normal((3, n)).astype(np.float32)
        tdt = torch.float32
    else:
        x = rng.integers(-32768, 32768, size=(3, n)).astype(np.int16)
        tdt = torch.int16
    targs = dict(sample_rate=16000, n_fft=n_fft, hop_length=hop, n_mels=64)
    ref = oracle(x, **targs)
    assert_parity(run_gpu(x, **targs), ref, f"copy {dtype} {n_fft} hop {hop}")
    base = torch.empty(3 * n + 1, dtype=tdt, device="cuda")
    base[1:] = torch.from_numpy(x.reshape(-1)).to("cuda")
    shifted = base[1:].view(3, n)
    y = MelSpectrogram(**targs)(shifted)
    torch.cuda.synchronize()
    assert_parity(y.cpu().numpy(), ref, f"copy {dtype} {n_fft} hop {hop} misaligned")


@pytest.mark.parametrize("n_fft,tiles", [(400, [1, 7, 16, 17, 32, 33, 48, 49, 64]),
                                         (128, [5, 64]), (1024, [1, 9, 16]), (4096, [3, 8])])
def test_forced_tile_sizes(monkeypatch, n_fft, tiles):
    """Every tile width the kernel has: 1..4 sixteen-frame column groups in
    the mel stage, direct stores (<= 32 frames) and staged row stores (>= 33),
    ragged last tiles; f32 and f16 output (FM_TILE_FRAMES forces the size)."""
    x = np.random.default_rng(n_fft).standard_normal((2, 12_345)).astype(np.float32)
    targs = dict(sample_rate=16000, n_fft=n_fft, hop_length=n_fft // 3, n_mels=72)
    ref = oracle(x, **targs)
    for g in tiles:
        monkeypatch.setenv("FM_TILE_FRAMES", str(g))
        assert_parity(run_gpu(x, **targs), ref, f"n_fft={n_fft} tile={g}")
        assert_parity_f16(run_gpu(x, out_dtype=torch.float16, **targs), ref, f"f16 n_fft={n_fft} tile={g}")
    monkeypatch.delenv("FM_TILE_FRAMES")


@pytest.mark.parametrize("n_mels", [1, 8, 16])
@pytest.mark.parametrize("tile", [0, 7, 33, 47])
def test_few_mels_full_band_ragged_tiles(monkeypatch, n_mels, tile):
    """n_fft 400 with at most 16 mels up to Nyquist: the one 16-filter block
    spans every bin (52 four-bin steps over a 201-float row), so the mel
    stage reads past each frame's row; in the last, ragged tile of a signal
    those floats must be zero, not whatever the LDS held before.  Ragged
    length, forced tile widths (0: the width the launch chooses), f32 and f16
    output, and a first launch of a wide many-mel plan that leaves non-zero
    LDS behind."""
    rng = np.random.default_rng(100 + n_mels)
    x = (rng.standard_normal((3, 16_321)) * 0.2).astype(np.float32)
    # fill the LDS of every compute unit with large values first
    run_gpu((rng.standard_normal((8, 48_000)) * 1e3).astype(np.float32), sample_rate=16000,
            n_fft=400, hop_length=160, n_mels=256)
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=n_mels, f_max=8000.0)
    ref = oracle(x, **targs)
    if tile:
        monkeypatch.setenv("FM_TILE_FRAMES", str(tile))
    assert_parity(run_gpu(x, **targs), ref, f"mels={n_mels} tile={tile}")
    assert_parity_f16(run_gpu(x, out_dtype=torch.float16, **targs), ref, f"f16 mels={n_mels} tile={tile}")


def test_int16_odd_length_and_misaligned_input():
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    q = np.random.default_rng(5).integers(-32768, 32768, size=(2, 6001)).astype(np.int16)
    targs = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=80)
    assert_parity(run_gpu(q, **targs), oracle(q, **targs), "i16 odd length")
    # input that starts one sample into an allocation: no paired loads allowed
    x = np.random.default_rng(6).standard_normal((2, 6001)).astype(np.float32)
    base = torch.empty(2 * 6000 + 1, device="cuda")
    base[1:] = torch.from_numpy(x[:, :6000].reshape(-1)).to("cuda")
    shifted = base[1:].view(2, 6000)          # data_ptr is 4 bytes past a 256-B boundary
    assert shifted.data_ptr() % 8 == 4
    y = MelSpectrogram(**targs)(shifted)
    torch.cuda.synchronize()
    assert_parity(y.cpu().numpy(), oracle(x[:, :6000], **targs), "misaligned f32")


def test_every_output_written_and_deterministic():
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    cfg = W.workload("whisper", batch=2, length=30_000)
    x = torch.from_numpy(W.make_signal(cfg)).cuda()
    mel = MelSpectrogram(**W.transform_args(cfg))
    T = mel.out_frames(30_000)
    out1 = torch.full((2, 128, T), float("nan"), device="cuda")
    out2 = torch.full((2, 128, T), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        mel(x, out=out1)
        mel(x, out=out2)
    torch.cuda.synchronize()
    assert not torch.isnan(out1).any()
    assert torch.equal(out1, out2)
    # empty filters (no bin inside) are exactly zero
    for m in (0, 3, 6, 13):
        assert torch.all(out1[:, m] == 0)


def test_maximum_length_sampled_frames():
    """length = 2^29 (the largest one launch takes; 2 GB of f32): frames at
    both ends and inside against the oracle on excerpts (a prefix for the
    first frames, a hop-aligned suffix for the last, exact slices inside);
    one sample more is rejected."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    from stft_mel_spectrogram_amd._native import FmError
    _require_gpu()
    n, hop, nfft = 1 << 29, 160, 400
    targs = dict(sample_rate=16000, n_fft=nfft, hop_length=hop, n_mels=80)
    rng = np.random.default_rng(29)
    x = (rng.standard_normal(n, dtype=np.float32) * np.float32(0.1))
    mel = MelSpectrogram(**targs)
    xd = torch.from_numpy(x).cuda()
    y = mel(xd)
    torch.cuda.synchronize()
    T = y.shape[-1]
    assert T == 1 + n // hop
    # first frames: the oracle on a prefix (centre padding reflects inside it)
    pre = 20 * hop
    ref = oracle(x[:pre], **targs)
    assert_parity(y[:, :10].cpu().numpy(), ref[:, :10], "max length: first frames")
    # last frames: a suffix starting on the frame grid
    start = (n // hop - 20) * hop
    ref = oracle(x[start:], **targs)
    assert_parity(y[:, -5:].cpu().numpy(), ref[:, -5:], "max length: last frames")
    # interior frames: exactly their samples, no centring
    for t in (T // 3, T // 2, T - 40):
        a0 = t * hop - nfft // 2
        ref = oracle(x[a0:a0 + nfft], center=False, **targs)
        assert_parity(y[:, t:t + 1].cpu().numpy(), ref, f"max length: frame {t}")
    del y
    with pytest.raises(FmError):
        mel.plan.forward_ptr(xd.data_ptr(), 0, 1, n + 1, xd.data_ptr())


def test_one_plan_on_two_streams():
    """A plan is immutable: two streams may run it at the same time."""
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    cfg = W.workload("whisper", batch=4, length=64_000)
    mel = MelSpectrogram(**W.transform_args(cfg))
    xa = torch.from_numpy(W.make_signal(cfg)).cuda()
    xb = torch.from_numpy(W.make_signal(W.workload("whisper", batch=4, length=64_000, seed=9))).cuda()
    ref_a, ref_b = mel(xa).clone(), mel(xb).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(5):
        with torch.cuda.stream(s1):
            ya = mel(xa)
        with torch.cuda.stream(s2):
            yb = mel(xb)
        outs.append((ya, yb))
    torch.cuda.synchronize()
    for ya, yb in outs:
        assert torch.equal(ya, ref_a) and torch.equal(yb, ref_b)


def test_leading_dims_and_empty_batch():
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    mel = MelSpectrogram(sample_rate=16000, n_fft=400, hop_length=160, n_mels=40)
    x = np.random.default_rng(7).standard_normal((2, 3, 4000)).astype(np.float32)
    y = mel(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert tuple(y.shape) == (2, 3, 40, 26)
    assert_parity(y.cpu().numpy(), oracle(x, sample_rate=16000, n_fft=400, hop_length=160, n_mels=40),
                  "leading dims")
    z = mel(torch.empty((0, 4000), device="cuda"))
    assert tuple(z.shape) == (0, 40, 26)


def test_rejects_bad_inputs():
    from stft_mel_spectrogram_amd import MelSpectrogram
    _require_gpu()
    mel = MelSpectrogram(n_fft=400, hop_length=160, n_mels=40)
    with pytest.raises(ValueError):
        mel(torch.zeros(4000))                                  # host tensor
    with pytest.raises(TypeError):
        mel(torch.zeros(4000, dtype=torch.float64, device="cuda"))
    assert mel(torch.zeros(4000, device="cuda", requires_grad=True)).requires_grad  # autograd node
    with pytest.raises(ValueError):
        mel(torch.zeros(2, 4000, device="cuda").t())             # non-contiguous
    from stft_mel_spectrogram_amd._native import FmError
    with pytest.raises(FmError):
        mel(torch.zeros(150, device="cuda"))                     # reflect needs L > 200
