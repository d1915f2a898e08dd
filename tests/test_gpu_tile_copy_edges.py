"""Tile copy at the signal ends: the whole-tile sample copy of the forward
kernel also serves the first and last tiles of a signal, whose spans reach
into the centre padding.  Against the f64 oracle at max |gpu - ref| <=
1e-4 * (1 + |ref|), and bit for bit against the per-sample gathering path
(both read the same samples and run the same operations)."""
import numpy as np
import pytest

from test_gpu_parity import _require_gpu, assert_parity, oracle, run_gpu

pytestmark = pytest.mark.gpu

EDGE_SHAPES = [(400, 160), (128, 32), (1024, 256), (2048, 512)]


@pytest.mark.parametrize("layout", ["rows", "split"])
@pytest.mark.parametrize("n_fft,hop", EDGE_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "i16"])
def test_tile_copy_edge_tiles(layout, n_fft, hop, dtype, monkeypatch):
    """Edge tiles copy their span too: the positions in the centre padding,
    and the partial 16-byte chunks at a signal's ends, are filled one sample
    each through the padding map.  Every padding mode, the `pad` zeros, a
    shorter window, centring off; a signal shorter than one tile (both ends
    in one tile), and lengths that start the signals of a batch at several
    alignments mod 16 (odd lengths: the misaligned signals gather).  Forced
    5-frame tiles (ragged last tiles), both second-pass layouts: against the
    oracle, and bit for bit against the same call with every tile gathering."""
    _require_gpu()
    monkeypatch.setenv("FM_FORWARD", layout)
    monkeypatch.setenv("FM_TILE_FRAMES", "5")
    rng = np.random.default_rng(n_fft + hop)
    for L in (n_fft * 3 // 4 + 2, 9 * hop + 6, 4322, 4321):
        if dtype == "f32":
            x = rng.standard_normal((3, L)).astype(np.float32)
        else:
            x = rng.integers(-32768, 32768, size=(3, L)).astype(np.int16)
        for extra in (dict(pad_mode="reflect"), dict(pad_mode="constant"), dict(pad_mode="replicate"),
                      dict(pad_mode="circular"), dict(center=False), dict(pad=2),
                      dict(win_length=n_fft - n_fft // 5, pad_mode="constant")):
            if extra.get("center") is False and L < n_fft:
                continue
            targs = dict(sample_rate=16000, n_fft=n_fft, hop_length=hop, n_mels=40, **extra)
            what = f"edge copy {layout} {dtype} {n_fft}/{hop} L={L} {extra}"
            print(f"[case] {what}", flush=True)
            monkeypatch.setenv("FM_TILE_COPY", "1")
            got = run_gpu(x, **targs)
            assert_parity(got, oracle(x, **targs), what)
            monkeypatch.setenv("FM_TILE_COPY", "0")
            assert np.array_equal(got, run_gpu(x, **targs)), what + ": copy != gather"
