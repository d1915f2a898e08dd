"""CPU tests of the C ABI: exported symbols, host-plan tables against the
oracle's own constructions, argument validation and error codes.  No GPU
work is launched (host-only plans)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import mel_oracle as O
from stft_mel_spectrogram_amd import _native as N
from stft_mel_spectrogram_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "fm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"fm_plan_create", "fm_forward", "fm_backward", "fm_plan_destroy", "fm_out_frames",
            "fm_strerror", "fm_last_error", "fm_plan_tables"} <= set(names)
    lib = ctypes.CDLL(N.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fm.h but not exported"


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "stft_mel_spectrogram_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(dirpath, f), errors="ignore").read()
                assert not re.search(r"^\s*(from|import)\s+oracle", src, re.M), f
                assert "mel_oracle" not in src, f


def host_plan(cfg, **kw):
    args = dict(W.transform_args(cfg))
    args.update(kw)
    return N.Plan(device=False, **args)


@pytest.mark.parametrize("name", ["tiny", "whisper", "pow2", "large"])
def test_window_matches_oracle(name):
    cfg = W.WORKLOADS[name]
    t = host_plan(cfg).tables()
    ref = O.analysis_window(cfg["n_fft"], cfg["win_length"], False)
    np.testing.assert_allclose(t["window"], ref, rtol=1.2e-7, atol=1e-30)


@pytest.mark.parametrize("normalized", [True, "window", "frame_length"])
@pytest.mark.parametrize("win", [400, 320, 257])
def test_window_normalisation_matches_oracle(normalized, win):
    p = N.Plan(device=False, n_fft=400, win_length=win, hop_length=100, n_mels=40,
               normalized=normalized)
    np.testing.assert_allclose(p.tables()["window"], O.analysis_window(400, win, normalized),
                               rtol=1.2e-7, atol=1e-30)
    assert p.info().normalized == (2 if normalized == "frame_length" else 1)


def test_args_defaults_are_torchaudios():
    a = N.Args()
    assert N.lib.fm_args_default(ctypes.byref(a)) == N.FM_OK
    got = {f: getattr(a, f) for f, _ in N.Args._fields_}
    assert got == dict(sample_rate=16000, n_fft=400, win_length=400, hop_length=200, n_mels=128,
                       f_min=0.0, f_max=8000.0, power=2.0, center=1, pad_mode=0, mel_scale=0,
                       norm=0, pad=0, normalized=0, out_dtype=N.FM_F32)
    assert N.lib.fm_args_default(None) == N.FM_E_INVAL


@pytest.mark.parametrize("pad", [1, 7, 200, 5000])
def test_out_frames_with_zero_pad(pad):
    for L in (1, 150, 201, 1000, 48_000):
        for center in (True, False):
            p = N.Plan(device=False, n_fft=400, hop_length=160, n_mels=40, pad=pad, center=center,
                       pad_mode="constant")
            lp = L + 2 * pad
            if not center and lp < 400:
                with pytest.raises(N.FmError):
                    p.out_frames(L)
                continue
            assert p.out_frames(L) == O.frame_count(L, 400, 160, center=center, pad=pad), (L, pad)
    # reflect needs the zero-extended signal to exceed n_fft/2
    r = N.Plan(device=False, n_fft=400, hop_length=160, n_mels=40, pad=30)
    assert r.out_frames(141) == O.frame_count(141, 400, 160, center=True, pad=30)
    with pytest.raises(N.FmError):
        r.out_frames(140)


def test_raw_args_validation():
    a = N.Args()
    N.lib.fm_args_default(ctypes.byref(a))
    h = ctypes.c_void_p()
    for field, bad in (("pad", -1), ("pad", (1 << 28) + 1), ("normalized", 3), ("out_dtype", N.FM_I16),
                       ("out_dtype", 7)):
        b = N.Args.from_buffer_copy(a)
        setattr(b, field, bad)
        assert N.lib.fm_plan_create_args_host(ctypes.byref(h), ctypes.byref(b)) == N.FM_E_INVAL, field
    assert N.lib.fm_plan_create_args_host(ctypes.byref(h), None) == N.FM_E_INVAL
    assert N.lib.fm_plan_create_args_host(ctypes.byref(h), ctypes.byref(a)) == N.FM_OK
    N.lib.fm_plan_destroy(h)


def test_window_shorter_than_nfft_is_centred():
    p = N.Plan(device=False, sample_rate=16000, n_fft=400, win_length=300, hop_length=100, n_mels=40)
    np.testing.assert_allclose(p.tables()["window"], O.analysis_window(400, 300, False), rtol=1.2e-7, atol=1e-30)


@pytest.mark.parametrize("name", ["tiny", "whisper", "pow2", "large"])
@pytest.mark.parametrize("scale,norm", [("htk", None), ("slaney", "slaney"), ("htk", "slaney")])
def test_csr_filterbank_matches_oracle(name, scale, norm):
    cfg = W.WORKLOADS[name]
    p = host_plan(cfg, mel_scale=scale, norm=norm)
    t = p.tables()
    fb = O.mel_filterbank(cfg["n_fft"] // 2 + 1, cfg["f_min"], cfg["f_max"], cfg["n_mels"],
                          cfg["sample_rate"], norm, scale)
    dense = np.zeros_like(fb)
    for m in range(cfg["n_mels"]):
        a, ln, off = t["first"][m], t["len"][m], t["off"][m]
        dense[a:a + ln, m] = t["weights"][off:off + ln]
        support = np.nonzero(fb[:, m] > 0)[0]
        if ln == 0:
            assert len(support) == 0 or fb[support, m].max() < 1e-12
        else:
            assert t["weights"][off] > 0 and t["weights"][off + ln - 1] > 0
    np.testing.assert_allclose(dense, fb, rtol=1.2e-7, atol=1e-12)
    assert p.info().nnz == int(np.sum(t["len"]))


def test_csr_statistics_of_the_workloads():
    # nonzeros / widest filter / empty filters of the four distinct filterbanks
    expect = {"tiny": (393, 14, []), "whisper": (395, 9, [0, 3, 6, 13]),
              "pow2": (1005, 34, []), "large": (2022, 46, [])}
    for name, (nnz, wmax, empty) in expect.items():
        p = host_plan(W.WORKLOADS[name])
        inf = p.info()
        t = p.tables()
        assert (inf.nnz, inf.w_max) == (nnz, wmax), name
        assert [m for m in range(inf.n_mels) if t["len"][m] == 0] == empty, name


@pytest.mark.parametrize("name,over", [("tiny", {}), ("whisper", {}), ("pow2", {}), ("large", {}),
                                       ("large", dict(n_mels=8)), ("whisper", dict(n_mels=256)),
                                       ("tiny", dict(n_fft=64, win_length=64, hop_length=16, n_mels=40)),
                                       ("tiny", dict(n_fft=512, win_length=512, hop_length=128)),
                                       ("large", dict(n_fft=4096, win_length=4096, hop_length=1024)),
                                       ("whisper", dict(n_mels=37)),
                                       ("whisper", dict(mel_scale="slaney", norm="slaney"))])
def test_mel_blocks_equal_the_csr_filterbank(name, over):
    """The kernel's mel layout (blocks of up to 16 consecutive filters, dense
    4-bin steps in the matrix-core lane order, split over 4 waves) holds
    exactly the CSR weights, stays inside the bins, and covers every filter
    once: the blocks' filter ranges tile 0 .. n_mels - 1."""
    cfg = dict(W.WORKLOADS[name])
    cfg.update(over)
    p = host_plan(cfg)
    t = p.tables()
    blocks, wave_beg, wts = p.mel_blocks()
    K = cfg["n_fft"] // 2 + 1
    M = cfg["n_mels"]
    nb = len(blocks)
    assert nb >= (M + 15) // 16 and wave_beg[0] == 0 and wave_beg[4] == nb
    assert all(wave_beg[w] <= wave_beg[w + 1] for w in range(4))
    mel0s, nrows = blocks[:, 3] & 0xFFFF, blocks[:, 3] >> 16
    assert np.all((nrows >= 1) & (nrows <= 16))
    order = np.argsort(mel0s)
    assert mel0s[order][0] == 0 and np.array_equal(mel0s[order][1:], (mel0s + nrows)[order][:-1])
    assert (mel0s + nrows)[order][-1] == M
    dense = np.zeros((M, K))
    for kb, ks, off, fw in blocks:
        mel0, nrow = fw & 0xFFFF, fw >> 16
        assert ks % 4 == 0
        assert 0 <= kb and (kb + 4 * ks <= K or (kb == 0 and 4 * ks <= K + 15))
        for s_ in range(ks):
            for lane in range(64):
                m, k = mel0 + lane % 16, kb + 4 * s_ + lane // 16
                v = wts[off + 64 * s_ + lane]
                if lane % 16 >= nrow or m >= M or k >= K:
                    assert v == 0.0
                elif v != 0.0:
                    assert dense[m, k] == 0.0
                    dense[m, k] = v
    slack = 32 * 64 if K - 1 >= 2048 else 0     # large FFTs read weights from L2 in 32-step chunks
    assert len(wts) == 64 * blocks[:, 1].sum() + slack and len(wts) % 256 == 0
    assert np.all(wts[len(wts) - slack:] == 0.0)
    # a wave's blocks are consecutive in the table
    for w in range(4):
        for j in range(wave_beg[w], wave_beg[w + 1] - 1):
            assert blocks[j + 1, 2] == blocks[j, 2] + 64 * blocks[j, 1]
    csr = np.zeros((M, K))
    for m in range(M):
        a, ln, o = t["first"][m], t["len"][m], t["off"][m]
        csr[m, a:a + ln] = t["weights"][o:o + ln]
    assert np.array_equal(dense, csr)
    # the tile's LDS holds the power tile, its overrun and the weights
    inf = p.info()
    G = inf.tile_frames
    assert inf.lds_bytes >= 4 * (-(-(G * K + 16) // 4) * 4 + (len(wts) if not slack else 0))
    # the waves' shares of 4-bin steps are balanced to within one block
    cost = [sum(blocks[j, 1] + 2 for j in range(wave_beg[w], wave_beg[w + 1])) for w in range(4)]
    assert max(cost) - min(cost) <= max(blocks[:, 1]) + 2


@pytest.mark.parametrize("name,over", [("whisper", {}), ("tiny", {}), ("pow2", {}), ("large", {}),
                                       ("tiny", dict(n_fft=64, win_length=64, hop_length=16, n_mels=40)),
                                       ("whisper", dict(n_mels=37)),
                                       ("whisper", dict(mel_scale="slaney", norm="slaney"))])
def test_mel_quads_equal_the_csr_filterbank(name, over):
    """The vector-unit mel layout (quads of 4 consecutive filters, runs
    padded to the quad's longest, 4 weights per step) holds exactly the CSR
    weights; every padded run lies inside the frame's bins (the kernel reads
    no float outside a valid power row); each quad's length is its longest
    filter's run; the 8 shares tile the quads in order."""
    cfg = dict(W.WORKLOADS[name])
    cfg.update(over)
    p = host_plan(cfg)
    t = p.tables()
    hdr, share, w = p.mel_quads()
    K = cfg["n_fft"] // 2 + 1
    M = cfg["n_mels"]
    nq = (M + 3) // 4
    assert len(hdr) == nq
    assert share[0] == 0 and share[8] == nq and np.all(np.diff(share) >= 0)
    dense = np.zeros((M, K))
    for q, (s0, s1, s2, s3, L, off) in enumerate(hdr):
        lens = [t["len"][m] for m in range(4 * q, min(M, 4 * q + 4))]
        assert L == max(lens)
        for a, st in enumerate((s0, s1, s2, s3)):
            assert 0 <= st and st + L <= K
            for i in range(L):
                v = w[4 * (off + i) + a]
                m = 4 * q + a
                if m >= M:
                    assert v == 0.0
                elif v != 0.0:
                    assert dense[m, st + i] == 0.0
                    dense[m, st + i] = v
    assert len(w) == 4 * int(hdr[:, 4].sum())
    csr = np.zeros((M, K))
    for m in range(M):
        a, ln, o = t["first"][m], t["len"][m], t["off"][m]
        csr[m, a:a + ln] = t["weights"][o:o + ln]
    assert np.array_equal(dense, csr)


@pytest.mark.parametrize("n_fft", [64, 128, 256, 400, 512, 1024, 2048])
def test_mel_quad_runs_stay_in_the_row(n_fft):
    """For every n_mels 1..256 and f_max at or below Nyquist, every padded
    quad run starts at bin >= 0 and ends at the last bin at most: the vector
    units read only inside the rows of valid frames."""
    sr = 16000
    K = n_fft // 2 + 1
    for f_max in (sr / 2, 0.43 * sr):
        for n_mels in range(1, 257):
            p = N.Plan(device=False, sample_rate=sr, n_fft=n_fft, hop_length=n_fft // 4,
                       n_mels=n_mels, f_max=f_max)
            hdr, share, _ = p.mel_quads()
            assert len(hdr) == (n_mels + 3) // 4 and share[8] == len(hdr)
            assert np.all(hdr[:, :4] >= 0) and np.all(hdr[:, :4] + hdr[:, 4:5] <= K), (n_fft, n_mels, f_max)


# Floats the forward kernel zeroes after the last valid frame's power row
# (the mel stage may read that far past a row).
MEL_ROW_OVERRUN = 16


@pytest.mark.parametrize("n_fft", [64, 128, 256, 400, 512, 1024, 2048, 4096])
def test_mel_block_reads_stay_in_written_or_zeroed_floats(n_fft):
    """For every n_mels 1..256 and f_max at or below Nyquist: a block's bin
    run starts at bin >= 0 and ends at most MEL_ROW_OVERRUN - 1 floats past
    the frame's last bin, and every weight on a bin past the row is 0.  The
    kernel writes the power rows of the tile's valid frames and zeroes
    MEL_ROW_OVERRUN floats after the last valid one, so in any tile (ragged
    or full) the mel stage reads only written or zeroed floats, and what it
    reads past a row is multiplied by 0."""
    sr = 16000
    K = n_fft // 2 + 1
    worst = 0
    for f_max in (sr / 2, 0.43 * sr):
        for n_mels in range(1, 257):
            p = N.Plan(device=False, sample_rate=sr, n_fft=n_fft, hop_length=n_fft // 4,
                       n_mels=n_mels, f_max=f_max)
            blocks, _, wts = p.mel_blocks()
            for kb, ks, off, fw in blocks:
                assert kb >= 0
                end = kb + 4 * ks                       # one past the last bin read
                assert end - K < MEL_ROW_OVERRUN, (n_fft, n_mels, f_max, kb, ks)
                worst = max(worst, end - K)
                if end > K:
                    w = wts[off:off + 64 * ks].reshape(ks, 4, 16)   # [step, bin, filter]
                    bins = kb + 4 * np.arange(ks)[:, None] + np.arange(4)[None, :]
                    assert np.all(w[bins >= K] == 0.0), (n_fft, n_mels, f_max)
    if n_fft == 400:
        assert worst > 0          # this shape does read past its rows (few mels, f_max = sr/2)


@pytest.mark.parametrize("n_fft", [64, 128, 256, 400, 512, 1024, 2048, 4096, 8192, 16384])
def test_twiddles(n_fft):
    p = N.Plan(device=False, sample_rate=16000, n_fft=n_fft, hop_length=n_fft // 4, n_mels=40)
    t = p.tables()
    M = n_fft // 2
    j = np.arange(M)
    np.testing.assert_allclose(t["tw_m"], np.exp(-2j * np.pi * j / M), rtol=0, atol=6e-8)
    np.testing.assert_allclose(t["tw_n"], np.exp(-2j * np.pi * j / n_fft), rtol=0, atol=6e-8)
    inf = p.info()
    assert inf.fft_n1 * inf.fft_n2 * (inf.fft_n3 or 1) == M


@pytest.mark.parametrize("L", [201, 202, 1000, 16000, 480000, 220500])
def test_out_frames_closed_form(L):
    for n_fft, hop in ((64, 16), (256, 64), (400, 160), (512, 100), (1024, 256), (2048, 512),
                       (4096, 1024), (8192, 2048), (16384, 4096)):
        if L <= n_fft // 2:
            continue
        p = N.Plan(device=False, n_fft=n_fft, hop_length=hop, n_mels=40)
        assert p.out_frames(L) == O.frame_count(L, n_fft, hop, center=True)
        if L >= n_fft:
            q = N.Plan(device=False, n_fft=n_fft, hop_length=hop, n_mels=40, center=False)
            assert q.out_frames(L) == O.frame_count(L, n_fft, hop, center=False)


def test_geometry_fits_the_hardware():
    plans = [host_plan(W.WORKLOADS[name]) for name in ("tiny", "whisper", "pow2", "large")]
    plans += [N.Plan(device=False, n_fft=n, hop_length=n // 4, n_mels=m)
              for n in (64, 128, 256, 512, 4096) for m in (8, 128, 256)]
    for p in plans:
        inf = p.info()
        assert inf.lds_bytes <= 160 * 1024
        assert 1 <= inf.tile_frames <= 64
        assert inf.tile_frames * inf.fft_n1 // 2 <= inf.threads
        assert inf.fft_n1 * inf.fft_n2 == inf.n_fft // 2
        assert inf.has_device == 0


@pytest.mark.parametrize("n_fft,shape", [(8192, (16, 16, 16)), (16384, (16, 16, 32))])
def test_large_fft_geometry(n_fft, shape):
    """n_fft 8192 and 16384 take the three-pass kernel: n_fft/2 = a*c*d
    complex points, c*d threads (one pass-1 DFT each), one frame's exchange
    buffer (strides d+1 per c and c(d+1)+1 per a, complex) in LDS, which
    also holds the frame's power row."""
    for n_mels in (1, 128, 256):
        p = N.Plan(device=False, sample_rate=44100, n_fft=n_fft, hop_length=n_fft // 4,
                   n_mels=n_mels, f_max=22050.0)
        inf = p.info()
        a, c, d = shape
        assert (inf.fft_n1, inf.fft_n2, inf.fft_n3) == shape and a * c * d == n_fft // 2
        assert inf.forward_variant == N.FM_FWD_LARGE
        assert inf.threads == c * d and inf.threads % 64 == 0 and inf.threads <= 1024
        ybytes = a * (c * (d + 1) + 1) * 8                   # exchange buffer (complex)
        assert inf.lds_bytes == ybytes + 16 * (-(-inf.nnz // 4)) <= 160 * 1024   # + CSR weights
        assert ybytes >= 4 * (n_fft // 2 + 1)                 # the power row fits the buffer
        assert n_mels <= 256 and -(-256 // inf.threads) >= -(-n_mels // inf.threads)  # filters tid + threads r
        # the largest position the passes touch is inside the buffer
        assert ((a - 1) * (c * (d + 1) + 1) + (c - 1) * (d + 1) + d - 1) * 8 < ybytes
    # every bin position (ka, kc, kd) maps to a distinct buffer slot
    pos = {(ka * (c * (d + 1) + 1) + kc * (d + 1) + kd) for ka in range(a) for kc in range(c)
           for kd in range(d)}
    assert len(pos) == n_fft // 2


BAD = [
    (dict(n_fft=32768, hop_length=8192, f_max=8000.0), N.FM_E_UNSUPPORTED),
    (dict(n_fft=2000, hop_length=500), N.FM_E_UNSUPPORTED),
    (dict(n_fft=300), N.FM_E_UNSUPPORTED),
    (dict(n_mels=257), N.FM_E_UNSUPPORTED),
    (dict(f_min=8000.0, f_max=8000.0), N.FM_E_INVAL),
    (dict(f_max=8001.0), N.FM_E_INVAL),
    (dict(f_min=-1.0), N.FM_E_INVAL),
    (dict(hop_length=0), N.FM_E_INVAL),
    (dict(win_length=401), N.FM_E_INVAL),
    (dict(power=0.0), N.FM_E_INVAL),
    (dict(sample_rate=0), N.FM_E_INVAL),
    (dict(n_mels=0), N.FM_E_INVAL),
]


@pytest.mark.parametrize("kw,code", BAD)
def test_invalid_arguments(kw, code):
    args = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=80, f_max=8000.0)
    args.update(kw)
    with pytest.raises(N.FmError) as e:
        N.Plan(device=False, **args)
    assert e.value.status == code


def test_raw_enum_validation_and_null_handling():
    lib = N.lib
    h = ctypes.c_void_p()
    base = [16000, 400, 400, 160, 80, 0.0, 8000.0, 2.0]
    assert lib.fm_plan_create_host(ctypes.byref(h), *base, 1, 9, 0, 0) == N.FM_E_INVAL   # pad_mode
    assert lib.fm_plan_create_host(ctypes.byref(h), *base, 1, 0, 5, 0) == N.FM_E_INVAL   # mel_scale
    assert lib.fm_plan_create_host(ctypes.byref(h), *base, 1, 0, 0, 7) == N.FM_E_INVAL   # norm
    assert lib.fm_plan_create_host(ctypes.byref(h), *base, 2, 0, 0, 0) == N.FM_E_INVAL   # center
    assert lib.fm_plan_create_host(None, *base, 1, 0, 0, 0) == N.FM_E_INVAL
    assert lib.fm_plan_destroy(None) == N.FM_OK
    assert lib.fm_forward(None, None, 0, 1, 1000, None, None) == N.FM_E_INVAL
    assert lib.fm_backward(None, None, 1, 1000, None, None, None) == N.FM_E_INVAL
    assert lib.fm_out_frames(None, 100) == N.FM_E_INVAL
    assert b"NULL" in lib.fm_last_error()
    assert lib.fm_strerror(N.FM_E_UNSUPPORTED) == b"unsupported configuration"


def test_forward_on_host_plan_and_bad_lengths():
    p = N.Plan(device=False, n_fft=400, hop_length=160, n_mels=80)
    with pytest.raises(N.FmError) as e:
        p.forward_ptr(0, N.FM_F32, 1, 1000, 0)
    assert e.value.status == N.FM_E_NODEVICE
    with pytest.raises(N.FmError) as e:
        p.backward_ptr(0, 1, 1000, 0, 0)
    assert e.value.status == N.FM_E_NODEVICE
    with pytest.raises(N.FmError) as e:
        p.out_frames(200)          # reflect needs length > n_fft/2
    assert e.value.status == N.FM_E_INVAL
    assert p.out_frames(201) == 2
    q = N.Plan(device=False, n_fft=400, hop_length=160, n_mels=80, pad_mode="constant")
    assert q.out_frames(1) == 1     # zero padding has no length bound beyond one sample
    r = N.Plan(device=False, n_fft=400, hop_length=160, n_mels=80, center=False)
    with pytest.raises(N.FmError):
        r.out_frames(399)


def test_build_rejects_kernels_that_use_scratch():
    """The build fails on any kernel whose resource remarks report scratch
    (a launch of such a kernel costs about 20 us on the MI355X); the parser
    picks out exactly the kernels with a non-zero scratch size."""
    from stft_mel_spectrogram_amd.build import RESOURCE_FLAGS, scratch_users
    assert "-Rpass-analysis=kernel-resource-usage" in RESOURCE_FLAGS
    remarks = "\n".join([
        "k.hip:10:1: remark: Function Name: _Z4kern1v [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:10:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:20:1: remark: Function Name: _Z4kern2v [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:20:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:30:1: remark: Function Name: _Z4kern3v [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:30:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert scratch_users(remarks) == [("_Z4kern2v", 12), ("_Z4kern3v", 8)]
    assert scratch_users("") == []


def test_forward_variant_choice(monkeypatch):
    """n_fft 64 ... 2048 choose between the pair and the row layout per call
    unless FM_FORWARD=rows or split (n_fft 400 also paired) is set at plan
    creation; n_fft 4096 takes the pair layout; n_fft 8192 and 16384 always
    take the three-pass kernel."""
    monkeypatch.delenv("FM_FORWARD", raising=False)
    p = N.Plan(device=False, sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    assert p.info().forward_variant == N.FM_FWD_AUTO
    monkeypatch.setenv("FM_FORWARD", "paired")
    p = N.Plan(device=False, sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    assert p.info().forward_variant == N.FM_FWD_PAIRED
    p = N.Plan(device=False, sample_rate=16000, n_fft=512, hop_length=160, n_mels=80)
    assert p.info().forward_variant == N.FM_FWD_AUTO        # paired: not built for other sizes
    p = N.Plan(device=False, sample_rate=44100, n_fft=16384, hop_length=4096, n_mels=256,
               f_max=22050.0)
    assert p.info().forward_variant == N.FM_FWD_LARGE
    monkeypatch.delenv("FM_FORWARD")
    for n_fft in (64, 128, 256, 512, 1024, 2048):
        p = N.Plan(device=False, sample_rate=16000, n_fft=n_fft, hop_length=n_fft // 4, n_mels=40)
        assert p.info().forward_variant == N.FM_FWD_AUTO, n_fft
    p = N.Plan(device=False, sample_rate=16000, n_fft=4096, hop_length=1024, n_mels=80)
    assert p.info().forward_variant == N.FM_FWD_SPLIT
    monkeypatch.setenv("FM_FORWARD", "rows")
    p = N.Plan(device=False, sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    assert p.info().forward_variant == N.FM_FWD_ROWS and p.info().threads == 512
    for n_fft in (64, 128, 256, 512, 1024, 2048):   # the row layout is built up to n1 = 32
        p = N.Plan(device=False, sample_rate=16000, n_fft=n_fft, hop_length=n_fft // 4, n_mels=40)
        assert p.info().forward_variant == N.FM_FWD_ROWS and p.info().threads == 512, n_fft
    p = N.Plan(device=False, sample_rate=16000, n_fft=4096, hop_length=1024, n_mels=80)
    assert p.info().forward_variant == N.FM_FWD_SPLIT and p.info().threads == 256
    monkeypatch.setenv("FM_FORWARD", "split")
    p = N.Plan(device=False, sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    assert p.info().forward_variant == N.FM_FWD_SPLIT and p.info().threads == 256


def test_forward_config(monkeypatch):
    """The per-call choice: n_fft 400 and 2048 take the row layout for every
    call; the other sizes take it while its workgroups fit one per compute
    unit (a host-only plan assumes 256 compute units, one workgroup each);
    the workgroup count is batch x tiles per signal."""
    monkeypatch.delenv("FM_FORWARD", raising=False)
    monkeypatch.delenv("FM_TILE_FRAMES", raising=False)
    p = N.Plan(device=False, sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    assert p.info().forward_variant == N.FM_FWD_AUTO and p.info().threads == 256
    T = p.out_frames(480000)
    assert T == 3001
    v, g, wg = p.forward_config(1, 16000)           # fewer tiles than compute units
    assert v == N.FM_FWD_ROWS and g == 1 and wg == 101
    for batch in (1, 2, 3, 4, 5, 8, 16, 64):
        for L in (16000, 160000, 480000):
            v, g, wg = p.forward_config(batch, L)
            T = p.out_frames(L)
            assert v == N.FM_FWD_ROWS and wg == batch * -(-T // g) and 1 <= g <= p.info().tile_frames
    assert p.forward_config(0, 480000)[2] == 0
    with pytest.raises(N.FmError):
        p.forward_config(-1, 480000)
    monkeypatch.setenv("FM_FORWARD", "split")
    ps = N.Plan(device=False, sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    monkeypatch.setenv("FM_FORWARD", "rows")
    pr = N.Plan(device=False, sample_rate=16000, n_fft=400, hop_length=160, n_mels=128)
    for batch in (1, 4, 8):
        assert ps.forward_config(batch, 480000)[0] == N.FM_FWD_SPLIT
        assert pr.forward_config(batch, 480000)[0] == N.FM_FWD_ROWS
    monkeypatch.delenv("FM_FORWARD")
    # n_fft 2048, 256 and 512: always rows; the other sizes: rows while its
    # workgroups fit one per compute unit
    p2 = N.Plan(device=False, sample_rate=22050, n_fft=2048, hop_length=512, n_mels=128)
    for batch in (1, 64, 512):
        assert p2.forward_config(batch, 220500)[0] == N.FM_FWD_ROWS
    for n in (256, 512):
        pn = N.Plan(device=False, sample_rate=16000, n_fft=n, hop_length=n // 4, n_mels=40)
        for batch in (1, 8, 64):
            assert pn.forward_config(batch, 480000)[0] == N.FM_FWD_ROWS
    monkeypatch.setenv("FM_FORWARD", "rows")
    forced = {n: N.Plan(device=False, sample_rate=16000, n_fft=n, hop_length=n // 4, n_mels=40)
              for n in (64, 128, 1024)}
    monkeypatch.delenv("FM_FORWARD")
    for n, pf in forced.items():
        pa = N.Plan(device=False, sample_rate=16000, n_fft=n, hop_length=n // 4, n_mels=40)
        for batch, L in ((1, 16000), (1, 480000), (8, 480000), (16, 32768), (64, 32768)):
            v, g, wg = pa.forward_config(batch, L)
            _, gr, wgr = pf.forward_config(batch, L)
            assert (v == N.FM_FWD_ROWS) == (wgr <= 256), (n, batch, L, v, wgr)
            if v == N.FM_FWD_ROWS:
                assert (g, wg) == (gr, wgr)
    pl = N.Plan(device=False, sample_rate=44100, n_fft=16384, hop_length=4096, n_mels=256,
                f_max=22050.0)
    v, g, wg = pl.forward_config(16, 441000)
    assert v == N.FM_FWD_LARGE and wg == 16 * -(-pl.out_frames(441000) // g)


def test_n_fft_4096_three_pass_choice(monkeypatch):
    """n_fft 4096 keeps its two-pass kernel (and the backward) and takes the
    three-pass kernel in calls whose two-pass tiles outnumber the compute
    units, or as FM_FORWARD says."""
    monkeypatch.delenv("FM_FORWARD", raising=False)
    p = N.Plan(device=False, sample_rate=44100, n_fft=4096, hop_length=1024, n_mels=128)
    assert p.info().fft_n3 == 0 and p.info().fft_n1 == 64  # its own (two-pass) shape
    v1, g1, w1 = p.forward_config(1, 1323000)
    assert v1 == N.FM_FWD_SPLIT and w1 <= 256
    for batch in (4, 16):
        v, g, wg = p.forward_config(batch, 1323000)
        T = p.out_frames(1323000)
        assert v == N.FM_FWD_LARGE and wg == batch * -(-T // g)
        assert batch * -(-T // (g - 1)) > 256 if g > 1 else True  # fewest frames in one round
    # more filters than its 128 threads: two per thread
    wide = N.Plan(device=False, sample_rate=44100, n_fft=4096, hop_length=1024, n_mels=256)
    assert wide.forward_config(16, 1323000)[0] == N.FM_FWD_LARGE
    monkeypatch.setenv("FM_FORWARD", "split")
    ps = N.Plan(device=False, sample_rate=44100, n_fft=4096, hop_length=1024, n_mels=128)
    monkeypatch.setenv("FM_FORWARD", "large")
    pl = N.Plan(device=False, sample_rate=44100, n_fft=4096, hop_length=1024, n_mels=128)
    assert ps.forward_config(16, 1323000)[0] == N.FM_FWD_SPLIT
    assert pl.forward_config(1, 16000)[0] == N.FM_FWD_LARGE
    # other sizes never take it
    monkeypatch.delenv("FM_FORWARD")
    for n in (1024, 2048):
        pn = N.Plan(device=False, sample_rate=44100, n_fft=n, hop_length=n // 4, n_mels=128)
        assert pn.forward_config(64, 1323000)[0] != N.FM_FWD_LARGE
