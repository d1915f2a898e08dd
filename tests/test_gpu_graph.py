"""fm_forward and fm_backward inside a captured HIP graph.

Neither entry point allocates, synchronises or records a memset: each is one
kernel launch on the caller's stream, so a graph can hold it.  The test
captures a forward pass (float32 and int16 input) and a backward pass once,
then replays the graph with new signals copied into the captured buffers,
with eager launches and synchronisations between the replays, and requires
every replay to equal the eager result bit for bit (the kernels are
deterministic).  The first replay is also checked against the oracle.
"""
import numpy as np
import pytest

from oracle import mel_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TARGS = dict(sample_rate=16000, n_fft=400, hop_length=160, n_mels=80)
B, L = 2, 16000


def _signal(seed):
    rng = np.random.default_rng(seed)
    x = (0.1 * rng.standard_normal((B, L))
         + 0.3 * np.sin(2 * np.pi * (220.0 + 50 * seed) * np.arange(L) / 16000.0)).astype(np.float32)
    pcm = rng.integers(-32768, 32768, size=(B, L), dtype=np.int16)
    return x, pcm


def test_graph_replays_match_eager():
    from stft_mel_spectrogram_amd import MelSpectrogram
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mel = MelSpectrogram(**{k: v for k, v in TARGS.items()})
    T = mel.out_frames(L)
    dev = "cuda"
    xs = torch.zeros(B, L, device=dev)
    ps = torch.zeros(B, L, dtype=torch.int16, device=dev)
    us = torch.zeros(B, TARGS["n_mels"], T, device=dev)
    y = torch.empty(B, TARGS["n_mels"], T, device=dev)
    y16 = torch.empty_like(y)
    gx = torch.empty(B, L, device=dev)

    def step():
        mel(xs, out=y)
        mel(ps, out=y16)
        mel.backward(xs, us, out=gx)

    # warm-up launches on a side stream before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    for seed in range(4):
        print(f"[case] graph replay {seed}", flush=True)
        x, pcm = _signal(seed)
        u = rng.standard_normal((B, TARGS["n_mels"], T)).astype(np.float32)
        xs.copy_(torch.from_numpy(x))
        ps.copy_(torch.from_numpy(pcm))
        us.copy_(torch.from_numpy(u))
        graph.replay()
        torch.cuda.synchronize()
        # eager launches between the replays, on fresh buffers
        ey = mel(xs.clone())
        ey16 = mel(ps.clone())
        egx = mel.backward(xs.clone(), us.clone())
        torch.cuda.synchronize()
        assert torch.equal(y, ey), seed
        assert torch.equal(y16, ey16), seed
        assert torch.equal(gx, egx), seed
        if seed == 0:
            ref = O.mel_spectrogram(x, **TARGS)
            got = y.cpu().numpy().astype(np.float64)
            err = np.abs(got - ref) / (1.0 + np.abs(ref))
            assert err.max() <= 1e-4, err.max()
            ref16 = O.mel_spectrogram(pcm, **TARGS)
            err16 = np.abs(y16.cpu().numpy().astype(np.float64) - ref16) / (1.0 + np.abs(ref16))
            assert err16.max() <= 1e-4, err16.max()
