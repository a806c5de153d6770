"""dust_head_estimate, dust_linear_estimate and dust_embedding_grad_noalloc under
HIP graph capture, and two estimates on two streams at once: the calls
only enqueue kernels on the caller's stream (no allocation, no host
synchronisation, no memset nodes), so a captured call replays to the same bits
as the eager call.  Each replay is checked, with unrelated eager work and
synchronisations between replays."""
import numpy as np
import pytest

from activation_perturbation_estimator_amd import synth
from util import need_gpu

pytestmark = pytest.mark.gpu


def _replay_matches(torch, call, outs, nrep=3):
    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call()
    for rep in range(nrep):
        for o in outs:
            o.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device="cuda") * 2.0  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager call"
        del scratch


def test_head_estimate_replays_bitwise():
    dust = need_gpu()
    import torch
    z, y, X = synth.head_inputs(512, 4096, 64, seed=31, bf16=True)
    z, y, X = z.cuda(), y.cuda(), X.cuda()
    g = torch.empty((512, 4096), device="cuda")
    G = torch.empty((4096, 64), device="cuda")
    ws = torch.empty(dust.head_workspace_size(512, 4096, 64, 16, 0.0), dtype=torch.uint8,
                     device="cuda")

    def call():
        dust.head_estimate(z, y, X, sigma=0.02, K=16, seed=3, seq_len=512, workspace=ws,
                           out=(g, G))
    _replay_matches(torch, call, [g, G])


def test_linear_estimate_replays_bitwise():
    dust = need_gpu()
    import torch
    T, d, N, K = 1024, 96, 256, 8
    rng = np.random.default_rng(32)
    X = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).cuda()
    c = torch.from_numpy(rng.standard_normal((K, T)).astype(np.float32)).cuda()
    g = torch.empty((T, N), device="cuda")
    G = torch.empty((N, d), device="cuda")
    ws = torch.empty(dust.linear_workspace_size(T, d, N, K, 0.9), dtype=torch.uint8,
                     device="cuda")

    def call():
        dust.linear_estimate(X, c, N=N, sigma=0.01, gamma=0.9, seed=5, seq_len=512,
                             workspace=ws, out=(g, G))
    _replay_matches(torch, call, [g, G])


def test_embedding_noalloc_replays_bitwise():
    """The allocation-free embedding call, which is for callers such as graph
    capture: its kernels use the library's fixed scratch and no memset, so each
    replay gives the eager call's bits (and the caller-workspace call's)."""
    dust = need_gpu()
    import torch
    T, N, vocab = 4096, 128, 1000
    rng = np.random.default_rng(33)
    ids = torch.from_numpy(synth.zipf_targets(rng, T, vocab)).cuda()
    g = torch.from_numpy(rng.standard_normal((T, N)).astype(np.float32)).cuda()
    G = torch.empty((vocab, N), device="cuda")

    def call():
        dust.embedding_grad_noalloc(ids, g, vocab, out=G)
    _replay_matches(torch, call, [G])
    assert torch.equal(G, dust.embedding_grad(ids, g, vocab))


def test_concurrent_streams_with_own_workspaces():
    """Two LM-head estimates enqueued on two streams at once, each with its own
    workspace and outputs, give the bits of the same calls made one after the
    other: the library keeps no state between calls."""
    dust = need_gpu()
    import torch
    args = [synth.head_inputs(384, 2048, 64, seed=40 + k, bf16=True) for k in range(2)]
    args = [tuple(a.cuda() for a in x) for x in args]
    outs = [(torch.empty((384, 2048), device="cuda"), torch.empty((2048, 64), device="cuda"))
            for _ in range(2)]
    wss = [torch.empty(dust.head_workspace_size(384, 2048, 64, 24, 0.0), dtype=torch.uint8,
                       device="cuda") for _ in range(2)]

    def call(k):
        z, y, X = args[k]
        dust.head_estimate(z, y, X, sigma=0.03, K=24, seed=7 + k, seq_len=384,
                           workspace=wss[k], out=outs[k])
    serial = []
    for k in range(2):
        call(k)
        torch.cuda.synchronize()
        serial.append([o.clone() for o in outs[k]])
    for o in outs:
        for t in o:
            t.fill_(float("nan"))
    streams = [torch.cuda.Stream() for _ in range(2)]
    torch.cuda.synchronize()
    for k in range(2):
        with torch.cuda.stream(streams[k]):
            call(k)
    torch.cuda.synchronize()
    for k in range(2):
        for got, ref in zip(outs[k], serial[k]):
            assert torch.equal(got, ref), f"stream {k} differs from the serial call"
