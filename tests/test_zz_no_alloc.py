"""dust_embedding_grad_noalloc (the embedding estimate with the library's own
fixed scratch, for callers that cannot allocate) through the C ABI: bitwise the
same result as dust_embedding_grad with a caller workspace, on two calls in a
row with the second smaller (the shared scratch keeps the first call's
contents), plus the oracle's parity bar and the size limit."""
import ctypes

import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import assert_parity, need_gpu

pytestmark = pytest.mark.gpu


def _inputs(T, N, vocab, seed):
    import torch
    rng = np.random.default_rng(seed)
    ids = synth.zipf_targets(rng, T, vocab).astype(np.int32)
    ids[::97] = vocab + 3  # out-of-range ids are skipped
    g = rng.standard_normal((T, N)).astype(np.float32)
    return torch.from_numpy(ids).cuda(), torch.from_numpy(g).cuda(), ids, g


def _noalloc(lib, ids, g, vocab, out):
    import torch
    T, N = g.shape
    st = lib.dust_embedding_grad_noalloc(ids.data_ptr(), g.data_ptr(), T, N, vocab,
                                         out.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


def test_noalloc_matches_workspace_call_twice():
    dust = need_gpu()
    import torch
    lib = dust._lib.load()
    for (T, N, vocab, seed) in ((16384, 512, 4096, 5), (3001, 264, 700, 6)):
        print(f"[no_alloc] T={T} N={N} vocab={vocab}", flush=True)
        assert lib.dust_embedding_noalloc_bytes(T, N, vocab) <= dust.DUST_EMBEDDING_NOALLOC_BYTES
        ids, g, ids_h, g_h = _inputs(T, N, vocab, seed)
        ref_ws = dust.embedding_grad(ids, g, vocab)
        out = torch.full((vocab, N), float("nan"), device="cuda")
        assert _noalloc(lib, ids, g, vocab, out) == 0
        assert torch.equal(out, ref_ws), "differs from dust_embedding_grad"
        assert_parity(out.cpu().numpy(), oracle.embedding_grad(ids_h, g_h, vocab), "G_E")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    dust = need_gpu()
    import torch
    lib = dust._lib.load()
    T, N, vocab = 1 << 20, 1024, 64
    assert lib.dust_embedding_noalloc_bytes(T, N, vocab) > dust.DUST_EMBEDDING_NOALLOC_BYTES
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    g = torch.zeros((1, N), device="cuda")  # never read: the call is rejected first
    out = torch.zeros((vocab, N), device="cuda")
    st = lib.dust_embedding_grad_noalloc(ids.data_ptr(), g.data_ptr(), T, N, vocab,
                                         out.data_ptr(), None)
    assert st == dust._lib.DUST_ERR_UNSUPPORTED
