"""The C ABI from plain C: tests/c_abi/head_consumer.c (built by build() with
gcc, linked against libdust.so and the HIP runtime, no C++, no torch) allocates
device memory itself, calls dust_head_estimate and writes g_hat and G_W; the
results are held to the same bar as the Python binding's against the oracle."""
import os
import struct
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from activation_perturbation_estimator_amd import synth
from util import (G_HAT_TERM_TOL, assert_elementwise, assert_gw, assert_parity, assert_rows,
                  need_gpu)

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "_build", "head_consumer")


@pytest.mark.parametrize("bf16", [False, True])
def test_c_consumer_head_estimate(bf16):
    dust = need_gpu()
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: __graft_entry__.build() compiles it")
    T, V, d, L, K, sigma, seed, stream = 192, 1000, 40, 64, 12, 0.05, 77, 3
    gamma = 0.0 if bf16 else 0.5  # the fused kernel and the staged path
    z, y, X = synth.head_inputs(T, V, d, seed=21, bf16=bf16)
    zdt = dust.DUST_BF16 if bf16 else dust.DUST_F32

    def raw(t):  # the tensor's bytes: fp32, or the bf16 bit patterns
        import torch
        return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).numpy().tobytes()

    with tempfile.TemporaryDirectory() as tmp:
        fin, fout = os.path.join(tmp, "in.bin"), os.path.join(tmp, "out.bin")
        with open(fin, "wb") as f:
            f.write(struct.pack("<5q2fQI2i", T, V, d, L, K, sigma, gamma, seed, stream, zdt, zdt))
            f.write(raw(z))
            f.write(y.numpy().astype(np.int32).tobytes())
            f.write(raw(X))
        res = subprocess.run([EXE, fin, fout], capture_output=True, text=True, timeout=120)
        assert res.returncode == 0, res.stdout + res.stderr
        out = np.fromfile(fout, dtype=np.float32)
    g, G = out[:T * V].reshape(T, V), out[T * V:].reshape(V, d)
    rg, rG, diag = oracle.head_estimate(synth.to_f64(z), y.numpy(), synth.to_f64(X), L, sigma, K,
                                        gamma, seed, stream, diagnostics=True)
    assert_parity(g, rg, "g_hat")
    assert_rows(g, rg, "g_hat rows")
    assert_elementwise(g, rg, diag["g_scale"], "g_hat elements", G_HAT_TERM_TOL)
    assert_parity(G, rG, "G_W")
    assert_gw(G, rg, synth.to_f64(X))
