"""The seeded synthetic inputs: shapes of the pages' workloads (tests/golden/
pages_facts.json, each fact cited there), determinism and the stated recipes."""
import json
import os

import numpy as np
import torch

from activation_perturbation_estimator_amd import synth

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def test_paper_workloads_match_the_pages():
    batch = FACTS["batch_sequences"]["value"] * FACTS["sequence_length"]["value"]
    assert batch == FACTS["batch_tokens"]["value"]
    lo, hi = FACTS["population_sweep_draws"]["value"]
    for name in ("paper", "k1024", "k16384"):
        w = synth.WORKLOADS[name]
        assert (w.T, w.seq_len, w.V, w.d) == (batch, FACTS["sequence_length"]["value"],
                                              FACTS["vocabulary"]["value"], FACTS["width"]["value"])
        assert lo <= w.K <= hi and w.gamma == 0.0 and w.bf16
    assert synth.WORKLOADS["k16384"].K == FACTS["public_code_default_population"]["value"]
    lin = synth.WORKLOADS["linear"]
    assert (lin.T, lin.seq_len, lin.d, lin.V) == (batch, 2048, 512, 4 * 512)


def test_inputs_are_seeded_and_shaped():
    a = synth.head_inputs(64, 128, 16, seed=3, bf16=True, zipf=True, logit_var=2.0,
                          target_boost=3.0)
    b = synth.head_inputs(64, 128, 16, seed=3, bf16=True, zipf=True, logit_var=2.0,
                          target_boost=3.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    z, t, X = a
    assert z.dtype == torch.bfloat16 and X.dtype == torch.bfloat16 and t.dtype == torch.int32
    assert z.shape == (64, 128) and X.shape == (64, 16) and t.shape == (64,)
    assert int(t.min()) >= 0 and int(t.max()) < 128


def test_zipf_targets():
    rng = np.random.default_rng(0)
    y = synth.zipf_targets(rng, 200_000, 4096)
    counts = np.bincount(y, minlength=4096)
    assert counts[0] == counts.max()
    # P(k) ~ (k+1)^-1.1: the ratio of the first two frequencies is 2^1.1
    assert abs(counts[0] / counts[1] - 2 ** 1.1) < 0.1


def test_target_boost_and_variance():
    z, y, X = synth.head_inputs(2048, 256, 64, seed=1, zipf=True, logit_var=2.0,
                                target_boost=3.0)
    zz = z.double().numpy()
    tgt = zz[np.arange(2048), y.numpy()]
    mask = np.ones_like(zz, bool)
    mask[np.arange(2048), y.numpy()] = False
    assert abs(zz[mask].var() - 2.0) < 0.05
    assert abs(tgt.mean() - 3.0) < 0.15
    assert abs(X.double().var().item() - 1.0 / 64) < 0.002


def test_linear_inputs():
    X, c = synth.linear_inputs(512, 64, 32, seed=1, c_seed=7, bf16=True)
    assert X.dtype == torch.bfloat16 and c.dtype == torch.float32 and c.shape == (32, 512)
    assert abs(c.double().var().item() - 1e-3) < 1e-4
