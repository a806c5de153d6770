"""Shared test helpers (comparison metrics, GPU gating, cross-check builds)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "pins")
PIN_BUILD = os.path.join(ROOT, "_build", "pins")


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def cosine(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# Parity bar on g_hat and G_W: relative L2 <= 1e-3 and cosine >= 0.99999,
# fp32 accumulation on the GPU against the fp64 oracle.
REL_L2_MAX = 1e-3
COS_MIN = 0.99999


def assert_parity(gpu, ref, what: str, rel=REL_L2_MAX, cos=COS_MIN):
    r = rel_l2(gpu, ref)
    c = cosine(gpu, ref)
    assert r <= rel and c >= cos, f"{what}: rel_l2={r:.3e} cos={c:.8f}"


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import activation_perturbation_estimator_amd as dust
    dust._lib.load()  # a missing library must fail, not skip
    return dust


def pin_lib(name: str, compiler: list, extra: list):
    """Build (once) and load a test-only cross-check library from tests/pins."""
    os.makedirs(PIN_BUILD, exist_ok=True)
    src = os.path.join(PINS, name + ".cpp")
    so = os.path.join(PIN_BUILD, "lib" + name + ".so")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        tmp = so + ".tmp%d" % os.getpid()
        subprocess.check_call(compiler + ["-O2", "-std=c++17", "-shared", "-fPIC", *extra, src,
                                          "-o", tmp], stderr=subprocess.DEVNULL)
        os.replace(tmp, so)
    return ctypes.CDLL(so)
