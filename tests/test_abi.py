"""The C ABI of libdust without a GPU: the library loads, exports every call
include/dust.h declares, and rejects bad arguments on the host before any HIP
call (so these run on a machine with no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from util import ROOT

HEADER = os.path.join(ROOT, "include", "dust.h")


def _lib():
    from activation_perturbation_estimator_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        subprocess.check_call(["python", "-m", "activation_perturbation_estimator_amd.build"],
                              cwd=ROOT)
    return L, L.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dust_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L, lib = _lib()
    names = _declared()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dust_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    # and the Python binding covers exactly the declared calls
    assert sorted(L.SIGNATURES) == names


def test_status_strings_and_version():
    L, lib = _lib()
    for code, name in ((0, "DUST_OK"), (1, "DUST_ERR_INVALID_ARG"), (2, "DUST_ERR_WORKSPACE"),
                       (3, "DUST_ERR_HIP"), (4, "DUST_ERR_UNSUPPORTED"), (5, "DUST_ERR_TARGETS")):
        assert L.status_string(code) == name
    assert "gfx950" in lib.dust_version().decode()


FAKE = 0x1000  # never dereferenced: every call below is rejected on the host


def _head(lib, **kw):
    a = dict(logits=FAKE, ldt=0, targets=FAKE, X=FAKE, xdt=0, T=256, V=512, d=64, L=128,
             sigma=0.05, K=16, gamma=0.0, seed=1, stream=0, g=FAKE, G=FAKE, losses=None,
             ws=FAKE, wsb=1 << 40, s=None, ev=None)
    a.update(kw)
    return lib.dust_head_estimate(a["logits"], a["ldt"], a["targets"], a["X"], a["xdt"], a["T"],
                                  a["V"], a["d"], a["L"], a["sigma"], a["K"], a["gamma"],
                                  a["seed"], a["stream"], a["g"], a["G"], a["losses"], a["ws"],
                                  a["wsb"], a["s"], a["ev"])


@pytest.mark.parametrize("bad", [
    dict(logits=None), dict(targets=None), dict(X=None), dict(g=None), dict(G=None),
    dict(ldt=7), dict(xdt=-1), dict(T=0), dict(T=-5), dict(V=0), dict(V=510), dict(V=65540),
    dict(d=0), dict(K=0), dict(K=-1), dict(L=0), dict(L=100), dict(sigma=0.0),
    dict(sigma=-1.0), dict(sigma=float("nan")), dict(sigma=float("inf")), dict(sigma=8.5),
    dict(gamma=-0.1), dict(gamma=1.5), dict(gamma=float("nan")),
])
def test_head_estimate_rejects(bad):
    L, lib = _lib()
    assert _head(lib, **bad) == L.DUST_ERR_INVALID_ARG


def test_head_estimate_workspace_checks():
    L, lib = _lib()
    need = lib.dust_head_workspace_size(256, 512, 64, 16, 0.0)
    assert need > 0
    assert _head(lib, ws=None) == L.DUST_ERR_WORKSPACE
    assert _head(lib, wsb=need - 1) == L.DUST_ERR_WORKSPACE
    # the non-fused path (gamma > 0) needs room for the [K,T] rewards
    assert (lib.dust_head_workspace_size(256, 512, 64, 16, 0.5)
            >= need + 16 * 256 * 4)


def test_linear_estimate_rejects():
    L, lib = _lib()
    def call(**kw):
        a = dict(X=FAKE, xdt=1, c=FAKE, T=4096, d_in=512, N=2048, L=2048, sigma=0.01, K=8,
                 gamma=0.9, seed=1, stream=0, draw0=0, K_total=8, g=FAKE, G=FAKE, ws=FAKE,
                 wsb=1 << 40)
        a.update(kw)
        return lib.dust_linear_estimate(a["X"], a["xdt"], a["c"], a["T"], a["d_in"], a["N"],
                                        a["L"], a["sigma"], a["K"], a["gamma"], a["seed"],
                                        a["stream"], a["draw0"], a["K_total"], a["g"], a["G"],
                                        a["ws"], a["wsb"], None, None)
    for bad in (dict(X=None), dict(c=None), dict(N=2046), dict(L=1000), dict(K=0),
                dict(gamma=2.0), dict(sigma=0.0), dict(d_in=0), dict(draw0=-1),
                dict(K_total=0), dict(draw0=(1 << 32) - 7)):
        assert call(**bad) == L.DUST_ERR_INVALID_ARG, bad
    assert call(wsb=16) == L.DUST_ERR_WORKSPACE


def test_stage_calls_reject():
    L, lib = _lib()
    E = L.DUST_ERR_INVALID_ARG
    assert lib.dust_noise(1, 0, 0, 4, 8, 6, FAKE, None) == E          # N % 4
    assert lib.dust_noise(1, 0, 0, 4, 8, 8, None, None) == E
    assert lib.dust_noise(1, 0, -1, 4, 8, 8, FAKE, None) == E
    assert lib.dust_philox4x32_10(1, None, FAKE, 5, None) == E
    assert lib.dust_philox4x32_10(1, FAKE, FAKE, -1, None) == E
    assert lib.dust_head_losses(FAKE, 0, FAKE, 8, 6, 0.1, 4, 1, 0, FAKE, None) == E
    assert lib.dust_head_losses(FAKE, 0, FAKE, 8, 8, 9.0, 4, 1, 0, FAKE, None) == E
    assert lib.dust_centre(None, 4, 8, FAKE, None) == E
    assert lib.dust_centre(FAKE, 0, 8, FAKE, None) == E
    assert lib.dust_reward_scan(FAKE, 4, 10, 3, 0.5, FAKE, None) == E  # T % L
    assert lib.dust_reward_scan(FAKE, 4, 12, 3, 1.5, FAKE, None) == E
    assert lib.dust_error_estimate(FAKE, 4, 8, 10, 0.1, 1, 0, 0, 4, FAKE, None) == E
    assert lib.dust_error_estimate(FAKE, 4, 8, 8, 0.1, 1, 0, -1, 4, FAKE, None) == E
    assert lib.dust_error_estimate(FAKE, 4, 8, 8, 0.1, 1, 0, 0, 0, FAKE, None) == E
    assert lib.dust_error_estimate(FAKE, 4, 8, 8, 0.1, 1, 0, (1 << 32) - 3, 4, FAKE, None) == E
    assert lib.dust_outer_sum(FAKE, FAKE, 0, 8, 0, 4, FAKE, FAKE, 1 << 30, None) == E
    assert lib.dust_outer_sum(FAKE, FAKE, 0, 8, 4, 4, FAKE, None, 0, None) == L.DUST_ERR_WORKSPACE
    assert lib.dust_check_targets(None, 8, 4, FAKE, None) == E


def test_workspace_sizes_are_host_only_and_sane():
    L, lib = _lib()
    # the paper-shape head: split-K partials of V x d fp32
    ws = lib.dust_head_workspace_size(16384, 4096, 512, 64, 0.0)
    assert ws >= 4096 * 512 * 4
    assert lib.dust_head_workspace_size(16384, 4096, 512, 64, 0.9) >= ws + 64 * 16384 * 4
    assert lib.dust_linear_workspace_size(16384, 512, 2048, 256, 0.9) >= 256 * 16384 * 4
    assert lib.dust_outer_sum_workspace_size(16, 8, 8) > 0


def test_size_limits_are_unsupported_not_invalid():
    """Shapes beyond the documented limits of the G_W-forming calls (T <= 2^22;
    N, d <= 2^20) are refused on the host with DUST_ERR_UNSUPPORTED."""
    L, lib = _lib()
    U = L.DUST_ERR_UNSUPPORTED
    assert _head(lib, T=(1 << 22) + 128, L=128) == U
    assert _head(lib, d=(1 << 20) + 1) == U
    assert lib.dust_outer_sum(FAKE, FAKE, 0, 8, (1 << 20) + 4, 4, FAKE, FAKE, 1 << 40, None) == U
    assert lib.dust_outer_sum(FAKE, FAKE, 0, 8, 4, (1 << 20) + 8, FAKE, FAKE, 1 << 40, None) == U
    assert lib.dust_linear_estimate(FAKE, 1, FAKE, 4096, (1 << 20) + 8, 2048, 2048, 0.01, 8,
                                    0.9, 1, 0, 0, 8, FAKE, FAKE, FAKE, 1 << 40, None, None) == U


def test_grid_and_overflow_limits():
    """Sizes whose launch grid would not fit a dispatch's 32-bit work-item count,
    or whose element counts would overflow a 64-bit product, are refused on the
    host (DUST_ERR_UNSUPPORTED) instead of reaching a kernel."""
    L, lib = _lib()
    U = L.DUST_ERR_UNSUPPORTED
    big = 1 << 24                                      # one workgroup per token: T < 2^24
    assert lib.dust_error_estimate(FAKE, 2, big, 4, 0.1, 1, 0, 0, 2, FAKE, None) == U
    assert lib.dust_head_losses(FAKE, 0, FAKE, big, 4, 0.1, 2, 1, 0, FAKE, None) == U
    assert lib.dust_centre(FAKE, 1, big, FAKE, None) == U
    assert lib.dust_ce_grad(FAKE, 0, FAKE, big, 4, FAKE, None) == U
    assert lib.dust_perturbed_linear(FAKE, FAKE, 1, big, 8, 8, 0.1, 1, 0, 0, 1, FAKE, None) == U
    # products that would overflow int64 if formed directly
    assert lib.dust_centre(FAKE, 1 << 40, 1 << 23, FAKE, None) == U
    assert lib.dust_reward_scan(FAKE, 1 << 62, 4, 4, 0.5, FAKE, None) == U
    assert lib.dust_ce_grad(FAKE, 0, FAKE, 8, 1 << 62, FAKE, None) == U
    assert lib.dust_noise(1, 0, 0, 1 << 32, 1 << 32, 4, FAKE, None) == U
    assert lib.dust_embedding_grad(FAKE, FAKE, 8, 1 << 60, 8, FAKE, FAKE, 1 << 40, None) == U
    # perturbed forward: more than 2^24 - 1 tiles of 128 x 128 outputs
    assert lib.dust_perturbed_linear(FAKE, FAKE, 1, 1 << 23, 8, 1 << 15, 0.1, 1, 0, 0, 1,
                                     FAKE, None) == U
    # outer product at widths whose tile grid alone exceeds 2^24 workgroups
    assert lib.dust_outer_sum(FAKE, FAKE, 1, 1024, 1 << 20, 1 << 20, FAKE, FAKE, 1 << 62,
                              None) == U


def test_embedding_noalloc_rejections_and_size():
    # host-side checks of the variant without a workspace: bad arguments, and
    # sizes whose scratch exceeds the library's fixed array, before any HIP call
    L, lib = _lib()
    cap = 16 << 20
    assert lib.dust_embedding_noalloc_bytes(16384, 512, 4096) < cap
    assert (lib.dust_embedding_noalloc_bytes(16384, 512, 4096) + 256 ==
            lib.dust_embedding_workspace_size(16384, 512, 4096))
    assert lib.dust_embedding_noalloc_bytes(1 << 20, 1024, 64) > cap
    assert lib.dust_embedding_noalloc_bytes(-1, 4, 4) == 0
    f = lib.dust_embedding_grad_noalloc
    assert f(FAKE, FAKE, 1 << 20, 1024, 64, FAKE, None) == L.DUST_ERR_UNSUPPORTED
    assert f(None, FAKE, 8, 4, 4, FAKE, None) == L.DUST_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 8, 6, 4, FAKE, None) == L.DUST_ERR_INVALID_ARG  # N % 4
    assert f(FAKE, FAKE, 8, 4, 0, FAKE, None) == L.DUST_ERR_INVALID_ARG
