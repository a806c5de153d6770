"""Build and run a hardware probe:

  python -m activation_perturbation_estimator_amd.probes [valu|gemm] [--build-only]

valu: issue rates of the VALU instructions the estimator kernels use.
gemm: bf16 and fp16 MFMA rates, LDS read and LDS-load rates, and the fp16 G_W
inner loop.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROBES = {"valu": "valu_rates", "gemm": "gemm_rates"}


def build(name: str) -> str:
    out = os.path.join(ROOT, "_build", PROBES[name])
    os.makedirs(os.path.dirname(out), exist_ok=True)
    subprocess.check_call(["hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang",
                           "-target-feature", "-Xclang", "-packed-fp32-ops",
                           os.path.join(HERE, PROBES[name] + ".hip"), "-o", out],
                          stderr=subprocess.DEVNULL)
    return out


def main() -> int:
    names = [a for a in sys.argv[1:] if not a.startswith("--")] or ["valu"]
    for name in names:
        if name not in PROBES:
            print(f"unknown probe {name!r}; choose from {sorted(PROBES)}")
            return 2
        exe = build(name)
        if "--build-only" not in sys.argv:
            rc = subprocess.call([exe])
            if rc:
                return rc
    return 0


if __name__ == "__main__":
    sys.exit(main())
