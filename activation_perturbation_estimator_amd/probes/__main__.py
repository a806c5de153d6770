"""Build and run the VALU issue-rate probe: python -m activation_perturbation_estimator_amd.probes"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))


def main() -> int:
    out = os.path.join(ROOT, "_build", "valu_rates")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    subprocess.check_call(["hipcc", "-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                           "-Xclang", "-packed-fp32-ops", os.path.join(HERE, "valu_rates.hip"),
                           "-o", out], stderr=subprocess.DEVNULL)
    if "--build-only" in sys.argv:
        return 0
    return subprocess.call([out])


if __name__ == "__main__":
    sys.exit(main())
