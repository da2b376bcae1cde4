"""Builds libspecverify.so for gfx950 with hipcc (in place, next to this file),
and libspecverify_t128.so, the same sources with 128-thread workgroups (a
test build: its results must equal the 256-thread library's).

    python -m lossless_token_verification_amd.build
"""

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OUT = os.path.join(HERE, "libspecverify.so")
OUT_T128 = os.path.join(HERE, "libspecverify_t128.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # no packed-fp32 instructions anywhere (only plain fp32 VALU)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _cmd(out, extra):
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    return [HIPCC, *FLAGS, *extra, "-I" + os.path.join(ROOT, "include"),
            "-I" + os.path.join(HERE, "csrc"), *srcs, "-o", out + ".tmp"]


def build(verbose=False):
    """Compiles both libraries (two hipcc processes side by side); returns the
    path of the product library."""
    jobs = [(OUT, []), (OUT_T128, ["-DSV_THREADS=128"])]
    procs = []
    for out, extra in jobs:
        cmd = _cmd(out, extra)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
    errors = []
    for (out, _), p in zip(jobs, procs):
        text, _ = p.communicate()
        msgs = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            errors.append(f"hipcc failed for {os.path.basename(out)}:\n" + "\n".join(msgs))
        elif verbose and msgs:
            print("\n".join(msgs))
    if errors:
        raise RuntimeError("\n".join(errors))
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
