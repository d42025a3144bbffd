"""Build libosattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m online_softmax_attn_amd.build          # builds in-tree
    python online_softmax_attn_amd/build.py --verbose

The library is written next to this file so that it travels with the source tree.
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libosattn.so")
SOURCES = ["api.hip", "fwd_mfma.hip", "bwd_mfma.hip", "f32_kernels.hip", "splitkv.hip",
           "rowsoftmax.hip", "fwd_fp8.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=fast",
    "-munsafe-fp-atomics",
    # Packed fp32 VALU instructions stay off: plain fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=None, out: str = LIB, csrc: str = CSRC) -> str:
    srcs = [os.path.join(csrc, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix=".libosattn.", suffix=".so.tmp", dir=os.path.dirname(os.path.abspath(out)))
    os.close(fd)
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags or []) + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--extra", action="append", default=[])
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--csrc", default=CSRC)
    args = ap.parse_args()
    path = build(args.verbose, args.extra, args.out, args.csrc)
    print(path)
    sys.exit(0)
