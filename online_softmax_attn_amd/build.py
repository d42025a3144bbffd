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
    "-ffp-contract=fast",
    "-munsafe-fp-atomics",
    # Packed fp32 VALU instructions stay off: plain fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)


def build(verbose: bool = False, extra_flags=None, out: str = LIB, csrc: str = CSRC,
          jobs: int = 0) -> str:
    """Compile every source to an object (in parallel, `jobs` at a time: default the
    usable cores, at most 16), link them into one shared library and move it into
    place only once the link has succeeded."""
    from concurrent.futures import ThreadPoolExecutor

    jobs = jobs or max(1, min(16, len(os.sched_getaffinity(0)), len(SOURCES)))
    flags = HIPCC_FLAGS + list(extra_flags or [])
    outdir = os.path.dirname(os.path.abspath(out))
    with tempfile.TemporaryDirectory(prefix=".osattn-build.") as objdir:
        objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc()] + flags + ["-c", os.path.join(csrc, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        fd, tmp = tempfile.mkstemp(prefix=".libosattn.", suffix=".so.tmp", dir=outdir)
        os.close(fd)
        try:
            _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        except BaseException:
            os.unlink(tmp)
            raise
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
