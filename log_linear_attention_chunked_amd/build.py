"""Build the gfx950 shared library in-tree: ``libloglinear_attn.so`` next to this file.

    python -m log_linear_attention_chunked_amd.build [--debug] [-j N]

Each ``csrc/*.hip`` translation unit is compiled by ``hipcc --offload-arch=gfx950`` in
parallel, then linked with ``-shared``. Always recompiles (it is also the "does it build"
check). Packed-FP32 instruction selection is disabled for all device code
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does not know that
feature, which is expected.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libloglinear_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def common_flags(debug: bool) -> list[str]:
    flags = [
        f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]
    flags += ["-O1", "-g"] if debug else ["-O3"]
    return flags


def build(debug: bool = False, jobs: int | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    tmp = tempfile.mkdtemp(prefix="lla_build_")
    try:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *common_flags(debug), "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            if verbose:
                errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
                if errs:
                    print("\n".join(errs), file=sys.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(compile_one, srcs))
        out_tmp = LIB_PATH + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--debug", action="store_true", help="-O1 -g instead of -O3")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(debug=a.debug, jobs=a.jobs, verbose=a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
