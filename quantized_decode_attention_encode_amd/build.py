"""Builds libkvq.so (the C-ABI library with the gfx950 HIP kernels) in-tree with hipcc.

Usage:  python quantized_decode_attention_encode_amd/build.py   (or call build())
Run it by path: importing the package loads the library this script builds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-variable",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    f"-I{os.path.join(HERE, '..', 'include')}",
]
PER_FILE = {
    # bit-exact quantizer: one rounding per fp32 operation; no NaN inputs assumed (min / max
    # need no canonicalizing step and fuse with their DPP lane moves)
    "encode.hip": ["-ffp-contract=off", "-fno-honor-nans"],
    "decode.hip": [],
    "decode_sink.hip": [],
    "decode_skvq.hip": [],
    # no NaN inputs assumed: a max then needs no canonicalizing step and fuses with its DPP lane move
    "decode_mfma.hip": ["-fno-honor-nans"],
    # multi-query attend on the matrix cores
    "attend_tiles.hip": [],
    # Kitty encode (bit-exact quantizer) and decode
    "kitty.hip": ["-ffp-contract=off"],
    "kvq.cpp": ["-x", "hip"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as tmp:
        objs = []
        procs = []
        for src, extra in PER_FILE.items():
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, cmd, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # the host pass does not know the packed-fp32 target feature; that warning is expected
            lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
            if p.returncode != 0:
                failed.append((src, text))
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = os.path.join(tmp, "libkvq.so")
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        shutil.move(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    t = build(verbose="-v" in sys.argv)
    print("built", t)
