"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc."""
import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCE = PKG / "csrc" / "specverify.hip"
LIBRARY = PKG / "libspecverify.so"
ARCH = os.environ.get("SPECV_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    # one rounding per written operation: no silent fma contraction, so every
    # kernel that evaluates the same expression gets the same bits
    "-ffp-contract=off",
    # no packed fp32 (v_pk_*_f32) instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build(verbose: bool = False, extra=()) -> Path:
    tmp = LIBRARY.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), *FLAGS, *extra, "-I", str(ROOT / "include"), "-I", str(PKG / "csrc"),
           str(SOURCE), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
