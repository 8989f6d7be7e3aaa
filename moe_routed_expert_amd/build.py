"""Build libmoe_epi.so (the HIP library behind the C ABI) for gfx950, in-tree.

hipcc cross-compiles for gfx950 without a GPU. Flags:
  -ffp-contract=off      every fp32 operation is rounded on its own, in source
                         order; fused multiply-adds only where the source asks
                         for one (__fmaf_rn).
  -packed-fp32-ops off   the compiler may not form v_pk_{add,mul,fma}_f32.
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_epi.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    cmd = [HIPCC, *FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so: harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


def device_asm(source: str, out: str) -> str:
    """gfx950 assembly of one source, built with the library's own flags."""
    flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", f"-I{INCLUDE}", f"-I{CSRC}", source, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed:\n" + res.stdout + res.stderr)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
