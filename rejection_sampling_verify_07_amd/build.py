"""Build libspecverify.so in-tree with hipcc for gfx950."""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspecverify.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-DSPECVERIFY_BUILDING",
]


def hipcc_path() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the argument
# checks, plan and workspace layout (the device code is built as usual): each
# -fsanitize applies to the host compilation only.
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
]


def build(verbose: bool = False, out: str = LIB, defines=(), host_sanitize: bool = False) -> str:
    """Compile the HIP sources into rejection_sampling_verify_07_amd/libspecverify.so
    (or `out`, with extra -D defines, for tuning builds; host_sanitize: a host
    ASan/UBSan build for the CPU tests of the argument checks)."""
    src = os.path.join(CSRC, "specverify.hip")
    tmp = out + ".tmp"
    extra = HOST_SANITIZE_FLAGS if host_sanitize else []
    cmd = [hipcc_path(), *HIPCC_FLAGS, *extra, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
