"""Build the HIP library liblinattn.so in-tree for gfx950 (hipcc)."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblinattn.so")

# translation unit -> its own extra flags
SOURCES = {
    "la_api.hip": [],
    # the temporal-convolution GEMM keeps its MFMA accumulators in VGPRs
    "la_tconv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 (v_pk_*_f32) instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")


def build(verbose: bool = False, extra=()) -> str:
    """Compile every translation unit for gfx950 and link liblinattn.so."""
    import tempfile
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    with tempfile.TemporaryDirectory(prefix="la_build_") as tmp:
        objs = []
        for src, flags in SOURCES.items():
            obj = os.path.join(tmp, src + ".o")
            _run([hipcc, *FLAGS, *flags, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                  os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


# Host-side sanitizers: the host code (argument checks, planning and alias
# logic) compiled with AddressSanitizer and UndefinedBehaviorSanitizer, any UB
# report fatal; the device code is built as usual, without sanitizers.
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime to preload into a non-sanitized host process."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """Compile the library's host code with ASan + UBSan into `out` (CPU tests only)."""
    import tempfile
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    host_flags = [f for f in FLAGS if f != "-O3"]  # -O1 from SANITIZE
    with tempfile.TemporaryDirectory(prefix="la_san_") as tmp:
        objs = []
        for src, flags in SOURCES.items():
            obj = os.path.join(tmp, src + ".o")
            _run([hipcc, *host_flags, *flags, *SANITIZE, "-I", INCLUDE, "-I", CSRC, "-c",
                  os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", out], verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
