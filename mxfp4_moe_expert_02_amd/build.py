"""Build the HIP library libmoe_mxfp4.so in-tree for gfx950.

Each .hip source is compiled to an object with hipcc (in parallel), then
linked into one shared library next to this file.  Packed-fp32 VALU ops are
disabled for device code (``-target-feature -packed-fp32-ops``): the kernels
never need them and the flag keeps the compiler from forming them.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_mxfp4.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, bdir: str, extra: list) -> str:
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str | None = None, defines: dict | None = None,
          build_dir: str | None = None) -> str:
    """Compile every .hip source and link the shared library (default: the
    in-tree libmoe_mxfp4.so).  ``defines`` adds -D tuning constants."""
    bdir = build_dir or BUILD
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    extra = [f"-D{k}={v}" for k, v in (defines or {}).items()]
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, bdir, extra), srcs))
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if out is None:
        write_build_info()
    if verbose:
        print(f"built {lib}")
    return lib


BUILD_INFO = os.path.join(HERE, "_build_info.json")  # git-ignored, beside the library


def write_build_info() -> None:
    """Record the commit the in-tree library was built from (and whether
    the tree had uncommitted changes), for reports made where the tree has
    no .git."""
    import json
    info = {"git_sha": None, "dirty": None}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        if r.returncode == 0:
            info["git_sha"] = r.stdout.strip()
            d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
            info["dirty"] = bool(d.stdout.strip()) if d.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        pass
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


# host-side sanitizers (each flag after -Xarch_host, so device code is not
# instrumented): AddressSanitizer and UndefinedBehaviorSanitizer, a UB report
# fatal
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def build_host_sanitized(build_dir: str | None = None) -> str:
    """The library with moe_abi.hip -- argument validation, workspace layout
    and ownership, launch sequencing -- compiled with host AddressSanitizer
    and UBSan, linked with the other objects of the regular build (build()
    first).  Loaded with the compiler's ASan runtime preloaded
    (asan_runtime()).  Returns the path of the .so (under _build/san/)."""
    bdir = build_dir or BUILD
    sdir = os.path.join(bdir, "san")
    os.makedirs(sdir, exist_ok=True)
    abi = os.path.join(CSRC, "moe_abi.hip")
    obj = _compile(abi, sdir, SAN_FLAGS)
    others = [os.path.join(bdir, os.path.basename(s) + ".o") for s in sources() if s != abi]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: {missing}")
    lib = os.path.join(sdir, "libmoe_mxfp4_san.so")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", obj, *others, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return lib


def asan_runtime() -> str:
    """The shared ASan runtime of hipcc's clang (to LD_PRELOAD)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = hits[0] if hits else ""
    if not path:
        raise RuntimeError("clang's ASan runtime not found")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
