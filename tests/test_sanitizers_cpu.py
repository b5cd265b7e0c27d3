"""CPU: the oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

oracle.c is rebuilt by gcc with -fsanitize=address,undefined (a UB report
fatal) and the oracle's own tests run against it with gcc's ASan runtime
preloaded.  moe_abi.hip -- argument validation, workspace layout and
ownership, launch sequencing -- is rebuilt with host-side ASan and UBSan
(device code untouched) and linked with the other objects of the regular
build; the C-ABI tests that need no GPU run against it with clang's ASan
runtime preloaded.  Each run first checks that the sanitized library and the
runtime are the ones loaded."""
import os
import subprocess
import sys

from tests.conftest import ROOT

SAN_DIR = os.path.join(ROOT, "_build", "san")
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run(args, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter is not instrumented
    r = subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    return out


def _loaded(module_code, names, env_extra):
    """The subprocess's mapped files include every name in `names`."""
    code = (f"{module_code}\n"
            "maps = open('/proc/self/maps').read()\n"
            f"missing = [n for n in {names!r} if n not in maps]\n"
            "assert not missing, missing\n")
    _run([sys.executable, "-c", code], env_extra)


def test_oracle_under_asan_ubsan():
    import oracle
    lib = oracle.build_sanitized(os.path.join(SAN_DIR, "liboracle_san.so"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = {"ORACLE_LIB": lib, "LD_PRELOAD": asan}
    _loaded("import oracle; oracle.lib()", ["liboracle_san.so", "libasan"], env)
    tests = ["tests/test_oracle_formats.py", "tests/test_oracle_forward.py", "tests/test_oracle_route.py",
             "tests/test_oracle_shared.py", "tests/test_oracle_router.py", "tests/test_oracle_h_stage.py"]
    out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests], env)
    assert " passed" in out


def test_host_code_under_asan_ubsan():
    from mxfp4_moe_expert_02_amd import build as hip_build
    if not all(os.path.exists(os.path.join(ROOT, "_build", os.path.basename(s) + ".o"))
               for s in hip_build.sources()):
        hip_build.build()
    lib = hip_build.build_host_sanitized()
    env = {"MOE_MXFP4_LIB": lib, "LD_PRELOAD": hip_build.asan_runtime()}
    _loaded("import mxfp4_moe_expert_02_amd as M; M.lib()", ["libmoe_mxfp4_san.so", "libclang_rt.asan"],
            env)
    out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_cpu.py"],
               env)
    assert " passed" in out
