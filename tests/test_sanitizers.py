"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only, no GPU code):

  - the oracle (oracle/hq_oracle.c) built with -fsanitize=address,undefined, under its pins;
  - the C-ABI layer (hq_api.cpp, hq_profile.cpp) built the same way, with stand-ins for the
    kernel launchers (tests/sanitize/launcher_stubs.cpp), under tests/test_abi.py: every call
    there fails its argument checks, or reaches the device check and fails there, so the
    checks themselves are what runs.

Each run is a pytest subprocess that preloads gcc's libasan and points the loaders at the
sanitized builds (HQ_ORACLE_LIB, HQ_LIB_PATH). A sanitizer report or a failing test fails
the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hadamard_rotated_precision_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _libasan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                           text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


LIBASAN = _libasan()
pytestmark = pytest.mark.skipif(LIBASAN is None, reason="gcc's libasan is not available")


def _run_pytest(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = LIBASAN
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    r = subprocess.run(cmd + args, cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, "sanitized run failed"
    for rep in REPORTS:
        assert rep not in out, rep


def test_oracle_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    lib = obuild.build(out=str(tmp_path / "libhq_oracle_san.so"), sanitize=True)
    pins = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_pins") and f.endswith(".py"))
    assert pins
    _run_pytest({"HQ_ORACLE_LIB": lib}, pins)


def test_abi_checks_under_sanitizers(tmp_path):
    objs = []
    for src in (os.path.join(CSRC, "hq_api.cpp"), os.path.join(CSRC, "hq_profile.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "launcher_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(["g++", "-std=c++17", "-w", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")] + SAN +
                       ["-c", src, "-o", obj], check=True)
        objs.append(obj)
    lib = str(tmp_path / "libhq_san.so")
    subprocess.run(["g++", "-shared"] + SAN + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-o", lib], check=True)
    _run_pytest({"HQ_LIB_PATH": lib}, [os.path.join("tests", "test_abi.py")])
