"""Run the CPU test tier (pytest -m "not gpu") against AddressSanitizer +
UndefinedBehaviorSanitizer builds of the host code: the planner and C ABI
(plan.cpp, api.cpp) and the C oracle (oracle/convt_oracle.c).

Host sources are compiled with gcc/g++ only (no .hip file on a sanitized
line); the kernel objects are the ordinary hipcc build, linked in unchanged so
the library still exports every entry point. The sanitized libraries go to
convt_forward_amd/_build/san/ and are selected through CONVT_LIB and
CONVT_ORACLE_LIB; gcc's ASan runtime is preloaded into the Python process.
Any sanitizer report aborts the run (non-zero exit).

    python tests/host_sanitizers.py [extra pytest args]
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from convt_forward_amd import build as hip_build  # noqa: E402

SAN_DIR = os.path.join(hip_build.BUILD_DIR, "san")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
HOST_SOURCES = ["plan.cpp", "api.cpp"]


def run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stderr)


def build_planner() -> str:
    """Sanitized host objects + the ordinary kernel objects -> libconvt_san.so."""
    hip_build.build()
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        run(["g++", "-std=c++17", "-O1", "-fPIC", "-Wall"] + SAN +
            ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + hip_build.INCLUDE, "-I" + hip_build.CSRC,
             "-c", os.path.join(hip_build.CSRC, src), "-o", obj])
        objs.append(obj)
    kernels = [os.path.join(hip_build.BUILD_DIR, os.path.splitext(s)[0] + ".o")
               for s in hip_build.SOURCES if s not in HOST_SOURCES]
    out = os.path.join(SAN_DIR, "libconvt_san.so")
    run(["g++", "-shared", "-fPIC"] + SAN + ["-o", out] + objs + kernels +
        ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    return out


def build_oracle() -> str:
    out = os.path.join(SAN_DIR, "libconvt_oracle_san.so")
    run(["gcc", "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall"] + SAN +
        ["-o", out, os.path.join(ROOT, "oracle", "convt_oracle.c"), "-lm"])
    return out


def main(argv) -> int:
    os.makedirs(SAN_DIR, exist_ok=True)
    lib = build_planner()
    olib = build_oracle()
    asan_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    env = dict(os.environ)
    env.update({
        "CONVT_LIB": lib,
        "CONVT_ORACLE_LIB": olib,
        "LD_PRELOAD": asan_rt,
        # the Python interpreter and torch keep allocations alive at exit
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    # the sanitized builds, not the in-tree ones, must be what the tests load
    probe = ("import convt_forward_amd as C, oracle; C.lib(); oracle.default(); "
             "m = open('/proc/self/maps').read(); "
             "assert 'libconvt_san.so' in m and 'libconvt_oracle_san.so' in m and 'libasan' in m, 'not sanitized'; "
             "assert '/libconvt.so' not in m and '/libconvt_oracle.so' not in m, 'in-tree library loaded'")
    subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, check=True)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q", "-m", "not gpu",
           "-p", "no:cacheprovider"] + list(argv)
    print("sanitized planner:", lib, "\nsanitized oracle:", olib, flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
