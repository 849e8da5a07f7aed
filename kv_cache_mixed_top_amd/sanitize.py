"""Build and run the host-side C-ABI checks under the host compiler's
AddressSanitizer and UndefinedBehaviorSanitizer.

    python -m kv_cache_mixed_top_amd.sanitize

Every library source is compiled as for the library (gfx950 code included,
so that the objects link as usual) with the sanitizers on the host side
only, and linked with sanitize/abi_host_check.cpp into
_build/san/abi_host_check, which is then run with no GPU visible: it drives
every entry point's argument checks, size queries and launch planning, and
each call that reaches a launch fails cleanly instead of touching a device.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from . import build as B

SAN_BUILD = os.path.join(B.BUILD, "san")
ROCM_INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(B.HIPCC))), "include")
EXE = os.path.join(SAN_BUILD, "abi_host_check")
DRIVER = os.path.join(B.HERE, "sanitize", "abi_host_check.cpp")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build_checker(verbose: bool = False) -> str:
    os.makedirs(SAN_BUILD, exist_ok=True)
    flags = [f for f in B.FLAGS if f not in ("-O3",)] + SAN_FLAGS
    jobs = []
    for src in B.SOURCES:
        obj = os.path.join(SAN_BUILD, src.replace(".hip", ".o"))
        jobs.append(([B.HIPCC, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj], obj))
    drv = os.path.join(SAN_BUILD, "abi_host_check.o")
    jobs.append(([B.HIPCC, "-std=c++17", *SAN_FLAGS, "-I", B.INCLUDE, "-I", ROCM_INCLUDE, "-x", "c++",
                  "-c", DRIVER, "-D__HIP_PLATFORM_AMD__", "-o", drv], drv))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda j: B._run(j[0], verbose), jobs))
    B._run([B.HIPCC, f"--offload-arch={B.ARCH}", *SAN_FLAGS, "-o", EXE, *[o for _, o in jobs]], verbose)
    return EXE


def run_checker() -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["HIP_VISIBLE_DEVICES"] = ""          # no device: nothing is ever launched
    env["ROCR_VISIBLE_DEVICES"] = ""
    env["ASAN_OPTIONS"] = "detect_leaks=0"   # the HIP runtime keeps allocations until exit
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return subprocess.run([EXE], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


if __name__ == "__main__":
    build_checker(verbose="-v" in sys.argv)
    p = run_checker()
    print(p.stdout, end="")
    sys.exit(p.returncode)
