"""Compile the C programs that drive libbeamstep.so through its C ABI alone
(no Python): plain C against include/beamstep.h and the HIP runtime API."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROGRAMS = ("table_9_5", "verify_and_resume")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> list:
    exes = []
    for name in PROGRAMS:
        src, exe = os.path.join(HERE, name + ".c"), os.path.join(HERE, name)
        cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
               "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), src,
               "-L", os.path.join(ROOT, "beam_search_step_amd"), "-lbeamstep",
               "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
               "-Wl,-rpath,$ORIGIN/../../beam_search_step_amd",
               "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(exe + ".tmp", exe)
        exes.append(exe)
    return exes


if __name__ == "__main__":
    print(build(verbose=True))
