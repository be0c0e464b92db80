"""Compile the plain-C consumer of libtsel (``tsel_consumer.c``) next to this
file.  gcc, C99, -Wall -Wextra -Werror; it links libtsel.so and the HIP
runtime's C API (libamdhip64) and finds both through its rpath."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "tsel_consumer.c")
BIN = os.path.join(HERE, "tsel_consumer")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib_dir = os.path.join(ROOT, "attention_score_selection_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), SRC, "-o", BIN + ".tmp",
           "-L", lib_dir, "-ltsel", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../attention_score_selection_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"consumer build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
