"""Build the plain-C client of the C ABI (test infrastructure), in-tree.

gcc compiles it as C11 against include/bitdelta.h and the HIP runtime's C
header; it opens libbitdelta.so itself at run time (dlopen), so the binary
does not link the library.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "bd_client.c")
BINARY = os.path.join(HERE, "bd_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = BINARY + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=gnu11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), SOURCE, "-o", tmp,
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-ldl"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, BINARY)
    return BINARY


if __name__ == "__main__":
    print("built", build())
