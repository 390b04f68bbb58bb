"""Build step for the attention oracle (test infrastructure).

Compiles ``attn_oracle.c`` with the host C compiler into
``liboracle_attn.so`` next to this file. Floating-point contraction and fast
math are off so that each double operation rounds as written.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "attn_oracle.c")
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-Wall", "-Wextra", "-Werror"]


def library_path() -> str:
    return os.path.join(HERE, "liboracle_attn.so")


def compile_source(source: str, out: str, extra: list[str] | None = None) -> str:
    """Compile one C source into a shared library at ``out``."""
    cc = os.environ.get("CC", "gcc")
    # a temporary name per process: concurrent builds (parallel test workers)
    # each replace the library atomically with a complete file
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [cc, *CFLAGS, *(extra or []), source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    return compile_source(SOURCE, library_path())


if __name__ == "__main__":
    print(build())
