"""CPU oracle of the neuron-sparse FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it imports neither of them.

The arithmetic lives in ``oracle.c`` (plain single-threaded C, binary64
accumulation, ascending loop order); ``oracle.py`` marshals numpy arrays into
it and writes out the per-layer decode glue.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c to load instead (the sanitizer
# build of the CPU tests)
LIB = os.environ.get("ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, out: str = None, sanitize: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math) into liboracle.so, or with
    AddressSanitizer and UndefinedBehaviorSanitizer into `out`."""
    out = out or os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           *(SANITIZE_FLAGS if sanitize else []), SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


from .oracle import *  # noqa: E402,F401,F403
