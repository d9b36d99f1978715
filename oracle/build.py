"""Builds the CPU oracle (test infrastructure) as oracle/liblq_oracle.so.

Plain gcc, -O2, no fused multiply-add contraction, no fast-math, so every
fp32 codec operation is one IEEE-rounded operation.

build(sanitize=True) builds the same source with AddressSanitizer and
UndefinedBehaviorSanitizer (any report aborts) as oracle/liblq_oracle_san.so.
The Python front end loads it when LQ_ORACLE_LIB names it; the process must
then preload gcc's ASan and UBSan runtimes (sanitizer_runtime()).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lq_oracle.c")
LIB = os.path.join(HERE, "liblq_oracle.so")
LIB_SAN = os.path.join(HERE, "liblq_oracle_san.so")

_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", *(_SAN_FLAGS if sanitize else []), "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitizer_runtime() -> str:
    """LD_PRELOAD value for a process that loads liblq_oracle_san.so."""
    libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                           check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    return ":".join(libs)


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
