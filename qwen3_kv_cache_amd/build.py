"""Compile the HIP library libqdec.so for gfx950, in-tree, with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqdec.so")
# diagnostic variant: the decode kernel records realtime-counter stamps at its
# phase boundaries (read back with qdec_debug_trace); never the product library
TRACE_LIB = os.path.join(HERE, "libqdec_trace.so")
SOURCES = ["qdec_api.cpp", "qdec_kernels.hip", "qdec_decode.hip", "qdec_encoder.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # keep the compiler from emitting packed fp32 math (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    log = (r.stdout + r.stderr).replace(
        "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)\n", "")
    if r.returncode != 0:
        sys.stderr.write(log)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    if verbose and log.strip():
        sys.stderr.write(log)
    os.replace(tmp, out)
    return out


def build_trace(verbose: bool = False) -> str:
    return build(verbose, TRACE_LIB, ("-DQDEC_TRACE",))


if __name__ == "__main__":
    print(build(verbose=True))
    if "--trace" in sys.argv[1:]:
        print(build_trace(verbose=True))
