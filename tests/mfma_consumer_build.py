"""Build the test-only scaled-MFMA consumer (``mfma_consumer.hip``) into
``tests/libmfma_consumer.so`` for gfx950.  It is a test instrument: the
library under test never links or loads it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_consumer.hip")
LIB = os.path.join(HERE, "libmfma_consumer.so")


def build() -> str:
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") \
        else "hipcc"
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(
        [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-shared", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", SRC, "-o", tmp],
        stderr=subprocess.DEVNULL if os.environ.get("QUIET_BUILD") else None)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
