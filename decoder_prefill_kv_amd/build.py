"""Build the dpk HIP library (_dpk.so) in-tree for gfx950."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_dpk.so")
SOURCES = ["runtime.hip", "skinny.hip", "gemv.hip", "attn_decode.hip", "attn_decode_mfma.hip", "misc.hip", "gemm.hip", "attn_prefill.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["hipcc"] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
