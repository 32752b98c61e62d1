"""Build the dpk HIP library (_dpk.so) in-tree for gfx950: one hipcc
compile per source (in parallel) into _build/, then one link."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_dpk.so")
SOURCES = ["runtime.hip", "skinny.hip", "gemv.hip", "attn_decode.hip", "attn_decode_mfma.hip", "misc.hip", "gemm.hip", "attn_prefill.hip", "decode_step.hip", "decode_step_kv8.hip", "sample.hip"]
BUILD = os.path.join(HERE, "_build")
# per-source additions: the int8 GEMV keeps its MFMA results in ordinary VGPRs
# (its block scales read each k-step's result, which from AGPRs costs a copy)
EXTRA = {"skinny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [["hipcc"] + FLAGS + EXTRA.get(s, []) + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = OUT + ".tmp%d" % os.getpid()
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
