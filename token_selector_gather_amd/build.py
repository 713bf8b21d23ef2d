"""Compile libsa.so (HIP, gfx950) in-tree with hipcc."""
import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libsa.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "attn.hip", "hisa.hip", "misa.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep hipcc from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file code generation options: the indexer keeps its MFMA results in plain VGPRs, which
# saves a copy per result element ahead of the ReLU / head-weighting arithmetic.
FILE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "misa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose=False, jobs=4):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [hipcc] + [f for f in FLAGS if f != "-shared"] + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(shlex.quote(c) for c in cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        errs = [l for l in text.splitlines() if "error" in l]
        if pr.returncode != 0:
            failed.append(src)
            sys.stderr.write(text)
        elif verbose and errs:
            sys.stderr.write(text)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    tmp = SO + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, SO)
    for o in objs:
        os.remove(o)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
