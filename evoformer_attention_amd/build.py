"""Build libevoattn.so in-tree with hipcc for gfx950.

    python -m evoformer_attention_amd.build

Every HIP source is compiled with packed-fp32 instruction selection turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops; hipcc's host pass
warns that it does not know that feature, which is harmless) and with MFMA
accumulators in ordinary VGPRs (-mllvm -amdgpu-mfma-vgpr-form), which spares
the accumulator-register copies around every softmax element."""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libevoattn.so")
SOURCES = ["evo_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "tri_project.hip",
           "tri_module_bwd.hip", "tri_mul.hip", "transition.hip", "opm.hip",
           "transition_bwd.hip", "measure.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libevoattn)")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep matrix-core accumulators in VGPRs (no AGPR copies)
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
            "-Wno-unused-variable", "-Wno-unused-but-set-variable"]


def _compile(src, obj):
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + flags()
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return out


def build(verbose=False):
    """Compile every source and link libevoattn.so (always rebuilds)."""
    with tempfile.TemporaryDirectory() as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
            logs = list(ex.map(_compile, SOURCES, objs))
        if verbose:
            for s, l in zip(SOURCES, logs):
                if l.strip():
                    print(f"[{s}]\n{l}")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o",
               tmp_lib] + objs
        r = subprocess.run(cmd, stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
