"""Build step for the HIP library: hipcc for gfx950, in-tree, no JIT.

Produces scale_deformable_attention_amd/libmsda_amd.so from csrc/. The flags:
  --offload-arch=gfx950                       MI355X only
  -munsafe-fp-atomics                         fp32 / packed fp16 / bf16 adds lower
                                              to native no-return atomics, not
                                              compare-and-swap loops
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                              keep packed fp32 ALU ops out of the
                                              generated code
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmsda_amd.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(HERE, "csrc", "msda_kernels.hip"),
           os.path.join(HERE, "csrc", "msda_prep_kernels.hip"),
           os.path.join(HERE, "csrc", "msda_probe.hip"),
           os.path.join(HERE, "csrc", "msda_prereduce.hip"),
           os.path.join(HERE, "csrc", "msda_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "--offload-arch=gfx950",
                "-munsafe-fp-atomics", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, asm_dir: str = None) -> str:
    """Compile and link the library; optionally also write device assembly
    of the kernels to `asm_dir` (used to check which atomic forms are emitted)."""
    objs, procs = [], []
    for src in SOURCES:  # the sources compile in parallel
        obj = os.path.join(HERE, "csrc", os.path.basename(src) + ".o")
        cmd = [HIPCC, "-c", "-x", "hip", src, "-o", obj] + COMMON_FLAGS
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    for proc, cmd in procs:
        if proc.wait() != 0:
            raise subprocess.CalledProcessError(proc.returncode, cmd)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    for o in objs:
        os.remove(o)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        out = os.path.join(asm_dir, "msda_kernels-gfx950.s")
        cmd = [HIPCC, "-S", "-x", "hip", "--cuda-device-only", SOURCES[0], "-o", out] + COMMON_FLAGS
        subprocess.run(cmd, check=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
