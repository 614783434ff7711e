"""Build libgdn.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.hip", "gdn_intra.hip", "gdn_chunk.hip", "gdn_cp.hip", "gdn_recurrent.hip", "gdn_bwd.hip", "gdn_bwd_mma.hip"]
# Packed fp32 VALU ops are kept out of the generated code on purpose.  Matrix-core results stay in
# ordinary VGPRs (the recurrence reads and rescales them with vector ALU ops every chunk; the
# accumulation registers would cost a copy each way).
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            ]


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", src.replace(".hip", ".o"))
        cmd = ["hipcc", *HIPFLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        objs.append(obj)
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
