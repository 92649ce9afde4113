"""Compile libgr.so (the HIP kernels and the C ABI of include/gr.h) for gfx950, in place.

Usage: python -m continuous_quantized_decode_amd.build  (or build() from Python).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libgr.so")
SOURCES = ["api.hip", "gemm.hip", "attn.hip", "attn_decode.hip", "pack.hip", "dequant.hip", "sample.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the epilogue math reads them directly (no AGPR copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 5) -> str:
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_obj_" + src.replace(".hip", ".o"))
        cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print(out, file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", SO + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SO + ".tmp", SO)
    for o in objs:
        os.remove(o)
    return SO


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
