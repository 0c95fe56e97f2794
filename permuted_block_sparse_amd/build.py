"""Build libsparse_attn.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "lib", "libsparse_attn.so")

SOURCES = ["plan_kernels.hip", "stop_kernels.hip", "topk_kernels.hip",
           "attn_kernel.hip", "sparse_attn.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (the code only uses scalar fp32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ArchVGPRs: the softmax reads S and rescales O with
    # VALU instructions, which cannot address AccVGPRs directly
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


# A build whose host code (argument checks, workspace layout, plan objects,
# launch set-up) runs under AddressSanitizer and UndefinedBehaviorSanitizer;
# the device code is built as usual. For CPU tests of the C ABI only: the
# process must preload the sanitizer runtime (sanitizer_runtime()).
SANITIZE_FLAGS = [
    "-O1", "-g",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def build(verbose: bool = False, out: str = LIB,
          sanitize: bool = False) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    flags = [f for f in FLAGS if not (sanitize and f == "-O3")]
    cmd = [hipcc(), *flags, *(SANITIZE_FLAGS if sanitize else []),
           "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (it also holds the undefined-
    behaviour handlers) that a process loading a sanitized build preloads."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..",
                         "lib", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/lib/llvm/bin/clang"):
        if os.path.exists(cand):
            res = subprocess.run([cand, "--print-resource-dir"],
                                 capture_output=True, text=True)
            path = os.path.join(res.stdout.strip(), "lib", "linux",
                                "libclang_rt.asan-x86_64.so")
            if res.returncode == 0 and os.path.exists(path):
                return path
    raise RuntimeError("clang's AddressSanitizer runtime not found")


if __name__ == "__main__":
    print(build(verbose=True))
