"""Host-sanitized build of libmla: the C-ABI layer (api.cpp) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code, linked with
the kernel objects of the regular build. For running the host-only ABI tests
under the sanitizers (the GPU code is not instrumented).

    python -m head_latent_attention_14_amd.build_sanitized OUT_DIR

Load the result with MLA_LIBRARY=<OUT_DIR>/libmla_asan.so and the clang ASan
runtime (asan_runtime()) in LD_PRELOAD.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_mla_build", os.path.join(HERE, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def asan_runtime() -> str | None:
    """The clang ASan runtime of the ROCm toolchain, if present."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(out_dir: str) -> str:
    b = _build_module()
    objs = [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES if s != "api.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"regular build objects missing (run the regular build first): {missing}")
    os.makedirs(out_dir, exist_ok=True)
    api_o = os.path.join(out_dir, "api_asan.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f for f in b.COMMON if f != "-O3"] + ["-O1", "-g"]
    cmd = [b.HIPCC, "-x", "hip", *flags, *host_san, "-c", os.path.join(b.CSRC, "api.cpp"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stderr}")
    lib = os.path.join(out_dir, "libmla_asan.so")
    cmd = [b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", lib, api_o, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "_build", "asan")))
