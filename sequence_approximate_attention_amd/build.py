"""Build libspava.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m sequence_approximate_attention_amd.build   (or build())
Every call recompiles all sources.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspava.so")
SOURCES = ["api.hip", "attn_bf16.hip", "score_bf16.hip", "attn_f32.hip", "score.hip", "aux.hip"]
ARCH = os.environ.get("SPAVA_ARCH", "gfx950")

# Packed-FP32 instructions are disabled for the device code: plain float math
# only (the flag is a device-side target feature; the host pass ignores it).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source device flags.  The attention kernel keeps every MFMA accumulator
# in the architectural VGPRs: with no AGPR use, two waves per SIMD get the
# whole 256-register budget as VGPRs instead of an even VGPR/AGPR split.
SOURCE_FLAGS = {"attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str, extra: list[str]) -> None:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
           os.path.join(CSRC, src), "-o", obj, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if l.strip() and noise not in l]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def _build_into(objdir: str, lib: str, extra: list[str], link_extra: list[str]) -> str:
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(SOURCES, objs)))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *link_extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every HIP source and link libspava.so; returns its path."""
    lib = _build_into(os.path.join(HERE, "_build"), LIB, list(extra or []), [])
    if verbose:
        print(f"built {lib}")
    return lib


# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
# argument checks, plan arithmetic and launch set-up behind the C ABI); the
# device code is built as usual.  The library then needs the shared ASan
# runtime loaded first (LD_PRELOAD of asan_runtime()).
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
HOST_SANITIZE_LINK = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -shared-libasan".split()


def build_host_sanitized(outdir: str) -> str:
    """Build the library with host-side sanitizers into outdir; returns its path."""
    return _build_into(os.path.join(outdir, "_build"), os.path.join(outdir, "libspava_host_sanitized.so"),
                       HOST_SANITIZE, HOST_SANITIZE_LINK)


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of hipcc's clang."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("the shared AddressSanitizer runtime of hipcc's clang was not found")


if __name__ == "__main__":
    build(verbose=True)
