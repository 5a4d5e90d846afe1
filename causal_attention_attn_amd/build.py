"""Build libattn.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m causal_attention_attn_amd.build           # libattn.so next to this file
    python -m causal_attention_attn_amd.build --asan    # also _build/libattn_asan.so

Every source compiles to its own object (in parallel), then one link makes the
shared library. The `asan` build is the same library with AddressSanitizer on
its host code only (the C ABI's validation and bookkeeping); its device code is
the ordinary gfx950 code. CPU tests load it through ATTN_LIBRARY with the
sanitizer runtime preloaded.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ASAN_LIB = os.path.join(BUILD_DIR, "libattn_asan.so")
SOURCES = ["api.hip", "rope_tables.hip", "fwd_16bit.hip", "bwd_prep.hip", "bwd_16bit.hip",
           "attn_f32.hip", "decode.hip", "layers.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off for every device pass; hipcc's host
# pass reports the feature as unknown, which is harmless.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-fno-honor-nans",
]
# host code only: each sanitizer flag goes to the host pass alone
ASAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()
_NOISE = "is not a recognized feature for this target"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)


def _build(out, objdir, extra, verbose):
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s.replace(".hip", ".o"))
        jobs.append((obj, [hipcc(), *FLAGS, *extra, *inc, "-c", os.path.join(CSRC, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra,
          *[obj for obj, _ in jobs], "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build(verbose=False, extra_flags=()):
    """Compile every HIP source into causal_attention_attn_amd/libattn.so (always rebuilds)."""
    return _build(LIB, os.path.join(BUILD_DIR, "obj"), list(extra_flags), verbose)


def build_asan(verbose=False):
    """The same library with AddressSanitizer on its host code, as _build/libattn_asan.so."""
    return _build(ASAN_LIB, os.path.join(BUILD_DIR, "obj_asan"), ASAN_FLAGS, verbose)


def asan_runtime():
    """Path of the AddressSanitizer runtime that matches hipcc's host compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found next to hipcc's clang")
    return path


if __name__ == "__main__":
    print(build(verbose=True))
    if "--asan" in sys.argv[1:]:
        print(build_asan(verbose=True))
    sys.exit(0)
