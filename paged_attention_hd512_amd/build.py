"""Builds libpa.so (host planner + gfx950 HIP kernels) in-tree with hipcc.

``python -m paged_attention_hd512_amd.build`` compiles every source each time it runs.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")

SOURCES = ["pa_host.cpp", "pa_decode.hip", "pa_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled: hipcc would otherwise form v_pk_* fp32 ops from
# ordinary float code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (device code is not
# instrumented): each -fsanitize= applies to the host compilation only.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
SANITIZED_DIR = os.path.join(BUILD_DIR, "sanitized")


def _compile(src, out_dir=BUILD_DIR, extra=()):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(PKG_DIR, "csrc", src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj, errs


def build(verbose=False, sanitize=False):
    """Builds libpa.so in the package (or, with sanitize, a host-sanitized copy under
    _build/sanitized/, for the CPU tests of the host code; load it with the ASan runtime
    preloaded and PA_LIBRARY pointing at it)."""
    out_dir = SANITIZED_DIR if sanitize else BUILD_DIR
    extra = SANITIZE_FLAGS if sanitize else []
    lib_path = os.path.join(SANITIZED_DIR, "libpa.so") if sanitize else LIB_PATH
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, out_dir, extra), SOURCES))
    if verbose:
        for _, msg in results:
            if msg.strip():
                print(msg)
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    if sanitize:
        cmd[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
