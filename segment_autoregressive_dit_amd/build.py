"""Build libnomas.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Run as ``python -m segment_autoregressive_dit_amd.build`` or through
``__graft_entry__.build()``. The library lands next to this file.
"""

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnomas.so")
DEBUG_LIB = os.path.join(HERE, "libnomas_debug.so")   # the checking build (NOMAS_DEVICE_CHECKS)
SOURCES = ["nomas_host.cpp", "rope3d.hip", "kvcache_append.hip", "kvcache_archive.cpp", "attention.hip",
           "sparse_select.hip", "qkv_gemm.hip", "calibrate.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # IEEE float32 division and denormals: the INT8 quantiser is bit-exact only with them
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # no packed-fp32 VALU forms anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the library's host
# code (argument checks, planning, ring arithmetic, archive bookkeeping); the
# device code is built as usual. Load such a build with the ASan runtime
# preloaded (ASAN_RUNTIME below).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_RUNTIME = os.path.join(os.path.dirname(HIPCC), "..", "lib", "llvm", "lib", "clang", "22", "lib", "linux",
                            "libclang_rt.asan-x86_64.so")


def build(verbose=True, jobs=4, sanitize=False, out=None, checks=False):
    """Compile every source for gfx950 and link ``out`` (default: libnomas.so
    next to this file, or libnomas_debug.so with ``checks``). ``sanitize``: host
    code with ASan + UBSan. ``checks``: the kernels test every cache slot, token
    range and tile row they address (NOMAS_DEVICE_CHECKS; see
    nomas_device_check_failures)."""
    lib = out or (DEBUG_LIB if checks else LIB)
    extra = (SANITIZE_FLAGS if sanitize else []) + (["-DNOMAS_DEVICE_CHECKS"] if checks else [])
    with tempfile.TemporaryDirectory(prefix="nomas_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [HIPCC] + FLAGS + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = False
        for src, cmd, p in procs:
            out = p.communicate()[0].decode()
            out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
            if p.returncode != 0:
                failed = True
                sys.stderr.write(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}\n")
            elif verbose and out.strip():
                sys.stderr.write(out + "\n")
        if failed:
            raise RuntimeError("libnomas build failed")
        tmp_lib = lib + ".tmp"
        # every symbol must resolve at link time: a kernel whose host stub the
        # compiler did not emit fails here, not when the library is loaded
        link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
                      "-shared-libsan"] if sanitize else ["-Wl,-z,defs"]
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + link_extra + ["-o", tmp_lib] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("libnomas link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp_lib, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
