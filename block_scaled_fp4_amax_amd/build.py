"""Build libfp4q.so (HIP kernels for gfx950 + the C-ABI host layer) in-tree.

Flags that matter for bit-exactness: -ffp-contract=off (no FMA contraction),
no fast-math, fp32 denormals kept, correctly rounded fp32 division; packed
fp32 instructions are disabled.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4q.so")
ARCH = os.environ.get("FP4Q_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(force: bool = True, verbose: bool = False) -> str:
    srcs = sources()
    deps = srcs + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(HERE, "..", "include", "fp4q.h")]
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(d) for d in deps):
        return LIB
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode().splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, text))
        if verbose and text.strip():
            print(text)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


# ---------------------------------------------------------------- sanitizer builds (host code)
# The host layer (validation, staging plans, the scratch lookup) is built with
# a sanitizer on its host side and linked with the kernels' objects of the
# normal build: "ubsan" gives libfp4q_ubsan.so, which the binding loads when
# FP4Q_SANITIZE=1 (UBSan's runtime needs no preloading into Python); "asan"
# gives an executable from a C++ driver (ASan's runtime must be in the
# executable).  Device code is never built with a sanitizer.
HOST_SOURCES = ("fp4q_api.cpp", "fp4q_noalloc.hip")
LIB_UBSAN = os.path.join(HERE, "libfp4q_ubsan.so")


def _clang_rt_dir():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.ubsan_standalone-x86_64.so")
    if not hits:
        raise RuntimeError("no clang sanitizer runtime under /opt/rocm/llvm")
    return os.path.dirname(hits[0])


def build_sanitized(kind: str, driver: str = None, out: str = None) -> str:
    """kind "ubsan": libfp4q_ubsan.so; kind "asan": the executable `out` built
    from `driver` (a C++ source calling the C ABI)."""
    build(force=False)
    objdir = os.path.join(HERE, "_build")
    san = ["-Xarch_host", "-fsanitize=undefined" if kind == "ubsan" else "-fsanitize=address,undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    if kind == "ubsan":
        san += ["-Xarch_host", "-shared-libsan"]
    objs, procs = [], []
    for src in sources():
        base = os.path.basename(src)
        if base in HOST_SOURCES:
            obj = os.path.join(objdir, base + "." + kind + ".o")
            procs.append((src, subprocess.Popen([HIPCC, *FLAGS, *san, "-g", "-c", src, "-o", obj],
                                                stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        else:
            obj = os.path.join(objdir, base + ".o")
        objs.append(obj)
    if kind == "asan":
        obj = os.path.join(objdir, os.path.basename(driver) + ".asan.o")
        procs.append((driver, subprocess.Popen([HIPCC, *FLAGS, *san, "-g", "-c", driver, "-o", obj],
                                               stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    for src, p in procs:
        text = p.communicate()[0].decode()
        if p.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, text))
    rt = _clang_rt_dir()
    if kind == "ubsan":
        target = LIB_UBSAN
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-shared-libsan", "-Wl,-rpath," + rt, *objs, "-o", target + ".tmp"]
    else:
        target = out
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-Xarch_host", "-fsanitize=address,undefined", *objs, "-o",
               target + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(target + ".tmp", target)
    return target


if __name__ == "__main__":
    if "--ubsan" in sys.argv:
        print(build_sanitized("ubsan"))
    else:
        print(build(force="--lazy" not in sys.argv, verbose="-v" in sys.argv))
