"""Host-sanitizer build of libdion3 (AddressSanitizer + UndefinedBehaviorSanitizer
on the host code only), for the CPU tests.

Each source is compiled twice: its device code alone (the same gfx950 code as
the regular build), then its host code with the sanitizers, embedding that
device binary.  The sanitizers instrument only host code (validation,
workspace planning, the step planner, launch set-up); the GPU code is the
regular one.  The result, _build_san/libdion3_san.so, needs the clang ASan
runtime preloaded (LD_PRELOAD) since Python itself is not instrumented.
Rebuilt only when a source, header or flag changed."""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess

from . import build as B

OUT_DIR = os.path.join(B.HERE, "_build_san")
LIB = os.path.join(OUT_DIR, "libdion3_san.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
BASE = [f for f in B.FLAGS if f != "--offload-arch=gfx950"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime matching hipcc's compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def _stamp() -> str:
    h = hashlib.sha256(" ".join(BASE + SAN).encode())
    inc = os.path.join(B.ROOT, "include")
    for d in (B.CSRC, inc):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _compile(src: str) -> str:
    name = os.path.basename(src)[:-4]
    fb = os.path.join(OUT_DIR, name + ".hipfb")
    obj = os.path.join(OUT_DIR, name + ".o")
    _run([B.HIPCC, "--offload-arch=gfx950", "--offload-device-only", *BASE, "-c", src, "-o", fb])
    _run([B.HIPCC, "--offload-arch=gfx950", "--offload-host-only", *BASE, *SAN,
          "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fb, "-c", src, "-o", obj])
    return obj


def build_sanitized() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    stamp_file = os.path.join(OUT_DIR, "stamp")
    stamp = _stamp()
    if os.path.exists(LIB) and os.path.exists(stamp_file) and open(stamp_file).read() == stamp:
        return LIB
    srcs = B.sources()
    with cf.ThreadPoolExecutor(min(len(srcs), max(1, min(8, os.cpu_count() or 1)))) as ex:
        objs = list(ex.map(_compile, srcs))
    _run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-shared-libsan", "-o", LIB, *objs])
    with open(stamp_file, "w") as fh:
        fh.write(stamp)
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
