"""Build libmla_decode.so for gfx950 in-tree with hipcc.

    python -m mla_latent_kv_fwd_amd.build [--isa DIR]

Every HIP source under csrc/ is compiled for gfx950 only and linked into
mla_latent_kv_fwd_amd/libmla_decode.so.  Packed-FP32 instruction selection is
switched off (-packed-fp32-ops).  --isa DIR keeps the generated assembly.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, obj: str, isa_dir: str | None) -> None:
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    if isa_dir:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, cwd=os.path.dirname(obj), capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)


def build(isa_dir: str | None = None) -> str:
    out_dir = isa_dir or os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(out_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], isa_dir), zip(srcs, objs)))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizers for the C ABI code (argument checks, sizing, launch set-up).  Each -fsanitize flag goes
# to the host compilation only; the device code is built as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build_host_sanitized(out_dir: str) -> str:
    """libmla_decode.so with the C ABI source (mla_api.hip) built with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host code, linked with the other sources' usual objects.  The process
    that loads it must preload the compiler's ASan runtime (tests/test_sanitizers.py does)."""
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    for src in srcs:
        obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
        if os.path.basename(src) == "mla_api.hip":
            cmd = [HIPCC, *FLAGS, *HOST_SANITIZE, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        else:
            _compile(src, obj, None)
        objs.append(obj)
    lib = os.path.join(out_dir, "libmla_decode.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs])
    return lib


def asan_runtime() -> str:
    """The clang ASan runtime that matches hipcc's host compiler."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = cands[0] if cands else ""
    return path


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None, help="directory to keep intermediate files (assembly) in")
    args = ap.parse_args()
    print(build(os.path.abspath(args.isa) if args.isa else None))
