"""Compile the plain-C client of libmla_decode.so (tests/c_client/mla_client.c) against the built library and the
C oracle.  Called by the repository's build step, after both libraries exist."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "mla_client")


def build() -> str:
    lib_dir = os.path.join(ROOT, "mla_latent_kv_fwd_amd")
    ora_dir = os.path.join(ROOT, "oracle")
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
        os.path.join(HERE, "mla_client.c"), "-o", BIN,
        "-L", lib_dir, "-lmla_decode", "-L", ora_dir, "-loracle", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm",
        "-Wl,-rpath,$ORIGIN/../../mla_latent_kv_fwd_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
        "-Wl,-rpath,/opt/rocm/lib"])
    return BIN


if __name__ == "__main__":
    print(build())
