"""Build of the plain C caller test program (kvq_c_caller.c): gcc, C99,
linked against the in-tree libkvq.so and the HIP runtime, with the oracle
compiled in under the oracle's own flags (no contraction, no fast math)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "kvq_c_caller")


def build() -> str:
    libdir = os.path.join(ROOT, "quantized_decode_attention_kivi_amd")
    tmp = BIN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-ffp-contract=off", "-fno-fast-math", "-fno-builtin",
           # the HIP runtime header needs its platform named when a plain C compiler reads it
           "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "kvq_c_caller.c"), os.path.join(ROOT, "oracle", "kvq_oracle.c"),
           "-o", tmp, "-L", libdir, "-lkvq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../quantized_decode_attention_kivi_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
