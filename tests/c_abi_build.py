"""Build tests/c_abi_check (test infrastructure): tests/c_abi_check.c as C11 with
gcc, linked against rotation_quantized_dit_amd/libconvrot.so, the HIP runtime
and the CPU oracle's C source.  __graft_entry__.build() calls it, so the
binary is in place before any GPU run; the GPU test only runs it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "c_abi_check")
LIBDIR = os.path.join(ROOT, "rotation_quantized_dit_amd")


def compile_only(lang: str = "c") -> None:
    """Syntax-check the check's source (C) or the public header alone (C or C++)."""
    inc = ["-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include")]
    if lang == "c":
        cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-fsyntax-only", *inc, os.path.join(HERE, "c_abi_check.c")]
    else:
        cmd = ["g++" if lang == "c++" else "gcc", "-x", lang, "-std=c++17" if lang == "c++" else "-std=c99",
               "-Wall", "-Wextra", "-Werror", "-fsyntax-only", *inc, os.path.join(ROOT, "include", "convrot.h")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stderr)


def build() -> str:
    """Compile the check (always); returns the executable's path."""
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wno-unknown-pragmas", "-ffp-contract=off", "-fno-fast-math",
           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi_check.c"), os.path.join(ROOT, "oracle", "convrot_oracle.c"),
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-L" + LIBDIR, "-lconvrot",
           "-Wl,-rpath,$ORIGIN/../rotation_quantized_dit_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm",
           "-o", EXE + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C ABI check failed:\n" + r.stderr)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
