"""In-tree build of libringag.so for gfx950 (hipcc cross-compiles; no GPU needed).

    python -m ring_all_gather_amd.build        # or __graft_entry__.build()

Steps:
  1. device code: csrc/device_kernels.hip -> one gfx950 code object (hipcc --genco), compiled with
     -Xclang -target-feature -Xclang -packed-fp32-ops so the compiler forms no packed fp32 VALU
     instructions (v_pk_*_f32);
  2. the code object is embedded as the symbol ringag_kernels_co (assembler .incbin);
  3. host code (csrc/runtime.cpp, csrc/launch.cpp) is compiled as plain C++ against the HIP
     runtime API and linked with the blob into ring_all_gather_amd/libringag.so.
The host objects contain no device code, so the library has no HIP registration constructors or
destructors; the kernels are loaded explicitly when a context is created.
"""
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libringag.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"
DEVICE_SRC = "device_kernels.hip"
HOST_SRCS = ["runtime.cpp", "launch.cpp"]
DEVICE_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "--genco",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
              "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build_code_object(extra=()) -> str:
    co = os.path.join(BUILD_DIR, "ringag_kernels.co")
    _run([HIPCC, *DEVICE_FLAGS, *extra, os.path.join(CSRC, DEVICE_SRC), "-o", co],
         "device compile")
    return co


def _blob_object(co: str) -> str:
    """Embed the code object, and its SHA-256 as the string ringag_kernels_sha256 (so that
    measurements taken with one build of the kernels can be told apart from another's)."""
    with open(co, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    asm = os.path.join(BUILD_DIR, "kernels_blob.S")
    with open(asm, "w") as f:
        f.write('    .section .rodata.ringag_kernels,"a"\n'
                "    .balign 4096\n"
                "    .globl ringag_kernels_co\n"
                "    .type ringag_kernels_co, @object\n"
                "ringag_kernels_co:\n"
                f'    .incbin "{co}"\n'
                "    .size ringag_kernels_co, . - ringag_kernels_co\n"
                "    .globl ringag_kernels_sha256\n"
                "    .type ringag_kernels_sha256, @object\n"
                "ringag_kernels_sha256:\n"
                f'    .asciz "{digest}"\n'
                "    .size ringag_kernels_sha256, . - ringag_kernels_sha256\n"
                '    .section .note.GNU-stack,"",@progbits\n')
    obj = os.path.join(BUILD_DIR, "kernels_blob.o")
    _run([CXX, "-c", asm, "-o", obj], "blob assembly")
    return obj


def _host_object(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    _run([CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], f"compile of {src}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=3) as ex:
        fco = ex.submit(build_code_object, list(extra))
        hosts = list(ex.map(_host_object, HOST_SRCS))
        co = fco.result()
    blob = _blob_object(co)
    tmp = LIB + ".tmp"
    _run([CXX, "-shared", "-fPIC", *hosts, blob, "-o", tmp, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"], "link")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
