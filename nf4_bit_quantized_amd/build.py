"""Build the HIP library in-tree: ``python -m nf4_bit_quantized_amd.build``.

Compiles every source under ``csrc/`` for gfx950 with hipcc (one process per
file, in parallel) and links ``libqlora_nf4.so`` next to this file.  Always
recompiles; the result replaces the old library atomically.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libqlora_nf4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (the validation,
# planning and dispatch code; device code is built as usual).  Every
# -fsanitize= goes after -Xarch_host, so it never reaches the GPU code.
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
]


def build(verbose: bool = False, jobs: int = 8, out_path: str = LIB_PATH, sanitize: bool = False) -> str:
    """Build the library to out_path (the in-tree library by default).  With
    sanitize, the host code carries ASan/UBSan checks; load such a library in
    a process that preloads the ASan runtime (the CPU tests do that)."""
    hipcc = _hipcc()
    srcs = sources()
    extra = SANITIZE_FLAGS if sanitize else []
    tmpdir = tempfile.mkdtemp(prefix="qlora_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc, *COMMON_FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
            if verbose:
                print("compiled", os.path.basename(src), flush=True)
            return obj

        with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp_lib = os.path.join(tmpdir, LIB_NAME)
        link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                      "-Xarch_host", "-shared-libsan"] if sanitize else []
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        shutil.copyfile(tmp_lib, out_path + ".tmp")
        os.replace(out_path + ".tmp", out_path)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    if verbose:
        print("built", out_path, flush=True)
    return out_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
