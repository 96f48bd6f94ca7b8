"""Build of libcsa2 whose host code (argument validation, dispatch, the
workspace arithmetic) is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is built as usual.  Used by the
CPU test that runs the C-ABI validation tests through it.  Output:
libcsa2_asan.so in the directory the caller gives."""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from . import build as B

# host-only instrumentation: each sanitizer flag goes to the host compile
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def runtime():
    """The clang ASan runtime the instrumented library needs preloaded into
    an uninstrumented host process (python)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return hits[-1]


def build(out_dir):
    cc = B.hipcc()
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libcsa2_asan.so")

    def one(src):
        obj = os.path.join(out_dir, src + ".o")
        cmd = [cc, *B.FLAGS, *B.EXTRA.get(src, []), *HOST_SAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(one, B.SOURCES))
    cmd = [cc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", *HOST_SAN, *objs,
           "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib
