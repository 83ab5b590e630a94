"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds every source of the library with the sanitizers on the host side only
(device code is compiled as usual and never runs), links the fuzz driver
`tests/sanitize/abi_fuzz.cpp`, and runs it: every entry point is called
thousands of times with edge-value arguments (null and misaligned pointers,
zero, negative, huge and overflowing sizes, non-finite floats).  The run must
end cleanly: statuses in range, error strings present, and no sanitizer
report (an out-of-bounds host access, signed overflow in a size computation,
a bad shift or cast in the validation layer aborts it).

Only where no GPU is visible: the driver passes host pointers as device
buffers, so it also refuses to start when a device exists.
"""
import glob
import os
import shutil
import subprocess
import concurrent.futures as cf

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_pool_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]

pytestmark = pytest.mark.skipif(
    os.path.exists("/dev/kfd") or not os.path.exists(HIPCC) or not os.path.exists(CLANG),
    reason="host sanitizer fuzz: needs hipcc and clang++, and runs only where no GPU is visible")


def _compile(src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    r = subprocess.run([HIPCC] + FLAGS + SAN + ["-c", src, "-o", obj], capture_output=True, text=True)
    assert r.returncode == 0, f"{src}:\n{r.stderr[-4000:]}"
    return obj


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(ROOT, "tests", "sanitize", "abi_fuzz.cpp")]
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, str(tmp_path)), srcs))
    exe = str(tmp_path / "abi_fuzz")
    # the link names no HIP source: clang++ with the sanitizer runtimes
    link = [CLANG, "-fsanitize=address,undefined", "-o", exe] + objs + [
        f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:])
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-6000:]
    assert "calls " in r.stdout
