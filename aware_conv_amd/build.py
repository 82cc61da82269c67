"""Build the HIP library (libwtconv.so) in-tree for gfx950.

    python -m aware_conv_amd.build              # libwtconv.so, valu_probe
    python -m aware_conv_amd.build --sanitize   # libwtconv_asan.so

compiles every source under ``csrc/`` with hipcc and links one shared object
next to this file.  Packed-FP32 instruction selection is switched off for the
device code (``-packed-fp32-ops``); hipcc's host pass warns that it does not
know that feature, which is harmless.

``--sanitize`` builds the same library with the host code (the C-ABI argument
checks, workspace sizing, dispatch) under AddressSanitizer and
UndefinedBehaviorSanitizer (``-Xarch_host`` before each ``-fsanitize=``: the
GPU code is built as usual).  The CPU ABI tests run against it with

    WTCONV_LIB=aware_conv_amd/libwtconv_asan.so ASAN_OPTIONS=detect_leaks=0 \
    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
    python -m pytest tests/test_abi.py -q -m "not gpu"
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libwtconv.so")
PROBE_SRC = os.path.join(CSRC, "probe", "valu_rate.hip")
PROBE_OUT = os.path.join(HERE, "valu_probe")
BUILD = os.path.join(HERE, "_build")
OUT_ASAN = os.path.join(HERE, "libwtconv_asan.so")
BUILD_ASAN = os.path.join(HERE, "_build_asan")
# host-only sanitizers: each -fsanitize= right after -Xarch_host
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
    "-fconstexpr-steps=200000000",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose=True):
    """Compile and link libwtconv.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, OUT)
    # the vector-ALU issue-rate probe (bench.py --valu-probe), same flags
    tmp = PROBE_OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + [f for f in FLAGS if f != "-fPIC"] + [PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s%s" % (PROBE_SRC, r.stdout, r.stderr))
    os.replace(tmp, PROBE_OUT)
    if verbose:
        print("built", OUT, "and", PROBE_OUT)
    return OUT


def build_sanitized(verbose=True):
    """libwtconv_asan.so: host code under ASan and UBSan (CPU checks only)."""
    os.makedirs(BUILD_ASAN, exist_ok=True)
    srcs = sources()
    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, BUILD_ASAN, SAN_FLAGS), srcs))
    tmp = OUT_ASAN + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libsan",
           "-fsanitize=address,undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, OUT_ASAN)
    if verbose:
        print("built", OUT_ASAN)
    return OUT_ASAN


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
    sys.exit(0)
