"""Build liblca.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Every .hip source under csrc/ is compiled by hipcc into an object in _build/,
then linked into long_context_attention_14_amd/liblca.so.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblca.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source extra flags.  attention.hip: MFMA accumulators in VGPRs.  The
# attention kernels rescale their O accumulators with VALU multiplies; with the
# accumulators in AGPRs every rescale and every MFMA moves them between the
# register files, and the decode kernel spills to scratch, whose reloads wait
# for the KV rows in flight.
# indexer.hip: no NaN-quieting before each ReLU.  max(x, 0) on an MFMA result
# is otherwise two instructions (a canonicalising max, then the max); the
# hardware max already returns 0 for a quiet NaN input, and MFMA results are
# never signalling NaNs.  Score keys handle NaN on the bit pattern.
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "indexer.hip": ["-fno-honor-nans"]}


# The host-sanitizer variant (CPU checks only): the host half of every source is
# built with AddressSanitizer and UndefinedBehaviorSanitizer (errors fatal);
# device code is built as usual.  Its library is loaded only by the CPU test
# that runs the C ABI's validation paths under the sanitizers, with the
# sanitizer runtime preloaded; nothing on a GPU loads it.
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "liblca_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


# The device-check variant (a debug build): the same sources with
# LCA_DEVICE_CHECKS=1, so that the kernels count index data that breaks the
# interface's rules and malformed selections (lca_device_checks reads the
# count).  Loaded only by the test that runs it in a child process.
DBG_BUILD = os.path.join(HERE, "_build_dbg")
DBG_LIB = os.path.join(DBG_BUILD, "liblca_dbg.so")
DBG_FLAGS = ["-DLCA_DEVICE_CHECKS=1"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, out_dir=BUILD, extra=()):
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return obj, warn


def build(verbose: bool = False, sanitize: bool = False, device_checks: bool = False) -> str:
    if sanitize:
        out_dir, lib, extra = SAN_BUILD, SAN_LIB, SAN_FLAGS
    elif device_checks:
        out_dir, lib, extra = DBG_BUILD, DBG_LIB, DBG_FLAGS
    else:
        out_dir, lib, extra = BUILD, LIB, []
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        results = list(ex.map(lambda src: _compile(src, out_dir, extra), sources()))
    for _, warn in results:
        if verbose and warn.strip():
            print(warn, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def sanitizer_runtime() -> str:
    """The ASan runtime of the compiler that built the sanitized library (it also
    carries the UBSan handlers), for LD_PRELOAD into an uninstrumented Python."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so next to hipcc")
    return hits[-1]


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv,
                device_checks="--device-checks" in sys.argv))
