"""Builds libtrimkv.so (HIP for gfx950) in place, next to this file.

    python -m retention_scored_decode_amd.build
"""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.environ.get("TRIMKV_BUILD_DIR", os.path.join(ROOT, "_build"))
LIB = os.environ.get("TRIMKV_LIB_OUT", os.path.join(HERE, "libtrimkv.so"))
# per-unit flags: attention keeps MFMA accumulators in ordinary VGPRs (its
# occasional rescale is VALU work on the same registers)
UNIT_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
# extra hipcc flags, e.g. -DTRIMKV_CHA_PLAIN=24 (tuning knobs of the kernels)
EXTRA = os.environ.get("TRIMKV_EXTRA_FLAGS", "").split()

SOURCES = ["abi.hip", "score.hip", "select.hip", "compact.hip", "attn.hip", "alloc.hip"]
# units whose results must be bit-reproducible: no contraction into FMA
EXACT = {"score.hip", "alloc.hip"}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          # packed fp32 VALU forms stay off (compiler-generated v_pk_* fp32 ops)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


# the compiler's per-kernel resource report, read for register spills
REPORT = ["-Rpass-analysis=kernel-resource-usage"]


def scratch_users(report):
    """(kernel, bytes per lane) for every kernel of a resource report that
    uses scratch memory.  No kernel may: after a kernel with scratch has run,
    later kernels of the process measured about 1% slower on an MI355X
    (the same mask-mode attention, 3.00 -> 3.04 ms), and register spills are
    the only scratch these kernels would have."""
    out, name = [], None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC] + COMMON + EXTRA + UNIT_FLAGS.get(src, []) + (["-ffp-contract=off"] if src in EXACT else []) + \
        REPORT + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    spills = scratch_users(r.stderr)
    if spills:
        raise RuntimeError("%s: kernels use scratch (register spills): %s" % (src, spills))
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
