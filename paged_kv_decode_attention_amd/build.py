"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_decode_attention_amd.build [--jobs N] [--save-temps]

Every HIP source is compiled with packed-fp32 instructions disabled (the
compiler may not form v_pk_* fp32 arithmetic).  Objects go to
``paged_kv_decode_attention_amd/_build/``; the library lands next to this
file, where ``ops.load_library()`` looks for it.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")
ARCH = "gfx950"

SOURCES = [
    "pa_api.cpp",
    "pa_decode_mfma_d128.hip",
    "pa_decode_mfma_d256.hip",
    "pa_decode_mfma_d64.hip",
    "pa_decode_mfma.hip",
    "pa_decode_generic.hip",
    "pa_merge.hip",
    "pa_cache.hip",
    "pa_bench.hip",
    "pa_pool.cpp",
    "pa_check.cpp",
    "pa_noalloc.hip",
]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# -amdgpu-mfma-vgpr-form: keep matrix-core results in VGPRs (no AGPR copies).
# -amdgpu-kernarg-preload-count: the first kernel arguments arrive in scalar
# registers (the balanced decode and merge kernels put there what their
# first loads need).
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=true",
          "-mllvm", "-amdgpu-kernarg-preload-count=6"]


# Sources whose change changes what the decode call's kernels do; hashed to
# tell whether stored counter readings still describe the built kernels.
DECODE_SOURCES = ["pa_decode_mfma.h", "pa_decode_mfma.hip", "pa_decode_mfma_d64.hip",
                  "pa_decode_mfma_d128.hip", "pa_decode_mfma_d256.hip", "pa_decode_generic.hip",
                  "pa_merge.hip", "pa_finalize.h", "pa_device.h", "pa_internal.h", "pa_api.cpp"]


def decode_source_hash():
    """First 16 hex digits of the SHA-256 of the decode sources, in order."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src, save_temps=False):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE
    if save_temps:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    return obj, err


def build(jobs=None, save_temps=False, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(os.cpu_count() or 8, len(SOURCES))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    objs = []
    for obj, warn in results:
        objs.append(obj)
        if verbose and warn.strip():
            print(warn, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + ["--offload-arch=" + ARCH, "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.save_temps, a.verbose))


if __name__ == "__main__":
    main()
