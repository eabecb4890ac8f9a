"""Builds libtopk_cols.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m drafter_vocab_top_amd.build

The library is placed next to this file; the Python binding loads it from
there.  hipcc cross-compiles for gfx950 without a GPU.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libtopk_cols.so")
SOURCES = [os.path.join(CSRC, n) for n in ("topk_col.hip", "topk_row.hip", "topk_onewave.hip",
                                            "topk_sample.hip", "topk_noalloc.hip", "topk_cols_api.cpp")]
OBJDIR = os.path.join(ROOT, "_build")
# Per-source flags.  The column kernel takes its ticket before ranking and
# publishing its list and reads the reply afterwards; the compiler's atomic
# optimizer would otherwise wait for the reply right after the atomic (it
# broadcasts the returned value at once), so it is off for that file.  Its
# kernel's leading scalar arguments are preloaded into registers.  The
# row scan asks for three waves per SIMD, which its instantiations with the
# larger candidate area cannot reach; the note saying so is silenced.
EXTRA_FLAGS = {"topk_col.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
                                 "-mllvm", "-amdgpu-kernarg-preload-count=16"],
               "topk_row.hip": ["-Wno-pass-failed"]}
# A plain streaming-read kernel that the benchmark times beside the top-k (not
# part of the top-k library).
STREAM_SOURCE = os.path.join(CSRC, "stream_read.hip")
STREAM_LIBRARY = os.path.join(HERE, "libstream_read.so")
HEADERS = [os.path.join(CSRC, n) for n in ("topk_device.hpp", "topk_col_common.hpp", "topk_internal.hpp")] + \
          [os.path.join(INCLUDE, "topk_cols.h")]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            # keep the compiler from emitting packed fp32 instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def command(output=LIBRARY):
    """One hipcc line that builds the whole library (for reference; the
    per-source flags of EXTRA_FLAGS then apply to every source)."""
    extra = [f for fl in EXTRA_FLAGS.values() for f in fl]
    return [hipcc()] + flags() + extra + ["-shared", "-o", output] + SOURCES


def _check(res, what, verbose):
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose=False):
    """Compiles every source to an object in parallel, then links the library."""
    os.makedirs(OBJDIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES + [STREAM_SOURCE]:
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmd = [hipcc()] + flags() + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for src, pr in procs:
        out, err = pr.communicate()
        _check(subprocess.CompletedProcess(pr.args, pr.returncode, out, err), os.path.basename(src), verbose)
    for lib, lib_objs in ((LIBRARY, objs[:-1]), (STREAM_LIBRARY, objs[-1:])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + lib_objs
        if verbose:
            print(" ".join(cmd), flush=True)
        _check(subprocess.run(cmd, capture_output=True, text=True), "link", verbose)
        os.replace(tmp, lib)
    return LIBRARY


def stale():
    if not os.path.exists(LIBRARY):
        return True
    t = os.path.getmtime(LIBRARY)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
