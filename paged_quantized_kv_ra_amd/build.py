"""Build ``libra_kv.so`` in-tree for gfx950.

Every HIP translation unit under ``csrc/`` is compiled with hipcc for
gfx950 only, then linked into one shared library.  The library is linked
against the HIP runtime that PyTorch-ROCm ships (``torch/lib``), by the
plain name ``libamdhip64.so``: the Python binding loads it after importing
torch, so the dynamic loader reuses torch's runtime and device pointers,
streams and events are shared with torch instead of living in a second
runtime instance.

Usage: ``python -m paged_quantized_kv_ra_amd.build [--jobs N] [--timeline]``.
``--timeline`` builds the timing variant ``libra_kv_timeline.so`` instead
(-DRA_TIMELINE: the attention kernel records per-workgroup timestamps that
``bench.py --timeline`` reads); the product library is left as it is.
"""
import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libra_kv.so")
PROBE_SRC = os.path.join(HERE, "probe", "read_ceiling.hip")
PROBE_LIB = os.path.join(HERE, "libra_probe.so")
TIMELINE_LIB = os.path.join(HERE, "libra_kv_timeline.so")
TIMELINE_OBJDIR = os.path.join(ROOT, "_build", "timeline")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # correctly rounded fp32 division: the store's quantiser divides
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def torch_lib_dir():
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        raise RuntimeError("PyTorch-ROCm is required: its HIP runtime is linked")
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so in {d}")
    return d


# Per-file code-generation options.  The matrix-core attention keeps its MFMA
# accumulators in architectural VGPRs: with everything in VGPRs it fits two
# waves per SIMD and avoids AGPR <-> VGPR copies around the softmax.
FILE_FLAGS = {
    "attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src, extra, objdir=OBJDIR):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + HIP_FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs, out):
    tl = torch_lib_dir()
    tmp = out + ".tmp"
    cmd = [CLANGXX, "-shared", "-fPIC", "-o", tmp] + objs + [
        f"-L{tl}", "-l:libamdhip64.so", f"-Wl,-rpath,{tl}", "-Wl,--no-undefined",
        "-Wl,-z,defs"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, out)
    return out


def build_probe(objdir=OBJDIR):
    """The HBM read-rate probe (libra_probe.so, a measurement aid that
    bench.py --read-ceiling loads; not part of libra_kv.so)."""
    os.makedirs(objdir, exist_ok=True)
    obj, _ = _compile(PROBE_SRC, [], objdir)
    return _link([obj], PROBE_LIB)


def build(jobs=None, verbose=False, extra=None, out=LIB, objdir=OBJDIR):
    """Compile every csrc/*.hip for gfx950 and link libra_kv.so, then the
    read-rate probe libra_probe.so.  Always rebuilds.

    ``extra``: additional hipcc flags; ``out`` / ``objdir``: where the library
    and the objects go (the in-tree paths by default).
    """
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources")
    extra = list(extra or [])
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra, objdir), srcs))
    objs = [o for o, _ in results]
    if verbose:
        for (o, err), s in zip(results, srcs):
            warn = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l
                             and "target-feature" not in l and l.strip())
            if warn:
                print(f"[{os.path.basename(s)}]\n{warn}", file=sys.stderr)
    _link(objs, out)
    if out == LIB:
        build_probe(objdir)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--timeline", action="store_true",
                    help="build the timing variant libra_kv_timeline.so (per-workgroup timestamps)")
    a = ap.parse_args()
    if a.timeline:
        print(build(a.jobs, a.verbose, extra=["-DRA_TIMELINE=1"], out=TIMELINE_LIB, objdir=TIMELINE_OBJDIR))
    else:
        print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
