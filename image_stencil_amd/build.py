"""Build libimgstencil.so (gfx950 HIP kernels + C ABI) in the package directory.

hipcc cross-compiles for gfx950 without a GPU. Packed FP32 instructions are
switched off for the device code (-packed-fp32-ops): the kernels use plain
v_fma_f32. The host pass warns that it does not know that target feature.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libimgstencil.so")
# Debug variant for the tests: every LDS-staging kernel first fills its LDS
# with NaN (IMGSTENCIL_LDS_POISON), so that reading LDS that was never written
# shows up in the results. Never loaded by the binding.
LIB_LDS_POISON = os.path.join(HERE, "libimgstencil_ldspoison.so")
# Measurement kernels of the benchmark (matrix-core rate and shader clock, LDS
# bank probes): a library of their own, never loaded by the binding.
PROBES_SRC = os.path.join(HERE, "probes", "probes.hip")
LIB_PROBES = os.path.join(HERE, "libimgstencil_probes.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Build the library and its LDS-poison debug variant; returns the library's path."""
    variants = [(LIB, "_build", []), (LIB_LDS_POISON, "_build_ldspoison", ["-DIMGSTENCIL_LDS_POISON"])]
    _compile_and_link(variants, verbose, jobs)
    _build_probes(verbose)
    return LIB


def _build_probes(verbose):
    tmp = LIB_PROBES + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-shared", PROBES_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(r.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for " + PROBES_SRC)
    os.replace(tmp, LIB_PROBES)


def _compile_and_link(variants, verbose, jobs):
    """Compile every csrc/*.hip of every variant to objects in parallel, then
    link each variant's library."""
    procs, objs = [], {}
    running = []
    for lib, objname, defines in variants:
        objdir = os.path.join(HERE, objname)
        os.makedirs(objdir, exist_ok=True)
        objs[lib] = []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            objs[lib].append(obj)
            cmd = [HIPCC] + FLAGS + defines + ["-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            p = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
            procs.append((src, p))
            running.append(p)
            while len([q for q in running if q.poll() is None]) >= jobs:
                running[0].wait()
                running = [q for q in running if q.poll() is None]
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines()
                         if "packed-fp32-ops" not in l and l.strip() != "1 warning generated.")
        if text.strip() and (verbose or p.returncode != 0):
            print(text, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    for lib, _, _ in variants:
        _link(lib, objs[lib], verbose)


def _link(lib, objs, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # Every symbol of the library's own namespace must be defined in it: the
    # host pass can drop a kernel's launch stub (a struct declared inside a
    # template kernel did) and leave an undefined reference that only fails
    # when the library is loaded.
    nm = subprocess.run(["nm", "-u", "-C", tmp], capture_output=True, text=True)
    if nm.returncode == 0:
        missing = [l.strip() for l in nm.stdout.splitlines() if "is::" in l]
        if missing:
            os.remove(tmp)
            raise RuntimeError("%s has undefined symbols of its own:\n  %s" % (os.path.basename(lib),
                                                                              "\n  ".join(missing)))
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
