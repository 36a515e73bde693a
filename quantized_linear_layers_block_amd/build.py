"""Builds libqlinear.so (the gfx950 kernels and the C ABI) in place with hipcc.

    python -m quantized_linear_layers_block_amd.build      (or build() from Python)

Every .hip/.cpp file under csrc/ is compiled for gfx950 only, in parallel, and
linked into quantized_linear_layers_block_amd/libqlinear.so.  Packed-FP32 VALU
instructions are disabled for the device code.  The measured-ceiling probe under
ceiling/ (benchmark infrastructure, not part of the layer's ABI) is built into
libqlinear_ceiling.so the same way.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqlinear.so")
CEIL_SRC = os.path.join(HERE, "ceiling", "ceiling.hip")
CEIL_OUT = os.path.join(HERE, "libqlinear_ceiling.so")
BUILD = os.path.join(HERE, "_build")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast"]


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else []) + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "is not a recognized feature for this target" not in l)
    return src, obj, r.returncode, errs


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        results = list(ex.map(_compile, srcs + [CEIL_SRC]))
    results, ceil = results[:-1], results[-1:]
    failed = [r for r in results + ceil if r[2] != 0]
    for src, _, rc, errs in results + ceil:
        if errs.strip() and (verbose or rc != 0):
            print(f"--- {src}\n{errs}", file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(f[0] for f in failed))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [r[1] for r in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    _link([r[1] for r in ceil], CEIL_OUT)
    return OUT


def _link(objs, out):
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
