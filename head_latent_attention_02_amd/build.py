"""Build libmla.so (HIP for gfx950) in-tree, and its checked variant.

Every ``csrc/*.hip`` file is compiled by hipcc into ``_build/`` and linked into
``head_latent_attention_02_amd/libmla.so``; the same sources compiled with ``MLA_CHECKED``
(objects in ``_build/checked/``) make ``libmla_checked.so``, whose decode kernels
bounds-check the page-table entries and lengths they read.  ``calib/calib.hip`` (the
bench's HBM-read and matrix-core calibration loops, no part of the method) becomes
``libmla_calib.so``.  Packed-fp32 instruction selection is
disabled for device code (``-packed-fp32-ops``); the host pass warns that it does not know
that feature, which is harmless.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libmla.so")
CHECKED_LIB_PATH = os.path.join(PKG, "libmla_checked.so")
# calibration microbenchmarks for the bench's measured roofline denominators
CALIB_SRC = os.path.join(PKG, "calib", "calib.hip")
CALIB_LIB_PATH = os.path.join(PKG, "libmla_calib.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", f"-I{INCLUDE}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def _compile(src, extra, out_dir=BUILD_DIR):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stderr}")
    return obj


def _build_one(lib_path, out_dir, flags, jobs, verbose):
    os.makedirs(out_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(flags), out_dir), sources))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path} from {len(sources)} sources", file=sys.stderr)
    return lib_path


def build_calib(verbose=False):
    """Compile the calibration microbenchmarks (calib/calib.hip) into libmla_calib.so."""
    out_dir = os.path.join(BUILD_DIR, "calib")
    os.makedirs(out_dir, exist_ok=True)
    obj = _compile(CALIB_SRC, [], out_dir)
    tmp = CALIB_LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, CALIB_LIB_PATH)
    if verbose:
        print(f"built {CALIB_LIB_PATH}", file=sys.stderr)
    return CALIB_LIB_PATH


def build(verbose=False, jobs=8, extra_flags=(), checked=True):
    """Compile every HIP source and link libmla.so (and libmla_checked.so unless
    checked=False), plus the calibration library; returns the path of libmla.so."""
    _build_one(LIB_PATH, BUILD_DIR, extra_flags, jobs, verbose)
    if checked:
        _build_one(CHECKED_LIB_PATH, os.path.join(BUILD_DIR, "checked"),
                   [*extra_flags, "-DMLA_CHECKED"], jobs, verbose)
    build_calib(verbose)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
