"""Build ``libffd.so`` (the HIP kernels and the C ABI) in-tree for gfx950."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libffd.so")
SAN_LIB = os.path.join(PKG, "libffd_san.so")   # host layer with AddressSanitizer + UBSan (CPU tests)
SOURCES = ["ffd_api.hip", "ffd_quantize.hip", "ffd_decode.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # selection arithmetic must match the oracle bit for bit:
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


# ffd_decode.hip holds every decode kernel family; it is compiled once per
# (head dim, dense, key storage) family so that the families build in parallel.
DECODE_FAMILIES = [(d, dense, thumb) for d in (128, 64) for dense in (0, 1) for thumb in (0, 1)]


def _units():
    """(source, extra defines, object name) of every compilation unit."""
    units = [(s, [], s.replace(".hip", ".o")) for s in SOURCES if s != "ffd_decode.hip"]
    for d, dense, thumb in DECODE_FAMILIES:
        units.append(("ffd_decode.hip",
                      [f"-DFFD_VARIANT_D={d}", f"-DFFD_VARIANT_DENSE={'true' if dense else 'false'}",
                       f"-DFFD_VARIANT_THUMB={'true' if thumb else 'false'}"],
                      f"ffd_decode_d{d}_{'dense' if dense else 'sparse'}_{'thumb' if thumb else 'int4'}.o"))
    return units


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source into ``libffd.so`` (units in parallel); returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_unit(u):
        src, defs, obj = u
        cmd = [hipcc(), *flags, *inc, *defs, "-c", os.path.join(CSRC, src), "-o", os.path.join(objdir, obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        return cmd, subprocess.run(cmd, capture_output=True, text=True)

    units = _units()
    jobs = jobs or min(len(units), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_unit, units))
    for cmd, res in results:
        if res.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
            raise RuntimeError("hipcc failed building libffd.so")
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
            *[os.path.join(objdir, u[2]) for u in units], "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libffd.so")
    os.replace(tmp, LIB)
    return LIB


# Host-only sanitizer flags: each -fsanitize applies to the host pass alone
# (device code is not instrumented); UBSan traps nothing, it reports and the
# runtime's halt_on_error decides.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_UNITS = ("ffd_api.hip", "ffd_quantize.hip")


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to LD_PRELOAD into Python)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return res.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """``libffd_san.so``: the C-ABI host layer (argument validation, dispatch,
    workspace carving; ffd_api.hip and ffd_quantize.hip) built with
    AddressSanitizer and UBSan on the host, linked with the decode kernels
    of the ordinary build (their objects are reused when present)."""
    objdir = os.path.join(PKG, "_build")
    units = _units()
    if not all(os.path.exists(os.path.join(objdir, u[2])) for u in units if u[0] not in SAN_UNITS):
        build(verbose=verbose)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + SAN_FLAGS
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src, defs, obj in units:
        if src in SAN_UNITS:
            out = os.path.join(objdir, "san_" + obj)
            cmd = [hipcc(), *flags, *inc, *defs, "-c", os.path.join(CSRC, src), "-o", out]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed building the sanitized host layer")
            objs.append(out)
        else:
            objs.append(os.path.join(objdir, obj))
    tmp = SAN_LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libffd_san.so")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
