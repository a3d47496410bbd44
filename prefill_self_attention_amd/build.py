"""Build libprefill_attn.so (HIP, gfx950) in-tree with hipcc, and two
measurement libraries the benchmark reports beside the attention rate: the
small libpa_mfma_peak.so (a matrix-core rate probe) and
libprefill_attn_clock.so (the same sources built with PA_CLOCK_STAMPS: the
64-row kernel records per-wave clock stamps; never loaded by the product).

Run as ``python -m prefill_self_attention_amd.build`` or call ``build()``.
Prints a warning for every kernel that uses scratch (private) memory.
Flags: -O3 for gfx950 only; IEEE mode off with relaxed NaN handling (no
canonicalising moves before max/min); packed-fp32 VALU ops disabled in device code
(``-Xclang -target-feature -Xclang -packed-fp32-ops``; the host pass prints a
harmless "not a recognized feature" warning for it).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libprefill_attn.so")
SOURCES = ["api.hip", "prefill_fwd.hip", "splitkv.hip", "fwd64.hip"]
PEAK_LIB = os.path.join(HERE, "libpa_mfma_peak.so")
PEAK_SOURCES = ["mfma_peak.hip"]
CLOCK_LIB = os.path.join(HERE, "libprefill_attn_clock.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def scratch_kernels(remarks: str):
    """(kernel, bytes per lane) for every kernel whose resource-usage remark
    reports scratch memory."""
    found, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:", 1)[1].split(" [-R")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line and name is not None:
            n = int(line.split("ScratchSize [bytes/lane]:", 1)[1].split()[0])
            if n > 0:
                found.append((name, n))
    return found


def _start(sources, lib, verbose, defines=()):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           # no NaN canonicalisation around max/min (inputs are finite by contract)
           "-fno-honor-nans", "-mno-amdgpu-ieee",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-Rpass-analysis=kernel-resource-usage",
           "-I", INCLUDE, "-I", CSRC]
    cmd += ["-D" + d for d in defines]
    cmd += [os.path.join(CSRC, s) for s in sources]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return proc, tmp, lib


def _finish(job, verbose):
    proc, tmp, lib = job
    stdout, _ = proc.communicate()
    out = "\n".join(line for line in stdout.splitlines()
                    if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + out)
    for name, n in scratch_kernels(out):
        print("build.py: warning: kernel %s uses %d bytes/lane of scratch memory" % (name, n),
              file=sys.stderr, flush=True)
    if verbose:
        msgs = [l for l in out.splitlines() if "remark:" not in l and l.strip()]
        if msgs:
            print("\n".join(msgs), flush=True)
    # a kernel whose host-side launch stub was not emitted leaves an undefined
    # symbol that only shows when the library is loaded: fail here instead
    nm = subprocess.run(["nm", "-C", "--undefined-only", tmp], stdout=subprocess.PIPE,
                        stderr=subprocess.STDOUT, text=True)
    missing = [l.strip() for l in nm.stdout.splitlines() if "__device_stub" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("hipcc emitted no launch stub for:\n" + "\n".join(missing))
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compiles the three libraries at once (separate hipcc processes)."""
    jobs = [_start(SOURCES, LIB, verbose), _start(PEAK_SOURCES, PEAK_LIB, verbose),
            _start(SOURCES, CLOCK_LIB, verbose, defines=("PA_CLOCK_STAMPS",))]
    errors = []
    for job in jobs:
        try:
            _finish(job, verbose)
        except RuntimeError as e:
            errors.append(str(e))
    if errors:
        raise RuntimeError("\n".join(errors))
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
