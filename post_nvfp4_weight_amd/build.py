"""Build libnvq.so (gfx950) in-tree with hipcc.

Usage: python post_nvfp4_weight_amd/build.py   (run by path: importing the
package loads the library it builds)
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvq.so")
PEAKS_LIB = os.path.join(HERE, "libnvq_peaks.so")
SOURCES = ["api.cpp", "gemm.hip", "syrk.hip", "factor.hip", "sweep.hip", "consumer.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def _objects(build_dir):
    return [os.path.join(build_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]


def build(verbose=False, jobs=None):
    """Compile every source for gfx950 and link libnvq.so; raises on failure."""
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    common = ["-O3", "-fPIC", "-std=c++20", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
              "-Wno-unused-result"]
    # Device code: no packed-fp32 instruction selection.
    device_flags = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    procs = []
    for src, obj in zip(SOURCES, _objects(build_dir)):
        path = os.path.join(CSRC, src)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC] + common + device_flags + lang + ["-c", path, "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, " ".join(cmd), text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n\n".join(f"[{s}] {c}\n{t}" for s, c, t in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", LIB + ".tmp"] + _objects(build_dir)
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(LIB + ".tmp", LIB)
    # The device-peak micro-benchmarks: a separate library that only the
    # benchmark loads.
    src = os.path.join(CSRC, "peaks.hip")
    r = subprocess.run([HIPCC] + common + device_flags + ["-shared", src, "-o", PEAKS_LIB + ".tmp"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on peaks.hip:\n" + r.stdout.decode(errors="replace"))
    os.replace(PEAKS_LIB + ".tmp", PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
