"""Build libringattn.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only, with packed-FP32
instructions disabled, and linked into one shared library next to this file.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libringattn.so")
SOURCES = ["ra_host.hip", "ra_fwd.hip", "ra_bwd.hip", "ra_elem.hip", "ra_decode.hip", "ra_ffn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fno-honor-nans",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False, jobs: int = 4) -> str:
    objs = []
    procs = []
    outdir = os.path.join(HERE, "_build")
    os.makedirs(outdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(outdir, src.replace(".hip", ".o"))
        cmd = [HIPCC] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    failed = []
    for p, src in procs:
        _, err = p.communicate()
        err = "\n".join(x for x in err.splitlines()
                        if "packed-fp32-ops" not in x)
        if p.returncode != 0:
            failed.append((src, err))
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        msg = "\n".join(f"--- {s}\n{e}" for s, e in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # every kernel launched from host code must have its host stub in the library
    und = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
    missing = [l for l in und.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("libringattn.so would miss kernel stubs:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
