"""Build the gfx950 HIP library in-tree: ``python -m moe_token_block_amd.build``.

One shared object, ``moe_token_block_amd/libmoe_token_block.so``, compiled by
hipcc for gfx950 only.  Flags that matter for results:

* ``-ffp-contract=off``: no multiply-add fusion the source does not spell out
  (the rounding sequence of every quantizer is part of its definition);
* packed FP32 instructions disabled (``-target-feature -packed-fp32-ops``);
* IEEE division and denormals are left at HIP's defaults (correctly rounded
  float division, FP32 denormals preserved).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_token_block.so")
SOURCES = ["abi.hip", "pack.hip", "unpack.hip", "route.hip", "receive.hip", "dswiglu.hip", "consumer.hip"]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=off",
            "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def build(verbose=False):
    """Compile every source (in parallel) and link the shared library; returns its path."""
    tmp = os.path.join(HERE, "_build")
    os.makedirs(tmp, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(tmp, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l
                        and "(ignoring feature)" not in l)
        if p.returncode != 0:
            failed.append((cmd, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(" ".join(c) + "\n" + o for c, o in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    tmp_lib = LIB + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp_lib] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
