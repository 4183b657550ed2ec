"""Build the HIP library libmoe_mi355x.so in-tree for gfx950.

    python -m routing_expert_grouped_amd.build        # compile every csrc/*.hip and link

Each source is compiled on its own (in parallel) with hipcc, then linked into one shared library
next to this file. Packed float32 instructions are disabled for all device code. The compiler's
per-kernel resource report (registers, spills, scratch, LDS) is kept in _build/kernel_resources.json.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import json
import re
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


RESOURCES = "kernel_resources.json"
_REMARK = re.compile(r"remark:\s+(.*?):\s+(\S+)\s+\[-Rpass-analysis=kernel-resource-usage\]")


def _resources(lines):
    """{kernel: {field: value}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for ln in lines:
        m = _REMARK.search(ln)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics",
           "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = (res.stdout + res.stderr).splitlines()
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    msgs = [ln for ln in lines
            if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj, _resources(lines)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    usage = {}
    for _, r in done:
        usage.update(r)
    with open(os.path.join(BUILD, RESOURCES), "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
