"""Builds libvla.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvla.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["vla_abi.hip", "scan_seq.hip", "chunked.hip", "state_pass.hip", "inverse_wy.hip", "residual_pass.hip",
           "decode.hip", "scan_split.hip", "project_u.hip", "validate.hip", "backward.hip", "linear_state.hip",
           "inverse_wy128.hip"]

# Packed-FP32 instructions stay off: hipcc would otherwise form v_pk_fma_f32
# and friends from ordinary float code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument", "-Werror",
    "-Rpass-analysis=kernel-resource-usage",
]

# Kernels whose waits count outstanding vector-memory operations (s_waitcnt
# vmcnt(N) with N > 0): a register spill would add scratch loads and stores
# to that count, so the build fails if any of them uses scratch.
COUNTED_WAIT_KERNELS = ["vla_res_chain_kernel"]

_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs|AGPRs|Dynamic Stack):\s*(\S+)")


def resource_usage(remarks: str) -> dict:
    """Per-kernel {vgprs, agprs, scratch, dynamic_stack} from kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(remarks):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[{"VGPRs": "vgprs", "AGPRs": "agprs", "Dynamic Stack": "dynamic_stack"}.get(key, "scratch")] = val
    return out


def check_counted_waits(usage: dict) -> None:
    for name in COUNTED_WAIT_KERNELS:
        hits = {k: v for k, v in usage.items() if name in k}
        if not hits:
            raise RuntimeError(f"kernel {name} not found in the resource-usage remarks")
        for k, v in hits.items():
            if v.get("scratch") != "0" or v.get("dynamic_stack") != "False":
                raise RuntimeError(f"{k} uses scratch ({v}); its counted s_waitcnt vmcnt would be wrong")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the VLA HIP library cannot be built")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libvla.so; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        return obj, _run([cc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(compile_one, SOURCES))
    usage = {}
    for _, msg in results:
        usage.update(resource_usage(msg))
    check_counted_waits(usage)
    with open(os.path.join(BUILD_DIR, "resource_usage.txt"), "w") as f:
        for k in sorted(usage):
            f.write(f"{k} {usage[k]}\n")
    if verbose:
        for obj, msg in results:
            msg = "\n".join(l for l in msg.splitlines() if "remark:" not in l and not re.match(r"\s*\d*\s*\|", l))
            if msg.strip():
                print(msg)
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
