"""Builds libdsv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m block_verification_attention_amd.build

The library has no PyTorch dependency: it links only the HIP runtime.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdsv.so")
SOURCES = ["dsv_pack.hip", "dsv_attn.hip", "dsv_accept.hip", "dsv_sample.hip", "dsv_features.hip", "dsv_rng.hip", "dsv_status.hip", "dsv_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


# attn_bf16_kernel<D, NW, PF, TILE, HV, MAP>
_ATTN_KERNEL = re.compile(r"attn_bf16_kernelILi(\d+)ELi(\d+)ELb([01])ELi(\d+)ELi(\d+)ELb([01])E")


def attn_kernel_resources(remarks: str) -> dict:
    """Per attention-kernel instantiation (D, waves, prefill, KV halves, cache map): VGPRs, AGPRs, scratch
    bytes per lane and occupancy (waves per SIMD), parsed from the compiler's resource-usage remarks."""
    res, cur = {}, None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            m = _ATTN_KERNEL.search(line)
            cur = (int(m.group(1)), int(m.group(2)), m.group(3) == "1", int(m.group(5)), m.group(6) == "1") if m else None
            if cur:
                res[cur] = {}
        elif cur is not None:
            for key, name in (("VGPRs:", "vgpr"), ("AGPRs:", "agpr"), ("ScratchSize [bytes/lane]:", "scratch"),
                              ("Occupancy [waves/SIMD]:", "occupancy")):
                if key in line:
                    res[cur][name] = int(line.rsplit(":", 1)[1].split()[0])
    return res


def build(verbose: bool = False) -> str:
    """Compiles every source and links libdsv.so; always rebuilds.  Returns the path."""
    objs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        if src == "dsv_attn.hip":
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for src, obj, proc in procs:
        out, err = proc.communicate()
        # hipcc's host pass reports the device-only target feature as unknown: harmless
        noise = "is not a recognized feature for this target"
        lines = [l for l in (out + err).splitlines() if noise not in l]
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
        if src == "dsv_attn.hip":
            res = attn_kernel_resources("\n".join(lines))
            if not res:
                raise RuntimeError("no attention kernel found in the resource report")
            if verbose:
                for (d, nw, pf, hv, mp), r in sorted(res.items()):
                    print(f"attn_bf16_kernel D={d} waves={nw} prefill={pf} halves={hv} map={mp}: {r}")
            lines = [l for l in lines if "remark:" not in l and "kernel-resource-usage" not in l]
        msg = "\n".join(lines)
        if msg.strip() and verbose:
            print(msg)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
