"""Builds libattn.so (the C-ABI library and its gfx950 kernels) in the package folder.

Each source is compiled in two passes: the gfx950 device pass produces the
code object bundle, and the host pass embeds it. Only the device pass takes
the target feature that keeps packed fp32 VALU forms out of the generated code
(the host compiler does not know the feature). The device pass also records
the compiler's per-kernel resource report (registers, scratch, occupancy,
LDS), written beside the library as kernel_resources.json together with a hash
of each source, so that tests can check the report of the current sources.
"""
import hashlib
import json
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "prefill.hip", "decode.hip", "backward.hip"]
LIB = os.path.join(HERE, "libattn.so")
RESOURCES = os.path.join(HERE, "kernel_resources.json")
BUILD_DIR = os.path.join(ROOT, "_build")

COMMON = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-I", os.path.join(ROOT, "include"),
          "-Wno-unused-command-line-argument"]
# device pass only: packed fp32 VALU forms are kept out of the generated code
DEVICE_ONLY = ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Rpass-analysis=kernel-resource-usage"]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def source_hash(name: str) -> str:
    """sha256 (16 hex digits) over a source and every header in csrc/ and include/."""
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, name)]
    for d in (CSRC, os.path.join(ROOT, "include")):
        paths += sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".h"))
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|VGPRs Spill|SGPRs Spill|LDS Size \[bytes/block\]):\s*(\S+)")
_KEYS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
         "Occupancy [waves/SIMD]": "occupancy", "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill",
         "LDS Size [bytes/block]": "lds_bytes"}


def parse_resources(stderr: str) -> dict:
    """Kernel name -> resource figures, from the kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = val
            out[cur] = {}
        elif cur is not None:
            out[cur][_KEYS[key]] = int(val) if val.isdigit() else val
    return out


def _compile(cc: str, name: str, verbose: bool, extra) -> tuple:
    src = os.path.join(CSRC, name)
    stem = os.path.splitext(name)[0]
    fatbin = os.path.join(BUILD_DIR, stem + ".hipfb")
    obj = os.path.join(BUILD_DIR, stem + ".o")
    dev = [cc, *COMMON, *DEVICE_ONLY, *extra, "-c", src, "-o", fatbin]
    host = [cc, *COMMON, *extra, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin,
            "-c", src, "-o", obj]
    res = {}
    for cmd in (dev, host):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {name} ({r.returncode}):\n{r.stderr[-4000:]}")
        if cmd is dev:
            res = parse_resources(r.stderr)
    return obj, res


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source for gfx950 and link libattn.so; returns the library path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        done = list(ex.map(lambda n: _compile(cc, n, verbose, list(extra_flags)), SOURCES))
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=HERE)
    os.close(fd)
    cmd = [cc, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *[o for o, _ in done]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"link failed ({r.returncode}):\n{r.stderr[-4000:]}")
    os.chmod(tmp, 0o755)
    os.replace(tmp, LIB)
    report = {"sources": {n: source_hash(n) for n in SOURCES},
              "kernels": {k: v for _, res in done for k, v in res.items()}}
    with open(RESOURCES, "w") as f:
        json.dump(report, f, indent=1, sort_keys=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
