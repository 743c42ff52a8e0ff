"""Register spills of the gfx950 kernels (CPU only: reads the compiler's
resource report that the build writes beside the library).

Every kernel must run without scratch memory, except the tuning alternatives
and corner forms listed here with the bytes per lane they are allowed; a new
spill anywhere else, or a listed one that grows, fails."""
import json
import os
import re

import pytest

from exact_attention_31_amd import build as B

if not os.path.exists(B.RESOURCES):
    pytest.skip("kernel_resources.json not built", allow_module_level=True)

REPORT = json.load(open(B.RESOURCES))

# (pattern over the mangled kernel name, allowed scratch bytes per lane, why)
ACCEPTED = [
    (r"prefill16_kernelI.*Li128ELb[01]ELi2ELi4ELb0E", 360,
     "prefill_variant 2 (two query blocks per wavefront at d = 128): a tuning alternative that "
     "needs more registers than two wavefronts per SIMD allow"),
    (r"prefill16_kernelI.*Li64ELb[01]ELi1ELi4ELb1E", 16,
     "prefill_variant 5 at d = 64 (staged form, persistent grid): a tuning alternative"),
    (r"prefill16_ring_kernelI.*Li64ELb[01]ELi4ELb1E", 8,
     "ring form at d = 64 on the persistent grid, which only many-item launches use (the "
     "23,400-step series runs one item per workgroup, without scratch)"),
    (r"prefill16_ring_kernelI.*Li128ELb[01]ELi8ELb1E", 8,
     "prefill_variant 4 at d = 128 (ring form on the persistent grid): a tuning alternative"),
    (r"decode_split_kernelI.*Li128ELi4ELi1ELb1ELb0E", 24,
     "paged decode with four column groups per wavefront (more than 32 query rows per KV head)"),
]


def test_report_matches_the_sources():
    for name, h in REPORT["sources"].items():
        assert B.source_hash(name) == h, f"{name} changed since the last build: rebuild the library"


def test_kernels_are_in_the_report():
    names = " ".join(REPORT["kernels"])
    for k in ("prefill16_kernel", "prefill16_ring_kernel", "prefill32_kernel", "decode_split_kernel",
              "decode_merge_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"):
        assert k in names, k


def test_no_unaccepted_scratch():
    bad = []
    for name, r in REPORT["kernels"].items():
        scratch = r.get("scratch_bytes", 0)
        allowed = 0
        for pat, limit, _ in ACCEPTED:
            if re.search(pat, name):
                allowed = limit
        if scratch > allowed:
            bad.append(f"{name}: {scratch} B/lane scratch (allowed {allowed})")
    assert not bad, "\n".join(bad)


def test_default_forms_do_not_spill():
    """The kernels the benchmarked workloads run: the persistent d = 128
    prefill (staged form), the one-item-per-workgroup d = 64 ring form, the
    decode split and merge kernels with one or two column groups, and the
    backward's dQ and dK/dV kernels."""
    pats = [r"prefill16_kernelI.*Li128ELb1ELi1ELi8ELb1E", r"prefill16_ring_kernelI.*Li64ELb1ELi4ELb0E",
            r"decode_split_kernelI.*Li128ELi1ELi2ELb0ELb0E", r"decode_split_kernelI.*Li128ELi1ELi2ELb0ELb1E",
            r"decode_merge_kernel", r"bwd_dq_kernelI.*Li128ELb1E", r"bwd_dkdv_kernelI.*Li128ELb1E"]
    for pat in pats:
        hits = [n for n in REPORT["kernels"] if re.search(pat, n)]
        assert hits, pat
        for n in hits:
            assert REPORT["kernels"][n].get("scratch_bytes", 0) == 0, n
