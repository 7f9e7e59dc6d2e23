"""Compiler-reported resources of every gfx950 kernel (CPU only: hipcc cross-compiles).

No kernel of the block step may use scratch memory: the step's kernels keep
their staging buffers in registers and LDS, and a buffer that falls back to
per-lane scratch (a struct copy the compiler does not promote, a dynamically
indexed array) costs the attention launch about a quarter of its time with no
other visible sign.
"""
import os
import shutil

import pytest

from block_diffusion_drafter_02_amd import build


@pytest.fixture(scope="module")
def usage():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    return build.resource_usage()


def test_every_kernel_reported(usage):
    names = " ".join(usage)
    for k in ("gemv_kernel", "attn_partial_kernel", "attn_combine_kernel", "gemm_kernel", "embed_kernel",
              "inject_kernel", "accept_kernel", "batch_epi_kernel"):
        assert k in names, k
    for name, u in usage.items():
        assert {"vgprs", "scratch", "occupancy"} <= set(u), (name, u)


def test_no_scratch(usage):
    with_scratch = {n: u["scratch"] for n, u in usage.items() if u["scratch"]}
    assert not with_scratch, with_scratch


def test_attention_occupancy(usage):
    # the 512-thread attention workgroup must fit with its LDS at >= 2 wavefronts per SIMD
    attn = {n: u for n, u in usage.items() if "attn_partial_kernel" in n}
    assert attn
    for n, u in attn.items():
        assert u["occupancy"] >= 2, (n, u)


def test_gate_up_grid_resident(usage):
    # The one-tile four-wave GEMV with bf16 or fp8 weights carries the gate/up projection of one sequence,
    # about five workgroups per compute unit: all of them must be resident at once (five wavefronts per
    # SIMD), otherwise the last ones start only when earlier ones finish.
    import re
    pat = re.compile(r"gemv_kernelILi([12])ELi(\d+)ELi1ELi(\d)ELi1ELi4ELi64E")
    hits = {n: u for n, u in usage.items() if pat.search(n)}
    assert hits
    low = {n: u["occupancy"] for n, u in hits.items() if u["occupancy"] < 5}
    assert not low, low
