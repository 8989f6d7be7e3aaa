"""Checks on the gfx950 machine code the library's sources compile to (CPU only).

- No mixed-precision fma with a half-precision result (v_fma_mix{lo,hi}_f16,
  v_mad_mix{lo,hi}_f16). hipcc folds `(float)a * b` feeding a float -> half
  conversion into one of these with a +0 addend. That rounds the exact product
  straight to half (the method rounds the binary32 product, then to half) and
  turns a -0 product into +0. The mixed forms with a float result only widen
  half sources, which is exact, and are allowed.
- No packed fp32 arithmetic (v_pk_{add,mul,fma}_f32): the build turns the
  feature off.
- The streaming kernels (SwiGLU, router multiply, combine) use no scratch
  memory, and the combine no LDS: a per-lane array indexed at run time is
  placed by the compiler in scratch or, multiplied by the lanes of a block, in
  LDS (a compacted row list in an earlier combine took 64 KiB per block and
  cut the CUs it could share).
"""
import os
import re

import pytest
import yaml

from moe_routed_expert_amd import build as hip_build

HALF_RESULT_MIX = re.compile(r"\bv_(fma|mad)_mix(lo|hi)_f16\b")
PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
KERNEL_LABEL = re.compile(r"^(_Z\S+):")


def _scan(path, pattern):
    hits, name = {}, None
    with open(path) as f:
        for line in f:
            m = KERNEL_LABEL.match(line)
            if m:
                name = m.group(1)
            elif pattern.search(line.split(";", 1)[0]):
                hits[name] = hits.get(name, 0) + 1
    return hits


@pytest.fixture(scope="module", params=[os.path.basename(s) for s in hip_build.sources()])
def asm(request, tmp_path_factory):
    src = os.path.join(hip_build.CSRC, request.param)
    out = tmp_path_factory.mktemp("asm") / (request.param + ".s")
    return hip_build.device_asm(src, str(out))


def test_no_half_result_mixed_fma(asm):
    hits = _scan(asm, HALF_RESULT_MIX)
    assert not hits, f"half-result mixed fma in {hits}"


def test_no_packed_fp32(asm):
    hits = _scan(asm, PACKED_F32)
    assert not hits, f"packed fp32 arithmetic in {hits}"


def test_scan_finds_a_planted_line(tmp_path):
    p = tmp_path / "k.s"
    p.write_text("_Zk:\n\tv_fma_mixlo_f16 v1, v2, v3, 0\n\tv_pk_mul_f32 v[0:1], v[2:3], v[4:5]\n"
                 "_Zj:\n\t; v_fma_mixhi_f16 in a comment\n\tv_fma_mix_f32 v1, v2, v3, v4\n")
    assert _scan(p, HALF_RESULT_MIX) == {"_Zk": 1}
    assert _scan(p, PACKED_F32) == {"_Zk": 1}


STREAMING = ("swiglu_clamped.hip", "router_weight_mul.hip", "moe_combine.hip")


def kernel_metadata(path):
    """{kernel symbol: its entry in the code object's amdhsa.kernels metadata}."""
    text = open(path).read()
    start = text.index(".amdgpu_metadata") + len(".amdgpu_metadata")
    meta = yaml.safe_load(text[start:text.index(".end_amdgpu_metadata")].rstrip())
    return {k[".symbol"]: k for k in meta["amdhsa.kernels"]}


@pytest.mark.parametrize("source", STREAMING)
def test_streaming_kernels_use_no_scratch_and_the_combine_no_lds(source, tmp_path):
    out = hip_build.device_asm(os.path.join(hip_build.CSRC, source), str(tmp_path / (source + ".s")))
    meta = kernel_metadata(out)
    assert meta, "no kernels found"
    for name, k in meta.items():
        assert k[".private_segment_fixed_size"] == 0, f"{name} uses scratch memory"
        if source == "moe_combine.hip":
            assert k[".group_segment_fixed_size"] == 0, f"{name} declares LDS"


def test_metadata_reader_sees_a_planted_scratch_entry(tmp_path):
    p = tmp_path / "k.s"
    p.write_text(".amdgpu_metadata\n---\namdhsa.kernels:\n  - .symbol: _Zk.kd\n"
                 "    .private_segment_fixed_size: 80\n    .group_segment_fixed_size: 65536\n"
                 "...\n.end_amdgpu_metadata\n")
    k = kernel_metadata(p)["_Zk.kd"]
    assert k[".private_segment_fixed_size"] == 80 and k[".group_segment_fixed_size"] == 65536
