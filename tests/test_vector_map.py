"""The vector map of the streaming kernels (quads_of in csrc/epi_common.h), checked on the CPU.

A host-only build of the library's own header walks the kernels' row loop
(c0 = lane; c0 < nvec; c0 += G*V; vectors c0 + k*G, k < V) for both maps, every
group width G the launchers use (and more), vectors per lane V from 1 to 16, and
ragged row widths. Every element of the row must be touched exactly once and
every access must stay inside the row.
"""
import os
import shutil
import subprocess

import pytest

from moe_routed_expert_amd import build as hip_build

GS = [8, 16, 32, 64, 128, 192, 256, 320, 384, 448, 512, 640, 768, 896, 1024]
VS = [1, 2, 3, 4, 6, 7, 8, 12, 16]


def widths(g, v):
    return sorted({w for w in (1, 2, 3, 7, g - 1, g, g + 1, 2 * g - 1, g * v - 1, g * v, g * v + 1,
                               g * v + g // 2 + 3, 3 * g * v - 5, 192, 193, 256, 257, 512, 896, 1024, 1025, 2053)
                   if w >= 1})


SOURCE = r'''
#include "epi_common.h"
#include <cstdio>
#include <vector>
using namespace moe_epi;
template <int G, bool kSplit>
int walk(int V, uint32_t nvec) {
    std::vector<int> seen(8 * (size_t)nvec, 0);
    for (uint32_t lane = 0; lane < (uint32_t)G; ++lane)
        for (uint32_t c0 = lane; c0 < nvec; c0 += G * V)
            for (int k = 0; k < V; ++k) {
                const uint32_t c = c0 + k * G;
                if (c >= nvec) continue;
                const Quads q = quads_of<G, kSplit>(c, lane, nvec);
                for (uint32_t e = 0; e < 4; ++e) {
                    if (q.a + e >= 8 * nvec || q.b + e >= 8 * nvec) return 1;
                    ++seen[q.a + e];
                    ++seen[q.b + e];
                }
            }
    for (int s : seen)
        if (s != 1) return 2;
    return 0;
}
int main() {
    int bad = 0, n = 0;
%s
    printf("walks %%d failed %%d\n", n, bad);
    return bad != 0;
}
'''


def test_every_element_once_and_in_bounds(tmp_path):
    hipcc = hip_build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    calls = []
    for g in GS:
        for v in VS:
            for w in widths(g, v):
                for split in ("false", "true"):
                    calls.append(f"    {{ int r = walk<{g}, {split}>({v}, {w}u); ++n; if (r) {{ ++bad; "
                                 f"printf(\"G=%d V=%d nvec=%d split=%d: %s\\n\", {g}, {v}, {w}, {int(split == 'true')}, "
                                 f"r == 1 ? \"out of bounds\" : \"not exactly once\"); }} }}")
    src = tmp_path / "walk.cpp"
    src.write_text(SOURCE % "\n".join(calls))
    exe = tmp_path / "walk"
    cmd = [hipcc, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", f"-I{hip_build.INCLUDE}",
           f"-I{hip_build.CSRC}", str(src), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "failed 0" in run.stdout
