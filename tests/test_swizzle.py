"""Host-side check of the LDS tile swizzle (csrc/fa_common.h, tile_swz).

The kernels stage bf16 tiles row-major with their 16-byte chunks permuted
per row. This compiles the header's constexpr function on the host, prints
its table and checks the properties the kernels rely on, for every head dim:
  * each row's chunk map is a permutation of the row's own chunks;
  * 16 consecutive rows read at one logical chunk (one ds_read_b128 per lane
    of a 16-lane group) touch 16 different 16-byte bank groups;
  * 4 aligned rows read over an aligned quad of chunks (a transpose read)
    touch 16 different bank groups;
  * 16 rows down the swizzle repeats (the kernels fold those row offsets
    into immediates).
The LDS has 64 banks of 4 bytes: 16 groups of 16 bytes.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_29_amd", "csrc")
DIMS = (32, 64, 96, 128, 256)
ROWS = 64

PROGRAM = r"""
#include <cstdio>
#include "fa_common.h"
template <int D> void dump() {
    for (int r = 0; r < %d; ++r) std::printf("%%d %%d %%d\n", D, r, fa::tile_swz<D>(r));
}
int main() { %s return 0; }
""" % (ROWS, " ".join(f"dump<{d}>();" for d in DIMS))


@pytest.fixture(scope="module")
def table(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("swz")
    src, exe = d / "swz.hip", d / "swz"
    src.write_text(PROGRAM)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    tab = {}
    for line in out.split("\n"):
        if line.strip():
            dim, r, s = map(int, line.split())
            tab[(dim, r)] = s
    return tab


@pytest.mark.parametrize("D", DIMS)
def test_swizzle_properties(table, D):
    C = D // 8
    swz = lambda r: table[(D, r)]
    group = lambda r, c: (r * C + (c ^ swz(r))) % 16
    for r in range(ROWS):
        assert sorted(c ^ swz(r) for c in range(C)) == list(range(C)), (D, r)
    for r0 in range(0, ROWS, 16):
        for c in range(C):
            assert len({group(r, c) for r in range(r0, r0 + 16)}) == 16, (D, r0, c)
    for r0 in range(0, ROWS, 4):
        for q in range(0, C, 4):
            cells = {group(r, c) for r in range(r0, r0 + 4) for c in range(q, q + 4)}
            assert len(cells) == 16, (D, r0, q)
    assert all(swz(r + 16) == swz(r) for r in range(ROWS - 16))
