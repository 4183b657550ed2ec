"""The large-tile GEMM's work order (moe_tile_order.h, compiled here with g++), checked on the host:
over every workgroup of the launch grid, each (M tile, N tile) is computed exactly once, for tile
counts 0..700 and N tile counts 1..40 in every band grouping; with one M group the order is the
plain N-major eighth of each band; and where the groups divide the band evenly, XCD x's tiles of a
band are exactly block x (N group x / gm, M group x % gm). The GPU is not used."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routing_expert_grouped_amd", "csrc")
# the host programs run under AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "moe_tile_order.h"
using namespace moe;
static int fail(const char* what, int mt, int Nt, int gm) {
  std::printf("FAIL %s mt=%d Nt=%d gm=%d\n", what, mt, Nt, gm);
  return 1;
}
int main() {
  long long checked = 0;
  for (int Nt = 1; Nt <= 40; ++Nt)
    for (int mt = 0; mt <= 700; mt += (mt < 64 ? 1 : 7))
      for (int gm : {1, 2, 4, 8}) {
        const int per = big_grid_per_xcd(mt, Nt);
        const int bm = band_rows_for(Nt);
        std::vector<int> hits((size_t)mt * Nt, 0);
        for (int x = 0; x < 8; ++x)
          for (int jx = 0; jx < per; ++jx) {
            int ti = -1, nt = -1;
            if (!big_tile_coords(mt, Nt, gm, x, jx, ti, nt)) continue;
            if (ti < 0 || ti >= mt || nt < 0 || nt >= Nt) return fail("range", mt, Nt, gm);
            ++hits[(size_t)ti * Nt + nt];
            const int band = ti / bm;
            const int rows = (band + 1) * bm <= mt ? bm : mt - band * bm;
            const int tb = rows * Nt;
            // the eighth of the band XCD x takes, as positions in the band's order
            const int lo = x * tb >> 3, hi = (x + 1) * tb >> 3;
            if (gm == 1) {  // plain N-major order: position nt * rows + (ti - band * bm)
              const int pos = nt * rows + (ti - band * bm);
              if (pos < lo || pos >= hi) return fail("N-major eighth", mt, Nt, gm);
            }
            if (Nt % (8 / gm) == 0 && rows % gm == 0) {  // even blocks: XCD x holds block x
              const int nn = Nt / (8 / gm), mm = rows / gm;
              if (nt / nn != x / gm || (ti - band * bm) / mm != x % gm)
                return fail("block", mt, Nt, gm);
            }
          }
        for (int h : hits)
          if (h != 1) return fail("exactly once", mt, Nt, gm);
        checked += (long long)mt * Nt;
      }
  std::printf("OK %lld\n", checked);
  return 0;
}
"""


def test_every_tile_exactly_once_in_every_grouping():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "order.cpp")
        exe = os.path.join(d, "order")
        with open(src, "w") as f:
            f.write(PROGRAM)
        subprocess.run([gxx, "-O2", "-std=c++17", *SAN, "-I", CSRC, src, "-o", exe], check=True,
                       capture_output=True, timeout=300)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout[-500:]
    assert out.stdout.startswith("OK ")


def test_band_groups_of_the_workload_shapes():
    """The grouping each launch of the workload shapes takes (tile rows, N tiles and mean routed
    rows per expert as the launchers pass them): four M groups where the experts hold at most two
    tiles (their weight panels are fetched once either way), the plain N-major order otherwise."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    cases = [  # (N tiles, tile rows, rows per expert, expected M groups)
        (16, 192, 256, 4),    # GLM-5.2-shaped GEMM-1 (MXFP8, 256 experts, top-8 of 8192 tokens)
        (24, 192, 256, 4),    # its GEMM-2
        (16, 192, 2730, 1),   # Kimi-shaped share GEMM-1 (6 local experts)
        (28, 192, 2730, 1),   # its GEMM-2
        (24, 256, 2048, 1),   # DeepSeek-V4-Pro-shaped share GEMM-1 (BF16)
        (8, 128, 80, 4),      # Qwen-shaped GEMM-1 (512 experts, top-10 of 4096 tokens)
        (16, 128, 80, 4),     # its GEMM-2
        (8, 192, 384, 4),     # two tiles per expert: still four M groups
        (8, 192, 385, 1),     # just over two tiles
    ]
    prog = '#include <cstdio>\n#include "moe_tile_order.h"\nint main() {\n'
    for nt, bm, rpe, _ in cases:
        prog += f'  std::printf("%d\\n", moe::band_groups_for({nt}, {bm}, {rpe}));\n'
    prog += "  return 0;\n}\n"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "g.cpp")
        exe = os.path.join(d, "g")
        with open(src, "w") as f:
            f.write(prog)
        subprocess.run([gxx, "-O2", "-std=c++17", *SAN, "-I", CSRC, src, "-o", exe], check=True,
                       capture_output=True, timeout=300)
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                              timeout=60).stdout.split()]
    assert got == [c[3] for c in cases]
