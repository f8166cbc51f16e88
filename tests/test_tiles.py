"""Host check of the materialised product kernel's tiling arithmetic
(csrc/tiles.hpp): the grid its launchers size and the workgroup -> (head,
row tile) decode the kernel runs agree, for many shapes, with every tile
taken exactly once and no head or row tile past the tensors.  The header is
plain constexpr C++, so a host compiler builds the check; no GPU is used."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_causal_head_attn_amd", "csrc")

CHECK = r"""
#include <cstdio>
#include <vector>
#include "tiles.hpp"
using namespace attn::tiles;
int main() {
    static_assert(kApplyRows == 64 * kApplyRB, "four waves of 16-row blocks");
    const int Ts[] = {1, 2, 63, 64, 65, 127, 128, 129, 196, 255, 256, 1000, 1024, 1025, 8192};
    const int BHs[] = {1, 2, 3, 7, 8, 12, 96, 97, 1536};
    long long checked = 0;
    for (int T : Ts) for (int BH : BHs) for (int heavy = 0; heavy < 2; ++heavy) {
        const int nrt = row_tiles(T, kApplyRows);
        if ((long long)nrt * kApplyRows < T || (long long)(nrt - 1) * kApplyRows >= T) {
            std::printf("row tiles do not cover T=%d exactly\n", T); return 1;
        }
        const long long grid = apply_grid(BH, T);
        if (grid != (long long)BH * nrt) { std::printf("grid mismatch\n"); return 1; }
        std::vector<int> seen((size_t)BH * nrt, 0);
        for (long long blk = 0; blk < grid; ++blk) {
            const TileId t = apply_tile(blk, BH, T, heavy != 0);
            if (!t.valid || t.bh < 0 || t.bh >= BH || t.rt < 0 || t.rt >= nrt) {
                std::printf("block %lld of BH=%d T=%d decodes out of range\n", blk, BH, T);
                return 1;
            }
            seen[(size_t)t.bh * nrt + t.rt] += 1;
            ++checked;
        }
        for (int v : seen) if (v != 1) { std::printf("a tile is not taken exactly once\n"); return 1; }
        // one workgroup past the grid (a launcher sized with another
        // constant) must decode as invalid, not as a head past the tensor
        if (apply_tile(grid, BH, T, heavy != 0).valid || apply_tile(-1, BH, T, heavy != 0).valid) {
            std::printf("out-of-grid block decodes as valid\n"); return 1;
        }
    }
    std::printf("ok %lld\n", checked);
    return 0;
}
"""


def test_apply_grid_and_decode_agree(tmp_path):
    src = tmp_path / "tiles_check.cpp"
    exe = tmp_path / "tiles_check"
    src.write_text(CHECK)
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, "-o", str(exe),
                    str(src)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok ")


RULE = r"""
#include <cstdio>
#include "tiles.hpp"
int main() {
    const int hss[] = {16, 32, 64, 128};
    for (int hs : hss)
        for (int T = 1; T <= 300; ++T) std::printf("%d %d %d\n", hs, T, (int)attn::tiles::bwd_short_applies(T, hs));
    return 0;
}
"""


def test_short_backward_rule_matches_bench(tmp_path):
    """bench.py times the fused 16-bit backward as one stage exactly where the
    library's dispatch (tiles::bwd_short_applies) runs the one-kernel
    backward: the two agree for every hs and T up to 300."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "rule.cpp"
    exe = tmp_path / "rule"
    src.write_text(RULE)
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, "-o", str(exe),
                    str(src)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, check=True)

    class W:
        pass
    n = 0
    for line in res.stdout.split("\n"):
        if not line:
            continue
        hs, T, lib = (int(v) for v in line.split())
        w = W()
        w.hs, w.T = hs, T
        assert bench.short_backward(w, "bf16") == bool(lib), (hs, T)
        n += 1
    assert n == 4 * 300
