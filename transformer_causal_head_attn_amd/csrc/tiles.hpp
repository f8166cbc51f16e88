// tiles.hpp -- integer tiling arithmetic of the materialised product kernel
// (apply_kernel in materialized.hip), shared by the kernel and its launchers
// so the grid and the workgroup -> (head, row tile) decode cannot drift
// apart.  Only constexpr integer functions: they compile for the device and
// the host alike and need no HIP header, so the host tests check them with
// a plain C++ compiler.
#pragma once

namespace attn {
namespace tiles {

// apply_kernel: 16-row output blocks per wave, output rows per workgroup
constexpr int kApplyRB = 1;
constexpr int kApplyRows = 4 * 16 * kApplyRB;

constexpr int row_tiles(int T, int rows) { return (T + rows - 1) / rows; }

// Workgroups of one apply_kernel launch over BH heads of T rows.
constexpr long long apply_grid(long long BH, int T) { return BH * row_tiles(T, kApplyRows); }

struct TileId {
    int bh;      // head index b * NH + h
    int rt;      // row tile of that head
    bool valid;  // false for a workgroup past the grid's tiles (never launched)
};

// Workgroup `block` of apply_grid(BH, T): heads run fastest; with
// heavy_first the row tiles run last to first (a causal row tile rt holds
// rt + 1 blocks of work, so the heaviest start first).
constexpr TileId apply_tile(long long block, int BH, int T, bool heavy_first) {
    const int nrt = row_tiles(T, kApplyRows);
    if (BH < 1 || block < 0 || block >= (long long)BH * nrt) return TileId{0, 0, false};
    const int rank = (int)(block / BH);
    const int bh = (int)(block - (long long)rank * BH);
    return TileId{bh, heavy_first ? nrt - 1 - rank : rank, true};
}

}  // namespace tiles
}  // namespace attn
