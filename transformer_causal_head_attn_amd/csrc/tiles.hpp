// tiles.hpp -- integer tiling and dispatch arithmetic shared by kernels and
// their launchers: the materialised product kernel's grid and workgroup ->
// (head, row tile) decode (apply_kernel in materialized.hip), and which
// 16-bit backward the fused entry points run.  Only constexpr integer
// functions: they compile for the device and the host alike and need no HIP
// header, so the host tests check them with a plain C++ compiler.
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

// The fused 16-bit backward runs one kernel with one workgroup per head
// (bwd_short_half_kernel) for T <= 256 and hs <= 64: at hs = 64 and 32 only
// above T = 128 (at or below it the dQ and dK/dV kernels, one workgroup per
// head each, measured 4-5% faster), at hs = 16 for every T.
constexpr bool bwd_short_applies(int T, int hs) {
    return hs <= 64 && T <= 256 && (T > 128 || hs == 16);
}

}  // namespace tiles
}  // namespace attn
