// streamk.hpp -- the stream-K work partition, shared by the planner (host), the hot
// kernel's stream-K mode and the fixup kernel (device).
//
// A tile grid that does not divide evenly over the resident workgroups leaves a last,
// partly filled round of tiles: 272 tiles on 256 compute units take two tile times, with
// 240 units idle in the second. The pages' own remedy is to pick the tile size ("Shared
// Memory Tiling", "Choosing a tile size"; "Visual walkthrough - Memory hierarchy",
// Step 7), which cannot fix a count just past a multiple of the CU count. Stream-K cuts
// the work finer: the unit is one K-panel of one tile (BM x BN x BK multiply-adds), and
// every workgroup gets an equal, contiguous range of those units. A range that covers a
// whole tile writes it to C; a tile shared by several ranges is summed afterwards.
//
// Layout of the work:
//   * tiles are numbered in the tile order (groups of kGroupM tile rows, column by column);
//   * tiles 0 .. tiles_dp - 1 run one per workgroup, as in the plain kernel;
//   * the next tiles_sk tiles form iters = tiles_sk * panels units, and stream-K
//     workgroup g (0 <= g < G) takes units [start(g), start(g + 1)): with iters = q G + r,
//     start(g) = g q + min(g, r), so the first r ranges hold q + 1 units and the rest q;
//   * inside its range a workgroup visits one segment per tile it touches; a segment that
//     is not the whole tile stores its partial sums to workspace slot 2g (the first
//     segment of the range) or 2g + 1 (the last one). A range touches at most one
//     partial tile at each end, so two slots per workgroup are enough.
//   * the fixup kernel adds, for each shared tile, the partial sums of its workgroups in
//     ascending g, which is ascending K; the result does not depend on timing.
// With q = tiles / G and r = tiles % G: r = 0 needs no stream-K; q = 0 shares every tile;
// otherwise either the last G + r tiles are shared (each stream-K range then holds more
// than one whole tile's worth of units, so no segment is very short) or only the last r
// (fewer partial tiles to write and add up), and the rest run plainly; the planner prices
// both.
// Every range holds at least one unit (G is lowered to the unit count when needed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sgemm {

// Contributors whose partial tiles the fixup kernel loads together before adding them.
constexpr int kFixupBatch = 8;

struct SkGeom {
    int G = 0;            // stream-K workgroups
    int tiles_dp = 0;     // tiles run one per workgroup before the shared ones
    int tiles_sk = 0;     // tiles shared out by K-panel
    int panels = 0;       // K-panels per tile
    int iters = 0;        // tiles_sk * panels units
    int q = 0, r = 0;     // iters = q G + r: the first r ranges hold q + 1 units, the rest q
};

// First unit of stream-K workgroup g (g = G gives the end of the last range).
__host__ __device__ inline int sk_start(const SkGeom &s, int g)
{
    return g * s.q + (g < s.r ? g : s.r);
}

// The workgroup whose range holds unit i: the largest g with start(g) <= i.
__host__ __device__ inline int sk_owner(const SkGeom &s, int i)
{
    const int long_units = s.r * (s.q + 1);
    return i < long_units ? i / (s.q + 1) : s.r + (i - long_units) / s.q;
}

// Workspace slot of workgroup g's partial sums of shared tile t (an index among the
// shared tiles): 2g if g's range starts inside t, else 2g + 1.
__host__ __device__ inline int sk_slot(const SkGeom &s, int g, int t)
{
    return 2 * g + (sk_start(s, g) / s.panels == t ? 0 : 1);
}

// The same slot, as the fixup kernel computes it for contributor g of shared tile t whose
// first contributor is g0: every later contributor's range starts inside t, and g0's does
// only when it starts at t's first unit (no division per contributor).
__host__ __device__ inline int sk_fixup_slot(const SkGeom &s, int g, int g0, int t)
{
    return g > g0 ? 2 * g : 2 * g + (sk_start(s, g) == t * s.panels ? 0 : 1);
}

// The partition for `tiles` tiles of `panels` K-panels over G resident workgroups. With
// q >= 1 full rounds, `remainder_only` shares just the r leftover tiles (short ranges,
// little partial-sum traffic) instead of the last G + r (ranges longer than a tile).
// Shares nothing (tiles_sk = 0) when the tiles divide evenly or the shared units would not
// fit in 31 bits.
inline SkGeom sk_geometry(int64_t tiles, int panels, int G, bool remainder_only = false)
{
    SkGeom s;
    s.G = G;
    s.panels = panels;
    const int64_t q = tiles / G, r = tiles % G;
    int64_t dp = tiles, sk = 0;
    if (r != 0) {
        dp = q == 0 ? 0 : (remainder_only ? q : q - 1) * G;
        sk = tiles - dp;
    }
    if (sk * panels > INT32_MAX || dp > INT32_MAX) {
        dp = tiles;
        sk = 0;
    }
    s.tiles_dp = int(dp);
    s.tiles_sk = int(sk);
    s.iters = int(sk * panels);
    // no empty ranges: a workgroup between two contributors of a tile must have written a
    // slot for it (only possible to violate when q = 0 and the tiles hold few units)
    if (s.tiles_sk > 0 && s.iters < G) s.G = s.iters;
    if (s.tiles_sk > 0) {
        s.q = s.iters / s.G;
        s.r = s.iters % s.G;
    }
    return s;
}

}  // namespace sgemm
