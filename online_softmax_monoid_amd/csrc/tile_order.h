// tile_order.h -- which (b, kv-head) unit, query head and query tile a
// prefill workgroup takes, from its id.
#pragma once

#include <hip/hip_runtime.h>

namespace miattn {

struct TileOrder {
    int unit;   // b * Hkv + kv-head
    int gq;     // query head within the kv-head's group
    int qtile;  // query tile
};

// Workgroup ids are dispatched round-robin over the 8 XCDs, and each XCD
// starts its next workgroup on whichever CU frees first. When the units split
// evenly over the XCDs, XCD x owns units [x*u, (x+1)*u), so their K and V stay
// in that XCD's L2, and walks them query-tile rank by rank. Rank 0 is the
// heaviest causal tile, so the short tiles come last and fill the gaps
// instead of leaving a long tile running alone at the end. Otherwise every
// unit walks the ranks together. The G query heads of a kv-head run next to
// each other.
__device__ __forceinline__ TileOrder tile_order(int id, int n_units, int G, int n_qtiles,
                                                bool causal)
{
    constexpr int kXcds = 8;
    int rank, unit, gq;
    if (n_units % kXcds == 0) {
        const int span = (n_units / kXcds) * G;  // one rank's tiles on one XCD
        const int xcd = id % kXcds, pos = id / kXcds;
        rank = pos / span;
        const int rest = pos - rank * span;
        unit = xcd * (n_units / kXcds) + rest / G;
        gq = rest % G;
    } else {
        const int span = n_units * G;
        rank = id / span;
        const int rest = id - rank * span;
        unit = rest / G;
        gq = rest % G;
    }
    return {unit, gq, causal ? n_qtiles - 1 - rank : rank};
}

// The order of the persistent kernels, which hold gx workgroups per XCD at
// once. When the units split evenly over the XCDs, XCD x walks its units in
// groups of U = gx / (query tiles per unit) units (at least one), whose items
// fill the XCD's workgroups about once; within a group, heaviest query-tile
// rank first, then unit, then query head. The workgroups in flight then read
// the K and V of about U units, which fit the XCD's 4 MB L2, instead of all
// of the XCD's units (measured at B2 H32 S4096 d128 causal: L2 misses fall
// from 2.45x to 1.23x of the algorithmic reads). Otherwise the plain order
// above.
__device__ __forceinline__ TileOrder tile_order_grouped(int id, int n_units, int G, int n_qtiles,
                                                        bool causal, int gx)
{
    constexpr int kXcds = 8;
    if (n_units % kXcds != 0)
        return tile_order(id, n_units, G, n_qtiles, causal);
    const int upx = n_units / kXcds, per_unit = n_qtiles * G;
    const int U = max(1, min(upx, gx / max(1, per_unit)));
    const int gsize = U * per_unit;
    const int x = id % kXcds, pos = id / kXcds;
    const int grp = pos / gsize, u0 = grp * U, Ug = min(U, upx - u0);
    const int rest = pos - grp * gsize;
    const int rank = rest / (Ug * G), r2 = rest - rank * (Ug * G);
    return {x * upx + u0 + r2 / G, r2 % G, causal ? n_qtiles - 1 - rank : rank};
}

}  // namespace miattn
