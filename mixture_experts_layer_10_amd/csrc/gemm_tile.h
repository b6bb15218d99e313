// Tile lookup shared by the grouped-GEMM kernels.
#pragma once

#include "moe_device.h"

namespace moe {

// One work item of a grouped GEMM launch.
struct Tile {
    int g;          // group (local expert, or n_local for the shared expert)
    int nt;         // column tile
    int ks;         // K slice
    bool shared;    // the shared-expert group
    int row0;       // first row of the group in the routed row space
    int m0;         // first row of the tile inside the group
    int rows;       // rows of the tile (1..BM)
};

// Work items are (group, n-tile, m-tile, k-slice), k-slice fastest, then
// m-tile: the workgroups that stream the same weight panel run side by side.
// Items are dealt to the 8 XCDs in contiguous ranges (the hardware deals
// workgroups round-robin over the XCDs), so neighbouring items share an XCD's
// L2: equal item counts, or the ranges of a.xcd_range (cut by estimated work,
// so that XCDs whose items have fewer rows are not left idle at the end).
// Group row counts come from device memory (dispatch offsets and the m-tile
// schedule), never from the host. Returns false for workgroups past the last
// item (the grid is an upper bound). Uniform across the workgroup.
//
// With `balanced`, a group's rows are split into its m-tiles evenly (each
// tile a multiple of 32 rows, at most BM) instead of BM, BM, ..., remainder:
// the m-tile count is the same, but no tile is left with a sliver of rows
// that still streams the whole weight panel.
__device__ __forceinline__ bool find_tile(const GemmArgs& a, int n_tiles, int BM, Tile& t, bool balanced = false) {
    const int KS = a.ksplit;
    const int n_groups = a.n_local + a.has_shared;
    const int per_item = n_tiles * KS;                 // items per m-tile
    // A null schedule means a single group of T rows.
    const int total = (a.sched ? a.sched[n_groups] : (a.T + BM - 1) / BM) * per_item;
    const int slot = static_cast<int>(blockIdx.x >> 3);
    int L;
    if (a.xcd_range) {
        const int x = static_cast<int>(blockIdx.x & 7);
        L = a.xcd_range[x] + slot;
        if (L >= a.xcd_range[x + 1]) return false;
    } else {
        const int per_xcd = (total + 7) >> 3;
        if (slot >= per_xcd) return false;
        L = static_cast<int>(blockIdx.x & 7) * per_xcd + slot;
    }
    if (L >= total) return false;
    if (a.tiles) {
        // one load (the search below takes a dependent load per step)
        const int4 d = a.tiles[L];
        t.g = d.x & 0xffff;
        t.nt = d.x >> 16;
        t.ks = 0;
        t.shared = a.has_shared && t.g == a.n_local;
        t.row0 = d.y;
        t.m0 = d.z;
        t.rows = d.w;
        return true;
    }
    int g = 0, mt_begin = 0, mt_count = (a.T + BM - 1) / BM;
    if (a.sched) {
        int lo = 0, hi = n_groups;                     // sched[lo]*per_item <= L < sched[hi]*per_item
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.sched[mid] * per_item <= L) lo = mid; else hi = mid;
        }
        g = lo;
        mt_begin = a.sched[g];
        mt_count = a.sched[g + 1] - mt_begin;
    }
    const int local = L - mt_begin * per_item;
    t.g = g;
    t.ks = local % KS;
    t.nt = (local / KS) / mt_count;
    const int mt = (local / KS) - t.nt * mt_count;
    t.shared = a.has_shared && g == a.n_local;
    int rows_g = a.T;
    t.row0 = 0;
    if (!t.shared && a.offsets) {
        t.row0 = a.offsets[g];
        rows_g = a.offsets[g + 1] - t.row0;
    }
    int tr = BM;
    if (balanced) {
        tr = (rows_g + mt_count - 1) / mt_count;
        tr = min(BM, (tr + 31) & ~31);
    }
    t.m0 = mt * tr;
    t.rows = min(tr, rows_g - t.m0);
    return true;
}

}  // namespace moe
