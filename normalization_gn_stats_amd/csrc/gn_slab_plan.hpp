// gn_slab_plan.hpp -- the schedule of the cooperative slab kernels as plain
// arithmetic: the grid plan (tiles per slab, team, teams, grid, partial-slot
// stride) and the tile geometry and walks the kernels follow.  Plain C++17
// with no HIP types, so that the host planner, the kernels and a CPU model of
// the schedule (built with g++ by the tests) run the very same code.
//
// The schedule is the one of apex PR #2018 ("Solution"): the cooperative grid
// holds at most as many workgroups as can be resident at once; a slab's tiles
// are spread over a team of workgroups, each taking several tiles when the
// slab has more tiles than the team has members (overflow tiles); every tile
// joins the slab's reductions in phase 1, and after the exchange phase 2
// writes every tile's output once -- the member's last tile from registers,
// the others reloaded.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define GN_HD __host__ __device__
#else
#define GN_HD
#endif

namespace gn {
namespace slab {

constexpr int kThreads = 256;   // threads per workgroup of the slab kernels

// ---- grid plan -----------------------------------------------------------------
struct Geometry {
    int64_t n_slabs;   // NHWC: samples; NCHW: (n, g) slices
    int64_t tiles;     // tiles per slab
    int64_t tpc;       // NCHW: tiles per channel plane (0 for NHWC)
    int64_t pstride;   // partial slots per slab: tiles rounded up to 16 (whole 128-byte lines of 8- and 16-byte slots)
    int64_t team;      // workgroups per slab
    int64_t nteams;    // teams in the grid (each walks slabs k, k + nteams, ...)
    int64_t grid;      // nteams * team
};

// NHWC: a tile is R iterations of kThreads / CPP pixels (CPP = C / V chunks per pixel).
GN_HD constexpr int64_t nhwc_tile_pixels(int64_t C, int V, int R) { return (int64_t)(kThreads / (int)(C / V)) * R; }

// NCHW: a tile is R chunks of V elements per thread, within one channel plane.
GN_HD constexpr int64_t nchw_tile_elems(int V, int R) { return (int64_t)kThreads * R * V; }

// The plan for a resident-workgroup cap `cap` (>= 1): the team is the slab's
// tile count, the cap or `max_team`, whichever is smallest; as many teams as
// the cap holds, at most one per slab.  Hence grid <= cap, and every slab is
// walked by exactly one team.
inline Geometry plan(bool nhwc, int64_t N, int64_t C, int64_t HW, int64_t G, int V, int R, int64_t cap,
                     int64_t max_team = INT64_MAX) {
    Geometry g{};
    const int64_t D = C / G;
    if (nhwc) {
        g.n_slabs = N;
        g.tpc = 0;
        const int64_t tp = nhwc_tile_pixels(C, V, R);
        g.tiles = (HW + tp - 1) / tp;
    } else {
        g.n_slabs = N * G;
        const int64_t te = nchw_tile_elems(V, R);
        g.tpc = (HW + te - 1) / te;
        g.tiles = D * g.tpc;
    }
    g.pstride = (g.tiles + 15) / 16 * 16;
    if (cap < 1) cap = 1;
    g.team = g.tiles < cap ? g.tiles : cap;
    if (g.team > max_team) g.team = max_team;
    if (g.team < 1) g.team = 1;
    g.nteams = cap / g.team;
    if (g.nteams > g.n_slabs) g.nteams = g.n_slabs;
    if (g.nteams < 1) g.nteams = 1;
    g.grid = g.nteams * g.team;
    return g;
}

// ---- NCHW: static walk ---------------------------------------------------------
// Member m of a team of `team` takes tiles m, m + team, ... in phase 1; its
// last tile stays in registers, and phase 2 walks the same tiles back down
// (last, last - team, ..., m): the most recently read first.
GN_HD inline int64_t nchw_last_tile(int64_t m, int64_t team, int64_t tiles) {
    if (m >= tiles) return -1;
    return m + (tiles - 1 - m) / team * team;
}

// Plane and first element of NCHW tile `tile` (tpc tiles per plane).
GN_HD inline void nchw_tile_pos(int64_t tile, int64_t tpc, int64_t te, int64_t* plane, int64_t* k0) {
    *plane = tile / tpc;
    *k0 = (tile - *plane * tpc) * te;
}

// Element (within its plane) of chunk j of thread t of a tile starting at k0;
// the chunk is part of the tile's work when the element is below HW.  Every
// thread still loads a whole chunk: from min(element, HW - V), in bounds.
GN_HD inline int64_t nchw_chunk_elem(int64_t k0, int j, int t, int V) {
    return k0 + (int64_t)(j * kThreads + t) * V;
}
GN_HD inline int64_t nchw_chunk_load(int64_t elem, int64_t HW, int V) { return elem < HW - V ? elem : HW - V; }

// Elements of NCHW tile `tile` (the last tile of each plane may be short).
// 32-bit index arithmetic: the planner keeps a slab's tiles below 2^31.
GN_HD inline int64_t nchw_tile_count(int64_t tile, int64_t tpc, int64_t te, int64_t HW) {
    const int64_t k0 = (int64_t)((uint32_t)tile % (uint32_t)tpc) * te;
    const int64_t rem = HW - k0;
    return rem < te ? rem : te;
}

// ---- NHWC: dynamic hand-out --------------------------------------------------------
// Phase 1: a member draws tile numbers from the slab's first counter until a
// draw reaches `tiles`; it keeps the last tile it reduced in registers and
// flags it resident.  Phase 2: draws k = 0, 1, ... of the second counter name
// tiles - 1 - k (reverse order: the most recently read first); resident
// tiles are skipped (their owner writes them from registers); a draw past
// the end means the member is done.
GN_HD inline int64_t nhwc_phase2_tile(int64_t k, int64_t tiles) { return k < tiles ? tiles - 1 - k : -1; }

// Pixel of chunk j of a thread at pixel row pi of an NHWC tile (PPI pixels per
// iteration); part of the tile's work when below HW; loads clamp to HW - 1.
GN_HD inline int64_t nhwc_pixel(int64_t tile, int64_t tile_pixels, int pi, int j, int ppi) {
    return tile * tile_pixels + pi + (int64_t)j * ppi;
}
GN_HD inline int64_t nhwc_pixel_load(int64_t p, int64_t HW) { return p < HW - 1 ? p : HW - 1; }

}  // namespace slab
}  // namespace gn
