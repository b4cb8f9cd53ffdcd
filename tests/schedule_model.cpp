// schedule_model.cpp -- CPU model of the cooperative slab kernels' schedule,
// built with g++ from the same header the kernels and the host planner use
// (normalization_gn_stats_amd/csrc/gn_slab_plan.hpp).
//
// For one problem and one resident-workgroup cap it checks:
//  * the plan: 1 <= team <= min(tiles, cap); grid = nteams * team <= cap;
//    nteams <= slabs; partial slots pstride >= tiles in whole 16-slot blocks;
//    tile indices below 2^31; every slab walked by exactly one team;
//  * NCHW (static walk): over the members of a team, phase 1 reduces every
//    tile exactly once, each member's last tile is nchw_last_tile, and the
//    phase-2 walk back down writes every tile exactly once; the chunks of
//    the tiles of a channel plane cover every element exactly once, their
//    loads stay inside the plane, and nchw_tile_count is each tile's share;
//  * NHWC (dynamic hand-out): the kernels' draw protocol -- phase 1 draws
//    from the first counter until a draw passes the end, the last tile is
//    kept resident; phase 2 writes the resident tile, then draws from the
//    second counter in reverse order skipping resident tiles -- run under
//    many interleavings of the members (random ones, round robin, one member
//    taking everything first): every tile is reduced exactly once and written
//    exactly once; the chunks of the tiles cover every (pixel, chunk) of the
//    sample exactly once and their loads stay inside the sample.
//
// Usage: schedule_model NHWC N C HW G V R CAP SEEDS
// Prints "OK tiles=.. team=.. nteams=.. grid=.." or "FAIL <reason>" (exit 1).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <string>
#include <vector>

#include "gn_slab_plan.hpp"

using namespace gn::slab;

static int fail(const std::string& why) {
    printf("FAIL %s\n", why.c_str());
    return 1;
}

#define CHECK(cond, ...)                                    \
    do {                                                    \
        if (!(cond)) {                                      \
            char buf[512];                                  \
            snprintf(buf, sizeof buf, __VA_ARGS__);         \
            return fail(buf);                               \
        }                                                   \
    } while (0)

// One member of a team in the NHWC protocol, advanced one counter draw at a time.
struct Member {
    int state = 0;        // 0: phase-1 first draw, 1: phase-1 loop, 2: phase-1 done
    int64_t tile = -1;    // current tile
    int64_t last = -1;    // last tile reduced (kept in registers)
    // phase 2
    int p2 = 0;           // 0: start, 1: loop, 2: done
    int64_t t2 = -1;
};

static int nhwc_run(int64_t tiles, int64_t team, int order, uint64_t seed, std::vector<int>& reduced,
                    std::vector<int>& written) {
    std::mt19937_64 rng(seed);
    std::vector<Member> mem((size_t)team);
    uint64_t ctr1 = 0, ctr2 = 0;
    std::vector<uint8_t> res((size_t)tiles, 0);
    reduced.assign((size_t)tiles, 0);
    written.assign((size_t)tiles, 0);
    // the members still running, and the one that takes the next step
    std::vector<int64_t> live;
    auto reset_live = [&]() {
        live.clear();
        for (int64_t m = 0; m < team; ++m) live.push_back(m);
    };
    uint64_t steps = 0;
    auto pick = [&]() -> size_t {
        ++steps;
        if (order == 0) return (size_t)(rng() % live.size());   // random interleaving
        if (order == 1) return (size_t)(steps % live.size());   // round robin
        return 0;                                               // one member runs ahead of all others
    };
    auto retire = [&](size_t i) {   // keeps the order of the others (member 0 stays first)
        live.erase(live.begin() + (std::ptrdiff_t)i);
    };
    // ---- phase 1: tile = draw(); while (tile < tiles) { next = draw(); reduce(tile);
    //      last = tile; if (next >= tiles) break; tile = next; } ----
    reset_live();
    while (!live.empty()) {
        const size_t i = pick();
        Member& x = mem[(size_t)live[i]];
        const int64_t d = (int64_t)ctr1++;
        if (x.state == 0) {
            x.tile = d;
            x.state = d < tiles ? 1 : 2;
        } else {
            ++reduced[(size_t)x.tile];   // reduce the current tile (its loads were issued at its draw)
            x.last = x.tile;
            if (d >= tiles) {
                x.state = 2;
            } else {
                x.tile = d;
            }
        }
        if (x.state == 2) retire(i);
    }
    for (auto& x : mem)
        if (x.last >= 0) res[(size_t)x.last] = 1;   // resident flags, published before the barrier
    // ---- phase 2: tile = last (or a draw); while (tile >= 0) { next = draw2(); write(tile);
    //      if (next < 0) break; tile = next; }, draw2 skipping resident tiles ----
    auto draw2 = [&]() -> int64_t {
        while (true) {
            const int64_t t = nhwc_phase2_tile((int64_t)ctr2++, tiles);
            if (t < 0) return -1;
            if (!res[(size_t)t]) return t;
        }
    };
    reset_live();
    while (!live.empty()) {
        const size_t i = pick();
        Member& x = mem[(size_t)live[i]];
        if (x.p2 == 0) {
            x.t2 = x.last >= 0 ? x.last : draw2();
            x.p2 = x.t2 >= 0 ? 1 : 2;
        } else {
            const int64_t next = draw2();
            ++written[(size_t)x.t2];
            if (next < 0) {
                x.p2 = 2;
            } else {
                x.t2 = next;
            }
        }
        if (x.p2 == 2) retire(i);
    }
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 10) {
        fprintf(stderr, "usage: %s NHWC N C HW G V R CAP SEEDS\n", argv[0]);
        return 2;
    }
    const bool nhwc = atoi(argv[1]) != 0;
    const int64_t N = atoll(argv[2]), C = atoll(argv[3]), HW = atoll(argv[4]), G = atoll(argv[5]);
    const int V = atoi(argv[6]), R = atoi(argv[7]);
    const int64_t cap = atoll(argv[8]);
    const int seeds = atoi(argv[9]);
    const Geometry g = plan(nhwc, N, C, HW, G, V, R, cap);

    // ---- the plan ----
    CHECK(g.tiles >= 1 && g.tiles < ((int64_t)1 << 31), "tiles %lld outside [1, 2^31)", (long long)g.tiles);
    CHECK(g.team >= 1 && g.team <= g.tiles && g.team <= (cap < 1 ? 1 : cap), "team %lld (tiles %lld, cap %lld)",
          (long long)g.team, (long long)g.tiles, (long long)cap);
    CHECK(g.grid == g.nteams * g.team && g.grid <= (cap < 1 ? 1 : cap), "grid %lld over cap %lld", (long long)g.grid,
          (long long)cap);
    CHECK(g.nteams >= 1 && g.nteams <= g.n_slabs, "nteams %lld (slabs %lld)", (long long)g.nteams,
          (long long)g.n_slabs);
    CHECK(g.pstride >= g.tiles && g.pstride % 16 == 0 && g.pstride - g.tiles < 16, "pstride %lld for %lld tiles",
          (long long)g.pstride, (long long)g.tiles);
    {   // teams walk slabs k, k + nteams, ...: each slab once
        std::vector<int> seen((size_t)g.n_slabs, 0);
        for (int64_t k = 0; k < g.nteams; ++k)
            for (int64_t sb = k; sb < g.n_slabs; sb += g.nteams) ++seen[(size_t)sb];
        for (int64_t sb = 0; sb < g.n_slabs; ++sb) CHECK(seen[(size_t)sb] == 1, "slab %lld walked %d times", (long long)sb, seen[(size_t)sb]);
        // partial slots of the last slab stay inside the block
        CHECK((g.n_slabs - 1) * g.pstride + g.tiles - 1 < g.n_slabs * g.pstride, "partial slot out of the block");
    }

    if (!nhwc) {
        const int64_t te = nchw_tile_elems(V, R);
        CHECK(HW >= V && HW % V == 0, "HW %lld not a multiple of V", (long long)HW);
        CHECK(g.tpc * te >= HW && (g.tpc - 1) * te < HW, "tpc %lld does not cover HW", (long long)g.tpc);
        // ---- member walks over one slab ----
        std::vector<int> red((size_t)g.tiles, 0), wr((size_t)g.tiles, 0);
        for (int64_t m = 0; m < g.team; ++m) {
            int64_t last = -1;
            for (int64_t t = m; t < g.tiles; t += g.team) {
                ++red[(size_t)t];
                last = t;
            }
            CHECK(last == nchw_last_tile(m, g.team, g.tiles), "member %lld: last %lld, nchw_last_tile %lld",
                  (long long)m, (long long)last, (long long)nchw_last_tile(m, g.team, g.tiles));
            for (int64_t t = last; t >= 0; t -= g.team) ++wr[(size_t)t];
        }
        for (int64_t t = 0; t < g.tiles; ++t) {
            CHECK(red[(size_t)t] == 1, "tile %lld reduced %d times", (long long)t, red[(size_t)t]);
            CHECK(wr[(size_t)t] == 1, "tile %lld written %d times", (long long)t, wr[(size_t)t]);
        }
        // ---- element coverage of each channel plane ----
        const int64_t D = C / G;
        for (int64_t plane = 0; plane < D; ++plane) {
            std::vector<uint8_t> cov((size_t)HW, 0);
            for (int64_t t = plane * g.tpc; t < (plane + 1) * g.tpc; ++t) {
                int64_t pl, k0;
                nchw_tile_pos(t, g.tpc, te, &pl, &k0);
                CHECK(pl == plane, "tile %lld in plane %lld, expected %lld", (long long)t, (long long)pl, (long long)plane);
                int64_t valid = 0;
                for (int th = 0; th < kThreads; ++th)
                    for (int j = 0; j < R; ++j) {
                        const int64_t e = nchw_chunk_elem(k0, j, th, V);
                        const int64_t ld = nchw_chunk_load(e, HW, V);
                        CHECK(ld >= 0 && ld + V <= HW, "load at %lld outside the plane", (long long)ld);
                        if (e < HW) {
                            CHECK(ld == e, "valid chunk at %lld loads %lld", (long long)e, (long long)ld);
                            for (int k = 0; k < V; ++k) ++cov[(size_t)(e + k)];
                            valid += V;
                        }
                    }
                CHECK(valid == nchw_tile_count(t, g.tpc, te, HW), "tile %lld: %lld valid elements, count %lld",
                      (long long)t, (long long)valid, (long long)nchw_tile_count(t, g.tpc, te, HW));
            }
            for (int64_t e = 0; e < HW; ++e)
                CHECK(cov[(size_t)e] == 1, "plane %lld element %lld covered %d times", (long long)plane, (long long)e,
                      cov[(size_t)e]);
        }
    } else {
        const int CPP = (int)(C / V);
        const int PPI = kThreads / CPP;
        const int64_t tp = nhwc_tile_pixels(C, V, R);
        CHECK(C % V == 0 && CPP >= 1 && kThreads % CPP == 0, "C %lld: chunks per pixel do not divide the workgroup",
              (long long)C);
        CHECK(tp == (int64_t)PPI * R && g.tiles * tp >= HW && (g.tiles - 1) * tp < HW, "tiles do not cover HW");
        // ---- (pixel, chunk) coverage of one sample ----
        std::vector<uint8_t> cov((size_t)(HW * CPP), 0);
        for (int64_t t = 0; t < g.tiles; ++t)
            for (int th = 0; th < kThreads; ++th) {
                const int q = th % CPP, pi = th / CPP;
                for (int j = 0; j < R; ++j) {
                    const int64_t p = nhwc_pixel(t, tp, pi, j, PPI);
                    const int64_t ld = nhwc_pixel_load(p, HW);
                    CHECK(ld >= 0 && ld < HW, "pixel load %lld outside the sample", (long long)ld);
                    if (p < HW) ++cov[(size_t)(p * CPP + q)];
                }
            }
        for (int64_t i = 0; i < HW * CPP; ++i)
            CHECK(cov[(size_t)i] == 1, "pixel %lld chunk %lld covered %d times", (long long)(i / CPP),
                  (long long)(i % CPP), cov[(size_t)i]);
        // ---- the draw protocol under interleavings ----
        std::vector<int> red, wr;
        for (int s = 0; s < seeds + 2; ++s) {
            const int order = s < seeds ? 0 : (s == seeds ? 1 : 2);
            nhwc_run(g.tiles, g.team, order, 0x9E3779B97F4A7C15ull * (uint64_t)(s + 1), red, wr);
            for (int64_t t = 0; t < g.tiles; ++t) {
                CHECK(red[(size_t)t] == 1, "order %d seed %d: tile %lld reduced %d times", order, s, (long long)t,
                      red[(size_t)t]);
                CHECK(wr[(size_t)t] == 1, "order %d seed %d: tile %lld written %d times", order, s, (long long)t,
                      wr[(size_t)t]);
            }
        }
    }
    printf("OK tiles=%lld team=%lld nteams=%lld grid=%lld\n", (long long)g.tiles, (long long)g.team,
           (long long)g.nteams, (long long)g.grid);
    return 0;
}
