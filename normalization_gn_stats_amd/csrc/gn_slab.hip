// gn_slab.hip -- GroupNorm forward and one-pass backward as cooperative
// kernels over contiguous "slabs", with the grid capped at the number of
// co-resident workgroups and overflow tiles handled by a grid-stride loop
// (the design of apex PR #2018: the cooperative grid is capped at the
// residency limit; resident blocks also process the extra activation tiles,
// which join the same reductions in the same launch and are reloaded for the
// dx store after the global reduction -- no fall back to a second pass).
//
// Slab: NHWC -> one sample n (HW pixels x C channels, all G groups
// interleaved, 16 bytes = V channels of one group per chunk); NCHW -> one
// slice (n, g), the contiguous D*HW elements of sample n in group g.
//
// A team of TW workgroups works on one slab at a time (teams walk slabs
// k, k + nteams, ...).  Member m takes the slab's tiles m, m + TW, ... (phase
// 1), keeps the last one in registers, and once the team's partials are in
// writes the outputs of that tile from registers and of the earlier tiles by
// reloading them in reverse order (the most recently read tiles first, the
// ones most likely still in the Infinity Cache).  NHWC members meet at
// counter barriers; NCHW members publish one self-flagging 64-bit word per
// tile and poll their slab's words, sleeping between reads of words not yet
// published.  Slabs of at most GN_SLAB_SOLO_BYTES take a team of one
// workgroup (no exchange, a normal launch); larger teams are launched
// cooperatively, so that every member is resident.  NCHW slabs that fit one
// workgroup's registers (up to GN_SLAB_MID_FWD_BYTES forward and
// GN_SLAB_MID_BWD_BYTES backward) skip the teams altogether: one workgroup
// of 256 or 1024 threads per slab holds the whole slab (small_nchw_*); a
// backward slab of up to GN_SLAB_MID_BWD_STREAM_BYTES keeps part of x and dy
// in registers and streams the rest twice (mid_nchw_bwd); small NCHW tensors
// with larger slabs take two ordinary launches (split_nchw_*).
//
// Reductions (all in a fixed order, no float atomics):
//  forward   per thread: exact two-pass (count, mean, M2) of each tile from
//            registers, merged across tiles and threads with Chan et al.'s
//            pairwise update;
//  backward  per-(n, c) sums of dy and dy*xhat (xhat from the saved mean/rstd);
//            per slice A = sum_c gamma_c*S1[n,c], B = sum_c gamma_c*S2[n,c]
//            (the per-group reduction of the baracuda-kernels backward plan,
//            regrouped by channel), dgamma_c = sum_n S2[n,c], dbeta_c = sum_n S1[n,c].
#include "gn_device.hpp"
#include "gn_internal.hpp"
#include "gn_slab_plan.hpp"

namespace gn {
namespace {

constexpr int kT = slab::kThreads;
constexpr int kNW = kT / kWave;

struct SlabCfg {
    int64_t N, C, HW, G, D;
    int64_t n_slabs;   // NHWC: N, NCHW: N*G
    int64_t tiles;     // tiles per slab
    int64_t tpc;       // NCHW: tiles per channel plane
    int64_t pstride;   // NCHW: partial slots per slab (tiles rounded up to whole 128-byte lines)
    int32_t team;      // workgroups per team
    int32_t nteams;
    float eps;
    int32_t want_dx;   // backward: write dx
    float* dgamma;     // backward, one-slab case: written by the finalizers
    float* dbeta;
    uint32_t spin_limit;   // polls before a wait between workgroups gives up
    uint32_t unmet;        // 1: every wait's target out of reach (failure-report tests)
};

__device__ inline float qnan() { return __uint_as_float(0x7FC00000u); }

// ============================================================================
// NHWC
// ============================================================================
// Thread t owns chunk q = t % CPP of each pixel it visits (channels q*V ..
// q*V+V-1, all in group q*V/D) and pixel t / CPP of each iteration; a tile is
// R iterations, i.e. R*PPI consecutive pixels.
//
// Tiles are handed out dynamically (an atomic tile counter per slab), so that
// faster workgroups take more of them -- the barrier then waits for less.  The
// partial statistics are kept per tile and merged in tile order, so the result
// does not depend on which workgroup took which tile.  Each member keeps its
// last tile in registers and flags it resident; after the barriers, phase 2
// hands out the remaining tiles from a second counter, in reverse order.
//
// Sync words per slab: [0] barrier 1, [1] barrier 2, [2] phase-1 tile counter,
// [3] phase-2 tile counter; res[slab][tile] = 1 for resident tiles.

// Takes the next tile of a counter (thread 0 draws, the workgroup shares it).
__device__ inline int64_t grab_tile(uint32_t* counter, int* s_slot) {
    if (threadIdx.x == 0) *s_slot = (int)__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t tile = *s_slot;
    __syncthreads();
    return tile;
}

// Phase-2 tiles: the second counter runs over all tiles in reverse order
// (most recently read first); resident tiles (flag set in phase 1, before the
// barriers) are skipped.  Returns -1 when the counter is exhausted.  The flags
// are read with plain loads: written once, through to the coherence point,
// before the first barrier and not read by anyone before it.
__device__ inline int64_t grab_phase2_tile(uint32_t* counter, const uint32_t* res, int64_t tiles, int* s_slot) {
    while (true) {
        const int64_t tile = slab::nhwc_phase2_tile(grab_tile(counter, s_slot), tiles);
        if (tile < 0) return -1;
        if (!res[tile]) return tile;
    }
}

template <typename T, int R>
__device__ inline void nhwc_load(const T* __restrict__ src, int64_t HW, int64_t C, int64_t p0, int PPI, u4v (&dst)[R]) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
        // in bounds; dropped by the caller if past HW
        const int64_t p = slab::nhwc_pixel_load(p0 + (int64_t)j * PPI, HW);
        dst[j] = ld16_nt(src + p * C);
    }
}

template <typename T, int R>
__global__ __launch_bounds__(kT) void slab_nhwc_fwd(const T* __restrict__ x, const float* __restrict__ gamma,
                                                    const float* __restrict__ beta, T* __restrict__ y,
                                                    float* mean, float* rstd, SlabCfg cfg, uint32_t* ctr,
                                                    uint32_t* err, float4* part, uint32_t* res) {
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int CPP = (int)(cfg.C / V);
    const int q = t % CPP;
    const int pi = t / CPP;
    const int PPI = kT / CPP;
    const int64_t TP = slab::nhwc_tile_pixels(cfg.C, V, R);
    const int gq = (q * V) / (int)cfg.D;
    const int qpg = (int)cfg.D / V;   // chunks per group
    const int team = blockIdx.x / cfg.team;
    const int m = blockIdx.x - team * cfg.team;
    const int G = (int)cfg.G;
    __shared__ Stat sst[kT];
    __shared__ float lds[kNW * 2];
    __shared__ int s_tile;

    for (int64_t sb = team; sb < cfg.n_slabs; sb += cfg.nteams) {
        const int64_t n = sb;
        uint32_t* sw = ctr + sb * 4;
        const uint32_t* rs_flags = res + sb * cfg.tiles;
        const T* xs = x + n * cfg.HW * cfg.C + q * V;
        u4v cur[R], nxt[R];
        int64_t last = -1;
        // ---- phase 1: statistics of every tile this member takes; the next
        // tile is drawn and its loads issued before the current one is used ----
        int64_t tile = grab_tile(&sw[2], &s_tile);
        if (tile < cfg.tiles) nhwc_load<T, R>(xs, cfg.HW, cfg.C, tile * TP + pi, PPI, cur);
        while (tile < cfg.tiles) {
            const int64_t ntile = grab_tile(&sw[2], &s_tile);
            if (ntile < cfg.tiles) nhwc_load<T, R>(xs, cfg.HW, cfg.C, ntile * TP + pi, PPI, nxt);
            const int64_t p0 = tile * TP + pi;
            float s = 0.f;
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                if (p0 + (int64_t)j * PPI < cfg.HW) {
                    float v[V];
                    Vec<T>::unpack(cur[j], v);
#pragma unroll
                    for (int k = 0; k < V; ++k) s += v[k];
                    cnt += V;
                }
            }
            Stat st = stat_empty();
            if (cnt > 0) {
                const float mt = s / (float)cnt;
                float m2 = 0.f;
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    if (p0 + (int64_t)j * PPI < cfg.HW) {
                        float v[V];
                        Vec<T>::unpack(cur[j], v);
#pragma unroll
                        for (int k = 0; k < V; ++k) {
                            const float d = v[k] - mt;
                            m2 = fmaf(d, d, m2);
                        }
                    }
                }
                st = Stat{(float)cnt, mt, m2};
            }
            // per-group statistics of the tile: the group's threads, in thread order
            sst[t] = st;
            __syncthreads();
            for (int g = t; g < G; g += kT) {
                Stat a = stat_empty();
                for (int i = 0; i < PPI; ++i)
                    for (int qq = g * qpg; qq < (g + 1) * qpg; ++qq) a = stat_merge(a, sst[i * CPP + qq]);
                xstore_stat(&part[(sb * G + g) * cfg.pstride + tile], a);
            }
            __syncthreads();
            last = tile;
            if (ntile >= cfg.tiles) break;   // cur keeps the last tile
#pragma unroll
            for (int j = 0; j < R; ++j) cur[j] = nxt[j];
            tile = ntile;
        }
        if (last >= 0 && t == 0) __hip_atomic_store(&res[sb * cfg.tiles + last], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // a member whose wait gave up merges incomplete partials: it writes
        // NaN statistics instead (and, after the second wait, NaN outputs)
        const bool all_tiles = team_barrier(&sw[0], (uint32_t)cfg.team, err, cfg.spin_limit, cfg.unmet);

        // ---- distributed finalize: member m owns groups m, m + team, ... ----
        // tile partials merged in tile order: mean = sum(n_i*mean_i)/sum(n_i),
        // M2 = sum(M2_i + n_i*(mean_i - mean)^2), each a fixed-order workgroup
        // sum.  Plain loads: each (slab, group) block of partials is written
        // once before the barrier, through to the coherence point, and padded
        // to whole 128-byte lines, so no XCD holds a stale copy.
        for (int g = m; g < G; g += cfg.team) {
            const float4* pg = part + (sb * G + g) * cfg.pstride;
            float sums[2] = {0.f, 0.f};
            for (int64_t i = t; i < cfg.tiles; i += kT) {
                const float4 v = pg[i];
                sums[0] = fmaf(v.x, v.y, sums[0]);
                sums[1] += v.x;
            }
            block_sum<2, kNW>(sums, lds);
            const float mu = sums[0] / sums[1];
            float m2[1] = {0.f};
            for (int64_t i = t; i < cfg.tiles; i += kT) {
                const float4 v = pg[i];
                const float d = v.y - mu;
                m2[0] += fmaf(v.x * d, d, v.z);
            }
            block_sum<1, kNW>(m2, lds);
            if (t == 0) {
                float var = m2[0] / (float)(cfg.D * cfg.HW);
                var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
                xstore(&mean[n * G + g], all_tiles ? mu : qnan());
                xstore(&rstd[n * G + g], all_tiles ? 1.0f / sqrtf(var + cfg.eps) : qnan());
            }
        }
        const bool all_stats = team_barrier(&sw[1], (uint32_t)cfg.team, err, cfg.spin_limit, cfg.unmet);
        if (y == nullptr) continue;

        // ---- phase 2: normalize + affine; the resident tile, then tiles
        // drawn in reverse order (next tile's loads issued before the current
        // one is written); streaming stores for y ----
        const float mu = all_stats ? xload(&mean[n * G + gq]) : qnan();
        const float r = all_stats ? xload(&rstd[n * G + gq]) : qnan();
        float a[V], b[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int c = q * V + k;
            a[k] = r * (gamma ? gamma[c] : 1.f);
            b[k] = beta ? beta[c] : 0.f;
        }
        T* ys = y + n * cfg.HW * cfg.C + q * V;
        tile = last;
        if (tile < 0) {
            tile = grab_phase2_tile(&sw[3], rs_flags, cfg.tiles, &s_tile);
            if (tile >= 0) nhwc_load<T, R>(xs, cfg.HW, cfg.C, tile * TP + pi, PPI, cur);
        }
        while (tile >= 0) {
            const int64_t ntile = grab_phase2_tile(&sw[3], rs_flags, cfg.tiles, &s_tile);
            if (ntile >= 0) nhwc_load<T, R>(xs, cfg.HW, cfg.C, ntile * TP + pi, PPI, nxt);
            const int64_t p0 = tile * TP + pi;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int64_t p = p0 + (int64_t)j * PPI;
                if (p < cfg.HW) {
                    float v[V], o[V];
                    Vec<T>::unpack(cur[j], v);
#pragma unroll
                    for (int k = 0; k < V; ++k) o[k] = fmaf(v[k] - mu, a[k], b[k]);
                    st16_nt(ys + p * cfg.C, Vec<T>::pack(o));
                }
            }
            if (ntile < 0) break;
#pragma unroll
            for (int j = 0; j < R; ++j) cur[j] = nxt[j];
            tile = ntile;
        }
    }
}

// part: [slab][C][pstride] float2 per-tile channel sums; stot: [N][C] float2.
template <typename T, int R>
__global__ __launch_bounds__(kT) void slab_nhwc_bwd(const T* __restrict__ dy, const T* __restrict__ x,
                                                    const float* __restrict__ mean,
                                                    const float* __restrict__ rstd,
                                                    const float* __restrict__ gamma, T* __restrict__ dx,
                                                    SlabCfg cfg, uint32_t* ctr, uint32_t* err, float2* part,
                                                    float2* stot, uint32_t* res) {
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int CPP = (int)(cfg.C / V);
    const int q = t % CPP;
    const int pi = t / CPP;
    const int PPI = kT / CPP;
    const int64_t TP = slab::nhwc_tile_pixels(cfg.C, V, R);
    const int gq = (q * V) / (int)cfg.D;
    const int team = blockIdx.x / cfg.team;
    const int m = blockIdx.x - team * cfg.team;
    const int G = (int)cfg.G;
    const int C = (int)cfg.C;
    __shared__ float lds[kNW * 2];
    __shared__ float2 lds_ch[kT * 8];   // [thread][k] per-thread channel sums (V <= 8)
    __shared__ int s_tile;

    for (int64_t sb = team; sb < cfg.n_slabs; sb += cfg.nteams) {
        const int64_t n = sb;
        uint32_t* sw = ctr + sb * 4;
        const uint32_t* rs_flags = res + sb * cfg.tiles;
        const int64_t off = n * cfg.HW * cfg.C + q * V;
        const float mu = mean[n * G + gq];
        const float r = rstd[n * G + gq];
        u4v cx[R], cd[R], nx[R], nd[R];
        int64_t last = -1;
        // ---- phase 1: per-tile channel sums of every tile this member takes ----
        int64_t tile = grab_tile(&sw[2], &s_tile);
        if (tile < cfg.tiles) {
            nhwc_load<T, R>(x + off, cfg.HW, cfg.C, tile * TP + pi, PPI, cx);
            nhwc_load<T, R>(dy + off, cfg.HW, cfg.C, tile * TP + pi, PPI, cd);
        }
        while (tile < cfg.tiles) {
            const int64_t ntile = grab_tile(&sw[2], &s_tile);
            if (ntile < cfg.tiles) {
                nhwc_load<T, R>(x + off, cfg.HW, cfg.C, ntile * TP + pi, PPI, nx);
                nhwc_load<T, R>(dy + off, cfg.HW, cfg.C, ntile * TP + pi, PPI, nd);
            }
            const int64_t p0 = tile * TP + pi;
            float s1[V], s2[V];
#pragma unroll
            for (int k = 0; k < V; ++k) { s1[k] = 0.f; s2[k] = 0.f; }
#pragma unroll
            for (int j = 0; j < R; ++j) {
                if (p0 + (int64_t)j * PPI < cfg.HW) {
                    float xv[V], dv[V];
                    Vec<T>::unpack(cx[j], xv);
                    Vec<T>::unpack(cd[j], dv);
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        s1[k] += dv[k];
                        s2[k] = fmaf(dv[k], (xv[k] - mu) * r, s2[k]);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < V; ++k) lds_ch[t * 8 + k] = make_float2(s1[k], s2[k]);
            __syncthreads();
            for (int c = t; c < C; c += kT) {
                const int cq = c / V, ck = c - cq * V;
                float2 acc = make_float2(0.f, 0.f);
                for (int i = 0; i < PPI; ++i) {
                    const float2 v = lds_ch[(i * CPP + cq) * 8 + ck];
                    acc.x += v.x;
                    acc.y += v.y;
                }
                xstore2(&part[(sb * C + c) * cfg.pstride + tile], acc);
            }
            __syncthreads();
            last = tile;
            if (ntile >= cfg.tiles) break;   // cx, cd keep the last tile
#pragma unroll
            for (int j = 0; j < R; ++j) { cx[j] = nx[j]; cd[j] = nd[j]; }
            tile = ntile;
        }
        if (last >= 0 && t == 0) __hip_atomic_store(&res[sb * cfg.tiles + last], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // a member whose wait gave up writes NaN channel sums (and dx below)
        const bool all_tiles = team_barrier(&sw[0], (uint32_t)cfg.team, err, cfg.spin_limit, cfg.unmet);

        // ---- distributed finalize: member m owns channels m, m + team, ...
        // (plain loads of the tile partials: see slab_nhwc_fwd) ----
        for (int c = m; c < C; c += cfg.team) {
            const float2* pc = part + (sb * C + c) * cfg.pstride;
            float acc[2] = {0.f, 0.f};
            for (int64_t i = t; i < cfg.tiles; i += kT) {
                const float2 v = pc[i];
                acc[0] += v.x;
                acc[1] += v.y;
            }
            block_sum<2, kNW>(acc, lds);
            if (t == 0) {
                if (!all_tiles) acc[0] = acc[1] = qnan();
                xstore2(&stot[n * C + c], make_float2(acc[0], acc[1]));
                if (cfg.dbeta) cfg.dbeta[c] = acc[0];     // one-slab case: final already
                if (cfg.dgamma) cfg.dgamma[c] = acc[1];
            }
        }
        if (!cfg.want_dx) continue;   // uniform over the grid: no member waits below
        const bool all_sums = team_barrier(&sw[1], (uint32_t)cfg.team, err, cfg.spin_limit, cfg.unmet);

        // ---- phase 2: dx = rstd*(gamma_c*dy - A/M - xhat*B/M) ----
        float A = 0.f, B = 0.f;
        for (int c = gq * (int)cfg.D; c < (gq + 1) * (int)cfg.D; ++c) {
            const float2 v = xload2(&stot[n * C + c]);
            const float ga = gamma ? gamma[c] : 1.f;
            A = fmaf(ga, v.x, A);
            B = fmaf(ga, v.y, B);
        }
        const float invM = 1.0f / (float)(cfg.D * cfg.HW);
        A = all_sums ? A * invM : qnan();
        B = all_sums ? B * invM : qnan();
        float ga[V];
#pragma unroll
        for (int k = 0; k < V; ++k) ga[k] = gamma ? gamma[q * V + k] : 1.f;
        tile = last;
        if (tile < 0) {
            tile = grab_phase2_tile(&sw[3], rs_flags, cfg.tiles, &s_tile);
            if (tile >= 0) {
                nhwc_load<T, R>(x + off, cfg.HW, cfg.C, tile * TP + pi, PPI, cx);
                nhwc_load<T, R>(dy + off, cfg.HW, cfg.C, tile * TP + pi, PPI, cd);
            }
        }
        while (tile >= 0) {
            const int64_t ntile = grab_phase2_tile(&sw[3], rs_flags, cfg.tiles, &s_tile);
            if (ntile >= 0) {
                nhwc_load<T, R>(x + off, cfg.HW, cfg.C, ntile * TP + pi, PPI, nx);
                nhwc_load<T, R>(dy + off, cfg.HW, cfg.C, ntile * TP + pi, PPI, nd);
            }
            const int64_t p0 = tile * TP + pi;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int64_t p = p0 + (int64_t)j * PPI;
                if (p < cfg.HW) {
#pragma clang fp contract(off)
                    float xv[V], dv[V], o[V];
                    Vec<T>::unpack(cx[j], xv);
                    Vec<T>::unpack(cd[j], dv);
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        const float xh = (xv[k] - mu) * r;
                        const float gd = dv[k] * ga[k];
                        o[k] = r * ((gd - A) - xh * B);
                    }
                    st16_nt(dx + off + p * cfg.C, Vec<T>::pack(o));
                }
            }
            if (ntile < 0) break;
#pragma unroll
            for (int j = 0; j < R; ++j) { cx[j] = nx[j]; cd[j] = nd[j]; }
            tile = ntile;
        }
    }
}

// ============================================================================
// NCHW
// ============================================================================
// Slab (n, g) is D contiguous channel planes of HW elements.  Tiles never
// straddle a plane: tile = (plane cl, k) covers elements [k*TE, (k+1)*TE) of
// plane cl, TE = kT*R*V; chunk j of thread t is element k*TE + (j*kT + t)*V.
//
// Tile partials of the NCHW kernels: one 64-bit word per tile, all ones until
// the tile's member publishes it (the launch's clear kernel fills the block).
// The value is its own ready flag: the writer issues one agent-scope atomic
// store and goes on (no counter, no fence, no wait for the store), and the
// readers poll the words they need.  Neither half of a published word holds
// the all-ones pattern (that NaN is stored as the canonical quiet NaN), and a
// reader takes a word only when neither half does, so it never takes a word
// that is unpublished or, were the 8-byte store ever seen in halves, half
// published.  A wave's memory operations complete in issue
// order, so a member that waits for its own store before signalling -- as a
// counter barrier must -- also waits for all the bulk traffic it issued
// before it; polling the data itself takes that drain off every round.

__device__ inline bool unpublished(uint64_t w) {
    return (uint32_t)w == 0xFFFFFFFFu || (uint32_t)(w >> 32) == 0xFFFFFFFFu;
}

__device__ inline void put_partial(uint64_t* p, float lo, float hi) {
    uint32_t l = __float_as_uint(lo), h = __float_as_uint(hi);
    if (l == 0xFFFFFFFFu) l = 0x7FC00000u;
    if (h == 0xFFFFFFFFu) h = 0x7FC00000u;
    const uint64_t w = (uint64_t)l | ((uint64_t)h << 32);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t peek_partial(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sleep between two reads of a word not yet published, in units of 64
// clocks (s_sleep), per kernel.  Every member of a team polls all of its
// slab's words at once, so each round of re-reads puts one agent-scope load
// per word and member in front of the bulk traffic at the coherence point;
// polling slowly leaves HBM to the data.  112 x 64 x 512 x 512, three
// alternating rounds: fp32 backward 4028-4042 us with a sleep of 1, 3988-4016
// with 8, 3886-3906 with 32, 3837-3871 with 64, 3877-3897 with 127; fp32
// forward 2632-2637 us with 1, 2597-2612 with 64, 2569-2575 with 127; bf16
// backward (twice the tiles per slab) 2206-2211 us with 32, 2173-2177 with 64,
// 2153-2157 with 127.
#ifndef GN_SLAB_POLL_SLEEP_F
#define GN_SLAB_POLL_SLEEP_F 127
#endif
#ifndef GN_SLAB_POLL_SLEEP_B
#define GN_SLAB_POLL_SLEEP_B 64     // fp32
#endif
#ifndef GN_SLAB_POLL_SLEEP_B16
#define GN_SLAB_POLL_SLEEP_B16 127  // fp16, bf16
#endif
static_assert(GN_SLAB_POLL_SLEEP_F >= 1 && GN_SLAB_POLL_SLEEP_F <= 127, "s_sleep takes 1..127");
static_assert(GN_SLAB_POLL_SLEEP_B >= 1 && GN_SLAB_POLL_SLEEP_B <= 127, "s_sleep takes 1..127");
static_assert(GN_SLAB_POLL_SLEEP_B16 >= 1 && GN_SLAB_POLL_SLEEP_B16 <= 127, "s_sleep takes 1..127");

// Waits until *p is published, w being a first read of it; returns (lo, hi).
// Bounded: after cfg.spin_limit polls it ORs kWaitExpired into *err and
// returns NaNs, which every sum, statistic and output derived from the
// partial then carries.  cfg.unmet (tests of the failure report) makes every
// word read as unpublished.
template <int kSleep>
__device__ inline float2 settle_partial(const uint64_t* p, uint64_t w, const SlabCfg& cfg, uint32_t* err) {
    uint32_t spins = 0;
    while (unpublished(w) || cfg.unmet) {
        if (cfg.team == 1)
            __builtin_amdgcn_s_sleep(1);   // the workgroup's own word, about to land
        else
            __builtin_amdgcn_s_sleep(kSleep);
        if (++spins > cfg.spin_limit) {
            __hip_atomic_fetch_or(err, kWaitExpired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            w = ~0ull;   // both halves NaN
            break;
        }
        w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return make_float2(__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32)));
}

template <int kSleep>
__device__ inline float2 poll_partial(const uint64_t* p, const SlabCfg& cfg, uint32_t* err) {
    return settle_partial<kSleep>(p, peek_partial(p), cfg, err);
}

// Elements of NCHW tile `tile` (the last tile of each channel plane may be
// short), as a float.
__device__ inline float nchw_tile_count(const SlabCfg& cfg, int64_t tile, int64_t TE) {
    return (float)slab::nchw_tile_count(tile, cfg.tpc, TE, cfg.HW);
}

// The thread index, opaque to the optimiser: the per-chunk element offsets of a
// tile derived from it are then recomputed in each phase instead of being
// hoisted out of the slab loop, where 32 of them, held in 64-bit registers
// next to two register tiles, spill.
__device__ inline int tile_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// A member prefetches its first tile of the team's next slab before it waits
// for the current slab's partials, so that HBM keeps streaming while the team
// synchronises (a second register tile).
// Non-temporal loads; the outputs are written with non-temporal stores too
// (forward on 112 x 64 x 512 x 512 against plain stores: fp32 2.72 -> 2.66 ms,
// bf16 1.48 -> 1.44 ms; then non-temporal forward loads: 2.65 -> 2.63 ms and
// 1.443 -> 1.429 ms).
template <typename T, int R>
__device__ inline void nchw_load_tile(const T* __restrict__ src, const SlabCfg& cfg, int64_t sb, int64_t tile,
                                      u4v (&dst)[R]) {
    constexpr int V = Vec<T>::V;
    constexpr int64_t TE = slab::nchw_tile_elems(V, R);
    const int64_t n = sb / cfg.G, g = sb - n * cfg.G;
    int64_t cl, k0;
    slab::nchw_tile_pos(tile, cfg.tpc, TE, &cl, &k0);
    const T* p = src + (n * cfg.C + g * cfg.D + cl) * cfg.HW;
    const int t = tile_tid();
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t e = slab::nchw_chunk_load(slab::nchw_chunk_elem(k0, j, t, V), cfg.HW, V);   // in bounds
        dst[j] = ld16_nt(p + e);
    }
}

// Phase 1 of the forward for slab sb: statistics of member m's tiles, one
// published (mean, M2) partial per tile -- an exact two-pass over the tile in registers: workgroup
// sum -> tile mean -> workgroup sum of squared deviations.  The last tile
// stays in buf; its channel's gamma/beta are fetched here so that phase 2 does
// not wait for them.  Returns the last tile index (-1 if the member has none).
template <typename T, int R>
__device__ inline int64_t nchw_fwd_phase1(const T* __restrict__ x, const float* __restrict__ gamma,
                                          const float* __restrict__ beta, const SlabCfg& cfg, int64_t sb, int m,
                                          u4v (&buf)[R], float2& gb, uint64_t* part, float* lds) {
    constexpr int V = Vec<T>::V;
    constexpr int64_t TE = slab::nchw_tile_elems(V, R);
    const int t = tile_tid();
    int64_t last = -1;
    for (int64_t tile = m; tile < cfg.tiles; tile += cfg.team) {
        int64_t cl, k0;
        slab::nchw_tile_pos(tile, cfg.tpc, TE, &cl, &k0);
        nchw_load_tile<T, R>(x, cfg, sb, tile, buf);
        const int64_t c = (sb - (sb / cfg.G) * cfg.G) * cfg.D + cl;
        gb = make_float2(gamma ? gamma[c] : 1.f, beta ? beta[c] : 0.f);
        const int64_t rem = cfg.HW - k0;
        const float cnt = (float)(rem < TE ? rem : TE);   // elements of this tile
        float acc[1] = {0.f};
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (slab::nchw_chunk_elem(k0, j, t, V) < cfg.HW) {
                float v[V];
                Vec<T>::unpack(buf[j], v);
#pragma unroll
                for (int k = 0; k < V; ++k) acc[0] += v[k];
            }
        }
        block_sum<1, kNW>(acc, lds);
        const float mt = acc[0] / cnt;
        if constexpr (sizeof(T) == 2) {
            // 16-bit tiles are unpacked again below rather than kept as
            // floats across the workgroup sum: bf16 tiles of 8 chunks then take
            // 122 instead of 167 VGPRs, four workgroups per CU instead of three
            // (112 x 64 x 512 x 512 bf16 forward 1.43 -> 1.37 ms)
#pragma unroll
            for (int j = 0; j < R; ++j) asm volatile("" : "+v"(buf[j]));
        }
        float q[1] = {0.f};
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (slab::nchw_chunk_elem(k0, j, t, V) < cfg.HW) {
                float v[V];
                Vec<T>::unpack(buf[j], v);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float d = v[k] - mt;
                    q[0] = fmaf(d, d, q[0]);
                }
            }
        }
        block_sum<1, kNW>(q, lds);
        if (t == 0) put_partial(&part[sb * cfg.pstride + tile], mt, q[0]);
        last = tile;
    }
    return last;
}

// Phase 2 of the forward for slab sb: every member waits for and combines all
// tile partials in the same order -- slab mean = sum(n_i*mean_i)/sum(n_i),
// then M2 = sum(M2_i + n_i*(mean_i - mean)^2) (the parallel form of Chan et
// al.'s update), each a fixed-order workgroup sum -- then writes y for its
// tiles (the last one from buf, the earlier ones reloaded in reverse order).
template <typename T, int R>
__device__ inline void nchw_fwd_phase2(const T* __restrict__ x, const float* __restrict__ gamma,
                                       const float* __restrict__ beta, T* __restrict__ y, float* mean,
                                       float* rstd, const SlabCfg& cfg, int64_t sb, int m, int64_t last,
                                       u4v (&buf)[R], float2 gb, const uint64_t* part, uint32_t* err, float* lds) {
    constexpr int V = Vec<T>::V;
    constexpr int64_t TE = slab::nchw_tile_elems(V, R);
    constexpr int kKeep = 1;   // partials a thread keeps in registers (slabs of up to kKeep * kT tiles)
    const int t = tile_tid();
    const int64_t n = sb / cfg.G, g = sb - n * cfg.G;
    const uint64_t* ps = part + sb * cfg.pstride;
    uint64_t w[kKeep];
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {   // all first reads in flight together
        const int64_t i = t + (int64_t)k * kT;
        w[k] = i < cfg.tiles ? peek_partial(ps + i) : 0;
    }
    float2 keep[kKeep];
    float sums[2] = {0.f, 0.f};   // sum n_i*mean_i, sum n_i
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
        const int64_t i = t + (int64_t)k * kT;
        keep[k] = make_float2(0.f, 0.f);
        if (i < cfg.tiles) {
            keep[k] = settle_partial<GN_SLAB_POLL_SLEEP_F>(ps + i, w[k], cfg, err);
            const float c = nchw_tile_count(cfg, i, TE);
            sums[0] = fmaf(c, keep[k].x, sums[0]);
            sums[1] += c;
        }
    }
    for (int64_t i = t + (int64_t)kKeep * kT; i < cfg.tiles; i += kT) {
        const float2 v = poll_partial<GN_SLAB_POLL_SLEEP_F>(ps + i, cfg, err);
        const float c = nchw_tile_count(cfg, i, TE);
        sums[0] = fmaf(c, v.x, sums[0]);
        sums[1] += c;
    }
    block_sum<2, kNW>(sums, lds);
    const float mu = sums[0] / sums[1];
    float m2[1] = {0.f};
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
        const int64_t i = t + (int64_t)k * kT;
        if (i < cfg.tiles) {
            const float c = nchw_tile_count(cfg, i, TE);
            const float d = keep[k].x - mu;
            m2[0] += fmaf(c * d, d, keep[k].y);
        }
    }
    for (int64_t i = t + (int64_t)kKeep * kT; i < cfg.tiles; i += kT) {
        const float2 v = poll_partial<GN_SLAB_POLL_SLEEP_F>(ps + i, cfg, err);   // published: returns at once
        const float c = nchw_tile_count(cfg, i, TE);
        const float d = v.x - mu;
        m2[0] += fmaf(c * d, d, v.y);
    }
    block_sum<1, kNW>(m2, lds);
    float var = m2[0] / (float)(cfg.D * cfg.HW);
    var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
    const float r = 1.0f / sqrtf(var + cfg.eps);
    if (m == 0 && t == 0) {
        mean[sb] = mu;
        rstd[sb] = r;
    }
    if (y == nullptr) return;
    const int64_t base = (n * cfg.C + g * cfg.D) * cfg.HW;
    for (int64_t tile = last; tile >= 0; tile -= cfg.team) {
        int64_t cl, k0;
        slab::nchw_tile_pos(tile, cfg.tpc, TE, &cl, &k0);
        float2 p = gb;
        if (tile != last) {
            nchw_load_tile<T, R>(x, cfg, sb, tile, buf);
            const int64_t c = g * cfg.D + cl;
            p = make_float2(gamma ? gamma[c] : 1.f, beta ? beta[c] : 0.f);
        }
        const float a_c = r * p.x;
        const float b_c = p.y;
        T* dst = y + base + cl * cfg.HW;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t e = slab::nchw_chunk_elem(k0, j, t, V);
            if (e < cfg.HW) {
                float v[V], o[V];
                Vec<T>::unpack(buf[j], v);
#pragma unroll
                for (int k = 0; k < V; ++k) o[k] = fmaf(v[k] - mu, a_c, b_c);
                st16_nt(dst + e, Vec<T>::pack(o));
            }
        }
    }
}

// Two slabs in flight per team: a member publishes the partials of slab s,
// then runs phase 1 of the team's next slab (loads, statistics, publish)
// before it needs the partials of s, so that they have had a whole phase to
// arrive.  (Measured slower: prefetching the next slab's first tile, then
// phase 2 of s while it streams, then phase 1 from registers.)
template <typename T, int R>
__global__ __launch_bounds__(kT) void slab_nchw_fwd(const T* __restrict__ x, const float* __restrict__ gamma,
                                                    const float* __restrict__ beta, T* __restrict__ y,
                                                    float* mean, float* rstd, SlabCfg cfg, uint32_t* /*ctr*/,
                                                    uint32_t* err, uint64_t* part, uint32_t* /*res: NHWC only*/) {
    const int team = blockIdx.x / cfg.team;
    const int m = blockIdx.x - team * cfg.team;
    __shared__ float lds[kNW * 2];
    u4v cur[R], nxt[R];
    float2 gcur = make_float2(1.f, 0.f), gnxt = gcur;
    int64_t sb = team;
    if (sb >= cfg.n_slabs) return;   // uniform over the team
    int64_t last = nchw_fwd_phase1<T, R>(x, gamma, beta, cfg, sb, m, cur, gcur, part, lds);
    while (true) {
        const int64_t nsb = sb + cfg.nteams;
        const bool more = nsb < cfg.n_slabs;   // uniform over the team
        int64_t nlast = -1;
        if (more) nlast = nchw_fwd_phase1<T, R>(x, gamma, beta, cfg, nsb, m, nxt, gnxt, part, lds);
        __builtin_amdgcn_sched_barrier(0);   // keep the two slabs' phases apart
        nchw_fwd_phase2<T, R>(x, gamma, beta, y, mean, rstd, cfg, sb, m, last, cur, gcur, part, err, lds);
        if (!more) break;
        // register moves (folded into one copy before unrolling: no pragma)
        for (int j = 0; j < R; ++j) cur[j] = nxt[j];
        gcur = gnxt;
        last = nlast;
        sb = nsb;
    }
}

// Phase 1 of the backward for slab sb: per-tile sums of dy and dy*xhat of
// member m's tiles, published per tile;
// the last tile of x and dy stays in bx, bd.  mu, r: the slab's saved
// statistics, loaded by the caller ahead of the bulk traffic (a wave's loads
// complete in issue order, so a late small load waits for all of it).
template <typename T, int R>
__device__ inline int64_t nchw_bwd_phase1(const T* __restrict__ dy, const T* __restrict__ x,
                                          const SlabCfg& cfg, int64_t sb, int m,
                                          float mu, float r, u4v (&bx)[R], u4v (&bd)[R], uint64_t* part,
                                          float* lds) {
    constexpr int V = Vec<T>::V;
    constexpr int64_t TE = slab::nchw_tile_elems(V, R);
    const int t = tile_tid();
    int64_t last = -1;
    for (int64_t tile = m; tile < cfg.tiles; tile += cfg.team) {
        int64_t cl, k0;
        slab::nchw_tile_pos(tile, cfg.tpc, TE, &cl, &k0);
        nchw_load_tile<T, R>(x, cfg, sb, tile, bx);
        nchw_load_tile<T, R>(dy, cfg, sb, tile, bd);
        float acc[2] = {0.f, 0.f};
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (slab::nchw_chunk_elem(k0, j, t, V) < cfg.HW) {
                float xv[V], dv[V];
                Vec<T>::unpack(bx[j], xv);
                Vec<T>::unpack(bd[j], dv);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    acc[0] += dv[k];
                    acc[1] = fmaf(dv[k], (xv[k] - mu) * r, acc[1]);
                }
            }
        }
        block_sum<2, kNW>(acc, lds);
        if (t == 0) put_partial(&part[sb * cfg.pstride + tile], acc[0], acc[1]);
        last = tile;
    }
    return last;
}

constexpr int kStage = 1024;   // tile partials staged in LDS per step of the channel sums

// Phase 2 of the backward for slab sb: per-channel sums of the slab (each in
// tile order, partials waited for and staged through LDS), A and B (channel
// order), then dx for the member's tiles (last from registers, the others
// reloaded).  gam: gamma of channel t of the slab's group (t < D), loaded by
// the caller ahead of the bulk traffic; shared through LDS (gch).
template <typename T, int R>
__device__ inline void nchw_bwd_phase2(const T* __restrict__ dy, const T* __restrict__ x,
                                       T* __restrict__ dx, const SlabCfg& cfg,
                                       int64_t sb, int m, int64_t last, float mu, float r, u4v (&bx)[R],
                                       u4v (&bd)[R], float gam, const uint64_t* part, uint32_t* err,
                                       float2* stot, float2* stage, float2* chan, float* gch) {
    constexpr int V = Vec<T>::V;
    constexpr int64_t TE = slab::nchw_tile_elems(V, R);
    constexpr int kPer = kStage / kT;
    const int t = tile_tid();
    const int64_t n = sb / cfg.G, g = sb - n * cfg.G;
    // channel sums: tiles cl*tpc .. cl*tpc+tpc-1 belong to channel cl
    float2 run = make_float2(0.f, 0.f);   // thread cl's running sum (cl < D <= kT)
    for (int64_t s0 = 0; s0 < cfg.tiles; s0 += kStage) {
        const int64_t cnt = cfg.tiles - s0 < kStage ? cfg.tiles - s0 : kStage;
        const uint64_t* ps = part + sb * cfg.pstride + s0;
        uint64_t w[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {   // all first reads in flight together
            const int64_t i = t + (int64_t)k * kT;
            w[k] = i < cnt ? peek_partial(ps + i) : 0;
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int64_t i = t + (int64_t)k * kT;
            if (i < cnt)
                stage[i] = settle_partial<sizeof(T) == 4 ? GN_SLAB_POLL_SLEEP_B : GN_SLAB_POLL_SLEEP_B16>(
                    ps + i, w[k], cfg, err);
        }
        __syncthreads();
        if (t < cfg.D) {
            const int64_t lo = (int64_t)t * cfg.tpc, hi = lo + cfg.tpc;
            for (int64_t i = lo > s0 ? lo : s0; i < hi && i < s0 + cnt; ++i) {
                run.x += stage[i - s0].x;
                run.y += stage[i - s0].y;
            }
        }
        __syncthreads();
    }
    if (t < cfg.D) {
        chan[t] = run;
        gch[t] = gam;
        if (m == 0) stot[n * cfg.C + g * cfg.D + t] = run;
    }
    __syncthreads();
    float A = 0.f, B = 0.f;
    for (int cl = 0; cl < cfg.D; ++cl) {
        A = fmaf(gch[cl], chan[cl].x, A);
        B = fmaf(gch[cl], chan[cl].y, B);
    }
    __syncthreads();
    if (!cfg.want_dx) return;
    const float invM = 1.0f / (float)(cfg.D * cfg.HW);
    A *= invM;
    B *= invM;
    const int64_t base = (n * cfg.C + g * cfg.D) * cfg.HW;
    for (int64_t tile = last; tile >= 0; tile -= cfg.team) {
        int64_t cl, k0;
        slab::nchw_tile_pos(tile, cfg.tpc, TE, &cl, &k0);
        const int64_t pb = base + cl * cfg.HW;
        const float ga = gch[cl];
        if (tile != last) {
            nchw_load_tile<T, R>(x, cfg, sb, tile, bx);
            nchw_load_tile<T, R>(dy, cfg, sb, tile, bd);
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t e = slab::nchw_chunk_elem(k0, j, t, V);
            if (e < cfg.HW) {
#pragma clang fp contract(off)
                float xv[V], dv[V], o[V];
                Vec<T>::unpack(bx[j], xv);
                Vec<T>::unpack(bd[j], dv);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float xh = (xv[k] - mu) * r;
                    const float gd = dv[k] * ga;
                    o[k] = r * ((gd - A) - xh * B);
                }
                st16_nt(dx + pb + e, Vec<T>::pack(o));
            }
        }
    }
}

// part: [slab][tile] published (sum dy, sum dy*xhat) words; stot: [N][C] float2.
// Two slabs in flight, as in the forward: a member runs phase 1 of the team's
// next slab (loads, sums, publish) before phase 2 of the current one needs
// its partials.  Requires D <= kT (checked on the host).  (fp32 112 x 64 x
// 512 x 512, tiles of 8 chunks, two workgroups per CU: 3.93 ms, against 4.38
// ms for tiles of 16 chunks, one workgroup per CU and the other order --
// the first tile of the next slab prefetched, phase 2 of the current slab
// while it streams, phase 1 of the next from registers.)
template <typename T, int R>
__global__ __launch_bounds__(kT) void slab_nchw_bwd(const T* __restrict__ dy, const T* __restrict__ x,
                                                    const float* __restrict__ mean,
                                                    const float* __restrict__ rstd,
                                                    const float* __restrict__ gamma, T* __restrict__ dx,
                                                    SlabCfg cfg, uint32_t* /*ctr*/, uint32_t* err, uint64_t* part,
                                                    float2* stot, uint32_t* /*res: NHWC only*/) {
    const int team = blockIdx.x / cfg.team;
    const int m = blockIdx.x - team * cfg.team;
    __shared__ float lds[kNW * 2];
    __shared__ float2 chan[kT];
    __shared__ float gch[kT];
    __shared__ float2 stage[kStage];
    u4v cx[R], cd[R], nx[R], nd[R];
    const int t = threadIdx.x;
    int64_t sb = team;
    if (sb >= cfg.n_slabs) return;   // uniform over the team
    float mu = mean[sb], r = rstd[sb];
    float gam = (gamma && t < cfg.D) ? gamma[(sb % cfg.G) * cfg.D + t] : 1.f;
    int64_t last = nchw_bwd_phase1<T, R>(dy, x, cfg, sb, m, mu, r, cx, cd, part, lds);
    while (true) {
        const int64_t nsb = sb + cfg.nteams;
        const bool more = nsb < cfg.n_slabs;   // uniform over the team
        float nmu = 0.f, nr = 0.f, ngam = 1.f;
        int64_t nlast = -1;
        if (more) {
            nmu = mean[nsb];
            nr = rstd[nsb];
            if (gamma && t < cfg.D) ngam = gamma[(nsb % cfg.G) * cfg.D + t];
            nlast = nchw_bwd_phase1<T, R>(dy, x, cfg, nsb, m, nmu, nr, nx, nd, part, lds);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the two slabs' phases apart
        nchw_bwd_phase2<T, R>(dy, x, dx, cfg, sb, m, last, mu, r, cx, cd, gam, part, err, stot, stage,
                              chan, gch);
        if (!more) break;
        for (int j = 0; j < R; ++j) { cx[j] = nx[j]; cd[j] = nd[j]; }   // register moves
        last = nlast;
        sb = nsb;
        mu = nmu;
        r = nr;
        gam = ngam;
    }
}

// ============================================================================
// Small NCHW slabs
// ============================================================================
// A slab that fits one workgroup's registers takes a workgroup of its own:
// BT threads (256, or 1024 for slabs past 64 KiB), R chunks of V elements per
// thread, chunk q = j*BT + t of the slab's D*HW contiguous elements (a chunk
// never straddles a channel plane: HW is a multiple of V).  The slab is read
// once, its statistics are an exact two-pass over the registers, and nothing
// is exchanged between workgroups: no sync words, no clear kernel, a normal
// launch.  grid: one workgroup per slab s = n*G + g.
template <typename T, int R, int BT>
__global__ __launch_bounds__(BT) void small_nchw_fwd(const T* __restrict__ x, const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, T* __restrict__ y,
                                                     float* __restrict__ mean, float* __restrict__ rstd, int64_t G,
                                                     int D, int HW, float eps) {
    constexpr int V = Vec<T>::V;
    constexpr int NW = BT / kWave;
    __shared__ float lds[NW * 2];
    __shared__ float sga[kT], sbe[kT];   // gamma, beta of the slab's channels (D <= kT <= BT)
    const int t = threadIdx.x;
    const int64_t sb = blockIdx.x;
    const int g = (int)(sb % G);
    const int M = D * HW;                // elements of the slab
    const int nq = M / V;                // chunks of the slab
    const int cpc = HW / V;              // chunks per channel plane
    const T* xs = x + sb * (int64_t)M;
    if (t < D) {
        sga[t] = gamma ? gamma[g * D + t] : 1.f;
        sbe[t] = beta ? beta[g * D + t] : 0.f;
    }
    u4v buf[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {   // branch-free: past the end, the last chunk again (not used)
        const int q = j * BT + t;
        buf[j] = ld16_nt(xs + (int64_t)(q < nq ? q : nq - 1) * V);
    }
    float sum[1] = {0.f};
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * BT + t < nq) {
            float v[V];
            Vec<T>::unpack(buf[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) sum[0] += v[k];
        }
    }
    block_sum<1, NW>(sum, lds);
    const float mu = sum[0] / (float)M;
    if constexpr (sizeof(T) == 2) {   // unpack again below rather than hold the floats
#pragma unroll
        for (int j = 0; j < R; ++j) asm volatile("" : "+v"(buf[j]));
    }
    float m2[1] = {0.f};
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * BT + t < nq) {
            float v[V];
            Vec<T>::unpack(buf[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = v[k] - mu;
                m2[0] = fmaf(d, d, m2[0]);
            }
        }
    }
    block_sum<1, NW>(m2, lds);
    float var = m2[0] / (float)M;
    var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
    const float r = 1.0f / sqrtf(var + eps);
    if (t == 0) {
        mean[sb] = mu;
        rstd[sb] = r;
    }
    if (y == nullptr) return;
    T* ys = y + sb * (int64_t)M;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int q = j * BT + t;
        if (q < nq) {
            const int cl = q / cpc;
            const float a_c = r * sga[cl];
            const float b_c = sbe[cl];
            float v[V], o[V];
            Vec<T>::unpack(buf[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = fmaf(v[k] - mu, a_c, b_c);
            st16_nt(ys + (int64_t)q * V, Vec<T>::pack(o));
        }
    }
}

// Backward of a small slab: A = sum gamma_c*dy and B = sum gamma_c*dy*xhat
// over the slab (one workgroup sum), dx from the registers, and the slab's
// per-channel sums of dy and dy*xhat (stot[n][c], for dgamma/dbeta over the
// samples): per-chunk sums staged in LDS, W lanes per channel (a power of two
// <= 64, so that a channel's lanes sit in one wave) add a channel's chunks
// with stride W, then a butterfly over the W lanes -- a fixed order.
template <typename T, int R, int BT>
__global__ __launch_bounds__(BT) void small_nchw_bwd(const T* __restrict__ dy, const T* __restrict__ x,
                                                     const float* __restrict__ mean,
                                                     const float* __restrict__ rstd,
                                                     const float* __restrict__ gamma, T* __restrict__ dx,
                                                     float2* __restrict__ stot, int64_t G, int64_t C, int D, int HW,
                                                     int want_dx) {
    constexpr int V = Vec<T>::V;
    constexpr int NW = BT / kWave;
    __shared__ float lds[NW * 2];
    __shared__ float sga[kT];          // D <= kT <= BT
    __shared__ float2 cpart[BT * R];   // per chunk: (sum dy, sum dy*xhat)
    const int t = threadIdx.x;
    const int64_t sb = blockIdx.x;
    const int64_t n = sb / G;
    const int g = (int)(sb - n * G);
    const int M = D * HW, nq = M / V, cpc = HW / V;
    const float mu = mean[sb], r = rstd[sb];
    if (t < D) sga[t] = gamma ? gamma[g * D + t] : 1.f;
    const T* xs = x + sb * (int64_t)M;
    const T* ds = dy + sb * (int64_t)M;
    u4v bx[R], bd[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {   // branch-free: past the end, the last chunk again (not used)
        const int q = j * BT + t;
        const int64_t e = (int64_t)(q < nq ? q : nq - 1) * V;
        bx[j] = ld16_nt(xs + e);
        bd[j] = ld16_nt(ds + e);
    }
    __syncthreads();   // sga
    float ab[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int q = j * BT + t;
        if (q < nq) {
            const float ga = sga[q / cpc];
            float xv[V], dv[V];
            Vec<T>::unpack(bx[j], xv);
            Vec<T>::unpack(bd[j], dv);
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float xh = (xv[k] - mu) * r;
                s1 += dv[k];
                s2 = fmaf(dv[k], xh, s2);
            }
            cpart[q] = make_float2(s1, s2);
            ab[0] = fmaf(ga, s1, ab[0]);
            ab[1] = fmaf(ga, s2, ab[1]);
        }
    }
    block_sum<2, NW>(ab, lds);   // its barriers also publish cpart
    int W = 64;
    while (W > 1 && W * D > BT) W >>= 1;
    const int ccl = t / W, cj = t & (W - 1);
    float2 run = make_float2(0.f, 0.f);
    if (ccl < D) {
        for (int i = cj; i < cpc; i += W) {
            const float2 v = cpart[ccl * cpc + i];
            run.x += v.x;
            run.y += v.y;
        }
    }
    for (int o = W >> 1; o > 0; o >>= 1) {   // every lane takes part
        run.x += __shfl_xor(run.x, o, kWave);
        run.y += __shfl_xor(run.y, o, kWave);
    }
    if (cj == 0 && ccl < D) stot[n * C + (int64_t)g * D + ccl] = run;
    if (!want_dx) return;
    const float invM = 1.0f / (float)M;
    const float A = ab[0] * invM, B = ab[1] * invM;
    T* dxs = dx + sb * (int64_t)M;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int q = j * BT + t;
        if (q < nq) {
#pragma clang fp contract(off)
            const float ga = sga[q / cpc];
            float xv[V], dv[V], o[V];
            Vec<T>::unpack(bx[j], xv);
            Vec<T>::unpack(bd[j], dv);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float xh = (xv[k] - mu) * r;
                const float gd = dv[k] * ga;
                o[k] = r * ((gd - A) - xh * B);
            }
            st16_nt(dxs + (int64_t)q * V, Vec<T>::pack(o));
        }
    }
}

// Backward of a slab past what 1024 threads hold of both x and dy (128 KiB
// each): the first RR chunk rounds of x and dy stay in registers; the other
// rounds (up to kMidBwdRounds in all) are streamed in batches of RB chunks in
// the sums pass and loaded again for dx.  Sums, channel sums and dx as in
// small_nchw_bwd, in chunk order.
constexpr int kMidBwdRounds = 16;
template <typename T, int RR, int RB>
__global__ __launch_bounds__(1024) void mid_nchw_bwd(const T* __restrict__ dy, const T* __restrict__ x,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     const float* __restrict__ gamma, T* __restrict__ dx,
                                                     float2* __restrict__ stot, int64_t G, int64_t C, int D, int HW,
                                                     int want_dx) {
    constexpr int V = Vec<T>::V;
    constexpr int BT = 1024, NW = BT / kWave;
    __shared__ float lds[NW * 2];
    __shared__ float sga[kT];                           // D <= kT
    __shared__ float2 cpart[BT * kMidBwdRounds];        // per chunk: (sum dy, sum dy*xhat)
    const int t = threadIdx.x;
    const int64_t sb = blockIdx.x;
    const int64_t n = sb / G;
    const int g = (int)(sb - n * G);
    const int M = D * HW, nq = M / V, cpc = HW / V;
    const int nr = (nq + BT - 1) / BT;                  // chunk rounds (RR < nr <= kMidBwdRounds)
    const float mu = mean[sb], r = rstd[sb];
    if (t < D) sga[t] = gamma ? gamma[g * D + t] : 1.f;
    const T* xs = x + sb * (int64_t)M;
    const T* ds = dy + sb * (int64_t)M;
    auto at = [&](int j) { const int q = j * BT + t; return (int64_t)(q < nq ? q : nq - 1) * V; };
    u4v bx[RR], bd[RR];
#pragma unroll
    for (int j = 0; j < RR; ++j) {   // branch-free: past the end, the last chunk again (not used)
        bx[j] = ld16_nt(xs + at(j));
        bd[j] = ld16_nt(ds + at(j));
    }
    __syncthreads();   // sga
    float ab[2] = {0.f, 0.f};
    // one chunk's sums into cpart and this thread's (A, B) terms
    auto sums = [&](int j, const u4v& cx, const u4v& cd) {
        const int q = j * BT + t;
        if (q >= nq) return;
        const float ga = sga[q / cpc];
        float xv[V], dv[V];
        Vec<T>::unpack(cx, xv);
        Vec<T>::unpack(cd, dv);
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const float xh = (xv[k] - mu) * r;
            s1 += dv[k];
            s2 = fmaf(dv[k], xh, s2);
        }
        cpart[q] = make_float2(s1, s2);
        ab[0] = fmaf(ga, s1, ab[0]);
        ab[1] = fmaf(ga, s2, ab[1]);
    };
#pragma unroll
    for (int j = 0; j < RR; ++j) sums(j, bx[j], bd[j]);
    for (int j0 = RR; j0 < nr; j0 += RB) {   // uniform
        u4v ox[RB], od[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            ox[i] = ld16_nt(xs + at(j0 + i));
            od[i] = ld16_nt(ds + at(j0 + i));
        }
#pragma unroll
        for (int i = 0; i < RB; ++i)
            if (j0 + i < nr) sums(j0 + i, ox[i], od[i]);
    }
    block_sum<2, NW>(ab, lds);   // its barriers also publish cpart
    int W = 64;
    while (W > 1 && W * D > BT) W >>= 1;
    const int ccl = t / W, cj = t & (W - 1);
    float2 run = make_float2(0.f, 0.f);
    if (ccl < D) {
        for (int i = cj; i < cpc; i += W) {
            const float2 v = cpart[ccl * cpc + i];
            run.x += v.x;
            run.y += v.y;
        }
    }
    for (int o = W >> 1; o > 0; o >>= 1) {   // every lane takes part
        run.x += __shfl_xor(run.x, o, kWave);
        run.y += __shfl_xor(run.y, o, kWave);
    }
    if (cj == 0 && ccl < D) stot[n * C + (int64_t)g * D + ccl] = run;
    if (!want_dx) return;
    const float invM = 1.0f / (float)M;
    const float A = ab[0] * invM, B = ab[1] * invM;
    T* dxs = dx + sb * (int64_t)M;
    auto out = [&](int j, const u4v& cx, const u4v& cd) {
#pragma clang fp contract(off)
        const int q = j * BT + t;
        if (q >= nq) return;
        const float ga = sga[q / cpc];
        float xv[V], dv[V], o[V];
        Vec<T>::unpack(cx, xv);
        Vec<T>::unpack(cd, dv);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const float xh = (xv[k] - mu) * r;
            const float gd = dv[k] * ga;
            o[k] = r * ((gd - A) - xh * B);
        }
        st16_nt(dxs + (int64_t)q * V, Vec<T>::pack(o));
    };
#pragma unroll
    for (int j = 0; j < RR; ++j) out(j, bx[j], bd[j]);
    for (int j0 = RR; j0 < nr; j0 += RB) {
        u4v ox[RB], od[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            ox[i] = ld16_nt(xs + at(j0 + i));
            od[i] = ld16_nt(ds + at(j0 + i));
        }
#pragma unroll
        for (int i = 0; i < RB; ++i)
            if (j0 + i < nr) out(j0 + i, ox[i], od[i]);
    }
}

// ============================================================================
// NCHW split form: statistics tiles, then outputs that combine them
// ============================================================================
// For tensors small enough that the cooperative kernels' fixed cost (launch,
// clear kernel, exchange) outweighs their single pass, two ordinary launches
// per call: a tile kernel writes each tile's statistics, and every workgroup
// of the output kernel combines its slab's few tile partials itself, in tile
// order (all of them derive the same values; workgroup 0 of a slab writes the
// saved statistics or the per-(n, c) sums).  Statistics tiles are plane
// aligned: tile k = c*tpc + i of slab s covers chunks [i*kT*R, (i+1)*kT*R) of
// channel plane c (the last tile of a plane may be short), so a backward
// tile's sums belong to one channel.  Output tiles are kT*RO consecutive
// chunks of the slab.

// grid (D*tpc, N*G); part[s*D*tpc + k] = (count, mean, M2, -), an exact
// two-pass over the tile
template <typename T, int R>
__global__ __launch_bounds__(kT) void split_nchw_stats(const T* __restrict__ x, int D, int HW, int tpc,
                                                       float4* __restrict__ part) {
    constexpr int V = Vec<T>::V;
    __shared__ float lds[kNW * 2];
    const int t = threadIdx.x;
    const int64_t sb = blockIdx.y;
    const int k = blockIdx.x, c = k / tpc, i = k - c * tpc;
    const int cpc = HW / V;
    const int q0 = i * kT * R;
    const int nv = min(kT * R, cpc - q0);   // chunks of this tile
    const T* xp = x + (sb * D + c) * (int64_t)HW;
    u4v buf[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {   // branch-free: past the tile, its last chunk again (not used)
        const int q = j * kT + t;
        buf[j] = ld16_nt(xp + (int64_t)(q0 + (q < nv ? q : nv - 1)) * V);
    }
    const float cnt = (float)nv * V;
    float sum[1] = {0.f};
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * kT + t < nv) {
            float v[V];
            Vec<T>::unpack(buf[j], v);
#pragma unroll
            for (int kk = 0; kk < V; ++kk) sum[0] += v[kk];
        }
    }
    block_sum<1, kNW>(sum, lds);
    const float mu = sum[0] / cnt;
    float m2[1] = {0.f};
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * kT + t < nv) {
            float v[V];
            Vec<T>::unpack(buf[j], v);
#pragma unroll
            for (int kk = 0; kk < V; ++kk) {
                const float d = v[kk] - mu;
                m2[0] = fmaf(d, d, m2[0]);
            }
        }
    }
    block_sum<1, kNW>(m2, lds);
    if (t == 0) part[sb * D * tpc + k] = make_float4(cnt, mu, m2[0], 0.f);
}

// grid (otiles or 1, N*G): the slab's statistics from its ntl = D*tpc tile
// partials (as the finalize of the stream path), then y for one output tile
template <typename T, int RO>
__global__ __launch_bounds__(kT) void split_nchw_apply(const T* __restrict__ x, const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, T* __restrict__ y,
                                                       const float4* __restrict__ part, float* __restrict__ mean,
                                                       float* __restrict__ rstd, int64_t G, int D, int HW, int ntl,
                                                       float eps) {
    constexpr int V = Vec<T>::V;
    __shared__ float sga[kT], sbe[kT];   // D <= kT
    const int t = threadIdx.x;
    const int64_t sb = blockIdx.y;
    const int g = (int)(sb % G);
    const float4* ps = part + sb * ntl;
    float s0 = 0.f, s1 = 0.f;
    for (int k = 0; k < ntl; ++k) {   // every thread, the same order
        const float4 v = ps[k];
        s0 = fmaf(v.x, v.y, s0);
        s1 += v.x;
    }
    const float mu = s0 / s1;
    float m2 = 0.f;
    for (int k = 0; k < ntl; ++k) {
        const float4 v = ps[k];
        const float d = v.y - mu;
        m2 += fmaf(v.x * d, d, v.z);
    }
    float var = m2 / ((float)D * (float)HW);
    var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
    const float r = 1.0f / sqrtf(var + eps);
    if (blockIdx.x == 0 && t == 0) {
        mean[sb] = mu;
        rstd[sb] = r;
    }
    if (y == nullptr) return;   // uniform
    if (t < D) {
        sga[t] = gamma ? gamma[g * D + t] : 1.f;
        sbe[t] = beta ? beta[g * D + t] : 0.f;
    }
    __syncthreads();
    const int cpc = HW / V, nq = D * cpc;
    const int64_t base = sb * (int64_t)D * HW;
    const int q0 = blockIdx.x * kT * RO;
    u4v buf[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
        const int q = q0 + j * kT + t;
        buf[j] = ld16_nt(x + base + (int64_t)(q < nq ? q : nq - 1) * V);
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) {
        const int q = q0 + j * kT + t;
        if (q < nq) {
            const int cl = q / cpc;
            const float a_c = r * sga[cl], b_c = sbe[cl];
            float v[V], o[V];
            Vec<T>::unpack(buf[j], v);
#pragma unroll
            for (int kk = 0; kk < V; ++kk) o[kk] = fmaf(v[kk] - mu, a_c, b_c);
            st16_nt(y + base + (int64_t)q * V, Vec<T>::pack(o));
        }
    }
}

// grid (D*tpc, N*G); part[s*D*tpc + k] = (sum dy, sum dy*xhat) over the tile
template <typename T, int R>
__global__ __launch_bounds__(kT) void split_nchw_sums(const T* __restrict__ dy, const T* __restrict__ x,
                                                      const float* __restrict__ mean,
                                                      const float* __restrict__ rstd, int D, int HW, int tpc,
                                                      float2* __restrict__ part) {
    constexpr int V = Vec<T>::V;
    __shared__ float lds[kNW * 2];
    const int t = threadIdx.x;
    const int64_t sb = blockIdx.y;
    const int k = blockIdx.x, c = k / tpc, i = k - c * tpc;
    const int cpc = HW / V;
    const int q0 = i * kT * R;
    const int nv = min(kT * R, cpc - q0);
    const int64_t off = (sb * D + c) * (int64_t)HW;
    const float mu = mean[sb], r = rstd[sb];
    u4v bx[R], bd[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int q = j * kT + t;
        const int64_t e = off + (int64_t)(q0 + (q < nv ? q : nv - 1)) * V;
        bx[j] = ld16_nt(x + e);
        bd[j] = ld16_nt(dy + e);
    }
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j * kT + t < nv) {
            float xv[V], dv[V];
            Vec<T>::unpack(bx[j], xv);
            Vec<T>::unpack(bd[j], dv);
#pragma unroll
            for (int kk = 0; kk < V; ++kk) {
                acc[0] += dv[kk];
                acc[1] = fmaf(dv[kk], (xv[kk] - mu) * r, acc[1]);
            }
        }
    }
    block_sum<2, kNW>(acc, lds);
    if (t == 0) part[sb * D * tpc + k] = make_float2(acc[0], acc[1]);
}

// grid (otiles or 1, N*G): per-channel sums of the slab from its tile sums (in
// tile order), A and B (one workgroup sum), then dx for one output tile;
// workgroup 0 writes the per-(n, c) sums into stot (for params_over_n)
template <typename T, int RO>
__global__ __launch_bounds__(kT) void split_nchw_dx(const T* __restrict__ dy, const T* __restrict__ x,
                                                    const float* __restrict__ mean, const float* __restrict__ rstd,
                                                    const float* __restrict__ gamma,
                                                    const float2* __restrict__ part, T* __restrict__ dx,
                                                    float2* __restrict__ stot, int64_t G, int64_t C, int D, int HW,
                                                    int tpc, int want_dx) {
    constexpr int V = Vec<T>::V;
    __shared__ float lds[kNW * 2];
    __shared__ float sga[kT];   // D <= kT
    const int t = threadIdx.x;
    const int64_t sb = blockIdx.y;
    const int64_t n = sb / G;
    const int g = (int)(sb - n * G);
    float ab[2] = {0.f, 0.f};
    if (t < D) {
        const float2* pc = part + sb * D * tpc + t * tpc;
        float2 v = make_float2(0.f, 0.f);
        for (int i = 0; i < tpc; ++i) {
            const float2 q = pc[i];
            v.x += q.x;
            v.y += q.y;
        }
        if (blockIdx.x == 0 && stot) stot[n * C + (int64_t)g * D + t] = v;
        const float ga = gamma ? gamma[g * D + t] : 1.f;
        sga[t] = ga;
        ab[0] = ga * v.x;
        ab[1] = ga * v.y;
    }
    if (!want_dx) return;   // kernel argument: uniform
    block_sum<2, kNW>(ab, lds);   // its barriers also publish sga
    const float mu = mean[sb], r = rstd[sb];
    const float invM = 1.0f / ((float)D * (float)HW);
    const float A = ab[0] * invM, B = ab[1] * invM;
    const int cpc = HW / V, nq = D * cpc;
    const int64_t base = sb * (int64_t)D * HW;
    const int q0 = blockIdx.x * kT * RO;
    u4v bx[RO], bd[RO];
#pragma unroll
    for (int j = 0; j < RO; ++j) {
        const int q = q0 + j * kT + t;
        const int64_t e = base + (int64_t)(q < nq ? q : nq - 1) * V;
        bx[j] = ld16_nt(x + e);
        bd[j] = ld16_nt(dy + e);
    }
#pragma unroll
    for (int j = 0; j < RO; ++j) {
        const int q = q0 + j * kT + t;
        if (q < nq) {
#pragma clang fp contract(off)
            const float ga = sga[q / cpc];
            float xv[V], dv[V], o[V];
            Vec<T>::unpack(bx[j], xv);
            Vec<T>::unpack(bd[j], dv);
#pragma unroll
            for (int kk = 0; kk < V; ++kk) {
                const float xh = (xv[kk] - mu) * r;
                const float gd = dv[kk] * ga;
                o[kk] = r * ((gd - A) - xh * B);
            }
            st16_nt(dx + base + (int64_t)q * V, Vec<T>::pack(o));
        }
    }
}

// ---- helpers ---------------------------------------------------------------
// Words [0, zeros) := 0, [zeros, total) := all ones.
__global__ void clear_words(uint32_t* p, int64_t zeros, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = i < zeros ? 0u : ~0u;
}

// dbeta_c = sum_n stot[n][c].x, dgamma_c = sum_n stot[n][c].y (n in order)
__global__ __launch_bounds__(kT) void params_over_n(const float2* __restrict__ stot, int64_t N, int64_t C,
                                                    float* __restrict__ dgamma, float* __restrict__ dbeta) {
    const int64_t c = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (c >= C) return;
    float a = 0.f, b = 0.f;
#pragma unroll 8
    for (int64_t n = 0; n < N; ++n) {
        const float2 v = stot[n * C + c];
        a += v.x;
        b += v.y;
    }
    if (dbeta) dbeta[c] = a;
    if (dgamma) dgamma[c] = b;
}

// ---- planning --------------------------------------------------------------
// 16-byte chunks per thread per tile (of x, and of dy in the backward)
#ifndef GN_SLAB_NHWC_RF
#define GN_SLAB_NHWC_RF 16
#endif
#ifndef GN_SLAB_NHWC_RB
#define GN_SLAB_NHWC_RB 8
#endif
// NCHW, largest tile per dtype and direction (measured on 112 x 64 x 512 x 512,
// G = 8): fp32 forward 16 -- its two register tiles leave room for two
// workgroups per CU, which 32 does not; fp32 backward 8 (four register tiles:
// x and dy of two slabs, two workgroups per CU; 16 leaves one workgroup per
// CU and is slower); 16-bit forward 8 -- 16 chunks of a 16-bit type, with
// their unpacked halves, hold two workgroups per CU instead of four and run
// slower; 16-bit backward 4 (121 VGPRs, four workgroups per CU: bf16 2.30 ->
// 2.27 ms against 8 chunks, 198 VGPRs and two workgroups per CU).  Smaller
// planes take the power of two at or above the
// plane's chunks per thread, so that a small plane does not leave most of a
// fixed-size tile empty.
#ifndef GN_SLAB_NCHW_RF
#define GN_SLAB_NCHW_RF 16
#endif
#ifndef GN_SLAB_NCHW_RB
#define GN_SLAB_NCHW_RB 8
#endif
#ifndef GN_SLAB_NCHW_RF16
#define GN_SLAB_NCHW_RF16 8
#endif
#ifndef GN_SLAB_NCHW_RB16
#define GN_SLAB_NCHW_RB16 4
#endif
constexpr int kNchwRF16 = GN_SLAB_NCHW_RF16 < 16 ? GN_SLAB_NCHW_RF16 : 16;
constexpr int kNchwRB16 = GN_SLAB_NCHW_RB16 < 16 ? GN_SLAB_NCHW_RB16 : 16;

int nchw_r(const Problem& p, bool backward) {
    const int64_t per_thread = (p.HW / (p.elem_bytes == 4 ? 4 : 8) + kT - 1) / kT;
    const int rmax = backward ? (p.elem_bytes == 4 ? GN_SLAB_NCHW_RB : kNchwRB16)
                              : (p.elem_bytes == 4 ? GN_SLAB_NCHW_RF : kNchwRF16);
    int r = 1;
    while (r < per_thread && r < rmax) r *= 2;
    return r;
}

int tile_chunks(const Problem& p, bool backward) {
    if (p.layout == GN_NHWC) return backward ? GN_SLAB_NHWC_RB : GN_SLAB_NHWC_RF;
    return nchw_r(p, backward);
}

size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

int vec_elems(const Problem& p) { return p.elem_bytes == 4 ? 4 : 8; }

struct Plan {
    SlabCfg cfg;
    int64_t grid;
    int64_t resident;
    size_t off_ctr, off_err, off_res, off_part, off_stot, total;
    size_t ones_end;   // [off_part, ones_end): filled with ones each call (NCHW partial words)
};

// Slabs of at most this many bytes (per tensor) are processed by one
// workgroup each, launched normally: there is no exchange between workgroups,
// and the cooperative launch, whose cost is fixed, would dominate such calls
// (graphs of 50 back-to-back calls: 2 x 32 x 16 x 16 fp32 forward 25 -> 9.2 us,
// backward 27.7 -> 11 us; 16 x 128 x 64 x 64 fp16 G=32 32.5 -> 16 us).  Up to
// 128 KiB slabs still gain on their own (8 x 64 x 64 x 64 fp32: 26.6 -> 18.4
// us), but graphs captured with such launches slowed later graphs of
// cooperative launches in the same process threefold, which eager launches
// did not; 512 KiB slabs run faster cooperatively.  (NCHW slabs past 64 KiB
// that fit a 1024-thread workgroup go to small_nchw_* instead, whose graphs
// leave later cooperative graphs at their speed: 33.2 / 34.1 us before, 32.4
// / 33.5 us after, 2 x 32 x 128 x 128 fp32 G4 around 2 x 320 x 64 x 64 fp16.)
#ifndef GN_SLAB_SOLO_BYTES
#define GN_SLAB_SOLO_BYTES 65536
#endif

// The schedule of this problem for a resident-workgroup cap (gn_slab_plan.hpp).
slab::Geometry geometry(const Problem& p, int R, int64_t cap) {
    const int64_t slab_bytes = (p.layout == GN_NHWC ? p.C : p.D) * p.HW * p.elem_bytes;
    const int64_t max_team = slab_bytes <= (int64_t)GN_SLAB_SOLO_BYTES ? 1 : INT64_MAX;
    return slab::plan(p.layout == GN_NHWC, p.N, p.C, p.HW, p.G, vec_elems(p), R, cap, max_team);
}

int64_t tiles_per_slab(const Problem& p, int R, int64_t* tpc) {
    const slab::Geometry g = geometry(p, R, 1);
    *tpc = g.tpc;
    return g.tiles;
}

template <typename K>
int64_t resident_cap(K kernel, int cu_count) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, (const void*)kernel, kT, 0) != hipSuccess) {
        (void)hipGetLastError();
        blocks = 1;
    }
    return (int64_t)(blocks > 0 ? blocks : 1) * cu_count;
}

// The grid plan for resident-workgroup cap `cap` and the workspace layout.
// The layout does not depend on the cap (the size queries pass the slab's tile
// count), so the size does not depend on the device.
Plan layout_ws(const Problem& p, bool backward, int64_t cap) {
    Plan pl{};
    const slab::Geometry g = geometry(p, tile_chunks(p, backward), cap);
    const int64_t tiles = g.tiles;
    const int64_t n_slabs = g.n_slabs;
    pl.cfg.tiles = tiles;
    pl.cfg.tpc = g.tpc;
    pl.cfg.pstride = g.pstride;
    pl.cfg.n_slabs = n_slabs;
    pl.cfg.team = (int32_t)g.team;
    pl.cfg.nteams = (int32_t)g.nteams;
    pl.grid = g.grid;
    size_t off = 256;            // [0, 256): error word
    pl.off_err = 0;
    pl.off_ctr = off;            // 4 sync words per slab
    off += al((size_t)n_slabs * 4 * sizeof(uint32_t));
    pl.off_res = off;            // NHWC: resident flag per tile
    if (p.layout == GN_NHWC) off += al((size_t)n_slabs * tiles * sizeof(uint32_t));
    pl.off_part = off;           // everything before this offset is cleared each call
    size_t part;
    if (p.layout == GN_NHWC)
        part = backward ? (size_t)n_slabs * p.C * pl.cfg.pstride * sizeof(float2)
                        : (size_t)n_slabs * p.G * pl.cfg.pstride * sizeof(float4);
    else
        part = (size_t)n_slabs * pl.cfg.pstride * sizeof(uint64_t);
    off += al(part);
    pl.ones_end = p.layout == GN_NHWC ? pl.off_part : off;
    pl.off_stot = off;
    if (backward) off += al((size_t)p.N * p.C * sizeof(float2));
    pl.total = off;
    return pl;
}

// Zeroes the error word, the sync words and the resident flags, and sets the
// NCHW partial words to the unpublished pattern (one fill kernel: no memset
// node, so the call stays safe to capture in a graph).
hipError_t clear_sync_words(char* ws, const Plan& pl, hipStream_t s) {
    const int64_t zeros = (int64_t)(pl.off_part / sizeof(uint32_t));
    const int64_t words = (int64_t)(pl.ones_end / sizeof(uint32_t));
    int64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(clear_words, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)ws, zeros, words);
    return hipGetLastError();
}

template <typename K>
hipError_t launch_coop(K kernel, int64_t grid, void** args, hipStream_t s, bool coop) {
    if (coop) return hipLaunchCooperativeKernel((const void*)kernel, dim3((unsigned)grid), dim3(kT), args, 0, s);
    return hipLaunchKernel((const void*)kernel, dim3((unsigned)grid), dim3(kT), args, 0, s);
}

template <typename T>
auto nchw_fwd_kernel(int R) -> decltype(&slab_nchw_fwd<T, 1>) {
    switch (R) {   // R as nchw_r gives it for this dtype
        case 1: return slab_nchw_fwd<T, 1>;
        case 2: return slab_nchw_fwd<T, 2>;
        case 4: return slab_nchw_fwd<T, 4>;
        case 8: return slab_nchw_fwd<T, 8>;
        case 16: return slab_nchw_fwd<T, 16>;
        default: return slab_nchw_fwd<T, sizeof(T) == 4 ? GN_SLAB_NCHW_RF : kNchwRF16>;
    }
}

template <typename T>
auto nchw_bwd_kernel(int R) -> decltype(&slab_nchw_bwd<T, GN_SLAB_NCHW_RB>) {
    switch (R) {
        case 1: return slab_nchw_bwd<T, 1>;
        case 2: return slab_nchw_bwd<T, 2>;
        case 4: return slab_nchw_bwd<T, 4>;
        case 8: return slab_nchw_bwd<T, 8>;
        default: return slab_nchw_bwd<T, sizeof(T) == 4 ? GN_SLAB_NCHW_RB : kNchwRB16>;
    }
}

// NCHW slabs that fit one workgroup's registers: one workgroup each (above).
// Up to GN_SLAB_SOLO_BYTES per tensor 256 threads, past that 1024 threads up
// to GN_SLAB_MID_FWD_BYTES in the forward (16 chunks per thread) and
// GN_SLAB_MID_BWD_BYTES in the backward (8 chunks each of x and dy; 16 would
// need about 200 VGPRs, more than a 1024-thread workgroup has).  Graphs of 20
// calls, forward / backward us, cooperative kernels -> one workgroup per slab:
// 2 x 320 x 64 x 64 fp16 G32 (80 KiB slabs) 32.0 / 36.4 -> 7.4 / 13.5;
// 16 x 320 x 64 x 64 fp16 G32 50.5 / 58.0 -> 13.6 / 30.6; 8 x 64 x 64 x 64
// fp32 G8 (128 KiB) 30.7 / 33.8 -> 7.5 / 12.4.
#ifndef GN_SLAB_MID_FWD_BYTES
#define GN_SLAB_MID_FWD_BYTES (256 << 10)
#endif
#ifndef GN_SLAB_MID_BWD_BYTES
#define GN_SLAB_MID_BWD_BYTES (128 << 10)
#endif
constexpr int kMidT = 1024;
static_assert(GN_SLAB_SOLO_BYTES <= kT * 16 * 16, "small slabs: at most 16 chunks per thread");
static_assert(GN_SLAB_MID_FWD_BYTES <= kMidT * 16 * 16, "mid-size forward: at most 16 chunks per thread");
static_assert(GN_SLAB_MID_BWD_BYTES <= kMidT * 8 * 16, "mid-size backward: at most 8 chunks per thread");
// Backward slabs past GN_SLAB_MID_BWD_BYTES up to this size: mid_nchw_bwd,
// eight chunk rounds of x and dy in registers and the rest streamed twice.
// Graphs of 20 calls, backward us, cooperative kernels -> mid_nchw_bwd with 8
// (4) rounds held: 2 x 640 x 64 x 64 fp16 G32 (160 KiB) 38.5 -> 21.9 (21.0);
// 16 x 640 x 64 x 64 fp16 G32 90.2 -> 58.9 (63.9); 4 x 32 x 64 x 64 fp32 G2
// (256 KiB) 33.0 -> 17.5 (17.4).
#ifndef GN_SLAB_MID_BWD_STREAM_BYTES
#define GN_SLAB_MID_BWD_STREAM_BYTES (256 << 10)
#endif
static_assert(GN_SLAB_MID_BWD_STREAM_BYTES <= kMidT * kMidBwdRounds * 16, "mid_nchw_bwd: at most 16 chunk rounds");
constexpr int kMidStreamT = -kMidT;   // small_bt's answer for mid_nchw_bwd

// Threads per workgroup of the one-workgroup-per-slab kernels for this call
// (kMidStreamT: mid_nchw_bwd's 1024), or 0 when they do not take it (other
// layouts, larger slabs, or a residency cap, which asks for the cooperative
// kernels' overflow tiles).
int small_bt(const Problem& p, const Launch& l, bool backward) {
    if (p.layout != GN_NCHW || l.max_resident_override > 0 || l.slab_coop || p.N * p.G > INT32_MAX) return 0;
    const int64_t b = p.D * p.HW * p.elem_bytes;
    if (b <= (int64_t)GN_SLAB_SOLO_BYTES) return kT;
    if (b <= (int64_t)(backward ? GN_SLAB_MID_BWD_BYTES : GN_SLAB_MID_FWD_BYTES)) return kMidT;
    if (backward && b <= (int64_t)GN_SLAB_MID_BWD_STREAM_BYTES) return kMidStreamT;
    return 0;
}

// chunks per thread: the smallest power of two that covers the slab
int small_r(const Problem& p, int bt) {
    const int64_t nq = p.D * p.HW / vec_elems(p);
    int r = 1;
    while ((int64_t)r * bt < nq) r *= 2;
    return r;
}

template <typename T>
auto small_fwd_kernel(int bt, int R) -> decltype(&small_nchw_fwd<T, 1, kT>) {
    if (bt == kMidT) return R <= 8 ? small_nchw_fwd<T, 8, kMidT> : R <= 16 ? small_nchw_fwd<T, 16, kMidT> : nullptr;
    return R == 1 ? small_nchw_fwd<T, 1, kT>
         : R == 2 ? small_nchw_fwd<T, 2, kT>
         : R == 4 ? small_nchw_fwd<T, 4, kT>
         : R == 8 ? small_nchw_fwd<T, 8, kT>
         : R == 16 ? small_nchw_fwd<T, 16, kT> : nullptr;
}

template <typename T>
auto small_bwd_kernel(int bt, int R) -> decltype(&small_nchw_bwd<T, 1, kT>) {
    if (bt == kMidT) return R <= 8 ? small_nchw_bwd<T, 8, kMidT> : nullptr;
    return R == 1 ? small_nchw_bwd<T, 1, kT>
         : R == 2 ? small_nchw_bwd<T, 2, kT>
         : R == 4 ? small_nchw_bwd<T, 4, kT>
         : R == 8 ? small_nchw_bwd<T, 8, kT>
         : R == 16 ? small_nchw_bwd<T, 16, kT> : nullptr;
}

template <typename T>
hipError_t small_fwd(const Problem& p, const FwdArgs& a, const Launch& l, int bt) {
    auto k = small_fwd_kernel<T>(bt, small_r(p, bt));
    if (k == nullptr) return hipErrorInvalidValue;   // the byte limits above rule this out
    const unsigned grid = (unsigned)(p.N * p.G);
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(bt), 0, l.stream, (const T*)a.x, a.gamma, a.beta, (T*)a.y, a.mean, a.rstd,
                       p.G, (int)p.D, (int)p.HW, a.eps);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_SLAB;
        l.info->kernels = 1;
        l.info->grid = grid;
        l.info->tiles = grid;
        l.info->resident_cap = 0;
        l.info->team = 1;
    }
    return hipSuccess;
}

template <typename T>
hipError_t small_bwd(const Problem& p, const BwdArgs& a, const Launch& l, int bt) {
    auto k = bt == kMidStreamT ? mid_nchw_bwd<T, 8, 4> : small_bwd_kernel<T>(bt, small_r(p, bt));
    if (k == nullptr) return hipErrorInvalidValue;   // the byte limits above rule this out
    if (bt == kMidStreamT) bt = kMidT;
    const Plan pl = layout_ws(p, true, 1);   // the layout does not depend on the cap
    float2* stot = (float2*)((char*)l.ws + pl.off_stot);
    const unsigned grid = (unsigned)(p.N * p.G);
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(bt), 0, l.stream, (const T*)a.dy, (const T*)a.x, a.mean, a.rstd, a.gamma,
                       (T*)a.dx, stot, p.G, p.C, (int)p.D, (int)p.HW, (a.mask & GN_GRAD_DX) ? 1 : 0);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    int kernels = 1;
    if (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) {
        hipLaunchKernelGGL(params_over_n, dim3((unsigned)((p.C + kT - 1) / kT)), dim3(kT), 0, l.stream, stot, p.N,
                           p.C, a.dgamma, a.dbeta);
        if ((e = hipGetLastError())) return e;
        ++kernels;
    }
    if (l.info) {
        l.info->path = GN_PATH_SLAB;
        l.info->kernels = kernels;
        l.info->grid = grid;
        l.info->tiles = grid;
        l.info->resident_cap = 0;
        l.info->team = 1;
    }
    return hipSuccess;
}

// NCHW split form (split_nchw_*): tensors up to GN_SLAB_SPLIT_FWD_BYTES
// (forward) or GN_SLAB_SPLIT_BWD_BYTES (backward) whose slabs are past the
// one-workgroup kernels, at most kSplitMaxTiles statistics tiles per slab.
// Past those sizes the cooperative kernels' single pass over the data wins.
// Graphs of 20 calls, forward / backward us, cooperative -> split: 2 x 32 x
// 128 x 128 fp32 G4 (4 MiB) 32.5 / 34.2 -> 9.9 / 9.7; 1 x 128 x 256 x 256 fp16
// G32 (16 MiB) 33.9 / 40.8 -> 14.9 / 18.7; 8 x 64 x 128 x 128 fp32 G8 (32 MiB)
// 35.7 / 45.4 -> 21.7 / 29.3; 1 x 512 x 256 x 256 fp16 G32 (64 MiB) 45.7 /
// 69.0 -> 50.3 / 58.6; at 128 MiB (2 x 512 x 256 x 256 fp16) 74.6 / 107.0 ->
// 95.8 / 108.9.
#ifndef GN_SLAB_SPLIT_FWD_BYTES
#define GN_SLAB_SPLIT_FWD_BYTES (32 << 20)
#endif
#ifndef GN_SLAB_SPLIT_BWD_BYTES
#define GN_SLAB_SPLIT_BWD_BYTES (64 << 20)
#endif
constexpr int kSplitR = 8, kSplitRO = 4, kSplitMaxTiles = 256;

struct SplitPlan {
    int R, tpc, ntl, otiles;
    size_t off_stot, total;   // workspace: tile partials, then (backward) [N][C] float2
};

// The split form's plan for this problem, or false when it does not apply
// (the caps and limits above; a residency cap asks for the cooperative kernels).
// any_size: the form wherever it can tile the slabs (the fallback of a refused
// cooperative launch), not only where it is the faster one.
bool split_plan(const Problem& p, int32_t max_resident_override, bool backward, SplitPlan* sp,
                bool any_size = false) {
    if (p.layout != GN_NCHW || p.N * p.G > 65535) return false;
    const int64_t limit = backward ? (int64_t)GN_SLAB_SPLIT_BWD_BYTES : (int64_t)GN_SLAB_SPLIT_FWD_BYTES;
    if (!any_size && (max_resident_override > 0 || (int64_t)p.N * p.C * p.HW * p.elem_bytes > limit)) return false;
    const int V = vec_elems(p);
    // the kernels take HW and a slab's chunk index (up to D*HW/V, plus one
    // output tile past it) as 32-bit integers
    if (p.HW > INT32_MAX || p.D * (p.HW / V) + (int64_t)kT * kSplitRO >= INT32_MAX) return false;
    const int64_t cpc = p.HW / V;
    int R = 1;
    while (R < kSplitR && (int64_t)kT * R < cpc) R *= 2;
    const int64_t tpc = (cpc + (int64_t)kT * R - 1) / ((int64_t)kT * R);
    if (p.D * tpc > kSplitMaxTiles) return false;
    sp->R = R;
    sp->tpc = (int)tpc;
    sp->ntl = (int)(p.D * tpc);
    sp->otiles = (int)((p.D * cpc + (int64_t)kT * kSplitRO - 1) / ((int64_t)kT * kSplitRO));
    const size_t part = al((size_t)p.N * p.G * sp->ntl * (backward ? sizeof(float2) : sizeof(float4)));
    sp->off_stot = part;
    sp->total = part + (backward ? al((size_t)p.N * p.C * sizeof(float2)) : 0);
    return true;
}

template <typename T>
hipError_t split_fwd(const Problem& p, const FwdArgs& a, const Launch& l, const SplitPlan& sp) {
    auto ks = sp.R == 1 ? split_nchw_stats<T, 1>
            : sp.R == 2 ? split_nchw_stats<T, 2>
            : sp.R == 4 ? split_nchw_stats<T, 4>
                        : split_nchw_stats<T, kSplitR>;
    float4* part = (float4*)l.ws;
    const unsigned slabs = (unsigned)(p.N * p.G);
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(ks, dim3((unsigned)sp.ntl, slabs), dim3(kT), 0, l.stream, (const T*)a.x, (int)p.D, (int)p.HW,
                       sp.tpc, part);
    hipLaunchKernelGGL((split_nchw_apply<T, kSplitRO>), dim3(a.y ? (unsigned)sp.otiles : 1u, slabs), dim3(kT), 0,
                       l.stream, (const T*)a.x, a.gamma, a.beta, (T*)a.y, (const float4*)part, a.mean, a.rstd, p.G,
                       (int)p.D, (int)p.HW, sp.ntl, a.eps);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_SLAB;
        l.info->kernels = 2;
        l.info->grid = (int64_t)sp.ntl * slabs;
        l.info->tiles = (int64_t)sp.ntl * slabs;
        l.info->resident_cap = 0;
        l.info->team = 0;
    }
    return hipSuccess;
}

template <typename T>
hipError_t split_bwd(const Problem& p, const BwdArgs& a, const Launch& l, const SplitPlan& sp) {
    auto ks = sp.R == 1 ? split_nchw_sums<T, 1>
            : sp.R == 2 ? split_nchw_sums<T, 2>
            : sp.R == 4 ? split_nchw_sums<T, 4>
                        : split_nchw_sums<T, kSplitR>;
    float2* part = (float2*)l.ws;
    float2* stot = (float2*)((char*)l.ws + sp.off_stot);
    const bool want_dx = (a.mask & GN_GRAD_DX) != 0;
    const bool params = (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) != 0;
    const unsigned slabs = (unsigned)(p.N * p.G);
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(ks, dim3((unsigned)sp.ntl, slabs), dim3(kT), 0, l.stream, (const T*)a.dy, (const T*)a.x,
                       a.mean, a.rstd, (int)p.D, (int)p.HW, sp.tpc, part);
    hipLaunchKernelGGL((split_nchw_dx<T, kSplitRO>), dim3(want_dx ? (unsigned)sp.otiles : 1u, slabs), dim3(kT), 0,
                       l.stream, (const T*)a.dy, (const T*)a.x, a.mean, a.rstd, a.gamma, (const float2*)part,
                       (T*)a.dx, params ? stot : nullptr, p.G, p.C, (int)p.D, (int)p.HW, sp.tpc, want_dx ? 1 : 0);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    int kernels = 2;
    if (params) {
        hipLaunchKernelGGL(params_over_n, dim3((unsigned)((p.C + kT - 1) / kT)), dim3(kT), 0, l.stream, stot, p.N,
                           p.C, (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr,
                           (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr);
        if ((e = hipGetLastError())) return e;
        ++kernels;
    }
    if (l.info) {
        l.info->path = GN_PATH_SLAB;
        l.info->kernels = kernels;
        l.info->grid = (int64_t)sp.ntl * slabs;
        l.info->tiles = (int64_t)sp.ntl * slabs;
        l.info->resident_cap = 0;
        l.info->team = 0;
    }
    return hipSuccess;
}

// ---- a refused cooperative launch --------------------------------------------
// The runtime refuses hipLaunchCooperativeKernel (hipErrorIllegalState) while
// another process on the device has made cooperative launches and is still
// running (measured on MI355X, ROCm 7).  Such a call takes kernels that need no
// co-residency instead: the split form wherever it can tile the slabs, else the
// generic kernels.  The workspace size queries cover both; the sync words the
// clear kernel already wrote are not read by them.
template <typename T>
hipError_t fwd_refused(const Problem& p, const FwdArgs& a, const Launch& l) {
    SplitPlan sp;
    if (split_plan(p, 0, false, &sp, true)) return split_fwd<T>(p, a, l, sp);
    return generic_fwd(p, dense_strides(p), a, l);
}

template <typename T>
hipError_t bwd_refused(const Problem& p, const BwdArgs& a, const Launch& l) {
    SplitPlan sp;
    if (split_plan(p, 0, true, &sp, true)) return split_bwd<T>(p, a, l, sp);
    return generic_bwd(p, dense_strides(p), a, l);
}

// Under stream capture a refused cooperative launch is not reported: it is
// recorded, and every replay of the graph then skips the kernel without an
// error (measured: y left as it was).  So a call recorded before this
// process's runtime has accepted a cooperative launch takes the kernels above.
bool coop_unsafe_to_record(hipStream_t s) {
    if (coop_accepted()) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

template <typename T>
hipError_t fwd_t(const Problem& p, const FwdArgs& a, const Launch& l) {
    if (const int bt = small_bt(p, l, false)) return small_fwd<T>(p, a, l, bt);
    SplitPlan sp;
    if (!l.slab_coop && split_plan(p, l.max_resident_override, false, &sp)) return split_fwd<T>(p, a, l, sp);
    const int cus = device_info().cu_count;
    const bool nhwc = p.layout == GN_NHWC;
    auto kn = slab_nhwc_fwd<T, GN_SLAB_NHWC_RF>;
    auto kc = nchw_fwd_kernel<T>(nchw_r(p, false));
    int64_t cap = nhwc ? resident_cap(kn, cus) : resident_cap(kc, cus);
    if (l.max_resident_override > 0 && l.max_resident_override < cap) cap = l.max_resident_override;
    Plan pl = layout_ws(p, false, cap);
    SlabCfg cfg = pl.cfg;
    cfg.N = p.N; cfg.C = p.C; cfg.HW = p.HW; cfg.G = p.G; cfg.D = p.D; cfg.eps = a.eps;
    cfg.want_dx = 0; cfg.dgamma = nullptr; cfg.dbeta = nullptr;
    cfg.spin_limit = l.spin_limit; cfg.unmet = l.unmet_waits;
    if (cfg.team > 1 && coop_unsafe_to_record(l.stream)) return fwd_refused<T>(p, a, l);
    const int64_t grid = pl.grid;   // <= cap: every workgroup co-resident
    char* ws = (char*)l.ws;
    uint32_t* ctr = (uint32_t*)(ws + pl.off_ctr);
    uint32_t* err = l.status_word ? l.status_word : (uint32_t*)(ws + pl.off_err);
    void* part = ws + pl.off_part;   // NHWC: float4 per (group, tile); NCHW: one word per tile
    uint32_t* res = (uint32_t*)(ws + pl.off_res);
    hipError_t e;
    if ((e = clear_sync_words(ws, pl, l.stream))) return e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    const T* x = (const T*)a.x;
    T* y = (T*)a.y;
    const float* gamma = a.gamma;
    const float* beta = a.beta;
    float* mean = a.mean;
    float* rstd = a.rstd;
    void* args[] = {&x, &gamma, &beta, &y, &mean, &rstd, &cfg, &ctr, &err, &part, &res};
    const bool coop = cfg.team > 1;
    e = nhwc ? launch_coop(kn, grid, args, l.stream, coop) : launch_coop(kc, grid, args, l.stream, coop);
    if (e && coop) {
        (void)hipGetLastError();
        return fwd_refused<T>(p, a, l);
    }
    if (e) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_SLAB;
        l.info->kernels = 2;
        l.info->grid = grid;
        l.info->tiles = cfg.tiles * cfg.n_slabs;
        l.info->resident_cap = cap;
        l.info->team = cfg.team;
    }
    return hipSuccess;
}

template <typename T>
hipError_t bwd_t(const Problem& p, const BwdArgs& a, const Launch& l) {
    if (const int bt = small_bt(p, l, true)) return small_bwd<T>(p, a, l, bt);
    SplitPlan sp;
    if (!l.slab_coop && split_plan(p, l.max_resident_override, true, &sp)) return split_bwd<T>(p, a, l, sp);
    const int cus = device_info().cu_count;
    const bool nhwc = p.layout == GN_NHWC;
    auto kn = slab_nhwc_bwd<T, GN_SLAB_NHWC_RB>;
    auto kc = nchw_bwd_kernel<T>(nchw_r(p, true));
    int64_t cap = nhwc ? resident_cap(kn, cus) : resident_cap(kc, cus);
    if (l.max_resident_override > 0 && l.max_resident_override < cap) cap = l.max_resident_override;
    Plan pl = layout_ws(p, true, cap);
    SlabCfg cfg = pl.cfg;
    cfg.N = p.N; cfg.C = p.C; cfg.HW = p.HW; cfg.G = p.G; cfg.D = p.D; cfg.eps = 0.f;
    cfg.want_dx = (a.mask & GN_GRAD_DX) ? 1 : 0;
    const bool one_slab_params = nhwc && p.N == 1;
    cfg.dgamma = one_slab_params ? a.dgamma : nullptr;
    cfg.dbeta = one_slab_params ? a.dbeta : nullptr;
    cfg.spin_limit = l.spin_limit; cfg.unmet = l.unmet_waits;
    if (cfg.team > 1 && coop_unsafe_to_record(l.stream)) return bwd_refused<T>(p, a, l);
    const int64_t grid = pl.grid;   // <= cap: every workgroup co-resident
    char* ws = (char*)l.ws;
    uint32_t* ctr = (uint32_t*)(ws + pl.off_ctr);
    uint32_t* err = l.status_word ? l.status_word : (uint32_t*)(ws + pl.off_err);
    void* part = ws + pl.off_part;   // NHWC: float2 per (channel, tile); NCHW: one word per tile
    float2* stot = (float2*)(ws + pl.off_stot);
    uint32_t* res = (uint32_t*)(ws + pl.off_res);
    hipError_t e;
    if ((e = clear_sync_words(ws, pl, l.stream))) return e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    const T* dy = (const T*)a.dy;
    const T* x = (const T*)a.x;
    const float* mean = a.mean;
    const float* rstd = a.rstd;
    const float* gamma = a.gamma;
    T* dx = (T*)a.dx;
    void* args[] = {&dy, &x, &mean, &rstd, &gamma, &dx, &cfg, &ctr, &err, &part, &stot, &res};
    const bool coop = cfg.team > 1;
    e = nhwc ? launch_coop(kn, grid, args, l.stream, coop) : launch_coop(kc, grid, args, l.stream, coop);
    if (e && coop) {
        (void)hipGetLastError();
        return bwd_refused<T>(p, a, l);
    }
    if (e) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    int kernels = 2;
    if ((a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) && !one_slab_params) {
        hipLaunchKernelGGL(params_over_n, dim3((unsigned)((p.C + kT - 1) / kT)), dim3(kT), 0, l.stream, stot, p.N,
                           p.C, a.dgamma, a.dbeta);
        if ((e = hipGetLastError())) return e;
        ++kernels;
    }
    if (l.info) {
        l.info->path = GN_PATH_SLAB;
        l.info->kernels = kernels;
        l.info->grid = grid;
        l.info->tiles = cfg.tiles * cfg.n_slabs;
        l.info->resident_cap = cap;
        l.info->team = cfg.team;
    }
    return hipSuccess;
}

}  // namespace

bool slab_ok(const Problem& p) {
    const int V = vec_elems(p);
    if (p.layout == GN_NHWC) {
        if (p.C % V != 0 || p.D % V != 0) return false;
        const int64_t cpp = p.C / V;
        if (cpp < 1 || cpp > kT || (kT % cpp) != 0) return false;   // chunks per pixel divide the workgroup
        return p.HW >= 1;
    }
    if (p.HW % V != 0) return false;   // every channel plane starts 16-byte aligned
    int64_t tpc;
    if (tiles_per_slab(p, tile_chunks(p, true), &tpc) >= ((int64_t)1 << 31) ||
        tiles_per_slab(p, tile_chunks(p, false), &tpc) >= ((int64_t)1 << 31))
        return false;                   // tile indices of a slab in 32 bits
    return p.HW >= V && p.D <= kT;      // channel sums of a slab: one thread per channel
}

// The largest of the cooperative kernels' layout and the other forms a call may
// take (the split form, or the generic kernels where the split form cannot
// tile the slabs): a size query does not know whether the call will cap the
// residency or find its cooperative launch refused.
size_t slab_fwd_ws(const Problem& p) {
    int64_t tpc;
    const size_t coop = layout_ws(p, false, tiles_per_slab(p, tile_chunks(p, false), &tpc)).total;
    SplitPlan sp;   // the split form (also a refused cooperative launch's), else the generic kernels
    const size_t other = split_plan(p, 0, false, &sp, true) ? sp.total : generic_fwd_ws(p, dense_strides(p));
    return std::max(coop, other);
}

size_t slab_bwd_ws(const Problem& p, int32_t mask) {
    int64_t tpc;
    const size_t coop = layout_ws(p, true, tiles_per_slab(p, tile_chunks(p, true), &tpc)).total;
    SplitPlan sp;
    const size_t other = split_plan(p, 0, true, &sp, true) ? sp.total : generic_bwd_ws(p, dense_strides(p), mask);
    return std::max(coop, other);
}

hipError_t slab_fwd(const Problem& p, const FwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return fwd_t<float>(p, a, l);
        case GN_F16: return fwd_t<_Float16>(p, a, l);
        default: return fwd_t<__bf16>(p, a, l);
    }
}

hipError_t slab_bwd(const Problem& p, const BwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return bwd_t<float>(p, a, l);
        case GN_F16: return bwd_t<_Float16>(p, a, l);
        default: return bwd_t<__bf16>(p, a, l);
    }
}

}  // namespace gn
