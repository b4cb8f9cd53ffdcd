// gn_stream.hip -- NHWC GroupNorm as a few streaming launches, one tile per
// workgroup: the planner's path for every NHWC shape these kernels take.
//
// In NHWC every group of a sample is spread over the whole image (16 bytes =
// V channels of one group per pixel), so the slab of one statistic is the
// whole sample.  When that slab exceeds what the co-resident grid can hold in
// registers, a cooperative one-pass kernel re-reads most tiles anyway and
// pays a per-tile hand-out and barrier cost on top; launching one workgroup
// per tile lets the hardware dispatcher balance the load instead.  On
// smaller images the cooperative launch and its two team barriers per slab
// cost more than the second read saves (2-6x slower than these kernels from
// 2x32x16x16 to 16x256x64x64, forward and backward).
//
//   forward   1. per tile: (count, mean, M2) of each group, an exact two-pass
//               over the tile from registers (fixed-order trees in LDS)
//             2. per slice: the tile partials in a fixed order -> mean, rstd
//               (sum n_i*mean_i, then sum M2_i + n_i*(mean_i - mean)^2)
//             3. per tile: y = (x - mean)*(rstd*gamma_c) + beta_c
//   backward  1. per tile: per-channel sums of dy and dy*xhat (xhat from the
//               saved mean/rstd)
//             2. per (n, c): those sums over the tiles, in two fixed-order
//               levels -> S1[n,c], S2[n,c]
//             3. per slice: A/M = sum_c gamma_c*S1/M, B/M = sum_c gamma_c*S2/M;
//               dbeta_c = sum_n S1[n,c], dgamma_c = sum_n S2[n,c]
//             4. per tile: dx = rstd*(gamma_c*dy - A/M - xhat*B/M)
// (POPCORNBENCH GroupNorm trace: statistics pass, then normalize-and-affine
// pass; baracuda-kernels GroupNorm backward plan: per-group reductions, then
// the elementwise dx.)  All reductions run in a fixed order, so the results
// are bitwise reproducible.  Activations are read with non-temporal loads and
// outputs written with non-temporal stores: nothing is read twice within the
// caches' reach.  A sample that fits one tile takes one workgroup, which runs
// all of the steps above from its registers in one launch (fwd_one_tile,
// bwd_one_tile); a sample of a few tiles skips step 2 (forward) or steps 2
// and 3 (backward), which its output kernels do themselves (fwd_apply_few,
// bwd_dx_few).
#include "gn_device.hpp"
#include "gn_internal.hpp"

namespace gn {
namespace {

constexpr int kT = 256;
constexpr int kNW = kT / kWave;

// 16-byte chunks per thread per tile (of x, and of dy in the backward), per
// kernel, as measured on the 1x128x1024x2048 fp16 image: 16 for the two
// reductions, 4 for the two output passes (forward output, rocprofv3 averages
// over 42 dispatches: 16 -> 178.0 us, 8 -> 166.5 us, 4 -> 161.2 us, 2 -> 162.8
// us; dx: 2 -> 268.0 us, 4 -> 253.5 us, 8 -> 271.9 us).  The output passes
// store what they load; fewer stores per thread in one burst keep the write
// stream from stalling the loads.
#ifndef GN_STREAM_R_STATS
#define GN_STREAM_R_STATS 16
#endif
#ifndef GN_STREAM_R_APPLY
#define GN_STREAM_R_APPLY 4
#endif
#ifndef GN_STREAM_R_SUMS
#define GN_STREAM_R_SUMS 16
#endif
#ifndef GN_STREAM_R_DX
#define GN_STREAM_R_DX 4
#endif

struct StreamCfg {
    int64_t N, C, HW, G, D;
    int64_t tiles;   // tiles per sample of the reduction kernel (partials per sample)
    int64_t otiles;  // tiles per sample of the output kernel
    float eps;
};

int vec_elems(const Problem& p) { return p.elem_bytes == 4 ? 4 : 8; }

// Thread t owns chunk q = t % CPP of each pixel it visits (channels q*V ..
// q*V+V-1, CPP = C/V chunks per pixel) and pixel row t / CPP of each of the
// tile's R iterations; a tile is R*PPI consecutive pixels of one sample,
// PPI = floor(kT / CPP).  When CPP does not divide kT, the last kT - PPI*CPP
// threads are idle.  A chunk's channels may belong to two or more groups (D
// need not be a multiple of V): every per-channel quantity looks up its own
// channel's group.
struct TileGeom {
    int V, CPP, q, pi, PPI;
    bool active;
    int64_t TP;
};

template <typename T, int R>
__device__ inline TileGeom tile_geom(int64_t C) {
    TileGeom g;
    g.V = Vec<T>::V;
    g.CPP = (int)(C / g.V);
    g.q = threadIdx.x % g.CPP;
    g.pi = threadIdx.x / g.CPP;
    g.PPI = kT / g.CPP;
    g.active = g.pi < g.PPI;
    g.TP = (int64_t)g.PPI * R;
    return g;
}

// R chunks of one tile; pixels past HW are clamped onto the last pixel (in
// bounds, no branch around the loads) and dropped by the caller.
template <typename T, int R>
__device__ inline void load_tile(const T* __restrict__ src, int64_t HW, int64_t C, int64_t p0, int PPI,
                                 u4v (&dst)[R]) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t p = min(p0 + (int64_t)j * PPI, HW - 1);
        dst[j] = ld16_nt(src + p * C);
    }
}

__device__ inline void add_to(float& a, const float& b) { a += b; }
__device__ inline void add_to(float2& a, const float2& b) {
    a.x += b.x;
    a.y += b.y;
}

// Fixed-order tree over the tile's PPI pixel rows of per-thread, per-channel
// values s[t*V + k]; afterwards row 0 holds the tile's channel totals, the
// value of channel c at s[c].  Every thread of the workgroup calls it.
template <int V, typename S>
__device__ inline void tree_rows(S* s, const TileGeom& tg) {
    int top = 1;
    while (top < tg.PPI) top *= 2;
    for (int h = top / 2; h > 0; h /= 2) {
        if (tg.active && tg.pi < h && tg.pi + h < tg.PPI) {
            const int t = threadIdx.x;
#pragma unroll
            for (int k = 0; k < V; ++k) add_to(s[t * V + k], s[(t + h * tg.CPP) * V + k]);
        }
        __syncthreads();
    }
}

// Fixed-order tree over consecutive segments of `seg` entries among the
// first `count` entries of s (a group's channels, or its chunks); afterwards
// s[g*seg] holds segment g's total.  Every thread calls it.
__device__ inline void tree_groups(float* s, int count, int seg) {
    int top = 1;
    while (top < seg) top *= 2;
    for (int h = top / 2; h > 0; h /= 2) {
        for (int c = threadIdx.x; c < count; c += kT) {
            const int l = c % seg;
            if (l < h && l + h < seg) s[c] += s[c + h];
        }
        __syncthreads();
    }
}

// Group totals of per-thread, per-channel values acc[k] over the tile: the
// values go through the pixel-row tree and the per-group tree; afterwards
// group g's total lies at s[group_slot(g)].  WHOLE (D % V == 0): each thread
// first adds its V channels, all of one group, so the trees carry one value
// per thread (the group's total then at s[g*D/V]); otherwise V values per
// thread and a tree over each group's channels (total at s[g*D]).
template <int V, bool WHOLE>
__device__ inline void group_totals(float* s, const float (&acc)[V], const TileGeom& tg, int C, int D) {
    const int t = threadIdx.x;
    if constexpr (WHOLE) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < V; ++k) a += acc[k];
        s[t] = a;
        __syncthreads();
        tree_rows<1>(s, tg);
        tree_groups(s, tg.CPP, D / V);
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k) s[t * V + k] = acc[k];
        __syncthreads();
        tree_rows<V>(s, tg);
        tree_groups(s, C, D);
    }
}

template <int V, bool WHOLE>
__device__ inline int group_slot(int g, int D) { return WHOLE ? g * (D / V) : g * D; }

// Slice (n, g) of each of a thread's V channels q*V .. q*V+V-1.  WHOLE: the
// groups are whole 16-byte chunks, so all V channels share one slice (one
// division, one load per quantity); otherwise one per channel (32-bit
// divisions: channels are below 2048).  A compile-time choice, so that
// neither form has a branch around loads.
template <int V, bool WHOLE>
__device__ inline void channel_slices(int q, int D, int64_t n, int64_t G, int64_t (&s)[V]) {
    if constexpr (WHOLE) {
        const int64_t s0 = n * G + (q * V) / D;
#pragma unroll
        for (int k = 0; k < V; ++k) s[k] = s0;
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k) s[k] = n * G + (q * V + k) / D;
    }
}

// Per-channel copies of a per-slice quantity.
template <int V, bool WHOLE, typename S>
__device__ inline void per_channel(const S* __restrict__ v, const int64_t (&s)[V], S (&o)[V]) {
    if constexpr (WHOLE) {
        const S a = v[s[0]];
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = a;
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = v[s[k]];
    }
}

// V per-channel parameters from c0 (a multiple of 4; p 16-byte aligned), or
// `dflt` when p is NULL: float4 loads.
template <int V>
__device__ inline void load_params(const float* __restrict__ p, int64_t c0, float dflt, float (&o)[V]) {
    if (!p) {
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = dflt;
        return;
    }
#pragma unroll
    for (int k = 0; k < V; k += 4) {
        const float4 q = *reinterpret_cast<const float4*>(p + c0 + k);
        o[k] = q.x; o[k + 1] = q.y; o[k + 2] = q.z; o[k + 3] = q.w;
    }
}

// Chunks j = 0 .. R-1 of a thread's tile that hold a pixel (p0 + j*PPI < HW),
// as one 32-bit count: the per-chunk tests of several passes then share one
// register instead of R 64-bit pixel indices kept live between the passes.
template <int R>
__device__ inline int valid_chunks(bool active, int64_t p0, int64_t HW, int PPI) {
    const int64_t rem = HW - p0;
    if (!active || rem <= 0) return 0;
    const int r = (int)(rem < (int64_t)R * PPI ? rem : (int64_t)R * PPI);
    return (r + PPI - 1) / PPI;
}

// ---- forward ----------------------------------------------------------------
// grid (tiles, N); part: [N*G][tiles] float4 (count, mean, M2, -) of each
// group over the tile -- an exact two-pass over the tile: per-channel sums ->
// group sums -> the tile's group means, then per-channel sums of squared
// deviations from them -> group M2, each reduction a fixed-order tree.
constexpr int kMaxC = kT * 8;   // channels of a pixel (C/V <= kT chunks of at most 8)
template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void fwd_tile_stats(const T* __restrict__ x, StreamCfg cfg,
                                                     float4* __restrict__ part) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int C = (int)cfg.C, D = (int)cfg.D, G = (int)cfg.G;
    const int64_t tile = blockIdx.x, n = blockIdx.y;
    __shared__ float s[kT * 8];      // [thread][k], then channel totals at s[c]
    __shared__ float gsum[kMaxC];    // group sums of pass 1 (G <= C)
    u4v reg[R];
    const int64_t p0 = tile * tg.TP + tg.pi;
    load_tile<T, R>(x + n * cfg.HW * cfg.C + tg.q * V, cfg.HW, cfg.C, p0, tg.PPI, reg);
    const int nv = valid_chunks<R>(tg.active, p0, cfg.HW, tg.PPI);
    float acc[V];
#pragma unroll
    for (int k = 0; k < V; ++k) acc[k] = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
            float v[V];
            Vec<T>::unpack(reg[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) acc[k] += v[k];
        }
    }
    group_totals<V, WHOLE>(s, acc, tg, C, D);
    const int64_t rows = min(tg.TP, cfg.HW - tile * tg.TP);   // pixels of this tile
    const float cnt = (float)(rows * D);                       // elements of a group in it
    float mu[V];
#pragma unroll
    for (int k = 0; k < V; ++k) mu[k] = s[group_slot<V, WHOLE>((tg.q * V + k) / D, D)] / cnt;
    for (int g = t; g < G; g += kT) gsum[g] = s[group_slot<V, WHOLE>(g, D)];
    __syncthreads();   // every read of pass 1's totals is done before s is reused
#pragma unroll
    for (int k = 0; k < V; ++k) acc[k] = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
            float v[V];
            Vec<T>::unpack(reg[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = v[k] - mu[k];
                acc[k] = fmaf(d, d, acc[k]);
            }
        }
    }
    group_totals<V, WHOLE>(s, acc, tg, C, D);
    for (int g = t; g < G; g += kT)
        part[(n * cfg.G + g) * cfg.tiles + tile] = make_float4(cnt, gsum[g] / cnt, s[group_slot<V, WHOLE>(g, D)], 0.f);
}

// one workgroup of kFinT threads per slice (blockIdx.x = n*G + g).  Each pass
// loads kFinB partials per thread at once (independent loads), so a slice of
// many thousand tiles costs a few load round trips, not one per tile.
constexpr int kFinT = 1024, kFinNW = kFinT / kWave, kFinB = 8;
__global__ __launch_bounds__(kFinT) void fwd_finalize(const float4* __restrict__ part, StreamCfg cfg,
                                                      float* __restrict__ mean, float* __restrict__ rstd) {
    __shared__ float lds[kFinNW * 2];
    const int64_t sg = blockIdx.x;
    const float4* pg = part + sg * cfg.tiles;
    const int t = threadIdx.x;
    float sums[2] = {0.f, 0.f};
    for (int64_t base = 0; base < cfg.tiles; base += (int64_t)kFinT * kFinB) {
        float4 v[kFinB];
#pragma unroll
        for (int j = 0; j < kFinB; ++j) {
            const int64_t i = base + (int64_t)j * kFinT + t;
            v[j] = i < cfg.tiles ? pg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < kFinB; ++j) {
            sums[0] = fmaf(v[j].x, v[j].y, sums[0]);
            sums[1] += v[j].x;
        }
    }
    block_sum<2, kFinNW>(sums, lds);
    const float mu = sums[0] / sums[1];
    float m2[1] = {0.f};
    for (int64_t base = 0; base < cfg.tiles; base += (int64_t)kFinT * kFinB) {
        float4 v[kFinB];
#pragma unroll
        for (int j = 0; j < kFinB; ++j) {
            const int64_t i = base + (int64_t)j * kFinT + t;
            v[j] = i < cfg.tiles ? pg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < kFinB; ++j) {
            const float d = v[j].y - mu;
            m2[0] += fmaf(v[j].x * d, d, v[j].z);
        }
    }
    block_sum<1, kFinNW>(m2, lds);
    if (t == 0) {
        float var = m2[0] / (float)(cfg.D * cfg.HW);
        var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
        mean[sg] = mu;
        rstd[sg] = 1.0f / sqrtf(var + cfg.eps);
    }
}

// grid (otiles, N)
template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void fwd_apply(const T* __restrict__ x, const float* __restrict__ gamma,
                                                const float* __restrict__ beta, T* __restrict__ y,
                                                const float* __restrict__ mean, const float* __restrict__ rstd,
                                                StreamCfg cfg) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    if (!tg.active) return;   // no barrier below
    const int64_t tile = blockIdx.x, n = blockIdx.y;
    const int64_t off = n * cfg.HW * cfg.C + tg.q * V;
    u4v reg[R];
    const int64_t p0 = tile * tg.TP + tg.pi;
    load_tile<T, R>(x + off, cfg.HW, cfg.C, p0, tg.PPI, reg);
    float mu[V], rs[V], a[V], b[V];
    int64_t sl[V];
    channel_slices<V, WHOLE>(tg.q, (int)cfg.D, n, cfg.G, sl);
    per_channel<V, WHOLE>(mean, sl, mu);
    per_channel<V, WHOLE>(rstd, sl, rs);
    load_params<V>(gamma, tg.q * V, 1.f, a);
    load_params<V>(beta, tg.q * V, 0.f, b);
#pragma unroll
    for (int k = 0; k < V; ++k) a[k] *= rs[k];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t p = p0 + (int64_t)j * tg.PPI;
        if (p < cfg.HW) {
            float v[V], o[V];
            Vec<T>::unpack(reg[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = fmaf(v[k] - mu[k], a[k], b[k]);
            st16_nt(y + off + p * cfg.C, Vec<T>::pack(o));
        }
    }
}

// ---- backward ---------------------------------------------------------------
// grid (tiles, N); part: [N][tiles][C] float2 (sum dy, sum dy*xhat)
template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void bwd_tile_sums(const T* __restrict__ dy, const T* __restrict__ x,
                                                    const float* __restrict__ mean,
                                                    const float* __restrict__ rstd, StreamCfg cfg,
                                                    float2* __restrict__ part) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int64_t tile = blockIdx.x, n = blockIdx.y;
    const int64_t off = n * cfg.HW * cfg.C + tg.q * V;
    __shared__ float2 lds[kT * 8];   // [thread][k], V <= 8
    u4v rx[R], rd[R];
    const int64_t p0 = tile * tg.TP + tg.pi;
    load_tile<T, R>(x + off, cfg.HW, cfg.C, p0, tg.PPI, rx);
    load_tile<T, R>(dy + off, cfg.HW, cfg.C, p0, tg.PPI, rd);
    const int nv = valid_chunks<R>(tg.active, p0, cfg.HW, tg.PPI);
    float mu[V], rs[V];
    int64_t sl[V];
    channel_slices<V, WHOLE>(tg.q, (int)cfg.D, n, cfg.G, sl);
    per_channel<V, WHOLE>(mean, sl, mu);
    per_channel<V, WHOLE>(rstd, sl, rs);
    float s1[V], s2[V];
#pragma unroll
    for (int k = 0; k < V; ++k) { s1[k] = 0.f; s2[k] = 0.f; }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
            float xv[V], dv[V];
            Vec<T>::unpack(rx[j], xv);
            Vec<T>::unpack(rd[j], dv);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                s1[k] += dv[k];
                s2[k] = fmaf(dv[k], (xv[k] - mu[k]) * rs[k], s2[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < V; ++k) lds[t * V + k] = make_float2(s1[k], s2[k]);
    __syncthreads();
    tree_rows<V>(lds, tg);
    // row 0 holds the tile's channel sums, channel c at lds[c]
    float2* dst = part + (n * cfg.tiles + tile) * cfg.C;
    for (int c = t; c < (int)cfg.C; c += kT) dst[c] = lds[c];
}

// Column sums of src [N][rows][C] float2 over row ranges of `per` rows:
// dst [N][chunks][C].  grid (ceil(C/(2*kColPairs)), chunks, N).  Each thread
// sums two adjacent channels (one float4) over its row lane in row order; the
// row lanes are then added in lane order.
constexpr int kColPairs = 8;
constexpr int kRowLanes = kT / kColPairs;
__global__ __launch_bounds__(kT) void col_sums(const float2* __restrict__ src, int64_t rows, int64_t C,
                                               int64_t per, float2* __restrict__ dst) {
    const int cp = threadIdx.x % kColPairs;
    const int rl = threadIdx.x / kColPairs;
    const int64_t c0 = ((int64_t)blockIdx.x * kColPairs + cp) * 2;
    const int64_t chunk = blockIdx.y, n = blockIdx.z;
    const int64_t r0 = chunk * per;
    const int64_t r1 = min(r0 + per, rows);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c0 < C) {
        const float2* s = src + n * rows * C + c0;
#pragma unroll 4
        for (int64_t b = r0 + rl; b < r1; b += kRowLanes) {
            const float4 q = *reinterpret_cast<const float4*>(s + b * C);
            acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
        }
    }
    __shared__ float4 red[kT];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (rl == 0 && c0 < C) {
        float4 tot = red[cp];
        for (int k = 1; k < kRowLanes; ++k) {
            const float4 q = red[k * kColPairs + cp];
            tot.x += q.x; tot.y += q.y; tot.z += q.z; tot.w += q.w;
        }
        *reinterpret_cast<float4*>(dst + (n * gridDim.y + chunk) * C + c0) = tot;
    }
}

// grid (G, N): ab[n*G + g] = (A/M, B/M); with one sample, dbeta/dgamma too
__global__ __launch_bounds__(kT) void bwd_group_ab(const float2* __restrict__ stot, const float* __restrict__ gamma,
                                                   StreamCfg cfg, float2* __restrict__ ab,
                                                   float* __restrict__ dgamma, float* __restrict__ dbeta) {
    __shared__ float lds[kNW * 2];
    const int64_t g = blockIdx.x, n = blockIdx.y;
    float acc[2] = {0.f, 0.f};
    for (int64_t c = g * cfg.D + threadIdx.x; c < (g + 1) * cfg.D; c += kT) {
        const float2 v = stot[n * cfg.C + c];
        const float ga = gamma ? gamma[c] : 1.f;
        acc[0] = fmaf(ga, v.x, acc[0]);
        acc[1] = fmaf(ga, v.y, acc[1]);
        if (cfg.N == 1) {
            if (dbeta) dbeta[c] = v.x;
            if (dgamma) dgamma[c] = v.y;
        }
    }
    block_sum<2, kNW>(acc, lds);
    if (threadIdx.x == 0) {
        const float invM = 1.0f / (float)(cfg.D * cfg.HW);
        ab[n * cfg.G + g] = make_float2(acc[0] * invM, acc[1] * invM);
    }
}

// dgamma/dbeta as sums over the samples, in sample order
__global__ __launch_bounds__(kT) void stream_params_over_n(const float2* __restrict__ stot, int64_t N, int64_t C,
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

// grid (otiles, N)
template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void bwd_dx(const T* __restrict__ dy, const T* __restrict__ x,
                                             const float* __restrict__ mean, const float* __restrict__ rstd,
                                             const float* __restrict__ gamma, const float2* __restrict__ ab,
                                             T* __restrict__ dx, StreamCfg cfg) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    if (!tg.active) return;   // no barrier below
    const int64_t tile = blockIdx.x, n = blockIdx.y;
    const int64_t off = n * cfg.HW * cfg.C + tg.q * V;
    u4v rx[R], rd[R];
    const int64_t p0 = tile * tg.TP + tg.pi;
    float mu[V], rs[V], Ak[V], Bk[V];
    int64_t sl[V];
    channel_slices<V, WHOLE>(tg.q, (int)cfg.D, n, cfg.G, sl);
    per_channel<V, WHOLE>(mean, sl, mu);
    per_channel<V, WHOLE>(rstd, sl, rs);
    float2 abk[V];
    per_channel<V, WHOLE>(ab, sl, abk);
#pragma unroll
    for (int k = 0; k < V; ++k) {
        Ak[k] = abk[k].x;
        Bk[k] = abk[k].y;
    }
    float ga[V];
    load_params<V>(gamma, tg.q * V, 1.f, ga);
    // the tile after the per-channel values (measured: 434 -> 428 us for the
    // 1x128x1024x2048 fp16 backward; the forward's apply is faster the other
    // way round)
    load_tile<T, R>(x + off, cfg.HW, cfg.C, p0, tg.PPI, rx);
    load_tile<T, R>(dy + off, cfg.HW, cfg.C, p0, tg.PPI, rd);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t p = p0 + (int64_t)j * tg.PPI;
        if (p < cfg.HW) {
#pragma clang fp contract(off)
            float xv[V], dv[V], o[V];
            Vec<T>::unpack(rx[j], xv);
            Vec<T>::unpack(rd[j], dv);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float xh = (xv[k] - mu[k]) * rs[k];
                const float gd = dv[k] * ga[k];
                o[k] = rs[k] * ((gd - Ak[k]) - xh * Bk[k]);
            }
            st16_nt(dx + off + p * cfg.C, Vec<T>::pack(o));
        }
    }
}

// ---- one tile per sample ----------------------------------------------------
// A sample whose HW pixels fit one tile of at most kOneTileR chunks per thread
// (HW <= PPI * kOneTileR) is one workgroup's whole call.  The forward's tile
// statistics are then the sample's: the exact two-pass above gives each
// group's mean and M2, the workgroup writes mean and rstd and then y from the
// registers.  The backward's per-channel tile sums of dy and dy*xhat are the
// sample's per-(n, c) sums: A and B of each group follow from a fixed-order
// tree over the group's channels, and dx is written from the registers.  One
// launch instead of three (forward) or four to five (backward).  grid (N).
constexpr int kOneTileR = 16;

template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void fwd_one_tile(const T* __restrict__ x, const float* __restrict__ gamma,
                                                   const float* __restrict__ beta, T* __restrict__ y,
                                                   float* __restrict__ mean, float* __restrict__ rstd,
                                                   StreamCfg cfg) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int C = (int)cfg.C, D = (int)cfg.D, G = (int)cfg.G;
    const int64_t n = blockIdx.x;
    __shared__ float s[kT * 8];     // [thread][k], then channel / group totals
    __shared__ float grp[kMaxC];    // each group's mean, then its rstd (G <= C)
    const int64_t off = n * cfg.HW * cfg.C + tg.q * V;
    u4v reg[R];
    load_tile<T, R>(x + off, cfg.HW, cfg.C, tg.pi, tg.PPI, reg);
    const int nv = valid_chunks<R>(tg.active, tg.pi, cfg.HW, tg.PPI);
    float acc[V];
#pragma unroll
    for (int k = 0; k < V; ++k) acc[k] = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
            float v[V];
            Vec<T>::unpack(reg[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) acc[k] += v[k];
        }
    }
    group_totals<V, WHOLE>(s, acc, tg, C, D);
    const float cnt = (float)(cfg.HW * D);   // elements of a group in the sample
    float mu[V];
#pragma unroll
    for (int k = 0; k < V; ++k) mu[k] = s[group_slot<V, WHOLE>((tg.q * V + k) / D, D)] / cnt;
    for (int g = t; g < G; g += kT) grp[g] = s[group_slot<V, WHOLE>(g, D)] / cnt;
    __syncthreads();   // every read of pass 1's totals is done before s is reused
#pragma unroll
    for (int k = 0; k < V; ++k) acc[k] = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
            float v[V];
            Vec<T>::unpack(reg[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = v[k] - mu[k];
                acc[k] = fmaf(d, d, acc[k]);
            }
        }
    }
    group_totals<V, WHOLE>(s, acc, tg, C, D);
    for (int g = t; g < G; g += kT) {   // thread t owns entries g = t, t + kT, ... of grp
        float var = s[group_slot<V, WHOLE>(g, D)] / cnt;
        var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
        const float r = 1.0f / sqrtf(var + cfg.eps);
        if (mean) mean[n * cfg.G + g] = grp[g];
        rstd[n * cfg.G + g] = r;
        grp[g] = r;
    }
    __syncthreads();
    if (y == nullptr || !tg.active) return;   // no barrier below
    float a[V], b[V];
    load_params<V>(gamma, tg.q * V, 1.f, a);
    load_params<V>(beta, tg.q * V, 0.f, b);
#pragma unroll
    for (int k = 0; k < V; ++k) a[k] *= grp[(tg.q * V + k) / D];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
            float v[V], o[V];
            Vec<T>::unpack(reg[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = fmaf(v[k] - mu[k], a[k], b[k]);
            st16_nt(y + off + (int64_t)(tg.pi + j * tg.PPI) * cfg.C, Vec<T>::pack(o));
        }
    }
}

// stot: [N][C] float2 per-(n, c) sums for stream_params_over_n (N > 1); with one
// sample dgamma/dbeta are the channel sums themselves and are written here.
template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void bwd_one_tile(const T* __restrict__ dy, const T* __restrict__ x,
                                                   const float* __restrict__ mean, const float* __restrict__ rstd,
                                                   const float* __restrict__ gamma, T* __restrict__ dx,
                                                   float2* __restrict__ stot, float* __restrict__ dgamma,
                                                   float* __restrict__ dbeta, StreamCfg cfg, int want_dx) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int C = (int)cfg.C, D = (int)cfg.D;
    const int64_t n = blockIdx.x;
    __shared__ float2 lds[kT * 8];   // [thread][k], then channel totals at lds[c]
    __shared__ float ga_s1[kMaxC], ga_s2[kMaxC];   // gamma_c * (sum dy, sum dy*xhat), then group totals
    const int64_t off = n * cfg.HW * cfg.C + tg.q * V;
    u4v rx[R], rd[R];
    load_tile<T, R>(x + off, cfg.HW, cfg.C, tg.pi, tg.PPI, rx);
    load_tile<T, R>(dy + off, cfg.HW, cfg.C, tg.pi, tg.PPI, rd);
    const int nv = valid_chunks<R>(tg.active, tg.pi, cfg.HW, tg.PPI);
    float mu[V], rs[V];
    int64_t sl[V];
    channel_slices<V, WHOLE>(tg.q, D, n, cfg.G, sl);
    per_channel<V, WHOLE>(mean, sl, mu);
    per_channel<V, WHOLE>(rstd, sl, rs);
    float s1[V], s2[V];
#pragma unroll
    for (int k = 0; k < V; ++k) { s1[k] = 0.f; s2[k] = 0.f; }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
            float xv[V], dv[V];
            Vec<T>::unpack(rx[j], xv);
            Vec<T>::unpack(rd[j], dv);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                s1[k] += dv[k];
                s2[k] = fmaf(dv[k], (xv[k] - mu[k]) * rs[k], s2[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < V; ++k) lds[t * V + k] = make_float2(s1[k], s2[k]);
    __syncthreads();
    tree_rows<V>(lds, tg);
    // row 0 holds the sample's channel sums, channel c at lds[c]
    for (int c = t; c < C; c += kT) {
        const float2 v = lds[c];
        if (cfg.N == 1) {
            if (dbeta) dbeta[c] = v.x;
            if (dgamma) dgamma[c] = v.y;
        } else if (stot) {
            stot[n * cfg.C + c] = v;
        }
    }
    if (!want_dx) return;   // kernel argument: uniform
    // gamma_c * (sum dy, sum dy*xhat) summed over each group's channels: with
    // whole 16-byte chunks per group a thread first adds its chunk's V
    // channels, then a tree over the group's chunks; otherwise a tree over
    // the group's channels.  Group g's A*M then lies at ga_s1[g*seg], B*M at
    // ga_s2[g*seg].
    const int seg = WHOLE ? D / V : D;
    if constexpr (WHOLE) {
        if (t < tg.CPP) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float2 v = lds[t * V + k];
                const float ga = gamma ? gamma[t * V + k] : 1.f;
                a = fmaf(ga, v.x, a);
                b = fmaf(ga, v.y, b);
            }
            ga_s1[t] = a;
            ga_s2[t] = b;
        }
    } else {
        for (int c = t; c < C; c += kT) {
            const float2 v = lds[c];
            const float ga = gamma ? gamma[c] : 1.f;
            ga_s1[c] = ga * v.x;
            ga_s2[c] = ga * v.y;
        }
    }
    __syncthreads();
    tree_groups(ga_s1, WHOLE ? tg.CPP : C, seg);
    tree_groups(ga_s2, WHOLE ? tg.CPP : C, seg);
    if (!tg.active) return;     // no barrier below
    const float invM = 1.0f / (float)(cfg.D * cfg.HW);
    float Ak[V], Bk[V], ga[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int g0 = ((tg.q * V + k) / D) * seg;
        Ak[k] = ga_s1[g0] * invM;
        Bk[k] = ga_s2[g0] * invM;
    }
    load_params<V>(gamma, tg.q * V, 1.f, ga);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < nv) {
#pragma clang fp contract(off)
            float xv[V], dv[V], o[V];
            Vec<T>::unpack(rx[j], xv);
            Vec<T>::unpack(rd[j], dv);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float xh = (xv[k] - mu[k]) * rs[k];
                const float gd = dv[k] * ga[k];
                o[k] = rs[k] * ((gd - Ak[k]) - xh * Bk[k]);
            }
            st16_nt(dx + off + (int64_t)(tg.pi + j * tg.PPI) * cfg.C, Vec<T>::pack(o));
        }
    }
}

// ---- a few tiles per sample ------------------------------------------------
// When a sample has at most kFewTiles statistics tiles, the output kernels
// combine the sample's tile partials themselves instead of a separate
// finalize (forward) or column-sum and per-group launches (backward): every
// workgroup of the sample reads the same partials (at most kFewTiles*G float4
// or kFewTiles*C float2, from L2) and combines them in tile order, so all of
// them derive the same statistics, and workgroup 0 of the sample writes the
// call's outputs (mean/rstd; dgamma/dbeta or the per-(n, c) sums).
constexpr int kFewTiles = 16;

// grid (otiles, N); part: [N*G][tiles] float4 from fwd_tile_stats
template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void fwd_apply_few(const T* __restrict__ x, const float* __restrict__ gamma,
                                                    const float* __restrict__ beta, T* __restrict__ y,
                                                    const float4* __restrict__ part, float* __restrict__ mean,
                                                    float* __restrict__ rstd, StreamCfg cfg) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int64_t tile = blockIdx.x, n = blockIdx.y;
    __shared__ float gmu[kMaxC], grs[kMaxC];
    for (int g = t; g < (int)cfg.G; g += kT) {   // the finalize of fwd_finalize, in tile order
        const float4* pg = part + (n * cfg.G + g) * cfg.tiles;
        float s0 = 0.f, s1 = 0.f;
        for (int64_t i = 0; i < cfg.tiles; ++i) {
            const float4 v = pg[i];
            s0 = fmaf(v.x, v.y, s0);
            s1 += v.x;
        }
        const float mu = s0 / s1;
        float m2 = 0.f;
        for (int64_t i = 0; i < cfg.tiles; ++i) {
            const float4 v = pg[i];
            const float d = v.y - mu;
            m2 += fmaf(v.x * d, d, v.z);
        }
        float var = m2 / (float)(cfg.D * cfg.HW);
        var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
        const float r = 1.0f / sqrtf(var + cfg.eps);
        gmu[g] = mu;
        grs[g] = r;
        if (tile == 0) {
            if (mean) mean[n * cfg.G + g] = mu;
            rstd[n * cfg.G + g] = r;
        }
    }
    __syncthreads();
    if (y == nullptr || !tg.active) return;   // no barrier below
    const int64_t off = n * cfg.HW * cfg.C + tg.q * V;
    u4v reg[R];
    const int64_t p0 = tile * tg.TP + tg.pi;
    load_tile<T, R>(x + off, cfg.HW, cfg.C, p0, tg.PPI, reg);
    float mu[V], a[V], b[V];
    load_params<V>(gamma, tg.q * V, 1.f, a);
    load_params<V>(beta, tg.q * V, 0.f, b);
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int g = (tg.q * V + k) / (int)cfg.D;
        mu[k] = gmu[g];
        a[k] *= grs[g];
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t p = p0 + (int64_t)j * tg.PPI;
        if (p < cfg.HW) {
            float v[V], o[V];
            Vec<T>::unpack(reg[j], v);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = fmaf(v[k] - mu[k], a[k], b[k]);
            st16_nt(y + off + p * cfg.C, Vec<T>::pack(o));
        }
    }
}

// grid (otiles, N) with dx, (1, N) without; part: [N][tiles][C] float2 from
// bwd_tile_sums.  Workgroup 0 of a sample writes dgamma/dbeta (one sample) or
// the sample's per-(n, c) sums into stot (several, for stream_params_over_n).
template <typename T, int R, bool WHOLE>
__global__ __launch_bounds__(kT) void bwd_dx_few(const T* __restrict__ dy, const T* __restrict__ x,
                                                 const float* __restrict__ mean, const float* __restrict__ rstd,
                                                 const float* __restrict__ gamma, const float2* __restrict__ part,
                                                 T* __restrict__ dx, float2* __restrict__ stot,
                                                 float* __restrict__ dgamma, float* __restrict__ dbeta,
                                                 StreamCfg cfg, int want_dx) {
    const TileGeom tg = tile_geom<T, R>(cfg.C);
    constexpr int V = Vec<T>::V;
    const int t = threadIdx.x;
    const int C = (int)cfg.C, D = (int)cfg.D;
    const int64_t tile = blockIdx.x, n = blockIdx.y;
    __shared__ float ga_s1[kMaxC], ga_s2[kMaxC];   // gamma_c * (sum dy, sum dy*xhat), then group totals
    const float2* pn = part + n * cfg.tiles * cfg.C;
    for (int c = t; c < C; c += kT) {   // the sample's channel sums, in tile order
        float2 v = make_float2(0.f, 0.f);
        for (int64_t i = 0; i < cfg.tiles; ++i) {
            const float2 q = pn[i * cfg.C + c];
            v.x += q.x;
            v.y += q.y;
        }
        if (tile == 0) {
            if (cfg.N == 1) {
                if (dbeta) dbeta[c] = v.x;
                if (dgamma) dgamma[c] = v.y;
            } else if (stot) {
                stot[n * cfg.C + c] = v;
            }
        }
        const float ga = gamma ? gamma[c] : 1.f;
        ga_s1[c] = ga * v.x;
        ga_s2[c] = ga * v.y;
    }
    if (!want_dx) return;   // kernel argument: uniform
    __syncthreads();
    const int seg = WHOLE ? D / V : D;
    if constexpr (WHOLE) {   // a chunk's V channels first (one group), then a tree over the group's chunks
        float a = 0.f, b = 0.f;
        if (t < tg.CPP) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                a += ga_s1[t * V + k];
                b += ga_s2[t * V + k];
            }
        }
        __syncthreads();   // every read of the per-channel values is done
        if (t < tg.CPP) {
            ga_s1[t] = a;
            ga_s2[t] = b;
        }
        __syncthreads();
    }
    tree_groups(ga_s1, WHOLE ? tg.CPP : C, seg);
    tree_groups(ga_s2, WHOLE ? tg.CPP : C, seg);
    if (!tg.active) return;   // no barrier below
    const int64_t off = n * cfg.HW * cfg.C + tg.q * V;
    const int64_t p0 = tile * tg.TP + tg.pi;
    const float invM = 1.0f / (float)(cfg.D * cfg.HW);
    float mu[V], rs[V], Ak[V], Bk[V], ga[V];
    int64_t sl[V];
    channel_slices<V, WHOLE>(tg.q, D, n, cfg.G, sl);
    per_channel<V, WHOLE>(mean, sl, mu);
    per_channel<V, WHOLE>(rstd, sl, rs);
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int g0 = ((tg.q * V + k) / D) * seg;
        Ak[k] = ga_s1[g0] * invM;
        Bk[k] = ga_s2[g0] * invM;
    }
    load_params<V>(gamma, tg.q * V, 1.f, ga);
    u4v rx[R], rd[R];
    load_tile<T, R>(x + off, cfg.HW, cfg.C, p0, tg.PPI, rx);
    load_tile<T, R>(dy + off, cfg.HW, cfg.C, p0, tg.PPI, rd);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t p = p0 + (int64_t)j * tg.PPI;
        if (p < cfg.HW) {
#pragma clang fp contract(off)
            float xv[V], dv[V], o[V];
            Vec<T>::unpack(rx[j], xv);
            Vec<T>::unpack(rd[j], dv);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float xh = (xv[k] - mu[k]) * rs[k];
                const float gd = dv[k] * ga[k];
                o[k] = rs[k] * ((gd - Ak[k]) - xh * Bk[k]);
            }
            st16_nt(dx + off + p * cfg.C, Vec<T>::pack(o));
        }
    }
}

// ---- planning ---------------------------------------------------------------
// (events, when given, bracket all kernels of a call)
size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

int64_t tiles_of(const Problem& p, int R) {
    const int CPP = (int)(p.C / vec_elems(p));
    const int64_t TP = (int64_t)(kT / CPP) * R;
    return (p.HW + TP - 1) / TP;
}

StreamCfg make_cfg(const Problem& p, int R, int RO, float eps) {
    StreamCfg c;
    c.N = p.N; c.C = p.C; c.HW = p.HW; c.G = p.G; c.D = p.D;
    c.tiles = tiles_of(p, R);
    c.otiles = tiles_of(p, RO);
    c.eps = eps;
    return c;
}

// Backward workspace: tile sums [N][tiles][C], chunk sums [N][chunks][C]
// (when there is more than one chunk), per-(n, c) totals [N][C] and (A/M,
// B/M) [N*G], all float2.
constexpr int64_t kRowsPerChunk = 64;

struct BwdPlan {
    int64_t tiles, chunks;
    size_t off_part, off_chunk, off_stot, off_ab, total;
};

BwdPlan bwd_plan(const Problem& p) {
    BwdPlan b{};
    b.tiles = tiles_of(p, GN_STREAM_R_SUMS);
    b.chunks = (b.tiles + kRowsPerChunk - 1) / kRowsPerChunk;
    size_t off = 0;
    b.off_part = off;
    off += al((size_t)p.N * b.tiles * p.C * sizeof(float2));
    b.off_chunk = off;
    if (b.chunks > 1) off += al((size_t)p.N * b.chunks * p.C * sizeof(float2));
    b.off_stot = off;
    off += al((size_t)p.N * p.C * sizeof(float2));
    b.off_ab = off;
    off += al((size_t)p.N * p.G * sizeof(float2));
    b.total = off;
    return b;
}

// Chunks per thread of the one-tile kernels for this call (4 or 16), or 0
// when a sample needs more than one tile of kOneTileR chunks per thread or
// the caller asked for the multi-kernel form.
int one_tile_r(const Problem& p, const Launch& l) {
    if (l.stream_split) return 0;
    const int64_t ppi = kT / (p.C / vec_elems(p));   // pixels per iteration of a tile
    if (p.HW > ppi * kOneTileR) return 0;
    return p.HW > ppi * 4 ? kOneTileR : 4;
}

template <typename T, bool WHOLE>
hipError_t fwd_one(const Problem& p, const FwdArgs& a, const Launch& l, int R) {
    const StreamCfg cfg = make_cfg(p, R, R, a.eps);
    auto k = R == 4 ? fwd_one_tile<T, 4, WHOLE> : fwd_one_tile<T, kOneTileR, WHOLE>;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)p.N), dim3(kT), 0, l.stream, (const T*)a.x, a.gamma, a.beta, (T*)a.y, a.mean,
                       a.rstd, cfg);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_STREAM;
        l.info->kernels = 1;
        l.info->grid = p.N;
        l.info->tiles = p.N;
    }
    return hipSuccess;
}

template <typename T, bool WHOLE>
hipError_t fwd_t(const Problem& p, const FwdArgs& a, const Launch& l) {
    if (const int r1 = one_tile_r(p, l)) return fwd_one<T, WHOLE>(p, a, l, r1);
    constexpr int R = GN_STREAM_R_STATS, RO = GN_STREAM_R_APPLY;
    const StreamCfg cfg = make_cfg(p, R, RO, a.eps);
    float4* part = (float4*)l.ws;
    const dim3 grid((unsigned)cfg.tiles, (unsigned)p.N), ogrid((unsigned)cfg.otiles, (unsigned)p.N);
    hipError_t e = record(l.ev_begin, l.stream);
    if (e) return e;
    hipLaunchKernelGGL((fwd_tile_stats<T, R, WHOLE>), grid, dim3(kT), 0, l.stream, (const T*)a.x, cfg, part);
    int kernels = 1;
    if (!l.stream_split && cfg.tiles <= kFewTiles) {   // the output kernel combines the partials itself
        const dim3 fgrid(a.y ? (unsigned)cfg.otiles : 1u, (unsigned)p.N);
        hipLaunchKernelGGL((fwd_apply_few<T, RO, WHOLE>), fgrid, dim3(kT), 0, l.stream, (const T*)a.x, a.gamma, a.beta,
                           (T*)a.y, (const float4*)part, a.mean, a.rstd, cfg);
        if ((e = hipGetLastError())) return e;
        ++kernels;
    } else {
        hipLaunchKernelGGL(fwd_finalize, dim3((unsigned)(p.N * p.G)), dim3(kFinT), 0, l.stream, part, cfg, a.mean,
                           a.rstd);
        if ((e = hipGetLastError())) return e;
        ++kernels;
        if (a.y) {
            hipLaunchKernelGGL((fwd_apply<T, RO, WHOLE>), ogrid, dim3(kT), 0, l.stream, (const T*)a.x, a.gamma, a.beta,
                               (T*)a.y, a.mean, a.rstd, cfg);
            if ((e = hipGetLastError())) return e;
            ++kernels;
        }
    }
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_STREAM;
        l.info->kernels = kernels;
        l.info->grid = cfg.tiles * p.N;
        l.info->tiles = cfg.tiles * p.N;
    }
    return hipSuccess;
}

template <typename T, bool WHOLE>
hipError_t bwd_one(const Problem& p, const BwdArgs& a, const Launch& l, int R) {
    const StreamCfg cfg = make_cfg(p, R, R, 0.f);
    float2* stot = (float2*)((char*)l.ws + bwd_plan(p).off_stot);
    float* dg = (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr;
    float* db = (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr;
    auto k = R == 4 ? bwd_one_tile<T, 4, WHOLE> : bwd_one_tile<T, kOneTileR, WHOLE>;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)p.N), dim3(kT), 0, l.stream, (const T*)a.dy, (const T*)a.x, a.mean, a.rstd,
                       a.gamma, (T*)a.dx, (p.N > 1 && (dg || db)) ? stot : nullptr, dg, db, cfg,
                       (a.mask & GN_GRAD_DX) ? 1 : 0);
    int kernels = 1;
    if (p.N > 1 && (dg || db)) {
        hipLaunchKernelGGL(stream_params_over_n, dim3((unsigned)((p.C + kT - 1) / kT)), dim3(kT), 0, l.stream,
                           (const float2*)stot, p.N, p.C, dg, db);
        ++kernels;
    }
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_STREAM;
        l.info->kernels = kernels;
        l.info->grid = p.N;
        l.info->tiles = p.N;
    }
    return hipSuccess;
}

template <typename T, bool WHOLE>
hipError_t bwd_t(const Problem& p, const BwdArgs& a, const Launch& l) {
    if (const int r1 = one_tile_r(p, l)) return bwd_one<T, WHOLE>(p, a, l, r1);
    constexpr int R = GN_STREAM_R_SUMS, RO = GN_STREAM_R_DX;
    const StreamCfg cfg = make_cfg(p, R, RO, 0.f);
    const BwdPlan b = bwd_plan(p);
    char* ws = (char*)l.ws;
    float2* part = (float2*)(ws + b.off_part);
    float2* chunk = (float2*)(ws + b.off_chunk);
    float2* stot = (float2*)(ws + b.off_stot);
    float2* ab = (float2*)(ws + b.off_ab);
    float* dg = (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr;
    float* db = (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr;
    const bool want_dx = (a.mask & GN_GRAD_DX) != 0;
    const dim3 grid((unsigned)cfg.tiles, (unsigned)p.N), ogrid((unsigned)cfg.otiles, (unsigned)p.N);
    const unsigned cblocks = (unsigned)((p.C + 2 * kColPairs - 1) / (2 * kColPairs));
    int kernels = 0;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL((bwd_tile_sums<T, R, WHOLE>), grid, dim3(kT), 0, l.stream, (const T*)a.dy, (const T*)a.x, a.mean,
                       a.rstd, cfg, part);
    ++kernels;
    if (!l.stream_split && b.tiles <= kFewTiles) {   // the dx kernel combines the tile sums itself
        const bool params = p.N > 1 && (dg || db);
        const dim3 fgrid(want_dx ? (unsigned)cfg.otiles : 1u, (unsigned)p.N);
        hipLaunchKernelGGL((bwd_dx_few<T, RO, WHOLE>), fgrid, dim3(kT), 0, l.stream, (const T*)a.dy, (const T*)a.x,
                           a.mean, a.rstd, a.gamma, (const float2*)part, (T*)a.dx, params ? stot : nullptr, dg, db, cfg,
                           want_dx ? 1 : 0);
        ++kernels;
        if (params) {
            hipLaunchKernelGGL(stream_params_over_n, dim3((unsigned)((p.C + kT - 1) / kT)), dim3(kT), 0, l.stream,
                               (const float2*)stot, p.N, p.C, dg, db);
            ++kernels;
        }
        if ((e = hipGetLastError())) return e;
        if ((e = record(l.ev_end, l.stream))) return e;
        if (l.info) {
            l.info->path = GN_PATH_STREAM;
            l.info->kernels = kernels;
            l.info->grid = cfg.tiles * p.N;
            l.info->tiles = cfg.tiles * p.N;
        }
        return hipSuccess;
    }
    if (b.chunks > 1) {
        hipLaunchKernelGGL(col_sums, dim3(cblocks, (unsigned)b.chunks, (unsigned)p.N), dim3(kT), 0, l.stream,
                           (const float2*)part, b.tiles, p.C, kRowsPerChunk, chunk);
        hipLaunchKernelGGL(col_sums, dim3(cblocks, 1, (unsigned)p.N), dim3(kT), 0, l.stream, (const float2*)chunk,
                           b.chunks, p.C, b.chunks, stot);
        kernels += 2;
    } else {
        hipLaunchKernelGGL(col_sums, dim3(cblocks, 1, (unsigned)p.N), dim3(kT), 0, l.stream, (const float2*)part,
                           b.tiles, p.C, b.tiles, stot);
        ++kernels;
    }
    if ((e = hipGetLastError())) return e;
    if (want_dx || p.N == 1) {
        hipLaunchKernelGGL(bwd_group_ab, dim3((unsigned)p.G, (unsigned)p.N), dim3(kT), 0, l.stream,
                           (const float2*)stot, a.gamma, cfg, ab, dg, db);
        ++kernels;
    }
    if (p.N > 1 && (dg || db)) {
        hipLaunchKernelGGL(stream_params_over_n, dim3((unsigned)((p.C + kT - 1) / kT)), dim3(kT), 0, l.stream,
                           (const float2*)stot, p.N, p.C, dg, db);
        ++kernels;
    }
    if ((e = hipGetLastError())) return e;
    if (want_dx) {
        hipLaunchKernelGGL((bwd_dx<T, RO, WHOLE>), ogrid, dim3(kT), 0, l.stream, (const T*)a.dy, (const T*)a.x, a.mean,
                           a.rstd, a.gamma, (const float2*)ab, (T*)a.dx, cfg);
        ++kernels;
        if ((e = hipGetLastError())) return e;
    }
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_STREAM;
        l.info->kernels = kernels;
        l.info->grid = cfg.tiles * p.N;
        l.info->tiles = cfg.tiles * p.N;
    }
    return hipSuccess;
}

}  // namespace

// NHWC whose pixels are whole 16-byte chunks (C a multiple of 4 fp32 / 8
// 16-bit channels) with at most kT chunks per pixel; any channels per group.
bool stream_ok(const Problem& p) {
    if (p.layout != GN_NHWC || p.HW < 1) return false;
    const int V = vec_elems(p);
    if (p.C % V != 0) return false;
    const int64_t cpp = p.C / V;
    if (cpp < 1 || cpp > kT) return false;
    // grid limits: samples and column-sum chunks on grid y (at most 65535)
    if (p.N > 65535) return false;
    const int64_t chunks = (tiles_of(p, GN_STREAM_R_SUMS) + kRowsPerChunk - 1) / kRowsPerChunk;
    return chunks <= 65535 && tiles_of(p, 1) <= INT32_MAX;   // grid x: tiles of the smallest size
}

size_t stream_fwd_ws(const Problem& p) {
    return al((size_t)p.N * p.G * tiles_of(p, GN_STREAM_R_STATS) * sizeof(float4));
}

size_t stream_bwd_ws(const Problem& p, int32_t) { return bwd_plan(p).total; }

// groups made of whole 16-byte chunks (the common case) or not
hipError_t stream_fwd(const Problem& p, const FwdArgs& a, const Launch& l) {
    const bool whole = p.D % vec_elems(p) == 0;
    switch (p.dtype) {
        case GN_F32: return whole ? fwd_t<float, true>(p, a, l) : fwd_t<float, false>(p, a, l);
        case GN_F16: return whole ? fwd_t<_Float16, true>(p, a, l) : fwd_t<_Float16, false>(p, a, l);
        default: return whole ? fwd_t<__bf16, true>(p, a, l) : fwd_t<__bf16, false>(p, a, l);
    }
}

hipError_t stream_bwd(const Problem& p, const BwdArgs& a, const Launch& l) {
    const bool whole = p.D % vec_elems(p) == 0;
    switch (p.dtype) {
        case GN_F32: return whole ? bwd_t<float, true>(p, a, l) : bwd_t<float, false>(p, a, l);
        case GN_F16: return whole ? bwd_t<_Float16, true>(p, a, l) : bwd_t<_Float16, false>(p, a, l);
        default: return whole ? bwd_t<__bf16, true>(p, a, l) : bwd_t<__bf16, false>(p, a, l);
    }
}

}  // namespace gn
