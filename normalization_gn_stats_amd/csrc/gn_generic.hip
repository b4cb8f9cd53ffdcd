// gn_generic.hip -- GroupNorm forward/backward for any shape, any element
// strides and any alignment (one element per lane).  It serves the dense
// layouts when a faster path cannot (odd shapes, unaligned pointers), and
// non-contiguous tensors -- slices, crops, permuted or broadcast views --
// without a copy.
//
// Forward (POPCORNBENCH GroupNorm trace: per (sample, group) mean and biased
// variance over (C/G)*H*W elements, then normalize and apply the per-channel
// weight and bias):
//   F1  per slice, per tile of the slice: (count, mean, M2) of the tile
//   F2  per slice: merge the tile statistics in tile order -> mean, rstd
//   F3  elementwise y = (x - mean)*(rstd*gamma_c) + beta_c
// Backward (the three stages of the baracuda-kernels GroupNorm backward plan:
// per-group reduction, per-cell dx, per-channel dgamma/dbeta):
//   B1  per slice, per tile: A = sum gamma_c*dy, B = sum gamma_c*dy*xhat
//   B2  per slice: sum the tile partials in tile order
//   B3  elementwise dx = rstd*(gamma_c*dy - A/M - xhat*B/M)
//   B4  per channel, per tile of the (n, h, w) range: sum dy, sum dy*xhat
//   B5  per channel: sum the tile partials in tile order -> dbeta, dgamma
// With large spatial planes (H*W >= kPlaneMinHW) stored in unit-stride runs
// of at least a wave in dy and x (NCHW-like: a plane is read coalesced), B1
// and B4 become one pass:
// A, B, dbeta and dgamma are all sums of the per-(n, c) plane sums
// S1 = sum dy and S2 = sum dy*xhat (A = sum over the group's channels of
// gamma_c*S1, dbeta_c = sum over n of S1, and likewise with S2), so
//   P1  per (n, c) plane, per tile: S1, S2
//   P2  per slice: A, B from the plane partials of its channels
//   P3  per channel: dbeta, dgamma from the plane partials of all samples
// read dy and x once instead of twice.
// Every sum has a fixed order, so results are bitwise reproducible.
//
// Addressing.  Each pass walks a box of "digits" -- the logical dimensions
// it iterates, each with an extent, an element stride per tensor, and its
// weight in the channel index c and in the slice index s = n*G + g (the
// channel dimension is split into the group g and the channel within the
// group, so that c = g*D + cl and s stay linear in the digits).  On the host
// the digits are sorted by the first tensor's strides and neighbours that
// are contiguous in every tensor are merged, so that digit 0 is the longest
// run of the smallest stride.  The box is then a matrix: rows (every digit
// but the first, decomposed once per row) by columns (digit 0, walked with a
// constant pointer step).  Tiles of that matrix are the unit of work: a
// tile spans a range of rows and a range of columns; when rows are shorter
// than a workgroup, one workgroup covers several rows at a time.
#include <algorithm>
#include <type_traits>

#include "gn_device.hpp"
#include "gn_internal.hpp"

namespace gn {
namespace {

constexpr int kT = 256;
constexpr int kNW = kT / kWave;
constexpr int kMaxD = 5;                 // digits: w, h, channel-in-group, group, sample
constexpr int kMaxTensors = 3;           // dy, x, dx
constexpr int64_t kRedTile = 16384;      // elements per workgroup in the reductions
constexpr int kMaxParts = 4096;          // partial results per slice / per channel
#ifndef GN_GEN_ELEM_TILE
#define GN_GEN_ELEM_TILE 8192
#endif
#ifndef GN_GEN_RED_U
#define GN_GEN_RED_U 8
#endif
#ifndef GN_GEN_ELEM_U
#define GN_GEN_ELEM_U 8
#endif
constexpr int64_t kElemTile = GN_GEN_ELEM_TILE;   // elements per tile in the elementwise passes
constexpr int kRedU = GN_GEN_RED_U;               // loads in flight per lane and tensor: reductions
constexpr int kElemU = GN_GEN_ELEM_U;             //   elementwise passes
constexpr int64_t kPlaneMinHW = 512;     // backward by plane sums from this plane size on

struct Box {
    int64_t ext[kMaxD];                  // extents, digit 0 innermost (unused digits: 1)
    int64_t st[kMaxTensors][kMaxD];      // element strides of each tensor
    int64_t cw[kMaxD];                   // weight in the channel index
    int64_t sw[kMaxD];                   // weight in the slice index
    int32_t nd;                          // digits in use (>= 1)
};

struct Tiling {
    int64_t e0, rows;                    // columns (digit 0) and rows (the other digits)
    int64_t ccols, cb;                   // columns per tile, column tiles per row
    int64_t rpt, rb;                     // rows per tile, row tiles
    int64_t tiles;                       // rb*cb
    int32_t cpr;                         // lanes per row (a power of two >= 64, or ccols < 64)
    int32_t rstep;                       // rows a workgroup covers at once, kT/cpr
};

struct DigitSpec {
    int64_t ext;
    int64_t st[kMaxTensors];
    int64_t cw, sw;
};

// Sorts the digits by the first tensor's stride (stable: ties keep the given
// order, which lists inner dimensions first), drops extent-1 digits and
// merges neighbours that are contiguous in every tensor and in both weights.
Box make_box(const DigitSpec* in, int count, int ntensors) {
    DigitSpec d[kMaxD];
    int n = 0;
    for (int k = 0; k < count; ++k)
        if (in[k].ext != 1) d[n++] = in[k];
    std::stable_sort(d, d + n, [](const DigitSpec& a, const DigitSpec& b) { return a.st[0] < b.st[0]; });
    int m = 0;
    for (int k = 0; k < n; ++k) {
        if (m > 0) {
            DigitSpec& a = d[m - 1];
            const DigitSpec& b = d[k];
            const __int128 e = a.ext;
            bool ok = (__int128)b.cw == e * a.cw && (__int128)b.sw == e * a.sw;
            for (int t = 0; t < ntensors && ok; ++t) ok = (__int128)b.st[t] == e * a.st[t];
            if (ok) {
                a.ext *= b.ext;
                continue;
            }
        }
        d[m++] = d[k];
    }
    Box box{};
    for (int k = 0; k < kMaxD; ++k) {
        box.ext[k] = 1;
        if (k < m) {
            box.ext[k] = d[k].ext;
            for (int t = 0; t < kMaxTensors; ++t) box.st[t][k] = t < ntensors ? d[k].st[t] : 0;
            box.cw[k] = d[k].cw;
            box.sw[k] = d[k].sw;
        }
    }
    box.nd = m > 0 ? m : 1;
    return box;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles of about `target` elements; at most `max_tiles` of them when
// max_tiles > 0 (the partial-result slots of a reduction).  Lanes per row:
// whole waves, as few as still give each lane `unroll` columns of a row (so
// that it keeps that many loads in flight), the rest of the workgroup taking
// further rows; rows narrower than a wave are packed several to a wave.
Tiling make_tiling(const Box& b, int64_t target, int64_t max_tiles, int unroll) {
    Tiling t{};
    t.e0 = b.ext[0];
    t.rows = 1;
    for (int k = 1; k < kMaxD; ++k) t.rows *= b.ext[k];
    if (t.e0 >= target) {
        t.ccols = target;
        t.rpt = 1;
    } else {
        t.ccols = t.e0;
        t.rpt = std::max<int64_t>(1, target / t.e0);
    }
    t.cb = cdiv(t.e0, t.ccols);
    if (max_tiles > 0 && t.cb > max_tiles) {
        t.ccols = cdiv(cdiv(t.e0, max_tiles), kT) * kT;
        t.cb = cdiv(t.e0, t.ccols);
    }
    t.rb = cdiv(t.rows, t.rpt);
    if (max_tiles > 0) {
        const int64_t rb_max = std::max<int64_t>(1, max_tiles / t.cb);
        if (t.rb > rb_max) {
            t.rpt = cdiv(t.rows, rb_max);
            t.rb = cdiv(t.rows, t.rpt);
        }
    }
    t.tiles = t.rb * t.cb;
    if (t.ccols < kWave) {
        t.cpr = (int32_t)t.ccols;
    } else {
        t.cpr = kWave;
        while (t.cpr * 2 <= kT && (int64_t)t.cpr * 2 * unroll <= t.ccols) t.cpr *= 2;
    }
    t.rstep = kT / t.cpr;
    return t;
}

__device__ inline int64_t udiv(int64_t a, int64_t b) {
    if ((((uint64_t)a | (uint64_t)b) >> 32) == 0) return (int64_t)((uint32_t)a / (uint32_t)b);
    return (int64_t)((uint64_t)a / (uint64_t)b);
}

// Adds the offsets (per tensor), channel and slice contributions of row r.
template <int NT>
__device__ inline void add_row(const Box& b, int64_t r, int64_t (&off)[NT], int64_t& c, int64_t& s) {
#pragma unroll
    for (int k = 1; k < kMaxD; ++k) {
        if (k < b.nd) {
            int64_t i = r;
            if (k + 1 < b.nd) {
                const int64_t q = udiv(r, b.ext[k]);
                i = r - q * b.ext[k];
                r = q;
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) off[t] += i * b.st[t][k];
            c += i * b.cw[k];
            s += i * b.sw[k];
        }
    }
}

// The rows and columns of tile `t` that this lane covers.
struct TileSpan {
    int64_t r0, r1, c0, c1;
};

__device__ inline TileSpan tile_span(const Tiling& tl, int64_t t) {
    const int64_t rt = udiv(t, tl.cb), ct = t - rt * tl.cb;
    TileSpan sp;
    sp.r0 = rt * tl.rpt;
    sp.r1 = min(sp.r0 + tl.rpt, tl.rows);
    sp.c0 = ct * tl.ccols;
    sp.c1 = min(sp.c0 + tl.ccols, tl.e0);
    return sp;
}

// Element loads and stores.  Every pass streams its tensors once, so by default
// they bypass the caches' retention (non-temporal), as the vector paths do.
#ifndef GN_GEN_NT
#define GN_GEN_NT 1
#endif
template <typename T>
using Bits = typename std::conditional<sizeof(T) == 4, uint32_t, uint16_t>::type;

template <typename T>
__device__ inline float ldf(const T* p, int64_t o) {
#if GN_GEN_NT
    const Bits<T> u = __builtin_nontemporal_load(reinterpret_cast<const Bits<T>*>(p + o));
    return Vec<T>::to_f(__builtin_bit_cast(T, u));
#else
    return Vec<T>::to_f(p[o]);
#endif
}

template <typename T>
__device__ inline void stf(T* p, float v) {
#if GN_GEN_NT
    __builtin_nontemporal_store(__builtin_bit_cast(Bits<T>, Vec<T>::from_f(v)), reinterpret_cast<Bits<T>*>(p));
#else
    *p = Vec<T>::from_f(v);
#endif
}

// ---- F1 --------------------------------------------------------------------
// box digits: w, h, channel in group (x only, no weights)
template <typename T, int U = kRedU>
__global__ __launch_bounds__(kT) void gen_stats_partial(const T* __restrict__ x, Box b, Tiling tl, int64_t G,
                                                        int64_t sn, int64_t sg, float4* __restrict__ part,
                                                        int P) {
    const int64_t s = blockIdx.x;
    const int64_t n = s / G, g = s - n * G;
    const int rsub = threadIdx.x / tl.cpr, lc = threadIdx.x - rsub * tl.cpr;
    const TileSpan sp = tile_span(tl, blockIdx.y);
    const int64_t step = (int64_t)tl.cpr * b.st[0][0];
    Stat st = stat_empty();
    if (rsub < tl.rstep) {
        for (int64_t r = sp.r0 + rsub; r < sp.r1; r += tl.rstep) {
            int64_t off[1] = {n * sn + g * sg};
            int64_t c = 0, sl = 0;
            add_row<1>(b, r, off, c, sl);
            int64_t col = sp.c0 + lc;
            const T* px = x + off[0] + col * b.st[0][0];
            for (; col < sp.c1; col += U * tl.cpr) {
                float v[U];
                int valid = 0;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool in = col + (int64_t)u * tl.cpr < sp.c1;
                    v[u] = in ? ldf(px, u * step) : 0.f;
                    valid += in ? 1 : 0;
                }
                px += U * step;
                st = stat_merge(st, stat_of<U>(v, valid));
            }
        }
    }
    st = wave_merge_strided(st, 1);
    __shared__ Stat lds[kNW];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) lds[wave] = st;
    __syncthreads();
    if (threadIdx.x == 0) {
        Stat r = lds[0];
        for (int w = 1; w < kNW; ++w) r = stat_merge(r, lds[w]);
        part[s * P + blockIdx.y] = make_float4(r.n, r.mean, r.m2, 0.f);
    }
}

// ---- F2 --------------------------------------------------------------------
__global__ __launch_bounds__(kWave) void gen_stats_final(const float4* __restrict__ part, int P, int64_t M,
                                                         float eps, float* __restrict__ mean,
                                                         float* __restrict__ rstd) {
    const int64_t s = blockIdx.x;
    const int lane = threadIdx.x;
    Stat st = stat_empty();
    for (int k = lane; k < P; k += kWave) {
        const float4 q = part[s * P + k];
        st = stat_merge(st, Stat{q.x, q.y, q.z});
    }
    st = wave_merge_strided(st, 1);
    if (lane == 0) {
        float var = st.m2 / (float)M;
        var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
        mean[s] = st.mean;
        rstd[s] = 1.0f / sqrtf(var + eps);
    }
}

// ---- F3 --------------------------------------------------------------------
// box digits: w, h, channel in group, group, sample (tensors x, y).  ROWCONST:
// digit 0 is spatial, so the channel and slice are constant along a row.
template <typename T, bool ROWCONST, int U = kElemU>
__global__ __launch_bounds__(kT) void gen_apply(const T* __restrict__ x, T* __restrict__ y,
                                                const float* __restrict__ gamma, const float* __restrict__ beta,
                                                const float* __restrict__ mean, const float* __restrict__ rstd,
                                                Box b, Tiling tl) {
    const int rsub = threadIdx.x / tl.cpr, lc = threadIdx.x - rsub * tl.cpr;
    if (rsub >= tl.rstep) return;   // no workgroup barrier below
    const int64_t sx = b.st[0][0], sy = b.st[1][0];
    for (int64_t t = blockIdx.x; t < tl.tiles; t += gridDim.x) {
        const TileSpan sp = tile_span(tl, t);
        for (int64_t r = sp.r0 + rsub; r < sp.r1; r += tl.rstep) {
            int64_t off[2] = {0, 0};
            int64_t c = 0, s = 0;
            add_row<2>(b, r, off, c, s);
            int64_t col = sp.c0 + lc;
            const T* px = x + off[0] + col * sx;
            T* py = y + off[1] + col * sy;
            if (ROWCONST) {
                const float a = rstd[s] * (gamma ? gamma[c] : 1.f);
                const float bb = beta ? beta[c] : 0.f;
                const float mu = mean[s];
                for (; col < sp.c1; col += U * tl.cpr) {
                    float v[U];
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[u] = col + (int64_t)u * tl.cpr < sp.c1 ? ldf(px, u * tl.cpr * sx) : 0.f;
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (col + (int64_t)u * tl.cpr < sp.c1)
                            stf(py + u * tl.cpr * sy, fmaf(v[u] - mu, a, bb));
                    px += U * tl.cpr * sx;
                    py += U * tl.cpr * sy;
                }
            } else {
                for (; col < sp.c1; col += tl.cpr) {
                    const int64_t ce = c + col * b.cw[0], se = s + col * b.sw[0];
                    const float a = rstd[se] * (gamma ? gamma[ce] : 1.f);
                    const float bb = beta ? beta[ce] : 0.f;
                    stf(py, fmaf(ldf(px, 0) - mean[se], a, bb));
                    px += tl.cpr * sx;
                    py += tl.cpr * sy;
                }
            }
        }
    }
}

// ---- B1 --------------------------------------------------------------------
// box digits: w, h, channel in group (tensors dy, x; channel weight)
template <typename T, bool ROWCONST, int U = kRedU>
__global__ __launch_bounds__(kT) void gen_ab_partial(const T* __restrict__ dy, const T* __restrict__ x,
                                                     const float* __restrict__ mean,
                                                     const float* __restrict__ rstd,
                                                     const float* __restrict__ gamma, Box b, Tiling tl, int64_t G,
                                                     int64_t D, int64_t dsn, int64_t dsg, int64_t xsn,
                                                     int64_t xsg, float2* __restrict__ part, int P) {
    const int64_t s = blockIdx.x;
    const int64_t n = s / G, g = s - n * G;
    const float mu = mean[s], rs = rstd[s];
    const int rsub = threadIdx.x / tl.cpr, lc = threadIdx.x - rsub * tl.cpr;
    const TileSpan sp = tile_span(tl, blockIdx.y);
    const int64_t sd = b.st[0][0], sx = b.st[1][0];
    float acc[2] = {0.f, 0.f};
    if (rsub < tl.rstep) {
        for (int64_t r = sp.r0 + rsub; r < sp.r1; r += tl.rstep) {
            int64_t off[2] = {n * dsn + g * dsg, n * xsn + g * xsg};
            int64_t c = g * D, sl = 0;
            add_row<2>(b, r, off, c, sl);
            int64_t col = sp.c0 + lc;
            const T* pd = dy + off[0] + col * sd;
            const T* px = x + off[1] + col * sx;
            if (ROWCONST) {
                const float gm = gamma ? gamma[c] : 1.f;
                for (; col < sp.c1; col += U * tl.cpr) {
                    float vd[U], vx[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool in = col + (int64_t)u * tl.cpr < sp.c1;
                        vd[u] = in ? ldf(pd, u * tl.cpr * sd) : 0.f;
                        vx[u] = in ? ldf(px, u * tl.cpr * sx) : mu;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const float gd = vd[u] * gm;
                        acc[0] += gd;
                        acc[1] = fmaf(gd, (vx[u] - mu) * rs, acc[1]);
                    }
                    pd += U * tl.cpr * sd;
                    px += U * tl.cpr * sx;
                }
            } else {
                for (; col < sp.c1; col += tl.cpr) {
                    const float gd = ldf(pd, 0) * (gamma ? gamma[c + col * b.cw[0]] : 1.f);
                    acc[0] += gd;
                    acc[1] = fmaf(gd, (ldf(px, 0) - mu) * rs, acc[1]);
                    pd += tl.cpr * sd;
                    px += tl.cpr * sx;
                }
            }
        }
    }
    __shared__ float lds[kNW * 2];
    block_sum<2, kNW>(acc, lds);
    if (threadIdx.x == 0) part[s * P + blockIdx.y] = make_float2(acc[0], acc[1]);
}

// ---- B2 / B5: fixed-order sum of P float2 partials per row ------------------
__global__ __launch_bounds__(kWave) void gen_sum_rows(const float2* __restrict__ part, int P,
                                                      float2* __restrict__ out_pair,
                                                      float* __restrict__ out0, float* __restrict__ out1) {
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    float a = 0.f, b = 0.f;
    for (int k = lane; k < P; k += kWave) {
        const float2 q = part[row * P + k];
        a += q.x;
        b += q.y;
    }
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
        if (out_pair) out_pair[row] = make_float2(a, b);
        if (out0) out0[row] = a;
        if (out1) out1[row] = b;
    }
}

// ---- B3 --------------------------------------------------------------------
// box digits: w, h, channel in group, group, sample (tensors dy, x, dx)
template <typename T, bool ROWCONST, int U = kElemU>
__global__ __launch_bounds__(kT) void gen_dx(const T* __restrict__ dy, const T* __restrict__ x,
                                             const float* __restrict__ mean, const float* __restrict__ rstd,
                                             const float* __restrict__ gamma, const float2* __restrict__ ab,
                                             T* __restrict__ dx, Box b, Tiling tl, int64_t M) {
    // gamma*dy is rounded exactly as in the partial sums, so that it cancels A/M
    // exactly where the slice makes dx vanish (one element per slice)
#pragma clang fp contract(off)
    const int rsub = threadIdx.x / tl.cpr, lc = threadIdx.x - rsub * tl.cpr;
    if (rsub >= tl.rstep) return;   // no workgroup barrier below
    const float invM = 1.0f / (float)M;
    const int64_t sd = b.st[0][0], sx = b.st[1][0], so = b.st[2][0];
    for (int64_t t = blockIdx.x; t < tl.tiles; t += gridDim.x) {
        const TileSpan sp = tile_span(tl, t);
        for (int64_t r = sp.r0 + rsub; r < sp.r1; r += tl.rstep) {
            int64_t off[3] = {0, 0, 0};
            int64_t c = 0, s = 0;
            add_row<3>(b, r, off, c, s);
            int64_t col = sp.c0 + lc;
            const T* pd = dy + off[0] + col * sd;
            const T* px = x + off[1] + col * sx;
            T* po = dx + off[2] + col * so;
            if (ROWCONST) {
                const float rs = rstd[s], mu = mean[s];
                const float gm = gamma ? gamma[c] : 1.f;
                const float2 q = ab[s];
                const float am = q.x * invM, bm = q.y * invM;
                for (; col < sp.c1; col += U * tl.cpr) {
                    float vd[U], vx[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool in = col + (int64_t)u * tl.cpr < sp.c1;
                        vd[u] = in ? ldf(pd, u * tl.cpr * sd) : 0.f;
                        vx[u] = in ? ldf(px, u * tl.cpr * sx) : 0.f;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        if (col + (int64_t)u * tl.cpr < sp.c1) {
                            const float xh = (vx[u] - mu) * rs;
                            const float gd = vd[u] * gm;
                            stf(po + u * tl.cpr * so, rs * (gd - am - xh * bm));
                        }
                    }
                    pd += U * tl.cpr * sd;
                    px += U * tl.cpr * sx;
                    po += U * tl.cpr * so;
                }
            } else {
                for (; col < sp.c1; col += tl.cpr) {
                    const int64_t ce = c + col * b.cw[0], se = s + col * b.sw[0];
                    const float rs = rstd[se];
                    const float xh = (ldf(px, 0) - mean[se]) * rs;
                    const float gd = ldf(pd, 0) * (gamma ? gamma[ce] : 1.f);
                    const float2 q = ab[se];
                    stf(po, rs * (gd - q.x * invM - xh * (q.y * invM)));
                    pd += tl.cpr * sd;
                    px += tl.cpr * sx;
                    po += tl.cpr * so;
                }
            }
        }
    }
}

// ---- B4 --------------------------------------------------------------------
// box digits: w, h, sample (tensors dy, x; slice weight G on the sample)
template <typename T, bool ROWCONST, int U = kRedU>
__global__ __launch_bounds__(kT) void gen_param_partial(const T* __restrict__ dy, const T* __restrict__ x,
                                                        const float* __restrict__ mean,
                                                        const float* __restrict__ rstd, Box b, Tiling tl,
                                                        int64_t D, int64_t dsc, int64_t xsc,
                                                        float2* __restrict__ part, int Q) {
    const int64_t c = blockIdx.x;
    const int rsub = threadIdx.x / tl.cpr, lc = threadIdx.x - rsub * tl.cpr;
    const TileSpan sp = tile_span(tl, blockIdx.y);
    const int64_t sd = b.st[0][0], sx = b.st[1][0];
    float acc[2] = {0.f, 0.f};
    if (rsub < tl.rstep) {
        for (int64_t r = sp.r0 + rsub; r < sp.r1; r += tl.rstep) {
            int64_t off[2] = {c * dsc, c * xsc};
            int64_t cc = 0, s = c / D;
            add_row<2>(b, r, off, cc, s);
            int64_t col = sp.c0 + lc;
            const T* pd = dy + off[0] + col * sd;
            const T* px = x + off[1] + col * sx;
            if (ROWCONST) {
                const float mu = mean[s], rs = rstd[s];
                for (; col < sp.c1; col += U * tl.cpr) {
                    float vd[U], vx[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool in = col + (int64_t)u * tl.cpr < sp.c1;
                        vd[u] = in ? ldf(pd, u * tl.cpr * sd) : 0.f;
                        vx[u] = in ? ldf(px, u * tl.cpr * sx) : mu;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        acc[0] += vd[u];
                        acc[1] += vd[u] * ((vx[u] - mu) * rs);
                    }
                    pd += U * tl.cpr * sd;
                    px += U * tl.cpr * sx;
                }
            } else {
                for (; col < sp.c1; col += tl.cpr) {
                    const int64_t se = s + col * b.sw[0];
                    const float d = ldf(pd, 0);
                    acc[0] += d;
                    acc[1] += d * ((ldf(px, 0) - mean[se]) * rstd[se]);
                    pd += tl.cpr * sd;
                    px += tl.cpr * sx;
                }
            }
        }
    }
    __shared__ float lds[kNW * 2];
    block_sum<2, kNW>(acc, lds);
    if (threadIdx.x == 0) part[c * Q + blockIdx.y] = make_float2(acc[0], acc[1]);
}

// ---- P1 --------------------------------------------------------------------
// box digits: w, h (tensors dy, x); one (n, c) plane per blockIdx.x
template <typename T, int U = kRedU>
__global__ __launch_bounds__(kT) void gen_plane_partial(const T* __restrict__ dy, const T* __restrict__ x,
                                                        const float* __restrict__ mean,
                                                        const float* __restrict__ rstd, Box b, Tiling tl,
                                                        int64_t C, int64_t D, int64_t G, int64_t dsn, int64_t dsc,
                                                        int64_t xsn, int64_t xsc, float2* __restrict__ part,
                                                        int P) {
    const int64_t pl = blockIdx.x;
    const int64_t n = pl / C, c = pl - n * C;
    const int64_t s = n * G + c / D;
    const float mu = mean[s], rs = rstd[s];
    const int rsub = threadIdx.x / tl.cpr, lc = threadIdx.x - rsub * tl.cpr;
    const TileSpan sp = tile_span(tl, blockIdx.y);
    const int64_t sd = b.st[0][0], sx = b.st[1][0];
    float acc[2] = {0.f, 0.f};
    if (rsub < tl.rstep) {
        for (int64_t r = sp.r0 + rsub; r < sp.r1; r += tl.rstep) {
            int64_t off[2] = {n * dsn + c * dsc, n * xsn + c * xsc};
            int64_t cc = 0, ss = 0;
            add_row<2>(b, r, off, cc, ss);
            int64_t col = sp.c0 + lc;
            const T* pd = dy + off[0] + col * sd;
            const T* px = x + off[1] + col * sx;
            for (; col < sp.c1; col += U * tl.cpr) {
                float vd[U], vx[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool in = col + (int64_t)u * tl.cpr < sp.c1;
                    vd[u] = in ? ldf(pd, u * tl.cpr * sd) : 0.f;
                    vx[u] = in ? ldf(px, u * tl.cpr * sx) : mu;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    acc[0] += vd[u];
                    acc[1] += vd[u] * ((vx[u] - mu) * rs);
                }
                pd += U * tl.cpr * sd;
                px += U * tl.cpr * sx;
            }
        }
    }
    __shared__ float lds[kNW * 2];
    block_sum<2, kNW>(acc, lds);
    if (threadIdx.x == 0) part[pl * P + blockIdx.y] = make_float2(acc[0], acc[1]);
}

// ---- P2 --------------------------------------------------------------------
// one wave per slice (n, g): A = sum over its channels and tiles of gamma_c*S1
__global__ __launch_bounds__(kWave) void gen_plane_ab(const float2* __restrict__ part, int P,
                                                      const float* __restrict__ gamma, int64_t C, int64_t D,
                                                      int64_t G, float2* __restrict__ ab) {
    const int64_t s = blockIdx.x;
    const int64_t n = s / G, g = s - n * G;
    const int lane = threadIdx.x;
    const float2* base = part + (n * C + g * D) * P;   // the group's planes are consecutive
    float a = 0.f, bb = 0.f;
    for (int64_t k = lane; k < D * P; k += kWave) {
        const int64_t cl = k / P;
        const float gm = gamma ? gamma[g * D + cl] : 1.f;
        const float2 q = base[k];
        a += gm * q.x;
        bb += gm * q.y;
    }
    a = wave_sum(a);
    bb = wave_sum(bb);
    if (lane == 0) ab[s] = make_float2(a, bb);
}

// ---- P3 --------------------------------------------------------------------
// one wave per channel: dbeta = sum over samples and tiles of S1, dgamma of S2
__global__ __launch_bounds__(kWave) void gen_plane_params(const float2* __restrict__ part, int P, int64_t N,
                                                          int64_t C, float* __restrict__ dbeta,
                                                          float* __restrict__ dgamma) {
    const int64_t c = blockIdx.x;
    const int lane = threadIdx.x;
    float a = 0.f, bb = 0.f;
    for (int64_t k = lane; k < N * P; k += kWave) {
        const int64_t n = k / P, t = k - n * P;
        const float2 q = part[(n * C + c) * P + t];
        a += q.x;
        bb += q.y;
    }
    a = wave_sum(a);
    bb = wave_sum(bb);
    if (lane == 0) {
        if (dbeta) dbeta[c] = a;
        if (dgamma) dgamma[c] = bb;
    }
}

// ---- boxes of each pass -------------------------------------------------------
// Digit specs list the dimensions innermost-first in the logical (n, c, h, w)
// order, which breaks stride ties.  Strides index: 0 n, 1 c, 2 h, 3 w.
Box slice_box(const Problem& p, const Strides& sd, const int64_t* const* st, int nt, bool channel_weight) {
    DigitSpec d[3] = {};
    d[0].ext = sd.W;
    d[1].ext = sd.H;
    d[2].ext = p.D;
    for (int t = 0; t < nt; ++t) {
        d[0].st[t] = st[t][3];
        d[1].st[t] = st[t][2];
        d[2].st[t] = st[t][1];
    }
    d[2].cw = channel_weight ? 1 : 0;
    return make_box(d, 3, nt);
}

Box elem_box(const Problem& p, const Strides& sd, const int64_t* const* st, int nt) {
    DigitSpec d[5] = {};
    d[0].ext = sd.W;
    d[1].ext = sd.H;
    d[2].ext = p.D;
    d[3].ext = p.G;
    d[4].ext = p.N;
    for (int t = 0; t < nt; ++t) {
        d[0].st[t] = st[t][3];
        d[1].st[t] = st[t][2];
        d[2].st[t] = st[t][1];
        d[3].st[t] = st[t][1] * p.D;
        d[4].st[t] = st[t][0];
    }
    d[2].cw = 1;
    d[3].cw = p.D;
    d[3].sw = 1;
    d[4].sw = p.G;
    return make_box(d, 5, nt);
}

Box param_box(const Problem& p, const Strides& sd, const int64_t* const* st, int nt) {
    DigitSpec d[3] = {};
    d[0].ext = sd.W;
    d[1].ext = sd.H;
    d[2].ext = p.N;
    for (int t = 0; t < nt; ++t) {
        d[0].st[t] = st[t][3];
        d[1].st[t] = st[t][2];
        d[2].st[t] = st[t][0];
    }
    d[2].sw = p.G;
    return make_box(d, 3, nt);
}

Box plane_box(const Strides& sd, const int64_t* const* st, int nt) {
    DigitSpec d[2] = {};
    d[0].ext = sd.W;
    d[1].ext = sd.H;
    for (int t = 0; t < nt; ++t) {
        d[0].st[t] = st[t][3];
        d[1].st[t] = st[t][2];
    }
    return make_box(d, 2, nt);
}

bool rowconst(const Box& b) { return b.cw[0] == 0 && b.sw[0] == 0; }

// Workgroups of the elementwise passes, which walk the tiles: at most 64 per
// CU (the 510 x 510 crops of the 112 x 64 x 512 x 512 fp32 images, two
// alternating rounds: 16 per CU 4.70 / 6.96-7.02 ms, 64 per CU 4.57 /
// 6.79-6.87 ms, one per tile 4.61-4.65 / 6.88-6.89 ms, forward / backward).
int elem_grid(const Tiling& t) {
    const int64_t cap = (int64_t)device_info().cu_count * 64;
    return (int)std::max<int64_t>(1, std::min<int64_t>(t.tiles, cap));
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct FwdPlan {
    Box sbox, ebox;
    Tiling stl, etl;
};

FwdPlan fwd_plan(const Problem& p, const Strides& sd) {
    const int64_t* xs[1] = {sd.x};
    const int64_t* xy[2] = {sd.x, sd.y};
    FwdPlan f;
    f.sbox = slice_box(p, sd, xs, 1, false);
    f.stl = make_tiling(f.sbox, kRedTile, kMaxParts, kRedU);
    f.ebox = elem_box(p, sd, xy, 2);
    f.etl = make_tiling(f.ebox, kElemTile, 0, kElemU);
    return f;
}

struct BwdPlan {
    bool planes;                 // reductions by per-(n, c) plane sums
    Box abox, ebox, pbox, lbox;
    Tiling atl, etl, ptl, ltl;
};

BwdPlan bwd_plan(const Problem& p, const Strides& sd) {
    const int64_t* dyx[2] = {sd.dy, sd.x};
    const int64_t* dyxdx[3] = {sd.dy, sd.x, sd.dx};
    BwdPlan b;
    b.abox = slice_box(p, sd, dyx, 2, true);
    b.atl = make_tiling(b.abox, kRedTile, kMaxParts, kRedU);
    b.ebox = elem_box(p, sd, dyxdx, 3);
    b.etl = make_tiling(b.ebox, kElemTile, 0, kElemU);
    b.pbox = param_box(p, sd, dyx, 2);
    b.ptl = make_tiling(b.pbox, kRedTile, kMaxParts, kRedU);
    b.lbox = plane_box(sd, dyx, 2);
    b.ltl = make_tiling(b.lbox, kRedTile, kMaxParts, kRedU);
    b.planes = p.HW >= kPlaneMinHW && b.lbox.st[0][0] == 1 && b.lbox.st[1][0] == 1 && b.lbox.ext[0] >= kWave;
    return b;
}

template <typename T>
hipError_t fwd_t(const Problem& p, const Strides& sd, const FwdArgs& a, const Launch& l) {
    const FwdPlan f = fwd_plan(p, sd);
    const int P = (int)f.stl.tiles;
    float4* part = (float4*)l.ws;
    const T* x = (const T*)a.x;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(gen_stats_partial<T>, dim3((unsigned)p.S, P), dim3(kT), 0, l.stream, x, f.sbox, f.stl,
                       p.G, sd.x[0], sd.x[1] * p.D, part, P);
    hipLaunchKernelGGL(gen_stats_final, dim3((unsigned)p.S), dim3(kWave), 0, l.stream, part, P, p.M, a.eps,
                       a.mean, a.rstd);
    int kernels = 2;
    if (a.y) {
        const int grid = elem_grid(f.etl);
        if (rowconst(f.ebox))
            hipLaunchKernelGGL((gen_apply<T, true>), dim3(grid), dim3(kT), 0, l.stream, x, (T*)a.y, a.gamma,
                               a.beta, a.mean, a.rstd, f.ebox, f.etl);
        else
            hipLaunchKernelGGL((gen_apply<T, false>), dim3(grid), dim3(kT), 0, l.stream, x, (T*)a.y, a.gamma,
                               a.beta, a.mean, a.rstd, f.ebox, f.etl);
        ++kernels;
    }
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_GENERIC;
        l.info->kernels = kernels;
        l.info->grid = (int64_t)P * p.S;
        l.info->tiles = f.etl.tiles;
    }
    return hipSuccess;
}

template <typename T>
hipError_t bwd_t(const Problem& p, const Strides& sd, const BwdArgs& a, const Launch& l) {
    const BwdPlan bp = bwd_plan(p, sd);
    const T* dy = (const T*)a.dy;
    const T* x = (const T*)a.x;
    char* ws = (char*)l.ws;
    hipError_t e;
    int kernels = 0;
    if ((e = record(l.ev_begin, l.stream))) return e;
    if (bp.planes) {
        const int P = (int)bp.ltl.tiles;
        float2* part = (float2*)ws;
        float2* ab = (float2*)(ws + align256((size_t)p.N * p.C * P * sizeof(float2)));
        hipLaunchKernelGGL(gen_plane_partial<T>, dim3((unsigned)(p.N * p.C), P), dim3(kT), 0, l.stream, dy, x,
                           a.mean, a.rstd, bp.lbox, bp.ltl, p.C, p.D, p.G, sd.dy[0], sd.dy[1], sd.x[0], sd.x[1],
                           part, P);
        kernels = 1;
        if (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) {
            hipLaunchKernelGGL(gen_plane_params, dim3((unsigned)p.C), dim3(kWave), 0, l.stream, part, P, p.N, p.C,
                               (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr,
                               (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr);
            ++kernels;
        }
        if (a.mask & GN_GRAD_DX) {
            hipLaunchKernelGGL(gen_plane_ab, dim3((unsigned)p.S), dim3(kWave), 0, l.stream, part, P, a.gamma, p.C,
                               p.D, p.G, ab);
            const int grid = elem_grid(bp.etl);
            if (rowconst(bp.ebox))
                hipLaunchKernelGGL((gen_dx<T, true>), dim3(grid), dim3(kT), 0, l.stream, dy, x, a.mean, a.rstd,
                                   a.gamma, ab, (T*)a.dx, bp.ebox, bp.etl, p.M);
            else
                hipLaunchKernelGGL((gen_dx<T, false>), dim3(grid), dim3(kT), 0, l.stream, dy, x, a.mean, a.rstd,
                                   a.gamma, ab, (T*)a.dx, bp.ebox, bp.etl, p.M);
            kernels += 2;
        }
    }
    if (!bp.planes && (a.mask & GN_GRAD_DX)) {
        const int P = (int)bp.atl.tiles;
        float2* part = (float2*)ws;
        float2* ab = (float2*)(ws + align256((size_t)p.S * P * sizeof(float2)));
        if (rowconst(bp.abox))
            hipLaunchKernelGGL((gen_ab_partial<T, true>), dim3((unsigned)p.S, P), dim3(kT), 0, l.stream, dy, x,
                               a.mean, a.rstd, a.gamma, bp.abox, bp.atl, p.G, p.D, sd.dy[0], sd.dy[1] * p.D,
                               sd.x[0], sd.x[1] * p.D, part, P);
        else
            hipLaunchKernelGGL((gen_ab_partial<T, false>), dim3((unsigned)p.S, P), dim3(kT), 0, l.stream, dy, x,
                               a.mean, a.rstd, a.gamma, bp.abox, bp.atl, p.G, p.D, sd.dy[0], sd.dy[1] * p.D,
                               sd.x[0], sd.x[1] * p.D, part, P);
        hipLaunchKernelGGL(gen_sum_rows, dim3((unsigned)p.S), dim3(kWave), 0, l.stream, part, P, ab,
                           (float*)nullptr, (float*)nullptr);
        const int grid = elem_grid(bp.etl);
        if (rowconst(bp.ebox))
            hipLaunchKernelGGL((gen_dx<T, true>), dim3(grid), dim3(kT), 0, l.stream, dy, x, a.mean, a.rstd,
                               a.gamma, ab, (T*)a.dx, bp.ebox, bp.etl, p.M);
        else
            hipLaunchKernelGGL((gen_dx<T, false>), dim3(grid), dim3(kT), 0, l.stream, dy, x, a.mean, a.rstd,
                               a.gamma, ab, (T*)a.dx, bp.ebox, bp.etl, p.M);
        kernels += 3;
    }
    if (!bp.planes && (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA))) {
        const int Q = (int)bp.ptl.tiles;
        float2* part = (float2*)ws;   // the dx stage above is ordered before on the stream
        if (rowconst(bp.pbox))
            hipLaunchKernelGGL((gen_param_partial<T, true>), dim3((unsigned)p.C, Q), dim3(kT), 0, l.stream, dy,
                               x, a.mean, a.rstd, bp.pbox, bp.ptl, p.D, sd.dy[1], sd.x[1], part, Q);
        else
            hipLaunchKernelGGL((gen_param_partial<T, false>), dim3((unsigned)p.C, Q), dim3(kT), 0, l.stream, dy,
                               x, a.mean, a.rstd, bp.pbox, bp.ptl, p.D, sd.dy[1], sd.x[1], part, Q);
        hipLaunchKernelGGL(gen_sum_rows, dim3((unsigned)p.C), dim3(kWave), 0, l.stream, part, Q,
                           (float2*)nullptr, (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr,
                           (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr);
        kernels += 2;
    }
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_GENERIC;
        l.info->kernels = kernels;
        l.info->tiles = bp.etl.tiles;
    }
    return hipSuccess;
}

}  // namespace

Strides dense_strides(const Problem& p) {
    Strides s{};
    s.H = 1;
    s.W = p.HW;
    int64_t d[4];
    if (p.layout == GN_NHWC) {
        d[0] = p.HW * p.C; d[1] = 1; d[2] = p.HW * p.C; d[3] = p.C;
    } else {
        d[0] = p.C * p.HW; d[1] = p.HW; d[2] = p.HW; d[3] = 1;
    }
    for (int k = 0; k < 4; ++k) s.x[k] = s.y[k] = s.dy[k] = s.dx[k] = d[k];
    return s;
}

size_t generic_fwd_ws(const Problem& p, const Strides& sd) {
    const FwdPlan f = fwd_plan(p, sd);
    return align256((size_t)p.S * f.stl.tiles * sizeof(float4));
}

size_t generic_bwd_ws(const Problem& p, const Strides& sd, int32_t mask) {
    const BwdPlan b = bwd_plan(p, sd);
    if (b.planes)
        return align256((size_t)p.N * p.C * b.ltl.tiles * sizeof(float2)) + align256((size_t)p.S * sizeof(float2));
    size_t need = 0;
    if (mask & GN_GRAD_DX)
        need = align256((size_t)p.S * b.atl.tiles * sizeof(float2)) + align256((size_t)p.S * sizeof(float2));
    if (mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) need = std::max(need, align256((size_t)p.C * b.ptl.tiles * sizeof(float2)));
    return need;
}

hipError_t generic_fwd(const Problem& p, const Strides& sd, const FwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return fwd_t<float>(p, sd, a, l);
        case GN_F16: return fwd_t<_Float16>(p, sd, a, l);
        default: return fwd_t<__bf16>(p, sd, a, l);
    }
}

hipError_t generic_bwd(const Problem& p, const Strides& sd, const BwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return bwd_t<float>(p, sd, a, l);
        case GN_F16: return bwd_t<_Float16>(p, sd, a, l);
        default: return bwd_t<__bf16>(p, sd, a, l);
    }
}

}  // namespace gn
