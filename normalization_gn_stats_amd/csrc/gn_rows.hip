// gn_rows.hip -- GroupNorm with one spatial position (HW == 1): slice (n, g)
// is the contiguous run of D channels starting at n*C + g*D, in NCHW and NHWC
// alike.  G == 1 is LayerNorm over the channel axis (the LayerNorm backward
// shapes of ROCm/pytorch PR #3564's benchmark table).
//
// Forward: one wavefront per slice.  The slice is loaded once with 16-byte
// loads into registers; the mean and then the sum of squared deviations are
// taken from the registers (an exact two-pass variance at one read of x), and
// y = (x - mean)*(rstd*gamma_c) + beta_c is written with 16-byte stores.
//
// Slices of at most 32 16-byte vectors (e.g. 64 fp16 channels) share a
// wavefront instead: LPR lanes per slice, segmented shuffle sums.
//
// Backward: waves are assigned per group g and walk samples n = w, w + W, ...
// For each slice: xhat = (x - mean)*rstd from the saved statistics,
// A = sum gamma_c*dy, B = sum gamma_c*dy*xhat (wave sums), dx =
// rstd*(gamma_c*dy - A/D - xhat*B/D).  Each lane keeps running per-channel sums
// of dy and dy*xhat for its columns; the four waves of a workgroup add theirs
// in wave order into LDS, and the workgroup writes one partial row.  A second
// kernel sums the partial rows in row order into dbeta and dgamma -- the
// "two pass" column reduction of ROCm/pytorch PR #3564 (per-block partial
// column sums, then a final reduce), deterministic and free of float atomics.
#include "gn_device.hpp"
#include "gn_internal.hpp"

namespace gn {
namespace {

constexpr int kT = 256;
constexpr int kNW = kT / kWave;

template <typename T, int NV>
__global__ __launch_bounds__(kT) void rows_fwd_k(const T* __restrict__ x, const float* __restrict__ gamma,
                                                 const float* __restrict__ beta, T* __restrict__ y,
                                                 float* __restrict__ mean, float* __restrict__ rstd, int64_t N,
                                                 int64_t G, int64_t C, int D, float eps, int rms) {
    constexpr int V = Vec<T>::V;
    const int lane = threadIdx.x & (kWave - 1);
    // grid: x = blocks of kNW samples, y = group; the wave index is uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t n = (int64_t)blockIdx.x * kNW + wave;
    const int64_t g = blockIdx.y;
    if (n >= N) return;
    const int64_t s = n * G + g;
    const int64_t base = n * C + g * D;
    const int nvec = D / V;
    // Loads are branch-free: a lane past the end of the slice reads the last
    // vector again (always in bounds) and its values are dropped afterwards,
    // so every load of the wave issues back to back.
    float v[NV][V];
    u4v raw[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int vi = min(j * kWave + lane, nvec - 1);
        raw[j] = ld16(x + base + (int64_t)vi * V);
    }
    // affine parameters of the lane's columns, fetched while x is in flight
    float ga[NV][V], be[NV][V];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c0 = (int)(g * D) + min(j * kWave + lane, nvec - 1) * V;
#pragma unroll
        for (int k = 0; k < V; k += 4) {
            const float4 q = gamma ? *reinterpret_cast<const float4*>(gamma + c0 + k) : make_float4(1.f, 1.f, 1.f, 1.f);
            const float4 t = beta ? *reinterpret_cast<const float4*>(beta + c0 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
            ga[j][k] = q.x; ga[j][k + 1] = q.y; ga[j][k + 2] = q.z; ga[j][k + 3] = q.w;
            be[j][k] = t.x; be[j][k + 1] = t.y; be[j][k + 2] = t.z; be[j][k + 3] = t.w;
        }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        Vec<T>::unpack(raw[j], v[j]);
        if (j * kWave + lane >= nvec) {
#pragma unroll
            for (int k = 0; k < V; ++k) v[j][k] = 0.f;   // not part of the slice
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int k = 0; k < V; ++k) sum += v[j][k];
    const float invD = 1.0f / (float)D;
    const float mu = rms ? 0.f : wave_sum(sum) * invD;   // RMSNorm: no mean
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (j * kWave + lane < nvec) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = v[j][k] - mu;
                q = fmaf(d, d, q);
            }
        }
    }
    float var = wave_sum(q) * invD;
    var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
    const float r = 1.0f / sqrtf(var + eps);
    if (lane == 0) {
        if (mean) mean[s] = mu;
        rstd[s] = r;
    }
    if (y == nullptr) return;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int vi = j * kWave + lane;
        if (vi >= nvec) continue;
        float o[V];
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = fmaf(v[j][k] - mu, r * ga[j][k], be[j][k]);
        st16_nt(y + base + (int64_t)vi * V, Vec<T>::pack(o));
    }
}

// Forward for wide slices (more than 64*8 16-byte vectors): CS waves share a
// slice -- wave w works on slot w / CS and on the vectors [part*NV*64,
// (part+1)*NV*64) of its slice, part = w % CS -- and the per-wave sums meet in
// LDS, added in part order.  Same arithmetic as rows_fwd_k otherwise; gamma
// and beta are fetched per vector in the output loop (from L1/L2) instead of
// being held in registers.
template <typename T, int NV, int CS>
__global__ __launch_bounds__(kT) void rows_fwd_cs_k(const T* __restrict__ x, const float* __restrict__ gamma,
                                                    const float* __restrict__ beta, T* __restrict__ y,
                                                    float* __restrict__ mean, float* __restrict__ rstd, int64_t N,
                                                    int64_t G, int64_t C, int D, float eps, int rms) {
    constexpr int V = Vec<T>::V;
    constexpr int SLOTS = kNW / CS;
    __shared__ float red[2][kNW];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slot = wave / CS;
    const int cpart = wave - slot * CS;
    const int64_t n_raw = (int64_t)blockIdx.x * SLOTS + slot;
    const bool live = n_raw < N;                       // uniform per wave
    const int64_t n = live ? n_raw : N - 1;            // past N: re-read the last slice, write nothing
    const int64_t g = blockIdx.y;
    const int64_t s = n * G + g;
    const int64_t base = n * C + g * D;
    const int nvec = D / V;
    const int vbase = cpart * NV * kWave;
    float v[NV][V];
    u4v raw[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int vi = min(vbase + j * kWave + lane, nvec - 1);   // branch-free: see rows_fwd_k
        raw[j] = ld16(x + base + (int64_t)vi * V);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        Vec<T>::unpack(raw[j], v[j]);
        if (vbase + j * kWave + lane >= nvec) {
#pragma unroll
            for (int k = 0; k < V; ++k) v[j][k] = 0.f;   // not part of the slice
        }
    }
    const float invD = 1.0f / (float)D;
    float mu = 0.f;
    if (!rms) {   // RMSNorm: no mean
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int k = 0; k < V; ++k) sum += v[j][k];
        sum = wave_sum(sum);
        if (lane == 0) red[0][wave] = sum;
        __syncthreads();
        float t = red[0][slot * CS];
#pragma unroll
        for (int q = 1; q < CS; ++q) t += red[0][slot * CS + q];
        mu = t * invD;
    }
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (vbase + j * kWave + lane < nvec) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = v[j][k] - mu;
                q = fmaf(d, d, q);
            }
        }
    }
    q = wave_sum(q);
    if (lane == 0) red[1][wave] = q;
    __syncthreads();
    float t = red[1][slot * CS];
#pragma unroll
    for (int k = 1; k < CS; ++k) t += red[1][slot * CS + k];
    float var = t * invD;
    var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
    const float r = 1.0f / sqrtf(var + eps);
    if (!live) return;
    if (cpart == 0 && lane == 0) {
        if (mean) mean[s] = mu;
        rstd[s] = r;
    }
    if (y == nullptr) return;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int vi = vbase + j * kWave + lane;
        if (vi >= nvec) continue;
        const int64_t c0 = g * D + (int64_t)vi * V;
        float o[V];
#pragma unroll
        for (int k = 0; k < V; k += 4) {
            const float4 ga = gamma ? *reinterpret_cast<const float4*>(gamma + c0 + k) : make_float4(1.f, 1.f, 1.f, 1.f);
            const float4 be = beta ? *reinterpret_cast<const float4*>(beta + c0 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
            o[k] = fmaf(v[j][k] - mu, r * ga.x, be.x);
            o[k + 1] = fmaf(v[j][k + 1] - mu, r * ga.y, be.y);
            o[k + 2] = fmaf(v[j][k + 2] - mu, r * ga.z, be.z);
            o[k + 3] = fmaf(v[j][k + 3] - mu, r * ga.w, be.w);
        }
        st16_nt(y + base + (int64_t)vi * V, Vec<T>::pack(o));
    }
}

// Forward for many slices per group: each wave walks slices n = w, w + W, ...
// of group g (W waves per group), with the next slice's loads issued before
// the current one is reduced and written.  gamma and beta of the group are
// staged once per workgroup in LDS ([D] each, dynamic shared memory) instead
// of being held per lane in registers (2*NV*V of them) and reloaded for every
// slice: fewer registers, so more waves per SIMD, and one parameter fetch per
// workgroup instead of one per slice.  In LDS a vector's parameters sit
// [quarter of a vector][vector]: the lanes of a wave read consecutive
// 16-byte quarters (no bank conflicts; with V = 8 the vector-major order put
// lanes 32 bytes apart).  Each wave keeps at most GN_ROWS_FWD_Y_INFLIGHT y
// stores in flight, as the wide backward does with dx.  Same arithmetic as
// rows_fwd_k.
#ifndef GN_ROWS_WALK_NT
#define GN_ROWS_WALK_NT 1   // non-temporal loads of x (measured: 420 -> 398 us on 131072 x 4096 bf16)
#endif
// Each y store is issued at wave priority 2 (s_setprio), back to 0 after it:
// 131072 x 4096 bf16, four alternating rounds on two boxes, 382.5-384.7 ->
// 379.2-380.7 us and 379.6-381.7 -> 375.9-376.9 us; priority 3 no better; the
// next slice's loads at priority 3 unchanged; the wide backward's dx stores at
// priority 2 slower (545-547 -> 552-554 us).
// y stores in flight per wave, 131072 x 4096 bf16 with the layout above,
// four alternating rounds: 3 -> 384-386 us, 4 -> 385-386, 5 -> 382-384,
// 6 -> 383-384, 8 -> 385-388, unlimited -> 391-392 (vector-major layout,
// unlimited: 391-400)
#ifndef GN_ROWS_FWD_Y_INFLIGHT
#define GN_ROWS_FWD_Y_INFLIGHT 5
#endif
static_assert(GN_ROWS_FWD_Y_INFLIGHT >= 0 && GN_ROWS_FWD_Y_INFLIGHT <= 16, "vmcnt holds 0..15 here");
template <typename T, int NV>
__global__ __launch_bounds__(kT) void rows_fwd_lds_k(const T* __restrict__ x, const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, T* __restrict__ y,
                                                     float* __restrict__ mean, float* __restrict__ rstd, int64_t N,
                                                     int64_t G, int64_t C, int D, float eps, int rms) {
    constexpr int V = Vec<T>::V;
    extern __shared__ float4 lds_par[];   // [V/4][nvec] gamma, then the same for beta
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t g = blockIdx.y;
    const int64_t stride = (int64_t)gridDim.x * kNW;
    const int nvec = D / V;
    int64_t n = (int64_t)blockIdx.x * kNW + wave;
    u4v cur[NV], nxt[NV];
    auto load = [&](int64_t nn, u4v (&dst)[NV]) {
        const int64_t base = nn * C + g * D;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vi = min(j * kWave + lane, nvec - 1);   // branch-free: see rows_fwd_k
            dst[j] = GN_ROWS_WALK_NT ? ld16_nt(x + base + (int64_t)vi * V) : ld16(x + base + (int64_t)vi * V);
        }
    };
    if (n < N) load(n, cur);
    for (int i = threadIdx.x; i < D / 4; i += kT) {
        const int at = (i % (V / 4)) * nvec + i / (V / 4);   // quarter i % (V/4) of vector i / (V/4)
        lds_par[at] = gamma ? *reinterpret_cast<const float4*>(gamma + g * D + 4 * i) : make_float4(1.f, 1.f, 1.f, 1.f);
        lds_par[D / 4 + at] = beta ? *reinterpret_cast<const float4*>(beta + g * D + 4 * i)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    const float invD = 1.0f / (float)D;
    // One slice: issue the loads of the slice after it into `nx`, then reduce
    // and write slice n from `c`.  The walk alternates the two register sets
    // (no copy between them: a copy would wait for loads still in flight and
    // delay the next slice's loads until they land).
    auto step = [&](int64_t n, const u4v (&c)[NV], u4v (&nx)[NV]) {
        const int64_t nn = n + stride;
        if (nn < N) load(nn, nx);
        float v[NV][V];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            Vec<T>::unpack(c[j], v[j]);
            if (j * kWave + lane >= nvec) {
#pragma unroll
                for (int k = 0; k < V; ++k) v[j][k] = 0.f;   // not part of the slice
            }
        }
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int k = 0; k < V; ++k) sum += v[j][k];
        const float mu = rms ? 0.f : wave_sum(sum) * invD;   // RMSNorm: no mean
        float q = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (j * kWave + lane < nvec) {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float d = v[j][k] - mu;
                    q = fmaf(d, d, q);
                }
            }
        }
        float var = wave_sum(q) * invD;
        var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
        const float r = 1.0f / sqrtf(var + eps);
        const int64_t sl = n * G + g;
        if (lane == 0) {
            if (mean) mean[sl] = mu;
            rstd[sl] = r;
        }
        if (y != nullptr) {
            const int64_t base = n * C + g * D;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int vi = j * kWave + lane;
                if (vi < nvec) {
                    float o[V];
#pragma unroll
                    for (int k = 0; k < V; k += 4) {
                        const float4 ga = lds_par[(k / 4) * nvec + vi];
                        const float4 be = lds_par[D / 4 + (k / 4) * nvec + vi];
                        o[k] = fmaf(v[j][k] - mu, r * ga.x, be.x);
                        o[k + 1] = fmaf(v[j][k + 1] - mu, r * ga.y, be.y);
                        o[k + 2] = fmaf(v[j][k + 2] - mu, r * ga.z, be.z);
                        o[k + 3] = fmaf(v[j][k + 3] - mu, r * ga.w, be.w);
                    }
                    if constexpr (GN_ROWS_FWD_Y_INFLIGHT > 0)
                        __builtin_amdgcn_s_waitcnt(0x0F70 | (GN_ROWS_FWD_Y_INFLIGHT - 1));   // vmcnt(K - 1)
                    // the wave's store goes out ahead of other waves' arithmetic
                    __builtin_amdgcn_s_setprio(2);
                    st16_nt(y + base + (int64_t)vi * V, Vec<T>::pack(o));
                    __builtin_amdgcn_s_setprio(0);
                }
            }
        }
    };
    for (; n < N; n += 2 * stride) {
        step(n, cur, nxt);
        if (n + stride >= N) break;
        step(n + stride, nxt, cur);
    }
}

// ---- narrow slices: several slices per wavefront ----------------------------
// A slice of at most 32 16-byte vectors takes LPR lanes (the power of two at
// or above its vector count), so a wave holds RPW = 64/LPR slices at a time
// instead of leaving most of its lanes idle; each lane loads RB such row sets
// up front.  Slice sums are butterfly shuffles within the LPR lanes of a
// slice (partners add the same two values, so every lane of the slice ends
// with the same bits).  Same arithmetic as the one-wave-per-slice kernels.
template <int LPR>
__device__ inline float seg_sum(float v) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

template <int V>
__device__ inline void load_vec_params(const float* __restrict__ p, int64_t c0, float dflt, float (&o)[V]) {
#pragma unroll
    for (int k = 0; k < V; k += 4) {
        const float4 q = p ? *reinterpret_cast<const float4*>(p + c0 + k) : make_float4(dflt, dflt, dflt, dflt);
        o[k] = q.x; o[k + 1] = q.y; o[k + 2] = q.z; o[k + 3] = q.w;
    }
}

// grid: x = blocks of kNW*RPW*RB samples, y = group
template <typename T, int LPR, int RB>
__global__ __launch_bounds__(kT) void rows_fwd_narrow_k(const T* __restrict__ x, const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, T* __restrict__ y,
                                                        float* __restrict__ mean, float* __restrict__ rstd,
                                                        int64_t N, int64_t G, int64_t C, int D, float eps, int rms) {
    constexpr int V = Vec<T>::V;
    constexpr int RPW = kWave / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int vi = lane % LPR;   // vector within the slice
    const int rl = lane / LPR;   // slice within the row set
    const int64_t g = blockIdx.y;
    const int nvec = D / V;
    const bool act = vi < nvec;
    const int vc = min(vi, nvec - 1);   // branch-free loads: idle lanes re-read the last vector
    const int64_t n0 = ((int64_t)blockIdx.x * kNW + wave) * (RPW * RB);
    u4v raw[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t n = min(n0 + r * RPW + rl, N - 1);   // rows past N re-read row N-1
        raw[r] = ld16(x + n * C + g * D + (int64_t)vc * V);
    }
    float ga[V], be[V];
    load_vec_params<V>(gamma, g * D + (int64_t)vc * V, 1.f, ga);
    load_vec_params<V>(beta, g * D + (int64_t)vc * V, 0.f, be);
    const float invD = 1.0f / (float)D;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t n = n0 + r * RPW + rl;
        float v[V];
        Vec<T>::unpack(raw[r], v);
        float sum = 0.f;
        if (act) {
#pragma unroll
            for (int k = 0; k < V; ++k) sum += v[k];
        }
        const float mu = rms ? 0.f : seg_sum<LPR>(sum) * invD;   // RMSNorm: no mean
        float q = 0.f;
        if (act) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = v[k] - mu;
                q = fmaf(d, d, q);
            }
        }
        float var = seg_sum<LPR>(q) * invD;
        var = var < 0.f ? 0.f : var;   // rounding below zero clamped; NaN passes through
        const float rs = 1.0f / sqrtf(var + eps);
        if (n < N) {
            if (vi == 0) {
                if (mean) mean[n * G + g] = mu;
                rstd[n * G + g] = rs;
            }
            if (y != nullptr && act) {
                float o[V];
#pragma unroll
                for (int k = 0; k < V; ++k) o[k] = fmaf(v[k] - mu, rs * ga[k], be[k]);
                st16_nt(y + n * C + g * D + (int64_t)vi * V, Vec<T>::pack(o));
            }
        }
    }
}

// grid: x = NB workgroups per group, y = group; part as for rows_bwd_k.  A
// workgroup takes blocks of RPB = kNW*RPW*RB samples (blocks b, b + NB, ...).
template <typename T, int LPR, int RB>
__global__ __launch_bounds__(kT) void rows_bwd_narrow_k(const T* __restrict__ dy, const T* __restrict__ x,
                                                        const float* __restrict__ mean,
                                                        const float* __restrict__ rstd,
                                                        const float* __restrict__ gamma, T* __restrict__ dx,
                                                        float2* __restrict__ part, int64_t N, int64_t G, int64_t C,
                                                        int D, int NB, int want_dx, int want_params,
                                                 int rms) {
    constexpr int V = Vec<T>::V;
    constexpr int RPW = kWave / LPR;
    constexpr int RPB = kNW * RPW * RB;
    __shared__ float2 red_cols[kNW][32 * 8];   // per-wave column sums (D <= 32 vectors of <= 8)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int vi = lane % LPR;
    const int rl = lane / LPR;
    const int64_t g = blockIdx.y;
    const int b = blockIdx.x;
    const int nvec = D / V;
    const bool act = vi < nvec;
    const int vc = min(vi, nvec - 1);
    const float invD = 1.0f / (float)D;
    float gam[V];
    load_vec_params<V>(gamma, g * D + (int64_t)vc * V, 1.f, gam);
    float cs1[V], cs2[V];
#pragma unroll
    for (int k = 0; k < V; ++k) { cs1[k] = 0.f; cs2[k] = 0.f; }
    for (int64_t blk = b; blk * RPB < N; blk += NB) {   // uniform over the workgroup
        const int64_t n0 = blk * RPB + (int64_t)wave * (RPW * RB);
        u4v rx[RB], rd[RB];
        float mu[RB], rs[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t n = min(n0 + r * RPW + rl, N - 1);   // rows past N re-read row N-1
            const int64_t off = n * C + g * D + (int64_t)vc * V;
            rx[r] = ld16(x + off);
            rd[r] = ld16(dy + off);
            mu[r] = rms ? 0.f : mean[n * G + g];
            rs[r] = rstd[n * G + g];
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t n = n0 + r * RPW + rl;
            const bool valid = act && n < N;
            float xv[V], dv[V];
            Vec<T>::unpack(rx[r], xv);
            Vec<T>::unpack(rd[r], dv);
            float a = 0.f, bb = 0.f;
            if (valid) {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float xh = (xv[k] - mu[r]) * rs[r];
                    const float gd = dv[k] * gam[k];
                    a += gd;
                    bb = fmaf(gd, xh, bb);
                    cs1[k] += dv[k];
                    cs2[k] = fmaf(dv[k], xh, cs2[k]);
                }
            }
            const float A = rms ? 0.f : seg_sum<LPR>(a) * invD;   // RMSNorm: no mean term
            const float B = seg_sum<LPR>(bb) * invD;
            if (want_dx && valid) {
                // gamma*dy rounded as it entered A, so that equal terms cancel exactly
#pragma clang fp contract(off)
                float o[V];
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float xh = (xv[k] - mu[r]) * rs[r];
                    const float gd = dv[k] * gam[k];
                    o[k] = rs[r] * ((gd - A) - xh * B);
                }
                st16_nt(dx + n * C + g * D + (int64_t)vi * V, Vec<T>::pack(o));
            }
        }
    }
    if (!want_params) return;
    // column sums: the wave's row sets (lanes of equal vi) by butterfly, then
    // the waves in wave order through LDS
#pragma unroll
    for (int k = 0; k < V; ++k) {
#pragma unroll
        for (int m = LPR; m < kWave; m <<= 1) {
            cs1[k] += __shfl_xor(cs1[k], m, kWave);
            cs2[k] += __shfl_xor(cs2[k], m, kWave);
        }
    }
    if (lane < LPR && act) {
#pragma unroll
        for (int k = 0; k < V; ++k) red_cols[wave][vi * V + k] = make_float2(cs1[k], cs2[k]);
    }
    __syncthreads();
    float2* dst = part + ((int64_t)g * NB + b) * D;
    for (int c = threadIdx.x; c < D; c += kT) {
        float2 t = red_cols[0][c];
#pragma unroll
        for (int w = 1; w < kNW; ++w) {
            t.x += red_cols[w][c].x;
            t.y += red_cols[w][c].y;
        }
        dst[c] = t;
    }
}

// part: [G][NB][D] float2 (sum dy, sum dy*xhat) -- one row per workgroup.
//
// CS waves share a slice: wave w works on row slot w / CS and column part
// w % CS, i.e. the 16-byte vectors [part*NV*64, (part+1)*NV*64) of the slice,
// so that wide slices keep few registers per lane.  A workgroup takes blocks
// of RPB = (4/CS)*RB consecutive samples (blocks b, b + NB, ...); all RB
// slices of a wave in a block are loaded before any is used.  The per-slice
// sums A and B are wave sums (CS = 1) or wave sums added in part order
// through LDS (CS > 1).
//
// With four waves per slice (wide slices: the large, bandwidth-bound shapes)
// x and dy are read with non-temporal loads, and each dx store first waits
// until at most one earlier memory operation of the wave is outstanding: two
// stores in flight per wave.  The bursts of dx stores from every wave
// otherwise slow the other waves' loads.  Measured on 131072 x 4096 bf16:
//   plain loads, stores in flight unlimited / 4 / 2 / 1: 610 / 597 / 580 / 574
//   us (graph of 20 calls);
//   non-temporal loads, 1 in flight: 577 -> 566 us (graph), dgamma/dbeta-only
//   backward 358 -> 320 us;
//   non-temporal loads, unlimited / 4 / 2 / 1 in flight: 597 / 564 / 563 /
//   595 us in alternating eager calls (medians of four rounds; 585 / 558 /
//   562 / 570 us in a graph).
// Narrower slices (the small, latency-bound shapes) keep plain loads and
// their store bursts: they ran 10-20% slower with non-temporal loads.
#ifndef GN_ROWS_BWD_DX_INFLIGHT
#define GN_ROWS_BWD_DX_INFLIGHT 2
#endif
static_assert(GN_ROWS_BWD_DX_INFLIGHT >= 0 && GN_ROWS_BWD_DX_INFLIGHT <= 16, "vmcnt holds 0..15 here");
#ifndef GN_ROWS_BWD_NT_WIDE
#define GN_ROWS_BWD_NT_WIDE 1
#endif
constexpr bool kBwdNtWide = GN_ROWS_BWD_NT_WIDE != 0;

template <typename T, int NV, int RB, int CS, int NW = kNW>
__global__ __launch_bounds__(NW * kWave) void rows_bwd_k(const T* __restrict__ dy, const T* __restrict__ x,
                                                 const float* __restrict__ mean, const float* __restrict__ rstd,
                                                 const float* __restrict__ gamma, T* __restrict__ dx,
                                                 float2* __restrict__ part, int64_t N, int64_t G, int64_t C,
                                                 int D, int NB, int want_dx, int want_params,
                                                 int rms) {
    constexpr int V = Vec<T>::V;
    constexpr int SLOTS = NW / CS;
    constexpr int RPB = SLOTS * RB;
    constexpr bool kHoistGamma = NV * V <= 16;   // gamma of the lane's columns kept in registers
    extern __shared__ float2 lds_cols[];         // [SLOTS][D] when want_params
    __shared__ float2 red[RB][NW];               // per-wave (a, b) of each slice of the block
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slot = wave / CS;
    const int cpart = wave - slot * CS;
    const int64_t g = blockIdx.y;   // grid: x = NB workgroups per group, y = group
    const int b = blockIdx.x;
    const int nvec = D / V;
    const int vbase = cpart * NV * kWave;
    const float invD = 1.0f / (float)D;
    const float* gcol = gamma ? gamma + g * D : nullptr;

    float gam[kHoistGamma ? NV : 1][kHoistGamma ? V : 1];
    // gamma of the V columns of vector vi (registers, or float4 loads that hit L1/L2)
    auto gamma_vec = [&](int j, int vi, float (&gv)[V]) {
        if constexpr (kHoistGamma) {
#pragma unroll
            for (int k = 0; k < V; ++k) gv[k] = gam[j][k];
        } else {
            const int vc = min(vi, nvec - 1);
#pragma unroll
            for (int k = 0; k < V; k += 4) {
                float4 q = gcol ? *reinterpret_cast<const float4*>(gcol + vc * V + k) : make_float4(1.f, 1.f, 1.f, 1.f);
                gv[k] = q.x; gv[k + 1] = q.y; gv[k + 2] = q.z; gv[k + 3] = q.w;
            }
        }
    };
    // gamma of the lane's columns into registers (issued after the first
    // block's activations, so that they do not wait behind it)
    auto hoist_gamma = [&]() {
        if constexpr (kHoistGamma) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int vc = min(vbase + j * kWave + lane, nvec - 1);
#pragma unroll
                for (int k = 0; k < V; k += 4) {
                    float4 q = gcol ? *reinterpret_cast<const float4*>(gcol + vc * V + k)
                                    : make_float4(1.f, 1.f, 1.f, 1.f);
                    gam[j][k] = q.x; gam[j][k + 1] = q.y; gam[j][k + 2] = q.z; gam[j][k + 3] = q.w;
                }
            }
        }
    };

    float cs1[NV][V], cs2[NV][V];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int k = 0; k < V; ++k) { cs1[j][k] = 0.f; cs2[j][k] = 0.f; }

    // Branch-free loads of block blk: rows past N re-read row N-1 and vectors
    // past the slice re-read its last vector; both are dropped in run_block.
    auto load_block = [&](int64_t blk, u4v (&rx)[RB][NV], u4v (&rd)[RB][NV], float (&mu)[RB], float (&rs)[RB]) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t n = min(blk * RPB + r * SLOTS + slot, N - 1);
            const int64_t base = n * C + g * D;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int vi = min(vbase + j * kWave + lane, nvec - 1);
                if constexpr (CS == 4 && kBwdNtWide) {
                    rx[r][j] = ld16_nt(x + base + (int64_t)vi * V);
                    rd[r][j] = ld16_nt(dy + base + (int64_t)vi * V);
                } else {
                    rx[r][j] = ld16(x + base + (int64_t)vi * V);
                    rd[r][j] = ld16(dy + base + (int64_t)vi * V);
                }
            }
            mu[r] = rms ? 0.f : mean[n * G + g];
            rs[r] = rstd[n * G + g];
        }
    };

    auto run_block = [&](int64_t blk, u4v (&rx)[RB][NV], u4v (&rd)[RB][NV], const float (&mu)[RB],
                         const float (&rs)[RB]) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (blk * RPB + r * SLOTS + slot >= N) {   // uniform per wave: contributes nothing
#pragma unroll
                for (int j = 0; j < NV; ++j) { rx[r][j] = u4v{0u, 0u, 0u, 0u}; rd[r][j] = u4v{0u, 0u, 0u, 0u}; }
            }
        }
        // per-slice partial sums of this wave and the running column sums
        float a[RB], bb[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            a[r] = 0.f;
            bb[r] = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int vi = vbase + j * kWave + lane;
                if (vi >= nvec) continue;
                float xv[V], dv[V], gv[V];
                Vec<T>::unpack(rx[r][j], xv);
                Vec<T>::unpack(rd[r][j], dv);
                gamma_vec(j, vi, gv);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float xh = (xv[k] - mu[r]) * rs[r];
                    const float gd = dv[k] * gv[k];
                    a[r] += gd;
                    bb[r] = fmaf(gd, xh, bb[r]);
                    cs1[j][k] += dv[k];
                    cs2[j][k] = fmaf(dv[k], xh, cs2[j][k]);
                }
            }
        }
        if (!want_dx) return;   // kernel argument: uniform
        float A[RB], B[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            A[r] = wave_sum(a[r]);
            B[r] = wave_sum(bb[r]);
        }
        if constexpr (CS > 1) {
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < RB; ++r) red[r][wave] = make_float2(A[r], B[r]);
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                float2 t = red[r][slot * CS];
#pragma unroll
                for (int p = 1; p < CS; ++p) {
                    t.x += red[r][slot * CS + p].x;
                    t.y += red[r][slot * CS + p].y;
                }
                A[r] = t.x;
                B[r] = t.y;
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            A[r] = rms ? 0.f : A[r] * invD;   // RMSNorm: no mean term
            B[r] *= invD;
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t n = blk * RPB + r * SLOTS + slot;
            if (n >= N) continue;
            const int64_t base = n * C + g * D;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                // gamma*dy rounded as it entered A, so that equal terms cancel exactly
#pragma clang fp contract(off)
                const int vi = vbase + j * kWave + lane;
                if (vi >= nvec) continue;
                float xv[V], dv[V], gv[V], o[V];
                Vec<T>::unpack(rx[r][j], xv);
                Vec<T>::unpack(rd[r][j], dv);
                gamma_vec(j, vi, gv);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float xh = (xv[k] - mu[r]) * rs[r];
                    const float gd = dv[k] * gv[k];
                    o[k] = rs[r] * ((gd - A[r]) - xh * B[r]);
                }
                if constexpr (CS == 4 && GN_ROWS_BWD_DX_INFLIGHT > 0)
                    __builtin_amdgcn_s_waitcnt(0x0F70 | (GN_ROWS_BWD_DX_INFLIGHT - 1));   // vmcnt(K - 1)
                st16_nt(dx + base + (int64_t)vi * V, Vec<T>::pack(o));
            }
        }
    };

    bool first = true;
    for (int64_t blk = b; blk * RPB < N; blk += NB) {   // uniform over the workgroup
        u4v rx[RB][NV], rd[RB][NV];
        float mu[RB], rs[RB];
        load_block(blk, rx, rd, mu, rs);
        if (first) hoist_gamma();
        first = false;
        run_block(blk, rx, rd, mu, rs);
    }
    if (!want_params) return;
    // column sums of the row slots: each slot's into its own LDS row (the parts
    // of one slot cover disjoint columns), then every column added over the
    // slots in slot order
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int vi = vbase + j * kWave + lane;
        if (vi >= nvec) continue;
#pragma unroll
        for (int k = 0; k < V; ++k) lds_cols[slot * D + vi * V + k] = make_float2(cs1[j][k], cs2[j][k]);
    }
    __syncthreads();
    float2* dst = part + ((int64_t)g * NB + b) * D;
    for (int c = threadIdx.x; c < D; c += NW * kWave) {
        float2 t = lds_cols[c];
#pragma unroll
        for (int sl = 1; sl < SLOTS; ++sl) {
            const float2 u = lds_cols[sl * D + c];
            t.x += u.x;
            t.y += u.y;
        }
        dst[c] = t;
    }
}

// dbeta[g*D + c] = sum_b part[g][b][c].x, dgamma likewise with .y, b in
// order.  A workgroup covers kColPairs pairs of channels (one float4 of
// partials per row) with kRowLanes lanes over the partial rows: lane rl sums
// rows rl, rl + kRowLanes, ... and the lanes are then added in lane order.
constexpr int kColPairs = 8;
constexpr int kRowLanes = kT / kColPairs;

__global__ __launch_bounds__(kT) void rows_colsum_k(const float2* __restrict__ part, int NB, int D,
                                                    float* __restrict__ dgamma, float* __restrict__ dbeta) {
    const int cp = threadIdx.x % kColPairs;
    const int rl = threadIdx.x / kColPairs;
    const int g = blockIdx.y;
    const int c0 = (blockIdx.x * kColPairs + cp) * 2;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c0 < D) {
        const float2* src = part + (int64_t)g * NB * D + c0;
#pragma unroll 8
        for (int b = rl; b < NB; b += kRowLanes) {
            const float4 q = *reinterpret_cast<const float4*>(src + (int64_t)b * D);
            acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
        }
    }
    __shared__ float4 red[kT];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (rl == 0 && c0 < D) {
        float4 t = red[cp];
        for (int k = 1; k < kRowLanes; ++k) {
            const float4 q = red[k * kColPairs + cp];
            t.x += q.x; t.y += q.y; t.z += q.z; t.w += q.w;
        }
        const int64_t o = (int64_t)g * D + c0;
        if (dbeta) { dbeta[o] = t.x; dbeta[o + 1] = t.z; }
        if (dgamma) { dgamma[o] = t.y; dgamma[o + 1] = t.w; }
    }
}

#ifndef GN_ROWS_FWD_MIN_SPW
#define GN_ROWS_FWD_MIN_SPW 2        // slices per wave from which the forward walks
#endif
#ifndef GN_ROWS_BWD_TARGET_WG
#define GN_ROWS_BWD_TARGET_WG 512
#endif
#ifndef GN_ROWS_BWD_RB
#define GN_ROWS_BWD_RB 4
#endif
// Slices per wave per block when four waves share a slice (the wide,
// bandwidth-bound shapes): 2.  131072 x 4096 bf16 backward with 2 instead of
// 4: 557 -> 538 us in a graph of 20 calls, 569 -> 549 us in alternating eager
// calls.  The narrower slices keep 4 (with 2, their column sums take twice
// the partial rows, and the calls measured no faster).
#ifndef GN_ROWS_BWD_RB_WIDE
#define GN_ROWS_BWD_RB_WIDE 2
#endif

// 16-byte vectors per lane of the forward (one wave per slice): 1, 2, 4, 8, or
// 0 when the slice does not fit one wave.
int nv_for(const Problem& p) {
    const int V = p.elem_bytes == 4 ? 4 : 8;
    const int64_t nvec = p.D / V;
    const int64_t nv = (nvec + kWave - 1) / kWave;
    return nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 8 ? 8 : 0;
}

// Vectors per lane of the forward with four waves per slice (slices wider
// than one wave takes): 4, 8, or 0 when the slice does not fit four waves.
int nv_cs4(const Problem& p) {
    const int V = p.elem_bytes == 4 ? 4 : 8;
    const int64_t nvec = p.D / V;
    const int64_t nv = (nvec + 4 * kWave - 1) / (4 * kWave);
    return nv <= 4 ? 4 : nv <= 8 ? 8 : 0;
}

// Backward split: CS waves per slice (1, 2, 4) and NV vectors per lane, the
// fewest waves that keep NV <= 2; wider slices go to CS = 4 with NV 4 or 8.
struct BwdShape { int cs, nv, rb; };
BwdShape bwd_shape(const Problem& p) {
    const int V = p.elem_bytes == 4 ? 4 : 8;
    const int64_t nvec = p.D / V;
    for (int cs : {1, 2, 4}) {
        const int64_t nv = (nvec + cs * kWave - 1) / (cs * kWave);
        if (nv <= 2) return BwdShape{cs, nv <= 1 ? 1 : 2, cs == 4 ? GN_ROWS_BWD_RB_WIDE : GN_ROWS_BWD_RB};
    }
    const int64_t nv = (nvec + 4 * kWave - 1) / (4 * kWave);
    if (nv <= 4) return BwdShape{4, 4, 2};
    if (nv <= 8) return BwdShape{4, 8, 1};
    return BwdShape{0, 0, 0};
}

// Workgroups per group in the backward: about two per compute unit of an
// MI355X (256 CUs) in total, fewer when the samples run out.  A constant, so
// that the workspace size does not depend on the device queried.
constexpr int64_t kBwdTargetWG = GN_ROWS_BWD_TARGET_WG;

int rows_nb(const Problem& p) {
    const BwdShape sh = bwd_shape(p);
    const int64_t rpb = (int64_t)(kNW / (sh.cs > 0 ? sh.cs : 1)) * (sh.rb > 0 ? sh.rb : 1);
    int64_t target = kBwdTargetWG / (p.G < 1 ? 1 : p.G);
    if (target < 1) target = 1;
    int64_t need = (p.N + rpb - 1) / rpb;
    if (need < 1) need = 1;
    return (int)(need < target ? need : target);
}

#ifndef GN_ROWS_NARROW_RBF
#define GN_ROWS_NARROW_RBF 2   // row sets per lane in the narrow forward
#endif
#ifndef GN_ROWS_NARROW_RBB
#define GN_ROWS_NARROW_RBB 8   // row sets per lane in the narrow backward
#endif

// Lanes per slice of the narrow kernels (1 .. 32), or 0 when the slice takes
// more than 32 vectors (one or more waves per slice instead).
int narrow_lpr(const Problem& p) {
    const int V = p.elem_bytes == 4 ? 4 : 8;
    const int64_t nvec = p.D / V;
    if (nvec > 32) return 0;
    int lpr = 1;
    while (lpr < nvec) lpr *= 2;
    return lpr;
}

int narrow_nb(const Problem& p) {
    const int lpr = narrow_lpr(p);
    const int64_t rpb = (int64_t)kNW * (kWave / lpr) * GN_ROWS_NARROW_RBB;
    int64_t target = kBwdTargetWG / (p.G < 1 ? 1 : p.G);
    if (target < 1) target = 1;
    int64_t need = (p.N + rpb - 1) / rpb;
    if (need < 1) need = 1;
    return (int)(need < target ? need : target);
}

template <typename T, int LPR>
hipError_t fwd_narrow(const Problem& p, const FwdArgs& a, const Launch& l) {
    constexpr int RB = GN_ROWS_NARROW_RBF;
    constexpr int64_t rows_per_wg = (int64_t)kNW * (kWave / LPR) * RB;
    const unsigned grid = (unsigned)((p.N + rows_per_wg - 1) / rows_per_wg);
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL((rows_fwd_narrow_k<T, LPR, RB>), dim3(grid, (unsigned)p.G), dim3(kT), 0, l.stream,
                       (const T*)a.x, a.gamma, a.beta, (T*)a.y, a.mean, a.rstd, p.N, p.G, p.C, (int)p.D, a.eps, a.rms);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_ROWS;
        l.info->kernels = 1;
        l.info->grid = (int64_t)grid * p.G;
    }
    return hipSuccess;
}

template <typename T, int LPR>
hipError_t bwd_narrow(const Problem& p, const BwdArgs& a, const Launch& l) {
    constexpr int RB = GN_ROWS_NARROW_RBB;
    const int NB = narrow_nb(p);
    const bool params = (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) != 0;
    float2* part = (float2*)l.ws;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL((rows_bwd_narrow_k<T, LPR, RB>), dim3((unsigned)NB, (unsigned)p.G), dim3(kT), 0, l.stream,
                       (const T*)a.dy, (const T*)a.x, a.mean, a.rstd, a.gamma, (T*)a.dx, part, p.N, p.G, p.C,
                       (int)p.D, NB, (a.mask & GN_GRAD_DX) ? 1 : 0, params ? 1 : 0, a.rms);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    int kernels = 1;
    if (params) {
        hipLaunchKernelGGL(rows_colsum_k, dim3((unsigned)((p.D + 2 * kColPairs - 1) / (2 * kColPairs)), (unsigned)p.G),
                           dim3(kT), 0, l.stream, part, NB, (int)p.D, (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr,
                           (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr);
        if ((e = hipGetLastError())) return e;
        ++kernels;
    }
    if (l.info) {
        l.info->path = GN_PATH_ROWS;
        l.info->kernels = kernels;
        l.info->grid = (int64_t)NB * p.G;
    }
    return hipSuccess;
}

template <typename T, int NV>
hipError_t fwd_nv(const Problem& p, const FwdArgs& a, const Launch& l) {
    unsigned grid = (unsigned)((p.N + kNW - 1) / kNW);
    // Many slices per group: a grid of as many workgroups as fit on the chip
    // at once, whose waves walk several slices each with the parameters in
    // LDS (every wave walks the same number of slices, give or take one, so
    // there is no tail of late workgroups); otherwise one slice per wave.
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)rows_fwd_lds_k<T, NV>, kT, (size_t)p.D * 8) !=
            hipSuccess || occ < 1) {
        (void)hipGetLastError();
        occ = 1;
    }
    const int64_t resident = (int64_t)occ * device_info().cu_count;
    int64_t cap = resident / p.G;
    if (cap < 1) cap = 1;
    const bool walk = p.N / (kNW * cap) >= GN_ROWS_FWD_MIN_SPW;   // whole slices per wave
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    if (walk) {
        grid = (unsigned)(cap < 1 ? 1 : cap);
        hipLaunchKernelGGL((rows_fwd_lds_k<T, NV>), dim3(grid, (unsigned)p.G), dim3(kT), (size_t)p.D * 8, l.stream,
                           (const T*)a.x, a.gamma, a.beta, (T*)a.y, a.mean, a.rstd, p.N, p.G, p.C, (int)p.D, a.eps, a.rms);
    } else {
        hipLaunchKernelGGL((rows_fwd_k<T, NV>), dim3(grid, (unsigned)p.G), dim3(kT), 0, l.stream, (const T*)a.x,
                           a.gamma, a.beta, (T*)a.y, a.mean, a.rstd, p.N, p.G, p.C, (int)p.D, a.eps, a.rms);
    }
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_ROWS;
        l.info->kernels = 1;
        l.info->grid = (int64_t)grid * p.G;
    }
    return hipSuccess;
}

template <typename T, int NV, int RB, int CS, int NW = kNW>
hipError_t bwd_launch(const Problem& p, const BwdArgs& a, const Launch& l) {
    const int NB = rows_nb(p);
    const bool params = (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) != 0;
    const unsigned grid = (unsigned)NB;
    const size_t lds = params ? (size_t)(NW / CS) * p.D * sizeof(float2) : 0;   // [slots][D]
    float2* part = (float2*)l.ws;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL((rows_bwd_k<T, NV, RB, CS, NW>), dim3(grid, (unsigned)p.G), dim3(NW * kWave), lds, l.stream,
                       (const T*)a.dy, (const T*)a.x, a.mean, a.rstd, a.gamma, (T*)a.dx, part, p.N, p.G, p.C,
                       (int)p.D, NB, (a.mask & GN_GRAD_DX) ? 1 : 0, params ? 1 : 0, a.rms);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    int kernels = 1;
    if (params) {
        hipLaunchKernelGGL(rows_colsum_k, dim3((unsigned)((p.D + 2 * kColPairs - 1) / (2 * kColPairs)), (unsigned)p.G), dim3(kT), 0,
                           l.stream, part, NB, (int)p.D, (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr,
                           (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr);
        if ((e = hipGetLastError())) return e;
        ++kernels;
    }
    if (l.info) {
        l.info->path = GN_PATH_ROWS;
        l.info->kernels = kernels;
        l.info->grid = (int64_t)grid * p.G;
    }
    return hipSuccess;
}

template <typename T, int NV>
hipError_t fwd_cs4(const Problem& p, const FwdArgs& a, const Launch& l) {
    constexpr int CS = 4;
    constexpr int SLOTS = kNW / CS;
    const unsigned grid = (unsigned)((p.N + SLOTS - 1) / SLOTS);
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL((rows_fwd_cs_k<T, NV, CS>), dim3(grid, (unsigned)p.G), dim3(kT), 0, l.stream, (const T*)a.x,
                       a.gamma, a.beta, (T*)a.y, a.mean, a.rstd, p.N, p.G, p.C, (int)p.D, a.eps, a.rms);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_ROWS;
        l.info->kernels = 1;
        l.info->grid = (int64_t)grid * p.G;
    }
    return hipSuccess;
}

template <typename T>
hipError_t fwd_t(const Problem& p, const FwdArgs& a, const Launch& l) {
    if (nv_for(p) == 0) {   // wider than one wave: four waves per slice
        if (nv_cs4(p) == 4) return fwd_cs4<T, 4>(p, a, l);
        return fwd_cs4<T, 8>(p, a, l);
    }
    switch (narrow_lpr(p)) {
        case 1: return fwd_narrow<T, 1>(p, a, l);
        case 2: return fwd_narrow<T, 2>(p, a, l);
        case 4: return fwd_narrow<T, 4>(p, a, l);
        case 8: return fwd_narrow<T, 8>(p, a, l);
        case 16: return fwd_narrow<T, 16>(p, a, l);
        case 32: return fwd_narrow<T, 32>(p, a, l);
        default: break;
    }
    switch (nv_for(p)) {
        case 1: return fwd_nv<T, 1>(p, a, l);
        case 2: return fwd_nv<T, 2>(p, a, l);
        case 4: return fwd_nv<T, 4>(p, a, l);
        default: return fwd_nv<T, 8>(p, a, l);
    }
}

template <typename T>
hipError_t bwd_t(const Problem& p, const BwdArgs& a, const Launch& l) {
    switch (narrow_lpr(p)) {
        case 1: return bwd_narrow<T, 1>(p, a, l);
        case 2: return bwd_narrow<T, 2>(p, a, l);
        case 4: return bwd_narrow<T, 4>(p, a, l);
        case 8: return bwd_narrow<T, 8>(p, a, l);
        case 16: return bwd_narrow<T, 16>(p, a, l);
        case 32: return bwd_narrow<T, 32>(p, a, l);
        default: break;
    }
    constexpr int RBS = GN_ROWS_BWD_RB, RBW = GN_ROWS_BWD_RB_WIDE;
    const BwdShape sh = bwd_shape(p);
    switch (sh.cs * 100 + sh.nv) {
        case 101: return bwd_launch<T, 1, RBS, 1>(p, a, l);
        case 102: return bwd_launch<T, 2, RBS, 1>(p, a, l);
        case 201: return bwd_launch<T, 1, RBS, 2>(p, a, l);
        case 202: return bwd_launch<T, 2, RBS, 2>(p, a, l);
        case 401: return bwd_launch<T, 1, RBW, 4>(p, a, l);
        case 402: return bwd_launch<T, 2, RBW, 4>(p, a, l);
        case 404: return bwd_launch<T, 4, 2, 4>(p, a, l);
        default: return bwd_launch<T, 8, 1, 4>(p, a, l);
    }
}

}  // namespace

bool rows_ok(const Problem& p) {
    if (p.HW != 1) return false;
    const int V = p.elem_bytes == 4 ? 4 : 8;
    if (p.D % V != 0 || p.C % V != 0) return false;   // every slice starts 16-byte aligned
    if ((nv_for(p) == 0 && nv_cs4(p) == 0) || bwd_shape(p).cs == 0) return false;   // slice fits the register budget
    return true;
}

size_t rows_fwd_ws(const Problem&) { return 0; }

size_t rows_bwd_ws(const Problem& p, int32_t mask) {
    if (!(mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA))) return 0;
    return (size_t)p.G * (narrow_lpr(p) ? narrow_nb(p) : rows_nb(p)) * p.D * sizeof(float2);
}

hipError_t rows_fwd(const Problem& p, const FwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return fwd_t<float>(p, a, l);
        case GN_F16: return fwd_t<_Float16>(p, a, l);
        default: return fwd_t<__bf16>(p, a, l);
    }
}

hipError_t rows_bwd(const Problem& p, const BwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return bwd_t<float>(p, a, l);
        case GN_F16: return bwd_t<_Float16>(p, a, l);
        default: return bwd_t<__bf16>(p, a, l);
    }
}

}  // namespace gn
