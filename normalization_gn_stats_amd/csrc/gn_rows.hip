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
                                                 float* __restrict__ mean, float* __restrict__ rstd, int64_t S,
                                                 int64_t G, int64_t C, int D, float eps) {
    constexpr int V = Vec<T>::V;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t s = (int64_t)blockIdx.x * kNW + threadIdx.x / kWave;
    if (s >= S) return;
    const int64_t n = s / G, g = s - n * G;
    const int64_t base = n * C + g * D;
    const int nvec = D / V;
    float v[NV][V];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int vi = j * kWave + lane;
        if (vi < nvec) {
            Vec<T>::unpack(ld16(x + base + (int64_t)vi * V), v[j]);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) v[j][k] = 0.f;
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int k = 0; k < V; ++k) sum += v[j][k];
    const float invD = 1.0f / (float)D;
    const float mu = wave_sum(sum) * invD;
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
    var = var > 0.f ? var : 0.f;
    const float r = 1.0f / sqrtf(var + eps);
    if (lane == 0) {
        mean[s] = mu;
        rstd[s] = r;
    }
    if (y == nullptr) return;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int vi = j * kWave + lane;
        if (vi >= nvec) continue;
        const int c0 = (int)(g * D) + vi * V;
        float o[V];
#pragma unroll
        for (int k = 0; k < V; k += 4) {
            float4 ga = gamma ? *reinterpret_cast<const float4*>(gamma + c0 + k) : make_float4(1.f, 1.f, 1.f, 1.f);
            float4 be = beta ? *reinterpret_cast<const float4*>(beta + c0 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
            o[k + 0] = fmaf(v[j][k + 0] - mu, r * ga.x, be.x);
            o[k + 1] = fmaf(v[j][k + 1] - mu, r * ga.y, be.y);
            o[k + 2] = fmaf(v[j][k + 2] - mu, r * ga.z, be.z);
            o[k + 3] = fmaf(v[j][k + 3] - mu, r * ga.w, be.w);
        }
        st16(y + base + (int64_t)vi * V, Vec<T>::pack(o));
    }
}

// part: [G][NB][D] float2 (sum dy, sum dy*xhat) -- one row per workgroup.
template <typename T, int NV>
__global__ __launch_bounds__(kT) void rows_bwd_k(const T* __restrict__ dy, const T* __restrict__ x,
                                                 const float* __restrict__ mean, const float* __restrict__ rstd,
                                                 const float* __restrict__ gamma, T* __restrict__ dx,
                                                 float2* __restrict__ part, int64_t N, int64_t G, int64_t C,
                                                 int D, int NB, int want_dx, int want_params) {
    constexpr int V = Vec<T>::V;
    extern __shared__ float2 lds_cols[];   // [D] when want_params
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t g = blockIdx.x / NB;
    const int b = blockIdx.x - (int)(g * NB);
    const int64_t W = (int64_t)NB * kNW;
    const int nvec = D / V;
    const float invD = 1.0f / (float)D;
    float cs1[NV][V], cs2[NV][V];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int k = 0; k < V; ++k) { cs1[j][k] = 0.f; cs2[j][k] = 0.f; }

    for (int64_t n = (int64_t)b * kNW + wave; n < N; n += W) {
        const int64_t s = n * G + g;
        const int64_t base = n * C + g * D;
        float xv[NV][V], dv[NV][V];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vi = j * kWave + lane;
            if (vi < nvec) {
                Vec<T>::unpack(ld16(x + base + (int64_t)vi * V), xv[j]);
                Vec<T>::unpack(ld16(dy + base + (int64_t)vi * V), dv[j]);
            } else {
#pragma unroll
                for (int k = 0; k < V; ++k) { xv[j][k] = 0.f; dv[j][k] = 0.f; }
            }
        }
        const float mu = mean[s], r = rstd[s];
        float a = 0.f, bb = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vi = j * kWave + lane;
            if (vi >= nvec) continue;
            const int c0 = (int)(g * D) + vi * V;
#pragma unroll
            for (int k = 0; k < V; k += 4) {
                float4 ga = gamma ? *reinterpret_cast<const float4*>(gamma + c0 + k) : make_float4(1.f, 1.f, 1.f, 1.f);
                const float gk[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float xh = (xv[j][k + u] - mu) * r;
                    const float gd = dv[j][k + u] * gk[u];
                    a += gd;
                    bb = fmaf(gd, xh, bb);
                    xv[j][k + u] = xh;            // keep xhat
                    cs1[j][k + u] += dv[j][k + u];
                    cs2[j][k + u] = fmaf(dv[j][k + u], xh, cs2[j][k + u]);
                    dv[j][k + u] = gd;            // keep gamma*dy
                }
            }
        }
        if (!want_dx) continue;
        {
            // gamma*dy stays the rounded product that entered A
#pragma clang fp contract(off)
            const float A = wave_sum(a) * invD;
            const float B = wave_sum(bb) * invD;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int vi = j * kWave + lane;
                if (vi >= nvec) continue;
                float o[V];
#pragma unroll
                for (int k = 0; k < V; ++k) o[k] = r * ((dv[j][k] - A) - xv[j][k] * B);
                st16(dx + base + (int64_t)vi * V, Vec<T>::pack(o));
            }
        }
    }
    if (!want_params) return;
    // waves add their column sums into LDS in wave order
    for (int w = 0; w < kNW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int vi = j * kWave + lane;
                if (vi >= nvec) continue;
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    float2 c = w == 0 ? make_float2(0.f, 0.f) : lds_cols[vi * V + k];
                    c.x += cs1[j][k];
                    c.y += cs2[j][k];
                    lds_cols[vi * V + k] = c;
                }
            }
        }
        __syncthreads();
    }
    float2* dst = part + ((int64_t)g * NB + b) * D;
    for (int c = threadIdx.x; c < D; c += kT) dst[c] = lds_cols[c];
}

// dbeta[g*D + c] = sum_b part[g][b][c].x, dgamma likewise with .y, b in order.
// Workgroup = 64 channels x 4 row lanes; each row lane sums rows rl, rl+4, ...
// then the four lanes are added in order.
__global__ __launch_bounds__(kT) void rows_colsum_k(const float2* __restrict__ part, int NB, int D,
                                                    float* __restrict__ dgamma, float* __restrict__ dbeta) {
    const int cb = blockIdx.x;
    const int g = blockIdx.y;
    const int cl = threadIdx.x & 63;
    const int rl = threadIdx.x >> 6;
    const int c = cb * 64 + cl;
    float s1 = 0.f, s2 = 0.f;
    if (c < D) {
        const float2* src = part + (int64_t)g * NB * D + c;
#pragma unroll 8
        for (int b = rl; b < NB; b += 4) {
            const float2 q = src[(int64_t)b * D];
            s1 += q.x;
            s2 += q.y;
        }
    }
    __shared__ float2 red[kT];
    red[threadIdx.x] = make_float2(s1, s2);
    __syncthreads();
    if (rl == 0 && c < D) {
        float2 t = red[cl];
        for (int k = 1; k < 4; ++k) {
            t.x += red[k * 64 + cl].x;
            t.y += red[k * 64 + cl].y;
        }
        if (dbeta) dbeta[(int64_t)g * D + c] = t.x;
        if (dgamma) dgamma[(int64_t)g * D + c] = t.y;
    }
}

constexpr int kMaxNV = 8;

int nv_for(const Problem& p) {
    const int V = p.elem_bytes == 4 ? 4 : 8;
    const int64_t nvec = p.D / V;
    const int64_t nv = (nvec + kWave - 1) / kWave;
    return nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 8 ? 8 : 0;
}

// Workgroups per group in the backward: about two per compute unit of an
// MI355X (256 CUs) in total, and at least ~4 slices per wave.  A constant, so
// that the workspace size does not depend on the device queried.
constexpr int64_t kBwdTargetWG = 512;

int rows_nb(const Problem& p) {
    int64_t target = kBwdTargetWG / (p.G < 1 ? 1 : p.G);
    if (target < 1) target = 1;
    int64_t need = (p.N + kNW * 4 - 1) / (kNW * 4);
    if (need < 1) need = 1;
    return (int)(need < target ? need : target);
}

template <typename T, int NV>
hipError_t fwd_nv(const Problem& p, const FwdArgs& a, const Launch& l) {
    const unsigned grid = (unsigned)((p.S + kNW - 1) / kNW);
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL((rows_fwd_k<T, NV>), dim3(grid), dim3(kT), 0, l.stream, (const T*)a.x, a.gamma, a.beta,
                       (T*)a.y, a.mean, a.rstd, p.S, p.G, p.C, (int)p.D, a.eps);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_ROWS;
        l.info->kernels = 1;
        l.info->grid = grid;
    }
    return hipSuccess;
}

template <typename T, int NV>
hipError_t bwd_nv(const Problem& p, const BwdArgs& a, const Launch& l) {
    const int NB = rows_nb(p);
    const bool params = (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) != 0;
    const unsigned grid = (unsigned)(p.G * NB);
    const size_t lds = params ? (size_t)p.D * sizeof(float2) : 0;
    float2* part = (float2*)l.ws;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL((rows_bwd_k<T, NV>), dim3(grid), dim3(kT), lds, l.stream, (const T*)a.dy, (const T*)a.x,
                       a.mean, a.rstd, a.gamma, (T*)a.dx, part, p.N, p.G, p.C, (int)p.D, NB,
                       (a.mask & GN_GRAD_DX) ? 1 : 0, params ? 1 : 0);
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    int kernels = 1;
    if (params) {
        hipLaunchKernelGGL(rows_colsum_k, dim3((unsigned)((p.D + 63) / 64), (unsigned)p.G), dim3(kT), 0,
                           l.stream, part, NB, (int)p.D, (a.mask & GN_GRAD_DGAMMA) ? a.dgamma : nullptr,
                           (a.mask & GN_GRAD_DBETA) ? a.dbeta : nullptr);
        if ((e = hipGetLastError())) return e;
        ++kernels;
    }
    if (l.info) {
        l.info->path = GN_PATH_ROWS;
        l.info->kernels = kernels;
        l.info->grid = grid;
    }
    return hipSuccess;
}

template <typename T>
hipError_t fwd_t(const Problem& p, const FwdArgs& a, const Launch& l) {
    switch (nv_for(p)) {
        case 1: return fwd_nv<T, 1>(p, a, l);
        case 2: return fwd_nv<T, 2>(p, a, l);
        case 4: return fwd_nv<T, 4>(p, a, l);
        default: return fwd_nv<T, 8>(p, a, l);
    }
}

template <typename T>
hipError_t bwd_t(const Problem& p, const BwdArgs& a, const Launch& l) {
    switch (nv_for(p)) {
        case 1: return bwd_nv<T, 1>(p, a, l);
        case 2: return bwd_nv<T, 2>(p, a, l);
        case 4: return bwd_nv<T, 4>(p, a, l);
        default: return bwd_nv<T, 8>(p, a, l);
    }
}

}  // namespace

bool rows_ok(const Problem& p) {
    if (p.HW != 1) return false;
    const int V = p.elem_bytes == 4 ? 4 : 8;
    if (p.D % V != 0 || p.C % V != 0) return false;   // every slice starts 16-byte aligned
    if (nv_for(p) == 0) return false;                 // slice fits the register budget
    (void)kMaxNV;
    return true;
}

size_t rows_fwd_ws(const Problem&) { return 0; }

size_t rows_bwd_ws(const Problem& p, int32_t mask) {
    if (!(mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA))) return 0;
    return (size_t)p.G * rows_nb(p) * p.D * sizeof(float2);
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
