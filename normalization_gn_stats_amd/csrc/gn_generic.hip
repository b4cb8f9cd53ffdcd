// gn_generic.hip -- GroupNorm forward/backward for any shape, layout and
// alignment (scalar loads).  This is the correctness path every other path is
// compared with on odd shapes; it is not tuned.
//
// Forward (POPCORNBENCH GroupNorm trace: per (sample, group) mean and biased
// variance over (C/G)*H*W elements, then normalize and apply the per-channel
// weight and bias):
//   F1  per slice, per chunk of the slice: (count, mean, M2) of the chunk
//   F2  per slice: merge the chunk statistics in chunk order -> mean, rstd
//   F3  elementwise y = (x - mean)*(rstd*gamma_c) + beta_c
// Backward (the three stages of the baracuda-kernels GroupNorm backward plan:
// per-group reduction, per-cell dx, per-channel dgamma/dbeta):
//   B1  per slice, per chunk: A = sum gamma_c*dy, B = sum gamma_c*dy*xhat
//   B2  per slice: sum the chunk partials in chunk order
//   B3  elementwise dx = rstd*(gamma_c*dy - A/M - xhat*B/M)
//   B4  per channel, per chunk of the (n, p) range: sum dy, sum dy*xhat
//   B5  per channel: sum the chunk partials in chunk order -> dbeta, dgamma
// Every sum has a fixed order, so results are bitwise reproducible.
#include "gn_device.hpp"
#include "gn_internal.hpp"

namespace gn {
namespace {

constexpr int kT = 256;
constexpr int kNW = kT / kWave;
constexpr int64_t kChunk = 16384;   // elements per workgroup in the chunked passes
constexpr int kMaxChunks = 4096;

__device__ inline int64_t slice_elem(int64_t i, int64_t n, int64_t g, int64_t C, int64_t HW,
                                     int64_t D, int layout, int64_t* c_out) {
    if (layout == GN_NCHW) {
        const int64_t cl = i / HW;
        *c_out = g * D + cl;
        return (n * C + g * D) * HW + i;   // a slice is contiguous in NCHW
    }
    const int64_t p = i / D;
    const int64_t cl = i - p * D;
    *c_out = g * D + cl;
    return (n * HW + p) * C + g * D + cl;
}

template <typename T>
__device__ inline float ldf(const T* p, int64_t o) { return Vec<T>::to_f(p[o]); }

// ---- F1 --------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kT) void gen_stats_partial(const T* __restrict__ x, int64_t C, int64_t HW,
                                                        int64_t G, int64_t D, int64_t M, int64_t chunk,
                                                        int layout, float4* __restrict__ part, int P) {
    const int64_t s = blockIdx.x;
    const int b = blockIdx.y;
    const int64_t n = s / G, g = s - n * G;
    const int64_t lo = (int64_t)b * chunk;
    const int64_t hi = lo + chunk < M ? lo + chunk : M;
    Stat st = stat_empty();
    for (int64_t i = lo + threadIdx.x; i < hi; i += kT) {
        int64_t c;
        const float v = ldf(x, slice_elem(i, n, g, C, HW, D, layout, &c));
        st.n += 1.f;                         // Welford update
        const float d = v - st.mean;
        st.mean += d / st.n;
        st.m2 += d * (v - st.mean);
    }
    st = wave_merge_strided(st, 1);
    __shared__ Stat lds[kNW];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) lds[wave] = st;
    __syncthreads();
    if (threadIdx.x == 0) {
        Stat r = lds[0];
        for (int w = 1; w < kNW; ++w) r = stat_merge(r, lds[w]);
        part[s * P + b] = make_float4(r.n, r.mean, r.m2, 0.f);
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
        var = var > 0.f ? var : 0.f;
        mean[s] = st.mean;
        rstd[s] = 1.0f / sqrtf(var + eps);
    }
}

// ---- F3 --------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kT) void gen_apply(const T* __restrict__ x, const float* __restrict__ gamma,
                                                const float* __restrict__ beta, T* __restrict__ y,
                                                const float* __restrict__ mean, const float* __restrict__ rstd,
                                                int64_t E, int64_t C, int64_t HW, int64_t G, int64_t D,
                                                int layout) {
    const int64_t stride = (int64_t)gridDim.x * kT;
    for (int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x; e < E; e += stride) {
        int64_t n, c;
        if (layout == GN_NCHW) { const int64_t nc = e / HW; n = nc / C; c = nc - n * C; }
        else { const int64_t np = e / C; c = e - np * C; n = np / HW; }
        const int64_t s = n * G + c / D;
        const float a = rstd[s] * (gamma ? gamma[c] : 1.f);
        const float b = beta ? beta[c] : 0.f;
        y[e] = Vec<T>::from_f(fmaf(ldf(x, e) - mean[s], a, b));
    }
}

// ---- B1 --------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kT) void gen_ab_partial(const T* __restrict__ dy, const T* __restrict__ x,
                                                     const float* __restrict__ mean,
                                                     const float* __restrict__ rstd,
                                                     const float* __restrict__ gamma, int64_t C, int64_t HW,
                                                     int64_t G, int64_t D, int64_t M, int64_t chunk,
                                                     int layout, float2* __restrict__ part, int P) {
    const int64_t s = blockIdx.x;
    const int b = blockIdx.y;
    const int64_t n = s / G, g = s - n * G;
    const float mu = mean[s], r = rstd[s];
    const int64_t lo = (int64_t)b * chunk;
    const int64_t hi = lo + chunk < M ? lo + chunk : M;
    float acc[2] = {0.f, 0.f};
    for (int64_t i = lo + threadIdx.x; i < hi; i += kT) {
        int64_t c;
        const int64_t o = slice_elem(i, n, g, C, HW, D, layout, &c);
        const float gd = ldf(dy, o) * (gamma ? gamma[c] : 1.f);
        acc[0] += gd;
        acc[1] = fmaf(gd, (ldf(x, o) - mu) * r, acc[1]);
    }
    __shared__ float lds[kNW * 2];
    block_sum<2, kNW>(acc, lds);
    if (threadIdx.x == 0) part[s * P + b] = make_float2(acc[0], acc[1]);
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
template <typename T>
__global__ __launch_bounds__(kT) void gen_dx(const T* __restrict__ dy, const T* __restrict__ x,
                                             const float* __restrict__ mean, const float* __restrict__ rstd,
                                             const float* __restrict__ gamma, const float2* __restrict__ ab,
                                             T* __restrict__ dx, int64_t E, int64_t C, int64_t HW, int64_t G,
                                             int64_t D, int64_t M, int layout) {
    // gamma*dy is rounded exactly as in the partial sums, so that it cancels A/M
    // exactly where the slice makes dx vanish (one element per slice)
#pragma clang fp contract(off)
    const int64_t stride = (int64_t)gridDim.x * kT;
    const float invM = 1.0f / (float)M;
    for (int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x; e < E; e += stride) {
        int64_t n, c;
        if (layout == GN_NCHW) { const int64_t nc = e / HW; n = nc / C; c = nc - n * C; }
        else { const int64_t np = e / C; c = e - np * C; n = np / HW; }
        const int64_t s = n * G + c / D;
        const float r = rstd[s];
        const float xh = (ldf(x, e) - mean[s]) * r;
        const float gd = ldf(dy, e) * (gamma ? gamma[c] : 1.f);
        const float2 q = ab[s];
        dx[e] = Vec<T>::from_f(r * (gd - q.x * invM - xh * (q.y * invM)));
    }
}

// ---- B4 --------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kT) void gen_param_partial(const T* __restrict__ dy, const T* __restrict__ x,
                                                        const float* __restrict__ mean,
                                                        const float* __restrict__ rstd, int64_t N, int64_t C,
                                                        int64_t HW, int64_t G, int64_t D, int64_t chunk,
                                                        int layout, float2* __restrict__ part, int Q) {
    const int64_t c = blockIdx.x;
    const int b = blockIdx.y;
    const int64_t L = N * HW;
    const int64_t lo = (int64_t)b * chunk;
    const int64_t hi = lo + chunk < L ? lo + chunk : L;
    const int64_t g = c / D;
    float acc[2] = {0.f, 0.f};
    for (int64_t j = lo + threadIdx.x; j < hi; j += kT) {
        const int64_t n = j / HW, p = j - n * HW;
        const int64_t o = layout == GN_NCHW ? (n * C + c) * HW + p : (n * HW + p) * C + c;
        const int64_t s = n * G + g;
        const float d = ldf(dy, o);
        acc[0] += d;
        acc[1] += d * ((ldf(x, o) - mean[s]) * rstd[s]);
    }
    __shared__ float lds[kNW * 2];
    block_sum<2, kNW>(acc, lds);
    if (threadIdx.x == 0) part[c * Q + b] = make_float2(acc[0], acc[1]);
}

int chunks_for(int64_t L, int64_t* chunk) {
    int64_t ch = kChunk;
    int64_t P = (L + ch - 1) / ch;
    if (P > kMaxChunks) {
        ch = (L + kMaxChunks - 1) / kMaxChunks;
        P = (L + ch - 1) / ch;
    }
    if (P < 1) P = 1;
    *chunk = ch;
    return (int)P;
}

int elem_grid(int64_t E) {
    int64_t b = (E + kT - 1) / kT;
    const int64_t cap = (int64_t)device_info().cu_count * 16;
    return (int)(b < cap ? (b > 0 ? b : 1) : cap);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

template <typename T>
hipError_t fwd_t(const Problem& p, const FwdArgs& a, const Launch& l) {
    int64_t chunk;
    const int P = chunks_for(p.M, &chunk);
    float4* part = (float4*)l.ws;
    const T* x = (const T*)a.x;
    hipError_t e;
    if ((e = record(l.ev_begin, l.stream))) return e;
    hipLaunchKernelGGL(gen_stats_partial<T>, dim3((unsigned)p.S, P), dim3(kT), 0, l.stream, x, p.C, p.HW,
                       p.G, p.D, p.M, chunk, (int)p.layout, part, P);
    hipLaunchKernelGGL(gen_stats_final, dim3((unsigned)p.S), dim3(kWave), 0, l.stream, part, P, p.M, a.eps,
                       a.mean, a.rstd);
    int kernels = 2;
    if (a.y) {
        hipLaunchKernelGGL(gen_apply<T>, dim3(elem_grid(p.E)), dim3(kT), 0, l.stream, x, a.gamma, a.beta,
                           (T*)a.y, a.mean, a.rstd, p.E, p.C, p.HW, p.G, p.D, (int)p.layout);
        ++kernels;
    }
    if ((e = hipGetLastError())) return e;
    if ((e = record(l.ev_end, l.stream))) return e;
    if (l.info) {
        l.info->path = GN_PATH_GENERIC;
        l.info->kernels = kernels;
        l.info->grid = (int64_t)P * p.S;
    }
    return hipSuccess;
}

template <typename T>
hipError_t bwd_t(const Problem& p, const BwdArgs& a, const Launch& l) {
    const T* dy = (const T*)a.dy;
    const T* x = (const T*)a.x;
    char* ws = (char*)l.ws;
    hipError_t e;
    int kernels = 0;
    if ((e = record(l.ev_begin, l.stream))) return e;
    if (a.mask & GN_GRAD_DX) {
        int64_t chunk;
        const int P = chunks_for(p.M, &chunk);
        float2* part = (float2*)ws;
        float2* ab = (float2*)(ws + align256((size_t)p.S * P * sizeof(float2)));
        hipLaunchKernelGGL(gen_ab_partial<T>, dim3((unsigned)p.S, P), dim3(kT), 0, l.stream, dy, x, a.mean,
                           a.rstd, a.gamma, p.C, p.HW, p.G, p.D, p.M, chunk, (int)p.layout, part, P);
        hipLaunchKernelGGL(gen_sum_rows, dim3((unsigned)p.S), dim3(kWave), 0, l.stream, part, P, ab,
                           (float*)nullptr, (float*)nullptr);
        hipLaunchKernelGGL(gen_dx<T>, dim3(elem_grid(p.E)), dim3(kT), 0, l.stream, dy, x, a.mean, a.rstd,
                           a.gamma, ab, (T*)a.dx, p.E, p.C, p.HW, p.G, p.D, p.M, (int)p.layout);
        kernels += 3;
    }
    if (a.mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) {
        int64_t chunk;
        const int Q = chunks_for(p.N * p.HW, &chunk);
        float2* part = (float2*)ws;   // the dx stage above is ordered before on the stream
        hipLaunchKernelGGL(gen_param_partial<T>, dim3((unsigned)p.C, Q), dim3(kT), 0, l.stream, dy, x, a.mean,
                           a.rstd, p.N, p.C, p.HW, p.G, p.D, chunk, (int)p.layout, part, Q);
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
    }
    return hipSuccess;
}

}  // namespace

size_t generic_fwd_ws(const Problem& p) {
    int64_t chunk;
    const int P = chunks_for(p.M, &chunk);
    return align256((size_t)p.S * P * sizeof(float4));
}

size_t generic_bwd_ws(const Problem& p, int32_t mask) {
    size_t need = 0;
    int64_t chunk;
    if (mask & GN_GRAD_DX) {
        const int P = chunks_for(p.M, &chunk);
        need = align256((size_t)p.S * P * sizeof(float2)) + align256((size_t)p.S * sizeof(float2));
    }
    if (mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) {
        const int Q = chunks_for(p.N * p.HW, &chunk);
        const size_t b = align256((size_t)p.C * Q * sizeof(float2));
        need = need > b ? need : b;
    }
    return need;
}

hipError_t generic_fwd(const Problem& p, const FwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return fwd_t<float>(p, a, l);
        case GN_F16: return fwd_t<_Float16>(p, a, l);
        default: return fwd_t<__bf16>(p, a, l);
    }
}

hipError_t generic_bwd(const Problem& p, const BwdArgs& a, const Launch& l) {
    switch (p.dtype) {
        case GN_F32: return bwd_t<float>(p, a, l);
        case GN_F16: return bwd_t<_Float16>(p, a, l);
        default: return bwd_t<__bf16>(p, a, l);
    }
}

}  // namespace gn
