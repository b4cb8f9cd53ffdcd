// gn_api.cpp -- the C ABI declared in include/gn.h: argument validation (the
// checks of the baracuda-kernels GroupNorm backward plan: non-negative sizes,
// G > 0 dividing C, supported dtype, affine all-or-none, workspace at least
// the queried size, zero extent is a successful no-op), path selection and
// dispatch to the kernel launchers.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "gn_internal.hpp"

namespace gn {

namespace {
DeviceInfo g_dev[64];
bool g_dev_ok[64];
std::mutex g_dev_mu;
}  // namespace

const DeviceInfo& device_info() {
    static DeviceInfo fallback{-1, 256, 0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return fallback;
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!g_dev_ok[dev]) {
        DeviceInfo d{dev, 256, 0};
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            d.cu_count = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess)
            d.coop_supported = v;
        (void)hipGetLastError();
        g_dev[dev] = d;
        g_dev_ok[dev] = true;
    }
    return g_dev[dev];
}

hipError_t record(hipEvent_t ev, hipStream_t s) {
    if (!ev) return hipSuccess;
    // under stream capture the event becomes a timing node of the graph
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive)
        return hipEventRecordWithFlags(ev, s, hipEventRecordExternal);
    return hipEventRecord(ev, s);
}

}  // namespace gn

using gn::Problem;

// A static device array for callers that cannot allocate: the workspace of
// gn_backward_scratch (each device holds its own copy).  In host code its name
// is only a handle; the device address of each device's copy comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to kernels.
static constexpr size_t kScratchBytes = (size_t)GN_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape/dtype/layout checks shared by every entry point.
gn_status make_problem(int64_t N, int64_t C, int64_t HW, int64_t G, gn_dtype dtype, gn_layout layout,
                       Problem* p) {
    if (dtype != GN_F32 && dtype != GN_F16 && dtype != GN_BF16) return GN_ERR_UNSUPPORTED;
    if (layout != GN_NCHW && layout != GN_NHWC) return GN_ERR_UNSUPPORTED;
    if (N < 0 || C < 0 || HW < 0 || G <= 0) return GN_ERR_INVALID;
    if (C > 0 && C % G != 0) return GN_ERR_INVALID;
    if (C == 0 && G > 0) { /* zero extent: G is irrelevant */ }
    // 64-bit element count must not overflow
    if (N > 0 && C > 0 && HW > 0) {
        const double e = (double)N * (double)C * (double)HW;
        if (e > 9.0e18) return GN_ERR_INVALID;
    }
    p->N = N; p->C = C; p->HW = HW; p->G = G;
    p->D = G > 0 ? C / G : 0;
    p->M = p->D * HW;
    p->S = N * G;
    p->E = N * C * HW;
    p->dtype = dtype;
    p->layout = layout;
    p->elem_bytes = dtype == GN_F32 ? 4 : 2;
    return GN_OK;
}

bool zero_extent(const Problem& p) { return p.N == 0 || p.C == 0 || p.HW == 0; }

int32_t forced(const gn_options* o) { return o ? o->force_path : GN_PATH_AUTO; }

// Path for these shapes assuming 16-byte aligned pointers; -1 if the forced
// path cannot serve them.
int32_t plan(const Problem& p, bool backward, const gn_options* opts) {
    const int32_t f = forced(opts);
    if (f == GN_PATH_GENERIC) return GN_PATH_GENERIC;
    if (f == GN_PATH_ROWS) return gn::rows_ok(p) ? GN_PATH_ROWS : -1;
    if (f == GN_PATH_SLAB) return gn::slab_ok(p) ? GN_PATH_SLAB : -1;
    if (f == GN_PATH_STREAM) return gn::stream_ok(p) ? GN_PATH_STREAM : -1;
    if (f != GN_PATH_AUTO) return -1;
    if (gn::rows_ok(p)) return GN_PATH_ROWS;
    // NHWC: the stream kernels whenever they take the shape.  Against the
    // cooperative slab kernels they measured 2-6x faster at every NHWC size
    // tried (fp16/fp32, 2x32x16x16 to 16x256x64x64 and 1x128x512x512,
    // forward and backward, graph or eager): at these sizes the cooperative
    // launch and the two team barriers per slab cost more than the second
    // read of each tile saves, and on the 1x128x1024x2048 image the slab
    // kernels re-read almost every tile anyway.  The slab kernels take the
    // NHWC shapes beyond the stream grid (more than 65535 samples), and NCHW.
    (void)backward;
    if (gn::stream_ok(p)) return GN_PATH_STREAM;
    if (gn::slab_ok(p)) return GN_PATH_SLAB;
    return GN_PATH_GENERIC;
}

size_t fwd_ws(const Problem& p, int32_t path) {
    switch (path) {
        case GN_PATH_ROWS: return gn::rows_fwd_ws(p);
        case GN_PATH_SLAB: return gn::slab_fwd_ws(p);
        case GN_PATH_STREAM: return gn::stream_fwd_ws(p);
        default: return gn::generic_fwd_ws(p, gn::dense_strides(p));
    }
}

size_t bwd_ws(const Problem& p, int32_t mask, int32_t path) {
    switch (path) {
        case GN_PATH_ROWS: return gn::rows_bwd_ws(p, mask);
        case GN_PATH_SLAB: return gn::slab_bwd_ws(p, mask);
        case GN_PATH_STREAM: return gn::stream_bwd_ws(p, mask);
        default: return gn::generic_bwd_ws(p, gn::dense_strides(p), mask);
    }
}

gn::Launch make_launch(void* ws, size_t ws_bytes, void* stream, const gn_options* opts) {
    gn::Launch l;
    l.stream = (hipStream_t)stream;
    l.ws = ws;
    l.ws_bytes = ws_bytes;
    l.ev_begin = opts ? (hipEvent_t)opts->kernel_begin : nullptr;
    l.ev_end = opts ? (hipEvent_t)opts->kernel_end : nullptr;
    l.max_resident_override = opts ? opts->max_resident_override : 0;
    l.info = opts ? opts->info : nullptr;
    l.status_word = opts ? opts->status_word : nullptr;
    l.spin_limit = (opts && opts->spin_limit) ? opts->spin_limit : gn::kDefaultSpinLimit;
    l.unmet_waits = (opts && (opts->debug_flags & GN_DEBUG_UNMET_WAITS)) ? 1u : 0u;
    l.stream_split = (opts && (opts->debug_flags & GN_DEBUG_STREAM_SPLIT)) ? 1u : 0u;
    l.slab_coop = (opts && (opts->debug_flags & GN_DEBUG_SLAB_COOP)) ? 1u : 0u;
    return l;
}

// ---- one empty cooperative launch per process and device, early --------------
// The HIP runtime sets, at a process's first cooperative launch, a state that
// then holds for every cooperative launch of the process.  Measured on MI355X
// (ROCm 7): when that first launch comes after three or more captured graphs of
// several kernel nodes each (of any kernels), every later cooperative launch,
// eager or in a graph, runs about three times slower (1x512x256x256 fp16 G32:
// 46 / 61 us -> 153 / 126 us per forward / backward call); when a cooperative
// launch came before those graphs, they change nothing.  So the library's first
// call on a device, whatever its path, makes one empty one-workgroup
// cooperative launch on its stream ahead of its own kernels, unless the stream
// is capturing (then a later call does); it counts as done once the runtime
// accepts it.  The price: while this process runs, other processes on the
// device find their cooperative launches refused (their slab calls then take
// the split or generic kernels).
__global__ void coop_first_k() {}

std::mutex g_coop_mu;
bool g_coop_done[64];
bool g_coop_refused[64];   // the last early launch was refused

// GN_EARLY_COOP=0 in the environment leaves the early launch out, for processes
// that should not hold the cooperative state (e.g. several processes on one
// device, only some of which need the cooperative kernels).
bool early_coop_wanted() {
    static const bool wanted = [] {
        const char* v = getenv("GN_EARLY_COOP");
        return !(v && v[0] == '0' && v[1] == '\0');
    }();
    return wanted;
}

void coop_first(hipStream_t s) {
    if (!early_coop_wanted()) return;
    const gn::DeviceInfo& d = gn::device_info();
    if (d.device < 0 || d.device >= 64 || !d.coop_supported) return;
    std::lock_guard<std::mutex> lk(g_coop_mu);
    if (g_coop_done[d.device]) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {   // e.g. the legacy stream while another captures
        (void)hipGetLastError();
        return;
    }
    if (cs != hipStreamCaptureStatusNone) return;
    void* none[1] = {nullptr};
    if (hipLaunchCooperativeKernel((const void*)coop_first_k, dim3(1), dim3(64), none, 0, s) == hipSuccess) {
        g_coop_done[d.device] = true;
        g_coop_refused[d.device] = false;
    } else {
        (void)hipGetLastError();   // refused (another process holds the state): a later call tries again
        g_coop_refused[d.device] = true;
    }
}

}  // namespace

bool gn::coop_accepted() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return false;
    }
    std::lock_guard<std::mutex> lk(g_coop_mu);
    return g_coop_done[dev];
}

namespace {

// Runs one launcher between the caller's whole-call events (if any).
template <typename F>
gn_status with_call_events(const gn_options* opts, void* stream, F&& launch) {
    hipStream_t s = (hipStream_t)stream;
    coop_first(s);
    if (opts && opts->event_begin && gn::record((hipEvent_t)opts->event_begin, s) != hipSuccess) return GN_ERR_HIP;
    if (launch() != hipSuccess) return GN_ERR_HIP;
    if (opts && opts->event_end && gn::record((hipEvent_t)opts->event_end, s) != hipSuccess) return GN_ERR_HIP;
    return GN_OK;
}

// ---- the backward, with the caller's workspace or the library's scratch ----
void* g_scratch[64];
bool g_scratch_ok[64];
std::mutex g_scratch_mu;

// This device's address of `scratch` (the current device), or NULL on failure.
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ok[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch[dev] = ptr;
        g_scratch_ok[dev] = true;
    }
    return g_scratch[dev];
}

gn_status backward_call(const void* dy, const void* x, const float* mean, const float* rstd, const float* gamma,
                        void* dx, float* dgamma, float* dbeta, int32_t mask, int64_t N, int64_t C, int64_t HW,
                        int64_t G, gn_dtype dtype, gn_layout layout, void* workspace, size_t ws_bytes,
                        bool use_scratch, void* stream, const gn_options* opts) {
    Problem p;
    gn_status st = make_problem(N, C, HW, G, dtype, layout, &p);
    if (st != GN_OK) return st;
    if (mask <= 0 || mask > 7) return GN_ERR_INVALID;
    if ((mask & GN_GRAD_DX) && dx == nullptr) return GN_ERR_INVALID;
    if ((mask & GN_GRAD_DGAMMA) && dgamma == nullptr) return GN_ERR_INVALID;
    if ((mask & GN_GRAD_DBETA) && dbeta == nullptr) return GN_ERR_INVALID;
    if ((mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) && gamma == nullptr) return GN_ERR_INVALID;
    if (zero_extent(p)) {
        if (opts && opts->info) *opts->info = gn_plan_info{GN_PATH_AUTO, 0, 0, 0, 0, 0};
        return GN_OK;
    }
    if (dy == nullptr || x == nullptr || mean == nullptr || rstd == nullptr) return GN_ERR_INVALID;
    int32_t path = plan(p, true, opts);
    if (path < 0) return GN_ERR_UNSUPPORTED;
    if (path != GN_PATH_GENERIC) {
        const bool al = aligned16(dy) && aligned16(x) && aligned16(gamma) &&
                        (!(mask & GN_GRAD_DX) || aligned16(dx));
        if (!al) {
            if (forced(opts) != GN_PATH_AUTO) return GN_ERR_UNSUPPORTED;
            path = GN_PATH_GENERIC;
        }
    }
    const size_t need = bwd_ws(p, mask, path);
    if (use_scratch) {
        if (need > kScratchBytes) return GN_ERR_WORKSPACE;
        workspace = need > 0 ? scratch_address() : nullptr;
        if (need > 0 && workspace == nullptr) return GN_ERR_HIP;
        ws_bytes = kScratchBytes;
    }
    if (ws_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace)))) return GN_ERR_WORKSPACE;
    gn::BwdArgs a{dy, x, mean, rstd, gamma,
                  (mask & GN_GRAD_DX) ? dx : nullptr,
                  (mask & GN_GRAD_DGAMMA) ? dgamma : nullptr,
                  (mask & GN_GRAD_DBETA) ? dbeta : nullptr, mask, 0};
    gn::Launch l = make_launch(workspace, ws_bytes, stream, opts);
    if (l.info) *l.info = gn_plan_info{path, 0, 0, 0, 0, 0};
    return with_call_events(opts, stream, [&] {
        return path == GN_PATH_ROWS ? gn::rows_bwd(p, a, l)
             : path == GN_PATH_SLAB ? gn::slab_bwd(p, a, l)
             : path == GN_PATH_STREAM ? gn::stream_bwd(p, a, l)
                                    : gn::generic_bwd(p, gn::dense_strides(p), a, l);
    });
}

}  // namespace

extern "C" {

size_t gn_forward_workspace_size(int64_t N, int64_t C, int64_t HW, int64_t G, gn_dtype dtype,
                                 gn_layout layout, const gn_options* opts) {
    Problem p;
    if (make_problem(N, C, HW, G, dtype, layout, &p) != GN_OK || zero_extent(p)) return 0;
    const int32_t path = plan(p, false, opts);
    if (path < 0) return 0;
    // the generic path is the fallback for unaligned pointers: cover it too
    size_t a = fwd_ws(p, path), b = gn::generic_fwd_ws(p, gn::dense_strides(p));
    return a > b ? a : b;
}

size_t gn_backward_workspace_size(int64_t N, int64_t C, int64_t HW, int64_t G, gn_dtype dtype,
                                  gn_layout layout, int32_t mask, const gn_options* opts) {
    Problem p;
    if (make_problem(N, C, HW, G, dtype, layout, &p) != GN_OK || zero_extent(p)) return 0;
    if (mask <= 0 || mask > 7) return 0;
    const int32_t path = plan(p, true, opts);
    if (path < 0) return 0;
    size_t a = bwd_ws(p, mask, path), b = gn::generic_bwd_ws(p, gn::dense_strides(p), mask);
    return a > b ? a : b;
}

int32_t gn_select_path(int32_t backward, int64_t N, int64_t C, int64_t HW, int64_t G, gn_dtype dtype,
                       gn_layout layout, const gn_options* opts) {
    Problem p;
    if (make_problem(N, C, HW, G, dtype, layout, &p) != GN_OK) return -1;
    return plan(p, backward != 0, opts);
}

gn_status gn_forward(const void* x, const float* gamma, const float* beta, void* y, float* mean, float* rstd,
                     int64_t N, int64_t C, int64_t HW, int64_t G, float eps, gn_dtype dtype, gn_layout layout,
                     void* workspace, size_t ws_bytes, void* stream, const gn_options* opts) {
    Problem p;
    gn_status st = make_problem(N, C, HW, G, dtype, layout, &p);
    if (st != GN_OK) return st;
    if (!(eps >= 0.f) || isinf(eps)) return GN_ERR_INVALID;
    if ((gamma == nullptr) != (beta == nullptr)) return GN_ERR_INVALID;
    if (zero_extent(p)) {
        if (opts && opts->info) *opts->info = gn_plan_info{GN_PATH_AUTO, 0, 0, 0, 0, 0};
        return GN_OK;
    }
    if (x == nullptr || mean == nullptr || rstd == nullptr) return GN_ERR_INVALID;
    int32_t path = plan(p, false, opts);
    if (path < 0) return GN_ERR_UNSUPPORTED;
    if (path != GN_PATH_GENERIC) {
        const bool al = aligned16(x) && (y == nullptr || aligned16(y)) && aligned16(gamma) && aligned16(beta);
        if (!al) {
            if (forced(opts) != GN_PATH_AUTO) return GN_ERR_UNSUPPORTED;
            path = GN_PATH_GENERIC;
        }
    }
    const size_t need = fwd_ws(p, path);
    if (ws_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace)))) return GN_ERR_WORKSPACE;
    gn::FwdArgs a{x, gamma, beta, y, mean, rstd, eps, 0};
    gn::Launch l = make_launch(workspace, ws_bytes, stream, opts);
    if (l.info) *l.info = gn_plan_info{path, 0, 0, 0, 0, 0};
    return with_call_events(opts, stream, [&] {
        return path == GN_PATH_ROWS ? gn::rows_fwd(p, a, l)
             : path == GN_PATH_SLAB ? gn::slab_fwd(p, a, l)
             : path == GN_PATH_STREAM ? gn::stream_fwd(p, a, l)
                                    : gn::generic_fwd(p, gn::dense_strides(p), a, l);
    });
}

gn_status gn_backward(const void* dy, const void* x, const float* mean, const float* rstd, const float* gamma,
                      void* dx, float* dgamma, float* dbeta, int32_t mask, int64_t N, int64_t C, int64_t HW,
                      int64_t G, gn_dtype dtype, gn_layout layout, void* workspace, size_t ws_bytes,
                      void* stream, const gn_options* opts) {
    return backward_call(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, mask, N, C, HW, G, dtype, layout, workspace,
                         ws_bytes, false, stream, opts);
}

gn_status gn_backward_scratch(const void* dy, const void* x, const float* mean, const float* rstd,
                              const float* gamma, void* dx, float* dgamma, float* dbeta, int32_t mask, int64_t N,
                              int64_t C, int64_t HW, int64_t G, gn_dtype dtype, gn_layout layout, void* stream,
                              const gn_options* opts) {
    return backward_call(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, mask, N, C, HW, G, dtype, layout, nullptr,
                         0, true, stream, opts);
}

// ---- strided tensors ---------------------------------------------------------
namespace {
// Checks one tensor's element strides (n, c, h, w) against its extents; an
// output must map distinct elements to distinct addresses.  Sets `dense` to
// the mask of dense layouts the strides describe (bit 0 NCHW, bit 1 NHWC).
gn_status check_strides(const int64_t* st, const Problem& p, int64_t H, int64_t W, bool output, int* dense) {
    if (st == nullptr) return GN_ERR_INVALID;
    const int64_t ext[4] = {p.N, p.C, H, W};
    __int128 span = 0;
    for (int k = 0; k < 4; ++k) {
        if (st[k] < 0) return GN_ERR_INVALID;
        span += (__int128)(ext[k] - 1) * st[k];
    }
    if (span >= ((__int128)1 << 62)) return GN_ERR_INVALID;
    if (output) {
        // injective iff, taking dimensions of extent > 1 by increasing stride,
        // each stride exceeds the span of all smaller ones
        int idx[4], m = 0;
        for (int k = 0; k < 4; ++k)
            if (ext[k] > 1) idx[m++] = k;
        for (int i = 1; i < m; ++i)
            for (int j = i; j > 0 && st[idx[j]] < st[idx[j - 1]]; --j) std::swap(idx[j], idx[j - 1]);
        __int128 below = 0;
        for (int i = 0; i < m; ++i) {
            if ((__int128)st[idx[i]] <= below) return GN_ERR_INVALID;
            below += (__int128)(ext[idx[i]] - 1) * st[idx[i]];
        }
    }
    const int64_t nchw[4] = {p.C * p.HW, p.HW, W, 1};
    const int64_t nhwc[4] = {p.HW * p.C, 1, W * p.C, p.C};
    bool a = true, b = true;
    for (int k = 0; k < 4; ++k) {
        if (ext[k] <= 1) continue;   // the stride of an extent-1 dimension is never used
        a = a && st[k] == nchw[k];
        b = b && st[k] == nhwc[k];
    }
    *dense &= (a ? 1 : 0) | (b ? 2 : 0);
    return GN_OK;
}

gn_status strided_problem(int64_t N, int64_t C, int64_t H, int64_t W, int64_t G, gn_dtype dtype, Problem* p) {
    if (H < 0 || W < 0) return GN_ERR_INVALID;
    if (H > 0 && W > INT64_MAX / H) return GN_ERR_INVALID;
    return make_problem(N, C, H * W, G, dtype, GN_NCHW, p);
}

void copy4(int64_t* d, const int64_t* s) {
    for (int k = 0; k < 4; ++k) d[k] = s ? s[k] : 0;
}

// Resolves a forward call: GN_OK with *layout >= 0 (every tensor dense in that
// layout: use the dense entry point) or -1 with *sd filled (generic kernels).
gn_status fwd_strides(const Problem& p, int64_t H, int64_t W, const int64_t* xs, const int64_t* ys, bool has_y,
                      int* layout, gn::Strides* sd) {
    int dense = 3;
    gn_status st = check_strides(xs, p, H, W, false, &dense);
    if (st == GN_OK && has_y) st = check_strides(ys, p, H, W, true, &dense);
    if (st != GN_OK) return st;
    *layout = (dense & 1) ? GN_NCHW : (dense & 2) ? GN_NHWC : -1;
    sd->H = H;
    sd->W = W;
    copy4(sd->x, xs);
    copy4(sd->y, has_y ? ys : xs);
    copy4(sd->dy, xs);
    copy4(sd->dx, xs);
    return GN_OK;
}

gn_status bwd_strides(const Problem& p, int64_t H, int64_t W, const int64_t* dys, const int64_t* xs,
                      const int64_t* dxs, bool has_dx, int* layout, gn::Strides* sd) {
    int dense = 3;
    gn_status st = check_strides(dys, p, H, W, false, &dense);
    if (st == GN_OK) st = check_strides(xs, p, H, W, false, &dense);
    if (st == GN_OK && has_dx) st = check_strides(dxs, p, H, W, true, &dense);
    if (st != GN_OK) return st;
    *layout = (dense & 1) ? GN_NCHW : (dense & 2) ? GN_NHWC : -1;
    sd->H = H;
    sd->W = W;
    copy4(sd->x, xs);
    copy4(sd->y, xs);
    copy4(sd->dy, dys);
    copy4(sd->dx, has_dx ? dxs : xs);
    return GN_OK;
}

bool generic_allowed(const gn_options* opts) {
    const int32_t f = forced(opts);
    return f == GN_PATH_AUTO || f == GN_PATH_GENERIC;
}
}  // namespace

size_t gn_forward_strided_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t G, gn_dtype dtype,
                                         const int64_t* x_strides, const int64_t* y_strides,
                                         const gn_options* opts) {
    Problem p;
    if (strided_problem(N, C, H, W, G, dtype, &p) != GN_OK || zero_extent(p)) return 0;
    int layout;
    gn::Strides sd;
    if (fwd_strides(p, H, W, x_strides, y_strides, y_strides != nullptr, &layout, &sd) != GN_OK) return 0;
    if (layout >= 0) return gn_forward_workspace_size(N, C, H * W, G, dtype, (gn_layout)layout, opts);
    if (!generic_allowed(opts)) return 0;
    return gn::generic_fwd_ws(p, sd);
}

gn_status gn_forward_strided(const void* x, const int64_t* x_strides, const float* gamma, const float* beta,
                             void* y, const int64_t* y_strides, float* mean, float* rstd, int64_t N, int64_t C,
                             int64_t H, int64_t W, int64_t G, float eps, gn_dtype dtype, void* workspace,
                             size_t ws_bytes, void* stream, const gn_options* opts) {
    Problem p;
    gn_status st = strided_problem(N, C, H, W, G, dtype, &p);
    if (st != GN_OK) return st;
    if (!(eps >= 0.f) || isinf(eps)) return GN_ERR_INVALID;
    if ((gamma == nullptr) != (beta == nullptr)) return GN_ERR_INVALID;
    if (zero_extent(p)) {
        if (opts && opts->info) *opts->info = gn_plan_info{GN_PATH_AUTO, 0, 0, 0, 0, 0};
        return GN_OK;
    }
    if (x == nullptr || mean == nullptr || rstd == nullptr) return GN_ERR_INVALID;
    int layout;
    gn::Strides sd;
    if ((st = fwd_strides(p, H, W, x_strides, y_strides, y != nullptr, &layout, &sd)) != GN_OK) return st;
    if (layout >= 0)
        return gn_forward(x, gamma, beta, y, mean, rstd, N, C, H * W, G, eps, dtype, (gn_layout)layout, workspace,
                          ws_bytes, stream, opts);
    if (!generic_allowed(opts)) return GN_ERR_UNSUPPORTED;
    const size_t need = gn::generic_fwd_ws(p, sd);
    if (ws_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace)))) return GN_ERR_WORKSPACE;
    gn::FwdArgs a{x, gamma, beta, y, mean, rstd, eps, 0};
    gn::Launch l = make_launch(workspace, ws_bytes, stream, opts);
    if (l.info) *l.info = gn_plan_info{GN_PATH_GENERIC, 0, 0, 0, 0, 0};
    return with_call_events(opts, stream, [&] { return gn::generic_fwd(p, sd, a, l); });
}

size_t gn_backward_strided_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t G, gn_dtype dtype,
                                          const int64_t* dy_strides, const int64_t* x_strides,
                                          const int64_t* dx_strides, int32_t mask, const gn_options* opts) {
    Problem p;
    if (strided_problem(N, C, H, W, G, dtype, &p) != GN_OK || zero_extent(p)) return 0;
    if (mask <= 0 || mask > 7) return 0;
    int layout;
    gn::Strides sd;
    if (bwd_strides(p, H, W, dy_strides, x_strides, dx_strides, (mask & GN_GRAD_DX) != 0, &layout, &sd) != GN_OK)
        return 0;
    if (layout >= 0) return gn_backward_workspace_size(N, C, H * W, G, dtype, (gn_layout)layout, mask, opts);
    if (!generic_allowed(opts)) return 0;
    return gn::generic_bwd_ws(p, sd, mask);
}

gn_status gn_backward_strided(const void* dy, const int64_t* dy_strides, const void* x, const int64_t* x_strides,
                              const float* mean, const float* rstd, const float* gamma, void* dx,
                              const int64_t* dx_strides, float* dgamma, float* dbeta, int32_t mask, int64_t N,
                              int64_t C, int64_t H, int64_t W, int64_t G, gn_dtype dtype, void* workspace,
                              size_t ws_bytes, void* stream, const gn_options* opts) {
    Problem p;
    gn_status st = strided_problem(N, C, H, W, G, dtype, &p);
    if (st != GN_OK) return st;
    if (mask <= 0 || mask > 7) return GN_ERR_INVALID;
    if ((mask & GN_GRAD_DX) && dx == nullptr) return GN_ERR_INVALID;
    if ((mask & GN_GRAD_DGAMMA) && dgamma == nullptr) return GN_ERR_INVALID;
    if ((mask & GN_GRAD_DBETA) && dbeta == nullptr) return GN_ERR_INVALID;
    if ((mask & (GN_GRAD_DGAMMA | GN_GRAD_DBETA)) && gamma == nullptr) return GN_ERR_INVALID;
    if (zero_extent(p)) {
        if (opts && opts->info) *opts->info = gn_plan_info{GN_PATH_AUTO, 0, 0, 0, 0, 0};
        return GN_OK;
    }
    if (dy == nullptr || x == nullptr || mean == nullptr || rstd == nullptr) return GN_ERR_INVALID;
    int layout;
    gn::Strides sd;
    if ((st = bwd_strides(p, H, W, dy_strides, x_strides, dx_strides, (mask & GN_GRAD_DX) != 0, &layout, &sd)) !=
        GN_OK)
        return st;
    if (layout >= 0)
        return gn_backward(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, mask, N, C, H * W, G, dtype,
                           (gn_layout)layout, workspace, ws_bytes, stream, opts);
    if (!generic_allowed(opts)) return GN_ERR_UNSUPPORTED;
    const size_t need = gn::generic_bwd_ws(p, sd, mask);
    if (ws_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace)))) return GN_ERR_WORKSPACE;
    gn::BwdArgs a{dy, x, mean, rstd, gamma,
                  (mask & GN_GRAD_DX) ? dx : nullptr,
                  (mask & GN_GRAD_DGAMMA) ? dgamma : nullptr,
                  (mask & GN_GRAD_DBETA) ? dbeta : nullptr, mask, 0};
    gn::Launch l = make_launch(workspace, ws_bytes, stream, opts);
    if (l.info) *l.info = gn_plan_info{GN_PATH_GENERIC, 0, 0, 0, 0, 0};
    return with_call_events(opts, stream, [&] { return gn::generic_bwd(p, sd, a, l); });
}

// ---- RMSNorm over rows: the rows kernels with the mean taken as 0 ----------
namespace {
// Rows problem of an [N, C] tensor; GN_OK, or the status to return.
gn_status rms_problem(int64_t N, int64_t C, int64_t G, gn_dtype dtype, const gn_options* opts, Problem* p) {
    gn_status st = make_problem(N, C, 1, G, dtype, GN_NCHW, p);
    if (st != GN_OK) return st;
    const int32_t f = forced(opts);
    if (f != GN_PATH_AUTO && f != GN_PATH_ROWS) return GN_ERR_UNSUPPORTED;
    if (!zero_extent(*p) && !gn::rows_ok(*p)) return GN_ERR_UNSUPPORTED;
    return GN_OK;
}
}  // namespace

size_t gn_rms_forward_workspace_size(int64_t N, int64_t C, int64_t G, gn_dtype dtype, const gn_options* opts) {
    Problem p;
    if (rms_problem(N, C, G, dtype, opts, &p) != GN_OK || zero_extent(p)) return 0;
    return gn::rows_fwd_ws(p);
}

gn_status gn_rms_forward(const void* x, const float* gamma, void* y, float* rstd, int64_t N, int64_t C, int64_t G,
                         float eps, gn_dtype dtype, void* workspace, size_t ws_bytes, void* stream,
                         const gn_options* opts) {
    Problem p;
    gn_status st = rms_problem(N, C, G, dtype, opts, &p);
    if (st != GN_OK) return st;
    if (!(eps >= 0.f) || isinf(eps)) return GN_ERR_INVALID;
    if (zero_extent(p)) {
        if (opts && opts->info) *opts->info = gn_plan_info{GN_PATH_AUTO, 0, 0, 0, 0, 0};
        return GN_OK;
    }
    if (x == nullptr || rstd == nullptr) return GN_ERR_INVALID;
    if (!aligned16(x) || (y != nullptr && !aligned16(y)) || !aligned16(gamma)) return GN_ERR_UNSUPPORTED;
    const size_t need = gn::rows_fwd_ws(p);
    if (ws_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace)))) return GN_ERR_WORKSPACE;
    gn::FwdArgs a{x, gamma, nullptr, y, nullptr, rstd, eps, 1};
    gn::Launch l = make_launch(workspace, ws_bytes, stream, opts);
    if (l.info) *l.info = gn_plan_info{GN_PATH_ROWS, 0, 0, 0, 0, 0};
    return with_call_events(opts, stream, [&] { return gn::rows_fwd(p, a, l); });
}

size_t gn_rms_backward_workspace_size(int64_t N, int64_t C, int64_t G, gn_dtype dtype, int32_t mask,
                                      const gn_options* opts) {
    Problem p;
    if (rms_problem(N, C, G, dtype, opts, &p) != GN_OK || zero_extent(p)) return 0;
    if (mask <= 0 || mask > (GN_GRAD_DX | GN_GRAD_DGAMMA)) return 0;
    return gn::rows_bwd_ws(p, mask);
}

gn_status gn_rms_backward(const void* dy, const void* x, const float* rstd, const float* gamma, void* dx,
                          float* dgamma, int32_t mask, int64_t N, int64_t C, int64_t G, gn_dtype dtype,
                          void* workspace, size_t ws_bytes, void* stream, const gn_options* opts) {
    Problem p;
    gn_status st = rms_problem(N, C, G, dtype, opts, &p);
    if (st != GN_OK) return st;
    if (mask <= 0 || mask > (GN_GRAD_DX | GN_GRAD_DGAMMA)) return GN_ERR_INVALID;   // no dbeta: no bias
    if ((mask & GN_GRAD_DX) && dx == nullptr) return GN_ERR_INVALID;
    if ((mask & GN_GRAD_DGAMMA) && (dgamma == nullptr || gamma == nullptr)) return GN_ERR_INVALID;
    if (zero_extent(p)) {
        if (opts && opts->info) *opts->info = gn_plan_info{GN_PATH_AUTO, 0, 0, 0, 0, 0};
        return GN_OK;
    }
    if (dy == nullptr || x == nullptr || rstd == nullptr) return GN_ERR_INVALID;
    if (!aligned16(dy) || !aligned16(x) || !aligned16(gamma) || ((mask & GN_GRAD_DX) && !aligned16(dx)))
        return GN_ERR_UNSUPPORTED;
    const size_t need = gn::rows_bwd_ws(p, mask);
    if (ws_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace)))) return GN_ERR_WORKSPACE;
    gn::BwdArgs a{dy, x, nullptr, rstd, gamma,
                  (mask & GN_GRAD_DX) ? dx : nullptr,
                  (mask & GN_GRAD_DGAMMA) ? dgamma : nullptr,
                  nullptr, mask, 1};
    gn::Launch l = make_launch(workspace, ws_bytes, stream, opts);
    if (l.info) *l.info = gn_plan_info{GN_PATH_ROWS, 0, 0, 0, 0, 0};
    return with_call_events(opts, stream, [&] { return gn::rows_bwd(p, a, l); });
}

gn_status gn_read_status(uint32_t* status_word, void* stream, int32_t reset, uint32_t* word_out) {
    if (status_word == nullptr) return GN_ERR_INVALID;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) {
        (void)hipGetLastError();
        return GN_ERR_HIP;
    }
    uint32_t w = 0;
    if (hipMemcpy(&w, status_word, sizeof(w), hipMemcpyDeviceToHost) != hipSuccess) {
        (void)hipGetLastError();
        return GN_ERR_HIP;
    }
    if (word_out) *word_out = w;
    if (reset) {
        const uint32_t zero = 0;
        if (hipMemcpy(status_word, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipGetLastError();
            return GN_ERR_HIP;
        }
    }
    return (w & GN_STATUS_WAIT_EXPIRED) ? GN_ERR_WAIT : GN_OK;
}

int32_t gn_cooperative_state(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return GN_COOP_NOT_TRIED;
    }
    std::lock_guard<std::mutex> lk(g_coop_mu);
    return g_coop_done[dev] ? GN_COOP_ACCEPTED : g_coop_refused[dev] ? GN_COOP_REFUSED : GN_COOP_NOT_TRIED;
}

const char* gn_status_string(gn_status s) {
    switch (s) {
        case GN_OK: return "ok";
        case GN_ERR_INVALID: return "invalid argument";
        case GN_ERR_UNSUPPORTED: return "unsupported dtype, layout or forced path";
        case GN_ERR_WORKSPACE: return "workspace too small";
        case GN_ERR_HIP: return "HIP launch failed";
        case GN_ERR_WAIT: return "a bounded wait between cooperating workgroups gave up; the call's outputs are NaN where affected";
        default: return "unknown status";
    }
}

int32_t gn_version(void) { return 400; }

}  // extern "C"
