// gn_internal.hpp -- host-side interfaces between the C ABI (gn_api.cpp) and
// the kernel launchers of each path.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gn.h"

namespace gn {

// One GroupNorm problem, validated by the C ABI.
struct Problem {
    int64_t N, C, HW, G;
    int64_t D;       // channels per group, C/G
    int64_t M;       // elements per slice, D*HW
    int64_t S;       // slices, N*G
    int64_t E;       // elements, N*C*HW
    gn_dtype dtype;
    gn_layout layout;
    int elem_bytes;  // 4 or 2
};

struct FwdArgs {
    const void* x;
    const float* gamma;  // NULL => 1
    const float* beta;   // NULL => 0
    void* y;             // NULL => statistics only
    float* mean;         // NULL for RMSNorm
    float* rstd;
    float eps;
    int32_t rms;         // RMSNorm over rows (rows path only): no mean, no beta
};

struct BwdArgs {
    const void* dy;
    const void* x;
    const float* mean;
    const float* rstd;
    const float* gamma;  // NULL => 1
    void* dx;            // NULL unless GN_GRAD_DX
    float* dgamma;       // NULL unless GN_GRAD_DGAMMA
    float* dbeta;        // NULL unless GN_GRAD_DBETA
    int32_t mask;
    int32_t rms;         // RMSNorm over rows (rows path only): mean unused, no mean term
};

// Launch context handed to every launcher.
struct Launch {
    hipStream_t stream;
    void* ws;              // device workspace (may be NULL when its size is 0)
    size_t ws_bytes;
    hipEvent_t ev_begin;   // recorded around the main kernel when not NULL (the
    hipEvent_t ev_end;     // C ABI records the whole-call events itself)
    int32_t max_resident_override;
    gn_plan_info* info;    // may be NULL
    uint32_t* status_word; // device word for failure reports, or NULL
    uint32_t spin_limit;   // polls before a bounded wait gives up (never 0)
    uint32_t unmet_waits;  // 1: every wait's target out of reach (failure-report tests)
    uint32_t stream_split;  // 1: the stream path's full multi-kernel form, no fused forms (tests)
    uint32_t slab_coop;     // 1: the slab path's cooperative kernels only (tests)
};

// Polls before a bounded wait between workgroups gives up: 2^20 polls, each
// after a sleep of 128 to 8128 clocks depending on the wait (about 0.1 to 3.4
// us), i.e. at most a few seconds -- far above the longest legitimate wait of
// a few milliseconds.
constexpr uint32_t kDefaultSpinLimit = 1u << 20;

// Device facts used by the planner (queried once per device).
struct DeviceInfo {
    int device;
    int cu_count;
    int coop_supported;
};
const DeviceInfo& device_info();

// Whether this process's runtime has accepted a cooperative launch on the
// current device (the library's early one, gn_api.cpp): it then keeps the
// cooperative state for the process, and later cooperative launches, eager or
// recorded into a graph, are not refused.
bool coop_accepted();

// Records ev (if any) on the stream; returns hipSuccess or the error.
hipError_t record(hipEvent_t ev, hipStream_t s);

// Element strides of each activation tensor, indexed 0 n, 1 c, 2 h, 3 w, over
// a spatial extent H x W (H*W == Problem::HW).  Validated by the C ABI: non-
// negative, offsets within int64, outputs free of self-overlap.
struct Strides {
    int64_t H, W;
    int64_t x[4], y[4], dy[4], dx[4];
};

// The strides of the dense layout p.layout (H = 1, W = HW) for every tensor.
Strides dense_strides(const Problem& p);

// ---- generic path: any shape, strides and alignment --------------------------
size_t generic_fwd_ws(const Problem& p, const Strides& s);
size_t generic_bwd_ws(const Problem& p, const Strides& s, int32_t mask);
hipError_t generic_fwd(const Problem& p, const Strides& s, const FwdArgs& a, const Launch& l);
hipError_t generic_bwd(const Problem& p, const Strides& s, const BwdArgs& a, const Launch& l);

// ---- rows path: HW == 1, one wavefront per slice ----------------------------
bool rows_ok(const Problem& p);   // shape condition (alignment checked separately)
size_t rows_fwd_ws(const Problem& p);
size_t rows_bwd_ws(const Problem& p, int32_t mask);
hipError_t rows_fwd(const Problem& p, const FwdArgs& a, const Launch& l);
hipError_t rows_bwd(const Problem& p, const BwdArgs& a, const Launch& l);

// ---- slab path: cooperative capped grid over contiguous slabs ---------------
bool slab_ok(const Problem& p);   // shape condition (alignment checked separately)
size_t slab_fwd_ws(const Problem& p);
size_t slab_bwd_ws(const Problem& p, int32_t mask);
hipError_t slab_fwd(const Problem& p, const FwdArgs& a, const Launch& l);
hipError_t slab_bwd(const Problem& p, const BwdArgs& a, const Launch& l);

// ---- stream path: NHWC as a few launches of one tile per workgroup ----------
bool stream_ok(const Problem& p);
size_t stream_fwd_ws(const Problem& p);
size_t stream_bwd_ws(const Problem& p, int32_t mask);
hipError_t stream_fwd(const Problem& p, const FwdArgs& a, const Launch& l);
hipError_t stream_bwd(const Problem& p, const BwdArgs& a, const Launch& l);

}  // namespace gn
