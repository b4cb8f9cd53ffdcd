/*
 * gn.h -- C ABI of the GroupNorm forward/backward library for AMD Instinct
 * MI355X (gfx950).
 *
 * Operation (POPCORNBENCH GroupNorm trace; baracuda-kernels GroupNorm backward
 * plan; apex PR #2018).  A dense activation tensor has N samples, C channels
 * and HW spatial positions (all spatial dimensions flattened).  The C channels
 * form G groups of D = C/G consecutive channels; a slice (n, g) holds the
 * M = D*HW elements of sample n in group g.
 *
 *   forward:  mean = average of the slice, var = biased variance (denominator
 *             M), rstd = 1/sqrt(var + eps), xhat = (x - mean)*rstd,
 *             y = gamma_c*xhat + beta_c.  mean and rstd are saved per slice.
 *   backward: with the saved mean/rstd, per slice A = sum gamma_c*dy and
 *             B = sum gamma_c*dy*xhat;  dx = rstd*(gamma_c*dy - A/M - xhat*B/M);
 *             dgamma_c = sum over n, p of dy*xhat;  dbeta_c = sum over n, p of dy.
 *
 * Memory layout of x, y, dy, dx (dense, element (n, c, p)):
 *   GN_NCHW: offset (n*C + c)*HW + p
 *   GN_NHWC: offset (n*HW + p)*C + c          (PyTorch channels_last)
 * Activations are float32, float16 or bfloat16 (IEEE binary16 / bfloat16
 * bit patterns); y and dx take x's dtype, rounded to nearest even.  gamma,
 * beta, dgamma, dbeta, mean and rstd are float32.  mean/rstd have N*G entries,
 * slice (n, g) at index n*G + g.  All arithmetic inside is float32.
 *
 * Ownership: every pointer argument except `opts` is a DEVICE pointer owned by
 * the caller; the library allocates and frees nothing.  Work is enqueued on
 * `stream` (a hipStream_t; NULL is the null stream) and the calls return
 * before it completes.  The workspace is borrowed until that work ends.
 * Once per process and device, the first call whose stream is not capturing
 * a graph also enqueues one empty one-workgroup cooperative launch ahead of
 * its own kernels (GN_EARLY_COOP=0 in the environment leaves it out): the HIP
 * runtime fixes a state at a process's first cooperative launch, and when
 * that launch comes after several captured multi-node graphs, all later
 * cooperative launches of the process run about three times slower.  While a process that has made cooperative launches
 * runs, the runtime refuses them to other processes on the device; a slab
 * call whose cooperative launch is refused takes the split form or the
 * generic kernels instead (same results within the tolerances; gn_plan_info
 * reports what ran).  Under stream capture a refusal would only show at
 * replay, as a kernel silently skipped, so a call captured before this
 * process has had a cooperative launch accepted records those kernels too.
 *
 * Determinism: every reduction runs in a fixed order and no float atomics are
 * used, so repeated calls with the same inputs and options give bitwise equal
 * results on the same device (baracuda-kernels GroupNorm backward plan,
 * precision guarantee: fp32 math and accumulators, deterministic).
 *
 * Errors are detected on the host, before anything is enqueued, and reported
 * by the return value; nothing is written to any output then.  A zero extent
 * (N, C or HW equal to 0) is a successful no-op (baracuda-kernels plan: run
 * returns early on a zero extent).
 */
#ifndef GN_MI355X_H
#define GN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gn_status {
    GN_OK = 0,
    GN_ERR_INVALID = 1,      /* bad sizes, G not dividing C, NULL where required,
                                affine pointers not all-or-none, bad mask */
    GN_ERR_UNSUPPORTED = 2,  /* dtype or layout outside the enums, or a forced
                                path that cannot serve these arguments */
    GN_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the size query returned */
    GN_ERR_HIP = 4,          /* the HIP runtime refused a launch */
    GN_ERR_WAIT = 5          /* reported by gn_read_status only: a bounded wait
                                between cooperating workgroups gave up (see
                                gn_options.status_word) */
} gn_status;

typedef enum gn_dtype { GN_F32 = 0, GN_F16 = 1, GN_BF16 = 2 } gn_dtype;

typedef enum gn_layout { GN_NCHW = 0, GN_NHWC = 1 } gn_layout;

/* Output mask of gn_backward (ROCm/pytorch PR #3564 tests: output_mask
 * selecting dgamma and dbeta, dbeta only, dgamma only). */
enum { GN_GRAD_DX = 1, GN_GRAD_DGAMMA = 2, GN_GRAD_DBETA = 4 };

/* Kernel families; GN_PATH_AUTO lets the planner choose. */
typedef enum gn_path {
    GN_PATH_AUTO = 0,
    GN_PATH_GENERIC = 1,  /* any shape, alignment or strides: partial sums, finalize,
                             elementwise */
    GN_PATH_ROWS = 2,     /* HW == 1: one wavefront per slice, slice kept in registers */
    GN_PATH_SLAB = 3,     /* cooperative capped grid over contiguous slabs with
                             grid-stride overflow tiles (one-pass backward);
                             NCHW slabs of up to 256 KiB (no
                             max_resident_override) take one workgroup each
                             instead (team 1, a normal launch), and NCHW
                             tensors of up to 32 MiB (forward) or 64 MiB
                             (backward) a two-launch split form (team 0) */
    GN_PATH_STREAM = 4    /* NHWC: a few launches of one tile per workgroup
                             (statistics, fixed-order combine, outputs), or one
                             workgroup per sample when a sample fits one tile;
                             the planner's choice for every NHWC shape it takes
                             (the slab path serves NHWC when forced, or past
                             the stream grid limits) */
} gn_path;

/* What a call ran (filled when gn_options.info is not NULL). */
typedef struct gn_plan_info {
    int32_t path;            /* gn_path actually used */
    int32_t kernels;         /* kernel launches enqueued by the call */
    int64_t grid;            /* workgroups of the main kernel */
    int64_t tiles;           /* work tiles of the main kernel (slab path) */
    int64_t resident_cap;    /* co-resident workgroup limit used for the cap */
    int64_t team;            /* workgroups cooperating on one slab (slab path) */
} gn_plan_info;

/* Bit that the kernels OR into gn_options.status_word when a bounded wait
 * gives up. */
#define GN_STATUS_WAIT_EXPIRED 1u

/* gn_options.debug_flags: GN_DEBUG_UNMET_WAITS raises the target of every
 * wait between cooperating workgroups out of reach, so that each of them
 * expires after spin_limit polls -- for tests of the failure report only. */
#define GN_DEBUG_UNMET_WAITS 1u
/* gn_options.debug_flags: GN_DEBUG_STREAM_SPLIT keeps the stream path (NHWC)
 * in its full multi-kernel form (tile statistics, finalize, apply; tile sums,
 * column sums, per-group terms, dx) also where one workgroup per sample would
 * take the whole call or the output kernels would combine a few tiles'
 * partials themselves -- for tests of that form only. */
#define GN_DEBUG_STREAM_SPLIT 2u
/* gn_options.debug_flags: GN_DEBUG_SLAB_COOP keeps the slab path on its
 * cooperative kernels at the natural residency cap also where the
 * one-workgroup-per-slab kernels or the split form would run -- for tests of
 * the cooperative kernels only. */
#define GN_DEBUG_SLAB_COOP 4u

/* Optional knobs (pass NULL for defaults).
 *
 * Failure report of the cooperative (slab) kernels.  Their workgroups
 * exchange partial results inside one launch (apex PR #2018, Solution: a
 * cooperative grid capped at the residency limit, so that every workgroup is
 * resident and the global reduction can complete).  Every such wait is
 * bounded: if the co-residency the launch guarantees were ever broken, a
 * waiting workgroup gives up after spin_limit polls instead of hanging,
 * ORs GN_STATUS_WAIT_EXPIRED into *status_word, and writes NaN to every
 * output it would have derived from the incomplete exchange (y or dx
 * elements, mean/rstd, dgamma/dbeta): no finite wrong value is written.
 * The call itself has already returned GN_OK (it returns before the
 * kernels run), so the report is read afterwards with gn_read_status. */
typedef struct gn_options {
    int32_t force_path;             /* gn_path; GN_PATH_AUTO = planner's choice */
    int32_t max_resident_override;  /* > 0: cap the cooperative grid at this many
                                       workgroups (forces overflow tiles) */
    gn_plan_info* info;             /* host pointer, may be NULL */
    void* event_begin;              /* hipEvent_t recorded on `stream` before the
                                       call's first kernel, or NULL */
    void* event_end;                /* hipEvent_t recorded after its last kernel, or NULL */
    void* kernel_begin;             /* hipEvent_t recorded right before the call's
                                       main kernel (GN_PATH_STREAM and
                                       GN_PATH_GENERIC: before the first kernel), or NULL */
    void* kernel_end;               /* recorded right after it (GN_PATH_STREAM and
                                       GN_PATH_GENERIC: after the last kernel), or NULL */
    uint32_t* status_word;          /* DEVICE pointer to one 32-bit word, or NULL:
                                       the kernels OR GN_STATUS_WAIT_EXPIRED into it
                                       when a wait gives up; never cleared by the
                                       library (the caller zeroes it) */
    uint32_t spin_limit;            /* polls before a wait gives up; 0 = default (2^20;
                                       a poll follows a sleep of 0.1 to 3.4 us,
                                       so the default gives up within seconds) */
    uint32_t debug_flags;           /* 0, or GN_DEBUG_* bits (tests only) */
} gn_options;

/* Workspace bytes gn_forward needs for these arguments (0 is possible).
 * Returns 0 as well for arguments gn_forward would reject. */
size_t gn_forward_workspace_size(int64_t N, int64_t C, int64_t HW, int64_t G,
                                 gn_dtype dtype, gn_layout layout,
                                 const gn_options* opts);

/*
 * Forward.  x: input; gamma, beta: [C] float32, both NULL (no affine: gamma 1,
 * beta 0) or both set; y: output (may be NULL to compute only the statistics);
 * mean, rstd: [N*G] float32 outputs (required).  eps >= 0.
 * workspace: 16-byte aligned device buffer of at least gn_forward_workspace_size() bytes
 * (may be NULL when that size is 0); its content on entry is irrelevant.
 */
gn_status gn_forward(const void* x, const float* gamma, const float* beta,
                     void* y, float* mean, float* rstd,
                     int64_t N, int64_t C, int64_t HW, int64_t G, float eps,
                     gn_dtype dtype, gn_layout layout,
                     void* workspace, size_t ws_bytes, void* stream,
                     const gn_options* opts);

/* Workspace bytes gn_backward needs for these arguments and mask. */
size_t gn_backward_workspace_size(int64_t N, int64_t C, int64_t HW, int64_t G,
                                  gn_dtype dtype, gn_layout layout, int32_t mask,
                                  const gn_options* opts);

/*
 * Backward.  dy, x: inputs in the same dtype/layout; mean, rstd: [N*G] saved
 * statistics of the forward; gamma: [C] or NULL (gamma = 1).
 * mask: OR of GN_GRAD_DX / GN_GRAD_DGAMMA / GN_GRAD_DBETA (non-zero); each
 * selected output must be non-NULL: dx (x's shape and dtype), dgamma [C],
 * dbeta [C] (float32).  dgamma/dbeta require gamma (affine all-or-none, as in
 * the baracuda-kernels plan's argument check).
 */
gn_status gn_backward(const void* dy, const void* x,
                      const float* mean, const float* rstd, const float* gamma,
                      void* dx, float* dgamma, float* dbeta, int32_t mask,
                      int64_t N, int64_t C, int64_t HW, int64_t G,
                      gn_dtype dtype, gn_layout layout,
                      void* workspace, size_t ws_bytes, void* stream,
                      const gn_options* opts);

/* Size of the static device array behind gn_backward_scratch (bytes). */
#define GN_SCRATCH_BYTES (32u << 20)

/*
 * gn_backward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The library's own workspace is a static device array
 * of GN_SCRATCH_BYTES (32 MiB), one per device the library runs on, held until
 * the process ends; the call allocates nothing and calls no allocating
 * routine.  Returns GN_ERR_WORKSPACE, before anything is enqueued, when the
 * call would need more than that (gn_backward_workspace_size for the same
 * arguments above GN_SCRATCH_BYTES; e.g. the generic path's partials for
 * large unaligned or oddly shaped tensors), and GN_ERR_HIP when the array's
 * device address cannot be obtained (the first call on each device looks it
 * up, with that device current).  Every call on one device shares that
 * device's array, and each call re-initialises what it needs of it: calls
 * whose work overlaps on one device (other streams, other host threads)
 * race and give undefined results -- serialise them.  Inputs, outputs,
 * options, errors and results are those of gn_backward.
 */
gn_status gn_backward_scratch(const void* dy, const void* x,
                              const float* mean, const float* rstd, const float* gamma,
                              void* dx, float* dgamma, float* dbeta, int32_t mask,
                              int64_t N, int64_t C, int64_t HW, int64_t G,
                              gn_dtype dtype, gn_layout layout, void* stream,
                              const gn_options* opts);

/* The path gn_forward (backward = 0) or gn_backward (backward = 1) would take
 * for these arguments, without enqueuing anything.  Returns a gn_path, or -1
 * for arguments the call would reject. */
int32_t gn_select_path(int32_t backward, int64_t N, int64_t C, int64_t HW, int64_t G,
                       gn_dtype dtype, gn_layout layout, const gn_options* opts);

/*
 * Strided tensors (ROCm/pytorch PR #3564's test run includes a correctness
 * test on non-contiguous input; the POPCORNBENCH GroupNorm trace weighs
 * reading arbitrary strides against copying the input first, and keeps a
 * scalar path for shapes its vector loads do not fit).  The same operation
 * on tensors of logical
 * shape (N, C, H, W) whose element (n, c, h, w) sits at offset
 *     n*s[0] + c*s[1] + h*s[2] + w*s[3]      (elements, not bytes)
 * from the tensor's pointer, for a host array s[4] of strides per tensor:
 * slices, crops, permuted and broadcast views are read and written where
 * they are, without a copy.  Strides must be non-negative and the largest
 * offset below 2^62; input tensors may overlap themselves (a stride of 0
 * broadcasts), an output must map distinct elements to distinct addresses
 * (GN_ERR_INVALID otherwise).  Outputs must not overlap inputs.  The stride
 * arrays are read during the call only.
 *
 * When every tensor of the call is dense in one layout (NCHW or NHWC, the
 * strides of extent-1 dimensions ignored), the call is exactly gn_forward /
 * gn_backward with HW = H*W and that layout, fast paths and forced paths
 * included.  Otherwise it runs the generic kernels (plan info: GN_PATH_GENERIC;
 * a forced path other than GN_PATH_GENERIC is GN_ERR_UNSUPPORTED), which take
 * any alignment.  Everything else -- dtypes, mean/rstd, gamma/beta, mask,
 * workspace, stream, errors, determinism -- is as for gn_forward / gn_backward.
 */

/* Workspace bytes gn_forward_strided needs; y_strides NULL when y will be
 * NULL.  0 for arguments the call would reject. */
size_t gn_forward_strided_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t G,
                                         gn_dtype dtype, const int64_t* x_strides,
                                         const int64_t* y_strides, const gn_options* opts);

/* x with strides x_strides (required); y with y_strides (ignored when y is
 * NULL); mean, rstd: [N*G]; other arguments as for gn_forward. */
gn_status gn_forward_strided(const void* x, const int64_t* x_strides,
                             const float* gamma, const float* beta,
                             void* y, const int64_t* y_strides, float* mean, float* rstd,
                             int64_t N, int64_t C, int64_t H, int64_t W, int64_t G, float eps,
                             gn_dtype dtype, void* workspace, size_t ws_bytes, void* stream,
                             const gn_options* opts);

/* Workspace bytes gn_backward_strided needs; dx_strides may be NULL when the
 * mask has no GN_GRAD_DX. */
size_t gn_backward_strided_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W, int64_t G,
                                          gn_dtype dtype, const int64_t* dy_strides,
                                          const int64_t* x_strides, const int64_t* dx_strides,
                                          int32_t mask, const gn_options* opts);

/* dy, x with their strides (required); dx with dx_strides (required with
 * GN_GRAD_DX); other arguments as for gn_backward. */
gn_status gn_backward_strided(const void* dy, const int64_t* dy_strides,
                              const void* x, const int64_t* x_strides,
                              const float* mean, const float* rstd, const float* gamma,
                              void* dx, const int64_t* dx_strides, float* dgamma, float* dbeta,
                              int32_t mask, int64_t N, int64_t C, int64_t H, int64_t W, int64_t G,
                              gn_dtype dtype, void* workspace, size_t ws_bytes, void* stream,
                              const gn_options* opts);

/*
 * RMSNorm over rows (ROCm/pytorch PR #3564 benchmarks an rms_norm operator
 * beside layer_norm; read as PyTorch's rms_norm).  x is a dense [N, C] row
 * major tensor (one row per sample; no spatial extent); each row is split
 * into G groups of D = C/G consecutive channels (G = 1: the whole row), and
 * every (n, g) segment is normalised by its root mean square:
 *     rstd = 1/sqrt((1/D) * sum x^2 + eps),   y = gamma_c * x * rstd
 * backward, per segment B = sum gamma_c * dy * x * rstd:
 *     dx = rstd * (gamma_c * dy - x * rstd * B/D),   dgamma_c = sum over n of dy * x * rstd
 * rstd: [N*G] float32, segment (n, g) at n*G + g (saved by the forward, read
 * by the backward).  gamma: [C] float32 or NULL (= 1); there is no bias.
 * dtypes as for gn_forward; y, dx take x's dtype.  These calls run on the
 * rows kernels only: they return GN_ERR_UNSUPPORTED when D or C is not a
 * multiple of 4 (float32) / 8 (16-bit) elements, when D exceeds 8192
 * (float32) / 16384 (16-bit) channels, when a pointer is not 16-byte aligned,
 * or for a forced path other than GN_PATH_ROWS.  Pointers, streams,
 * workspace, options and errors as for gn_forward / gn_backward.
 */
size_t gn_rms_forward_workspace_size(int64_t N, int64_t C, int64_t G, gn_dtype dtype,
                                     const gn_options* opts);

/* x, y: [N, C]; y may be NULL (rstd only); rstd required. eps >= 0. */
gn_status gn_rms_forward(const void* x, const float* gamma, void* y, float* rstd,
                         int64_t N, int64_t C, int64_t G, float eps, gn_dtype dtype,
                         void* workspace, size_t ws_bytes, void* stream,
                         const gn_options* opts);

/* Workspace bytes gn_rms_backward needs for these arguments and mask. */
size_t gn_rms_backward_workspace_size(int64_t N, int64_t C, int64_t G, gn_dtype dtype,
                                      int32_t mask, const gn_options* opts);

/* dy, x: [N, C]; rstd: [N*G] from gn_rms_forward; gamma: [C] or NULL.
 * mask: GN_GRAD_DX and/or GN_GRAD_DGAMMA (GN_GRAD_DBETA is invalid: there is
 * no bias); each selected output non-NULL; dgamma requires gamma. */
gn_status gn_rms_backward(const void* dy, const void* x, const float* rstd, const float* gamma,
                          void* dx, float* dgamma, int32_t mask,
                          int64_t N, int64_t C, int64_t G, gn_dtype dtype,
                          void* workspace, size_t ws_bytes, void* stream,
                          const gn_options* opts);

/* Reads a status word that calls of this library OR their failure reports
 * into (gn_options.status_word): waits for all work queued on `stream`
 * (hipStreamSynchronize), copies the word to the host, and returns GN_OK
 * when it is 0, GN_ERR_WAIT when it holds GN_STATUS_WAIT_EXPIRED, or
 * GN_ERR_HIP when the synchronisation or the copy fails.  reset != 0 zeroes
 * the word afterwards (a blocking copy).  *word_out (host pointer, may be
 * NULL) receives the word as read.  Not for use under stream capture. */
gn_status gn_read_status(uint32_t* status_word, void* stream, int32_t reset, uint32_t* word_out);

/* The state of this process's cooperative launches on the current device,
 * for callers that want to know why slab calls take the split or generic
 * kernels: GN_COOP_NOT_TRIED (no call has made the early empty cooperative
 * launch yet, or GN_EARLY_COOP=0 leaves it out), GN_COOP_ACCEPTED (the
 * runtime accepted it: the cooperative kernels run, eagerly and under
 * capture), GN_COOP_REFUSED (the runtime refused it, e.g. while another
 * process that has made cooperative launches runs on the device; later
 * calls try again).  Host only; enqueues nothing. */
enum { GN_COOP_NOT_TRIED = 0, GN_COOP_ACCEPTED = 1, GN_COOP_REFUSED = 2 };
int32_t gn_cooperative_state(void);

/* Static description of a status code (never NULL). */
const char* gn_status_string(gn_status status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t gn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GN_MI355X_H */
