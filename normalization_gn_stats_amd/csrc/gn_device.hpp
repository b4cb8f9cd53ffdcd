// gn_device.hpp -- device helpers shared by the GroupNorm kernels (gfx950, wave64).
//
// * 16-byte vector IO of float32 / float16 / bfloat16 activations with
//   conversion to float32 and back (round to nearest even, the hardware
//   v_cvt_pk_* conversions);
// * wavefront and workgroup sums in a fixed order (bitwise reproducible);
// * mean/M2 statistics merged with Chan, Golub and LeVeque's pairwise update
//   ("Algorithms for computing the sample variance", 1983), operands always
//   taken in a canonical order so that every lane agrees bitwise;
// * an arrival-counter barrier for co-resident workgroups whose exchanged
//   values travel through agent-scope atomics (no whole-L2 write-back or
//   invalidate), bounded so that no wave can spin forever.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gn {

constexpr int kWave = 64;

typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f8v __attribute__((ext_vector_type(8)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// element traits: V elements per 16-byte vector
// ---------------------------------------------------------------------------
template <typename T> struct Vec;

template <> struct Vec<float> {
    static constexpr int V = 4;
    __device__ static inline void load(const float* p, float (&o)[4]) {
        f4v v = *reinterpret_cast<const f4v*>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    __device__ static inline void unpack(const u4v& raw, float (&o)[4]) {
        f4v v = __builtin_bit_cast(f4v, raw);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    __device__ static inline u4v pack(const float (&o)[4]) {
        f4v v = {o[0], o[1], o[2], o[3]};
        return __builtin_bit_cast(u4v, v);
    }
    __device__ static inline float to_f(float v) { return v; }
    __device__ static inline float from_f(float v) { return v; }
};

template <> struct Vec<_Float16> {
    static constexpr int V = 8;
    __device__ static inline void unpack(const u4v& raw, float (&o)[8]) {
        f8v f = __builtin_convertvector(__builtin_bit_cast(h8v, raw), f8v);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = f[k];
    }
    __device__ static inline u4v pack(const float (&o)[8]) {
        f8v f;
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = o[k];
        return __builtin_bit_cast(u4v, __builtin_convertvector(f, h8v));
    }
    __device__ static inline float to_f(_Float16 v) { return (float)v; }
    __device__ static inline _Float16 from_f(float v) { return (_Float16)v; }
};

template <> struct Vec<__bf16> {
    static constexpr int V = 8;
    __device__ static inline void unpack(const u4v& raw, float (&o)[8]) {
        f8v f = __builtin_convertvector(__builtin_bit_cast(b8v, raw), f8v);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = f[k];
    }
    __device__ static inline u4v pack(const float (&o)[8]) {
        f8v f;
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = o[k];
        return __builtin_bit_cast(u4v, __builtin_convertvector(f, b8v));
    }
    __device__ static inline float to_f(__bf16 v) { return (float)v; }
    __device__ static inline __bf16 from_f(float v) { return (__bf16)v; }
};

__device__ inline u4v ld16(const void* p) { return *reinterpret_cast<const u4v*>(p); }
// Streaming load for activations: on MI355X a second read of a buffer gains
// nothing from the caches at these sizes, and the non-temporal hint raises
// the rate of a large read stream (about 6.2 -> 7.0 TB/s measured) and of a
// read-and-write stream (5.8 -> 6.4 TB/s, together with streaming stores).
#ifndef GN_NT_LOADS
#define GN_NT_LOADS 1
#endif
__device__ inline u4v ld16_nt(const void* p) {
#if GN_NT_LOADS
    return __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
#else
    return ld16(p);
#endif
}
__device__ inline void st16(void* p, const u4v& v) { *reinterpret_cast<u4v*>(p) = v; }
// Streaming store for outputs that are not read again by the kernel.
#ifndef GN_NT_STORES
#define GN_NT_STORES 1
#endif
__device__ inline void st16_nt(void* p, const u4v& v) {
#if GN_NT_STORES
    __builtin_nontemporal_store(v, reinterpret_cast<u4v*>(p));
#else
    st16(p, v);
#endif
}

// ---------------------------------------------------------------------------
// fixed-order reductions
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp_f(float v) {
    return __builtin_bit_cast(float,
        __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ inline float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes; every lane receives the same bits.  Steps: lane
// pairs, quads, half-rows and rows through DPP (each step adds a lane and its
// mirror, which is commutative and hence identical on both), then the four
// row sums combined as (r0 + r1) + (r2 + r3).
__device__ inline float wave_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Sum over lanes that are congruent modulo `stride` (stride a power of two,
// 1..32): lanes l, l+stride, l+2*stride, ... all receive the same bits.
__device__ inline float wave_sum_strided(float v, int stride) {
    for (int off = stride; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Workgroup sum of NV values per thread; `lds` holds NWAVES*NV floats.  All
// threads receive the same bits.  Contains __syncthreads (call uniformly).
template <int NV, int NWAVES>
__device__ inline void block_sum(float (&v)[NV], float* lds) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = wave_sum(v[k]);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < NV; ++k) lds[wave * NV + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        float s = lds[k];
#pragma unroll
        for (int w = 1; w < NWAVES; ++w) s += lds[w * NV + k];
        v[k] = s;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// (count, mean, M2) statistics
// ---------------------------------------------------------------------------
struct Stat {
    float n;     // element count (exact: counts stay far below 2^24 per merge operand
                 // only where noted; the merge uses the ratio, so large counts are fine)
    float mean;
    float m2;    // sum of squared deviations from mean
};

__device__ inline Stat stat_empty() { return Stat{0.f, 0.f, 0.f}; }

// Chan et al. pairwise merge; a is the "left" operand.
__device__ inline Stat stat_merge(const Stat& a, const Stat& b) {
    const float n = a.n + b.n;
    if (b.n == 0.f) return a;
    if (a.n == 0.f) return b;
    const float fb = b.n / n;
    const float delta = b.mean - a.mean;
    Stat r;
    r.n = n;
    r.mean = fmaf(delta, fb, a.mean);
    r.m2 = a.m2 + b.m2 + delta * delta * (a.n * fb);
    return r;
}

__device__ inline Stat shfl_xor_stat(const Stat& s, int off) {
    return Stat{__shfl_xor(s.n, off, kWave), __shfl_xor(s.mean, off, kWave), __shfl_xor(s.m2, off, kWave)};
}

// Butterfly merge over lanes congruent modulo `stride` (power of two).  The
// lower lane is always the left operand, so partners compute identical bits.
__device__ inline Stat wave_merge_strided(Stat s, int stride) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int off = stride; off < kWave; off <<= 1) {
        const Stat o = shfl_xor_stat(s, off);
        s = (lane & off) ? stat_merge(o, s) : stat_merge(s, o);
    }
    return s;
}

// Exact two-pass statistics of K values held in registers, `valid` of which
// count (the first `valid` ones).
template <int K>
__device__ inline Stat stat_of(const float (&v)[K], int valid) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) s += (k < valid) ? v[k] : 0.f;
    if (valid <= 0) return stat_empty();
    const float n = (float)valid;
    const float m = s / n;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float d = v[k] - m;
        q += (k < valid) ? d * d : 0.f;
    }
    return Stat{n, m, q};
}

// Failure report of a bounded wait (the bit the host API calls
// GN_STATUS_WAIT_EXPIRED): a wait that gives up ORs it into the call's status
// word instead of hanging, and its workgroup writes NaN wherever it would
// have used the missing data.
constexpr uint32_t kWaitExpired = 1u;

// ---------------------------------------------------------------------------
// exchange between the workgroups of one launch without cache maintenance
// ---------------------------------------------------------------------------
// gfx950 has one L2 per XCD and these L2s are not coherent with each other, so
// an agent-scope release/acquire fence writes back and invalidates the whole
// L2 of the XCD (buffer_wbl2 / buffer_inv).  A kernel that synchronises a team
// of workgroups once per slab would pay that for every workgroup at every
// slab.  Instead the few values that cross workgroups (partial sums, the slab
// statistics) are written and read with agent-scope relaxed atomics, which the
// hardware performs at the device coherence point (sc1), and the barrier only
// waits for the wave's own stores to complete before it signals arrival.
__device__ inline void xstore(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float xload(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void xstore2(float2* p, float2 v) {
    xstore(&p->x, v.x);
    xstore(&p->y, v.y);
}
__device__ inline float2 xload2(const float2* p) { return make_float2(xload(&p->x), xload(&p->y)); }
__device__ inline void xstore_stat(float4* p, const Stat& s) {
    xstore(&p->x, s.n);
    xstore(&p->y, s.mean);
    xstore(&p->z, s.m2);
}
__device__ inline Stat xload_stat(const float4* p) { return Stat{xload(&p->x), xload(&p->y), xload(&p->z)}; }

// Waits until every memory operation this wave issued has completed
// (s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15) in the gfx9 encoding); the
// signal fences keep the compiler from moving memory accesses across it.
__device__ inline void wait_own_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Barrier of `target` co-resident workgroups on counter *ctr (zero before the
// launch), in two halves so that loads for later work can be issued between
// them: team_arrive publishes (waits for this workgroup's stores, then counts
// one arrival), team_wait blocks until every member has arrived.  Data
// published before the arrival with xstore is visible to xload after the wait.
// Every thread of the workgroup calls both.
__device__ inline void team_arrive(uint32_t* ctr) {
    wait_own_stores();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Returns true when every member arrived; false when the wait gave up after
// `limit` polls (then kWaitExpired is ORed into *err).  `unmet` = 1 raises the
// target out of reach (tests of the failure report).  The result is the same
// for every thread of the workgroup.
__device__ inline bool team_wait(uint32_t* ctr, uint32_t target, uint32_t* err, uint32_t limit, uint32_t unmet) {
    __shared__ uint32_t s_gave_up;
    if (threadIdx.x == 0) {
        uint32_t spins = 0, gave_up = 0;
        const uint32_t goal = target + unmet;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < goal) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > limit) {   // bounded: report instead of hanging
                __hip_atomic_fetch_or(err, kWaitExpired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                gave_up = 1;
                break;
            }
        }
        s_gave_up = gave_up;
    }
    __syncthreads();
    const bool ok = s_gave_up == 0;
    __syncthreads();   // every thread has read the flag before thread 0 can write it again
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return ok;
}
__device__ inline bool team_barrier(uint32_t* ctr, uint32_t target, uint32_t* err, uint32_t limit, uint32_t unmet) {
    team_arrive(ctr);
    return team_wait(ctr, target, err, limit, unmet);
}

}  // namespace gn
