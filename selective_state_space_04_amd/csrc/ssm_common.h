// ssm_common.h -- helpers shared by the HIP sources of libssmscan.so: activation
// dtype conversion, the launch wrapper that records the optional per-launch HIP
// events, and host-side argument checks.  Internal header (not part of the ABI).
#ifndef SSM_COMMON_H
#define SSM_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_scan.h"

namespace ssm {

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
// f32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) {
    return __builtin_bit_cast(bf16_t, (__bf16)v);
}

// sigmoid(z) = 1 / (1 + exp(-|z|)) folded by the sign of z, with the hardware
// exp2 and reciprocal (both about 1 ulp).
__device__ __forceinline__ float sigmoid_f(float z) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(z) * 1.4426950408889634f);
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return z >= 0.0f ? r : e * r;
}

inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// Launches `kern` with `block` threads on the caller's stream; when the caller
// passed an ssm_timing, brackets the launch with its next two events and logs
// the kernel id.  A failed launch is reported as SSM_E_LAUNCH.
struct Launcher {
    hipStream_t s;
    ssm_timing* tm;
    template <typename... KArgs, typename... Args>
    ssm_status operator()(int kid, void (*kern)(KArgs...), dim3 grid, dim3 block, Args... args) {
        const bool rec = tm && tm->events && tm->count < tm->capacity && tm->count < SSM_TIMING_MAX;
        if (rec) (void)hipEventRecord(tm->events[2 * tm->count], s);
        hipLaunchKernelGGL(kern, grid, block, 0, s, args...);
        const hipError_t e = hipGetLastError();
        if (rec) {
            (void)hipEventRecord(tm->events[2 * tm->count + 1], s);
            tm->kernel_id[tm->count] = kid;
            tm->count++;
        }
        return e == hipSuccess ? SSM_OK : SSM_E_LAUNCH;
    }
};

}  // namespace ssm

#define SSM_TRY(expr)                       \
    do {                                    \
        const ssm_status st_ = (expr);      \
        if (st_ != SSM_OK) return st_;      \
    } while (0)

#endif  // SSM_COMMON_H
