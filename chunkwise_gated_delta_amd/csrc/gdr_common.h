// Shared device helpers and launch interfaces of libgdr (internal header).
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __hip_bfloat16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateNone = 0, kGateHead = 1, kGateChannel = 2;

// Bytes at the start of every workspace reserved for the device error flag.
constexpr size_t kWorkspaceHeader = 256;

__device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16 *p, size_t i) { return __bfloat162float(p[i]); }
__device__ __forceinline__ void st(float *p, size_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st(bf16 *p, size_t i, float x) { p[i] = __float2bfloat16(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two floats -> two bf16 (round to nearest even) packed low-first in one word
// (a single v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also waits for
// every outstanding global load and store, which would stall on loads issued
// early on purpose (prefetch of the next chunk).  Every barrier in the kernels
// here exists to hand LDS data between waves, so waiting on the LDS counter
// (lgkmcnt = 0, vmcnt and expcnt left at their maxima) before s_barrier is
// enough; the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Sequence bounds [t0, t1) of sequence n on the flattened token axis.  Packed
// offsets are clamped into [0, total] and made non-decreasing so that nothing
// is read or written outside the buffers; a clamp raises the error flag.
__device__ __forceinline__ void seq_bounds(const int32_t *cu, int n, int T, long total, long &t0,
                                           long &t1, int *err_flag) {
    if (cu == nullptr) {
        t0 = (long)n * T;
        t1 = t0 + T;
        return;
    }
    long a = cu[n], b = cu[n + 1];
    long ca = a < 0 ? 0 : (a > total ? total : a);
    long cb = b < ca ? ca : (b > total ? total : b);
    if ((ca != a || cb != b) && err_flag != nullptr) atomicOr(err_flag, 1);
    t0 = ca;
    t1 = cb;
}

struct FwdArgs {
    const void *q, *k, *v, *a, *b;
    const float *log_alpha, *beta, *S0;
    void *O;
    float *S_final;
    const int32_t *cu_seqlens;
    int n_seq, B, H, T, dk, dv, C, dtype, gate;
    void *workspace;
    size_t workspace_bytes;
};

// Launchers (return a hipError_t as int).  Each enqueues on `stream`.
bool f32_split_supported(const FwdArgs &a);
size_t f32_split_workspace_bytes(const FwdArgs &a, int n_seq_eff);
int launch_f32_split(const FwdArgs &a, int n_seq_eff, hipStream_t stream);
bool kda_split_supported(const FwdArgs &a);
size_t kda_split_workspace_bytes(const FwdArgs &a, int n_seq_eff);
int launch_kda_split(const FwdArgs &a, int n_seq_eff, hipStream_t stream);

}  // namespace gdr
