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

// Cross-lane moves.  DPP forms are VALU operand modifiers (no LDS round trip):
// quad_perm xor 1 / xor 2, row_half_mirror (lane i <-> 7 - i within 8) and
// row_mirror (i <-> 15 - i within 16).  Across the two 16-lane rows of a
// 32-lane group, ds_swizzle in its bit mode (offset = xor_mask << 10 | 0x1f).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float swizzle_xor16(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (16 << 10) | 0x1f));
}

// Sum of x over each group of G consecutive lanes (G a power of two, <= 32).
// After the quad steps every lane of a quad holds the quad sum, so the mirror
// steps pair whole quads (and then whole 8-lane halves).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G >= 1 && G <= 32 && (G & (G - 1)) == 0, "group of 1..32 lanes");
    if constexpr (G >= 2) x += dpp<kDppXor1>(x);
    if constexpr (G >= 4) x += dpp<kDppXor2>(x);
    if constexpr (G >= 8) x += dpp<kDppHalfMirror>(x);
    if constexpr (G >= 16) x += dpp<kDppMirror>(x);
    if constexpr (G >= 32) x += swizzle_xor16(x);
    return x;
}

// Spectral clip bound of one token ("How to make GDN2 more stable", eqs. 4 and 7):
// the gate is limited to 1 / rho with rho = ||I - b a^T||_2.  With eta = |a| |b|
// and cosine c, eq. 4 gives rho = (eta + sqrt(eta^2 - 4 eta c + 4)) / 2, and
// eta c = a.b.  The radicand is >= (eta - 2)^2 >= 0; max() absorbs rounding.
// Returns -log(rho) in the base the caller asks for (scale = log_base(2) factor:
// 1 for log2, ln 2 for the natural log).  Zero vectors give rho = 1, bound 0.
__device__ __forceinline__ float clip_bound(float aa, float bb, float ab, float scale) {
    const float eta = sqrtf(aa) * sqrtf(bb);
    const float disc = fmaxf(eta * eta - 4.f * ab + 4.f, 0.f);
    return -scale * __log2f(0.5f * (eta + sqrtf(disc)));
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
    int n_seq, B, H, T, dk, dv, C, dtype, gate;  // gate: the layout only (kGate*)
    bool clip;  // spectral clipping of the gate, alpha <- min(alpha, 1 / ||I - b a^T||_2)
    bool keep_states;  // also leave the per-chunk states for the backward (its workspace layout)
    void *workspace;
    size_t workspace_bytes;
    int *err;  // device error word; NULL: the one in the workspace header
};

// Arguments of the backward pass (a, b NULL: the KDA form a = k, b = beta k).
struct BwdArgs {
    const void *q, *k, *v, *a, *b, *dO;
    const float *log_alpha, *beta, *S0, *dS_final;
    void *grad_q, *grad_k, *grad_v, *grad_a, *grad_b;  // dL/dq, dL/dk, dL/dv, dL/da, dL/db
    float *grad_la, *grad_beta, *grad_S0;      // dL/dlog_alpha, dL/dbeta, dL/dS0
    const int32_t *cu_seqlens;
    int n_seq, B, H, T, dk, dv, C, dtype, gate;
    bool reuse_fwd;  // the workspace holds the forward's per-chunk blocks of the same inputs
    bool reuse_states;  // ... and the states entering each chunk (keep_states forward)
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
bool kda_bwd_supported(const BwdArgs &a);
size_t kda_bwd_workspace_bytes(const BwdArgs &a, int n_seq_eff);
int launch_kda_bwd(const BwdArgs &a, int n_seq_eff, hipStream_t stream);
BwdArgs bwd_view(const FwdArgs &a);  // the backward arguments that share a's shapes

}  // namespace gdr
