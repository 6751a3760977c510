// Matrix-core and LDS operand helpers for gfx950 (internal header).
//
// MFMA operand layouts used throughout (lane l of a 64-wide wave):
//   v_mfma_f32_16x16x32_bf16: A[l%16][8(l/16)+0..7], B[8(l/16)+0..7][l%16],
//                             D[4(l/16)+e][l%16] in register e.
//   v_mfma_f32_16x16x16_bf16: A[l%16][4(l/16)+0..3], B[4(l/16)+0..3][l%16], D as above.
//   v_mfma_f32_32x32x16_bf16: A[l%32][8(l/32)+0..7], B[8(l/32)+0..7][l%32],
//                             D[8q+4(l/32)+e][l%32] in register 4q+e.
// An operand whose eight contraction elements are contiguous in a row of a
// row-major LDS array is one 16-byte read (frag); an operand whose rows run along
// the contraction is gathered with the LDS transpose read (frag_tr, frag_tr32).
#pragma once

#include "gdr_common.h"

namespace gdr {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Fragment whose 8 contraction elements are contiguous in a row.
__device__ __forceinline__ bf16x8 frag(const uint16_t *base, int row, int stride, int col) {
    return *(const bf16x8 *)(base + row * stride + col);
}

// Fragment of a row-major array whose rows run along the contraction: lane l gets
// column col0 + l%16 at rows k0 + 8(l/16) + 0..7.  Each 16-lane group issues two
// transpose reads; source lane s of a group points at row (k0 + 8G + s/4 [+4]),
// columns col0 + 4(s%4) .. +3, and the hardware hands lane p element p%4 of source
// lanes 4e + p/4, i.e. column col0 + p, rows +e.
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t *base, int k0, int stride, int col0,
                                          int lane) {
    const int G = lane >> 4, s = lane & 15;
    const uint16_t *p = base + (k0 + 8 * G + (s >> 2)) * stride + col0 + 4 * (s & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 4 * stride));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// As frag_tr, for the 32x32x16 operand layout: lane l gets column col0 + l%32 at rows
// k0 + 8(l/32) + 0..7 (16-lane group G covers columns 16(G%2).. and rows 8(G/2)..).
__device__ __forceinline__ bf16x8 frag_tr32(const uint16_t *base, int k0, int stride, int col0,
                                            int lane) {
    const int G = lane >> 4, s = lane & 15;
    const uint16_t *p =
        base + (k0 + 8 * (G >> 1) + (s >> 2)) * stride + col0 + 16 * (G & 1) + 4 * (s & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 4 * stride));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
    return bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}
__device__ __forceinline__ bf16x8 to_bf16x8(float4 a, float4 b) {
    return bf16x8{(__bf16)a.x, (__bf16)a.y, (__bf16)a.z, (__bf16)a.w,
                  (__bf16)b.x, (__bf16)b.y, (__bf16)b.z, (__bf16)b.w};
}

// Four floats -> four bf16 (RNE), one 8-byte store.
__device__ __forceinline__ void store4(uint16_t *dst, float x0, float x1, float x2, float x3) {
    uint2 w;
    w.x = pack_bf16x2(x0, x1);
    w.y = pack_bf16x2(x2, x3);
    *(uint2 *)dst = w;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gdr
