// pkv_mfma.h -- matrix-core operations and LDS helpers shared by the decode
// and prefill kernels (gfx950, 16-bit inputs, fp32 accumulation).
//
// Operand layouts (lane l of a 64-wide wave; verified against numpy on MI355X):
//   v_mfma_f32_16x16x32_{bf16,f16}: A lane l = A[l % 16][8(l/16) .. 8(l/16)+7],
//     B lane l = B[8(l/16) .. +7][l % 16], C lane l = C[4(l/16) + r][l % 16];
//   v_mfma_f32_16x16x16{bf16_1k,f16}: the same with 4 instead of 8, so the C
//     layout of a 16x16 product is the B layout of the next one;
//   the order of the contracted index inside one product is free as long as
//     A and B agree, so two 4-element halves (from two 16x16 C tiles) make the
//     8 elements of a 16x16x32 operand (pv2): one instruction for the work of
//     two 16x16x16 ones;
//   ds_read_b64_tr_b16: within each 16-lane group, element r of lane j is
//     element j % 4 of the 8-byte row (4r + j / 4) of the 4 x 16 block read.
#pragma once

#include "pkv_device.h"

namespace pkv {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <class E>
struct MfmaOps;

template <>
struct MfmaOps<BF16> {
    typedef __bf16 v8_t __attribute__((ext_vector_type(8)));
    typedef __bf16 tr_t __attribute__((__vector_size__(4 * sizeof(__bf16))));
    typedef s16x4_t op4_t;
    __device__ static __forceinline__ f32x4_t qk(const Vec16& a, const Vec16& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8_t, a), __builtin_bit_cast(v8_t, b), c, 0,
                                                       0, 0);
    }
    __device__ static __forceinline__ op4_t read_tr(const char* p) {
        auto q = (__attribute__((address_space(3))) tr_t*)((__attribute__((address_space(3))) char*)(p));
        return __builtin_bit_cast(op4_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(q));
    }
    __device__ static __forceinline__ f32x4_t pv(op4_t a, op4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    // One 16x16x32 product over two 4-key halves: A = (a0, a1), B = (b0, b1).
    __device__ static __forceinline__ f32x4_t pv2(op4_t a0, op4_t a1, op4_t b0, op4_t b1, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7)),
            __builtin_bit_cast(v8_t, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7)), c, 0, 0, 0);
    }
    __device__ static __forceinline__ void split(float x, short& hi, short& lo) {
        const __bf16 h = (__bf16)x;
        hi = __builtin_bit_cast(short, h);
        lo = __builtin_bit_cast(short, (__bf16)(x - (float)h));
    }
};

template <>
struct MfmaOps<F16> {
    typedef _Float16 v8_t __attribute__((ext_vector_type(8)));
    typedef _Float16 v4h_t __attribute__((ext_vector_type(4)));
    typedef __fp16 tr_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
    typedef v4h_t op4_t;
    __device__ static __forceinline__ f32x4_t qk(const Vec16& a, const Vec16& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8_t, a), __builtin_bit_cast(v8_t, b), c, 0, 0,
                                                      0);
    }
    __device__ static __forceinline__ op4_t read_tr(const char* p) {
        auto q = (__attribute__((address_space(3))) tr_t*)((__attribute__((address_space(3))) char*)(p));
        return __builtin_bit_cast(op4_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(q));
    }
    __device__ static __forceinline__ f32x4_t pv(op4_t a, op4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4_t pv2(op4_t a0, op4_t a1, op4_t b0, op4_t b1, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                      __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c, 0,
                                                      0, 0);
    }
    __device__ static __forceinline__ void split(float x, short& hi, short& lo) {
        const _Float16 h = (_Float16)x;
        hi = __builtin_bit_cast(short, h);
        lo = __builtin_bit_cast(short, (_Float16)(x - (float)h));
    }
};

// 16-byte LDS store / load at a byte offset from an LDS base pointer.
__device__ __forceinline__ void lds_store16(char* base, uint32_t off, const Vec16& v) {
    typedef __attribute__((address_space(3))) v4u32_t lds_v4;
    typedef __attribute__((address_space(3))) char lds_c;
    *(lds_v4*)((lds_c*)base + off) = v4u32_t{v.w[0], v.w[1], v.w[2], v.w[3]};
}

__device__ __forceinline__ Vec16 lds_load16(const char* base, uint32_t off) {
    typedef const __attribute__((address_space(3))) v4u32_t lds_v4;
    typedef const __attribute__((address_space(3))) char lds_c;
    const v4u32_t u = *(lds_v4*)((lds_c*)base + off);
    return Vec16{{u.x, u.y, u.z, u.w}};
}

}  // namespace pkv
