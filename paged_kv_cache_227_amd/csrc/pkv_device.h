// pkv_device.h -- device-side building blocks of the HIP path (gfx950).
//
// Storage traits for the three element types, 16-byte vector loads, packed
// 16-bit dot products with fp32 accumulation, and wave64 cross-lane
// reductions.  Internal to the library: included by its .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr int kBlock = 16;  // tokens per KV block on the GPU path

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// 16 bytes as four 32-bit words; each word holds one fp32 or two 16-bit values.
struct alignas(16) Vec16 {
    uint32_t w[4];
};

__device__ __forceinline__ Vec16 load16(const void* p) {
    Vec16 v;
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    v.w[0] = u.x;
    v.w[1] = u.y;
    v.w[2] = u.z;
    v.w[3] = u.w;
    return v;
}

typedef uint32_t v4u32_t __attribute__((ext_vector_type(4)));

// Streaming load: the nontemporal hint marks the lines for early eviction, the
// right policy for K/V tiles that each step reads exactly once.
__device__ __forceinline__ Vec16 load16_stream(const void* p) {
    const v4u32_t u = __builtin_nontemporal_load(reinterpret_cast<const v4u32_t*>(p));
    Vec16 v;
    v.w[0] = u.x;
    v.w[1] = u.y;
    v.w[2] = u.z;
    v.w[3] = u.w;
    return v;
}

template <bool Stream>
__device__ __forceinline__ Vec16 load16_policy(const void* p) {
    if constexpr (Stream)
        return load16_stream(p);
    else
        return load16(p);
}

// The wave waits here until v has arrived: an empty asm statement reads v's
// registers.  Loads are counted in issue order, so a load on a rarely taken
// branch would otherwise be waited for where the branches join, together with
// every load issued before it.
__device__ __forceinline__ void settle(const Vec16& v) {
    asm volatile("" ::"v"(v.w[0]), "v"(v.w[1]), "v"(v.w[2]), "v"(v.w[3]));
}

__device__ __forceinline__ void store16(void* p, const Vec16& v) {
    *reinterpret_cast<uint4*>(p) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
}

// ---- element types ---------------------------------------------------------
// Each trait gives: element bytes, elements per 16-byte vector, the dot product
// of two vectors with fp32 accumulation, the expansion of a vector to fp32, and
// the round-to-nearest-even store of an fp32 value.

struct F32 {
    static constexpr int kBytes = 4;
    static constexpr int kPerVec = 4;
    __device__ static __forceinline__ float dot(const Vec16& a, const Vec16& b, float acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_fmaf(__uint_as_float(a.w[i]), __uint_as_float(b.w[i]), acc);
        return acc;
    }
    __device__ static __forceinline__ void expand(const Vec16& a, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(a.w[i]);
    }
    __device__ static __forceinline__ void store(void* p, float x) {
        *reinterpret_cast<float*>(p) = x;
    }
    __device__ static __forceinline__ uint32_t bits(float x) {
        return __float_as_uint(x);
    }
};

struct F16 {
    static constexpr int kBytes = 2;
    static constexpr int kPerVec = 8;
    __device__ static __forceinline__ float dot(const Vec16& a, const Vec16& b, float acc) {
        // v_dot2_f32_f16: both products are exact in fp32; the sum is fp32.
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.w[i]),
                                         __builtin_bit_cast(half2_t, b.w[i]), acc, false);
        return acc;
    }
    __device__ static __forceinline__ void expand(const Vec16& a, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            half2_t h = __builtin_bit_cast(half2_t, a.w[i]);
            f[2 * i] = (float)h.x;
            f[2 * i + 1] = (float)h.y;
        }
    }
    __device__ static __forceinline__ void store(void* p, float x) {
        *reinterpret_cast<_Float16*>(p) = (_Float16)x;  // v_cvt_f16_f32 rounds to nearest even
    }
    __device__ static __forceinline__ uint32_t bits(float x) {  // the rounded value's 16 bits
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
};

struct BF16 {
    static constexpr int kBytes = 2;
    static constexpr int kPerVec = 8;
    __device__ static __forceinline__ float dot(const Vec16& a, const Vec16& b, float acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a.w[i]),
                                                  __builtin_bit_cast(bf162_t, b.w[i]), acc, false);
        return acc;
    }
    __device__ static __forceinline__ void expand(const Vec16& a, float* f) {
        // bfloat16 is the top half of a binary32: widening is a shift / mask.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(a.w[i] << 16);
            f[2 * i + 1] = __uint_as_float(a.w[i] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ void store(void* p, float x) {
        *reinterpret_cast<__bf16*>(p) = (__bf16)x;  // round to nearest even
    }
    __device__ static __forceinline__ uint32_t bits(float x) {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
};

// Four consecutive elements, each rounded like E::store, in one store (8 bytes
// for 16-bit types, 16 for fp32; p aligned accordingly).
template <class E>
__device__ __forceinline__ void store4(char* p, float a, float b, float c, float d) {
    if constexpr (E::kBytes == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(E::bits(a) | (E::bits(b) << 16), E::bits(c) | (E::bits(d) << 16));
    } else {
        *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
    }
}

// ---- cross-lane helpers ------------------------------------------------------

// DPP control words (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of the
// group receives the total.  After the quad steps all lanes of a quad agree,
// so a mirror inside 8 (or 16) lanes acts as an exchange with the other half.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    static_assert(N <= 16, "group_sum: groups of at most 16 lanes");
    return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
    return __shfl_xor(x, mask, kWave);
}

// Maximum and sum over the four 16-lane rows' matching lanes (l, l^16, l^32,
// l^48), inside the vector ALU: v_permlane16_swap of a value with itself
// leaves lane l holding, in row order, its own and lane l^16's values (and
// v_permlane32_swap likewise for l^32), so both lanes of a pair combine the
// same two values in the same order.  (Lane mapping checked on gfx950.)
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ int wave_id_uniform() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

}  // namespace pkv
