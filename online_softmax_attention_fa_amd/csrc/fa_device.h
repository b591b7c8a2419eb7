// Device-side helpers shared by the forward and backward kernels (gfx950 only):
// vector types, MFMA wrappers per element type, the XCD-aware workgroup remap, lane-pair
// reductions, LDS tile swizzle and LDS reads.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;
// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;
// Largest per-lane sum of one tile's P accepted before the tile is redone with its own
// row maximum: keeps every P below 2^15, inside the fp16 range.
constexpr float kMaxTileSum = 32768.0f;

// ------------------------------------------------------------------ helpers ---

template <typename T> struct Elt;
template <> struct Elt<__bf16> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        f32x2 v = {x, y};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
    }
    // acc + x0 + x1 for a packed pair (v_dot2 against (1, 1))
    static __device__ __forceinline__ float sum2(unsigned packed, float acc) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
    }
    // acc + x0 y0 + x1 y1 for packed pairs
    static __device__ __forceinline__ float dot2(unsigned x, unsigned y, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc, false);
    }
};
template <> struct Elt<_Float16> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y) {
        f32x2 v = {x, y};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
    }
    static __device__ __forceinline__ float sum2(unsigned packed, float acc) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
    }
    static __device__ __forceinline__ float dot2(unsigned x, unsigned y, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), acc, false);
    }
};

// Maps the hardware workgroup id to a logical one so that the workgroups the
// dispatcher sends to one XCD (ids congruent mod 8) cover a contiguous logical range.
__device__ __forceinline__ int remap_xcd(int bid, int n) {
    const int xcd = bid % kXcds, local = bid / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// max(a, b, c) with NaN propagation: lowers to one v_maximum3_f32 and, unlike fmaxf,
// needs no canonicalisation of MFMA results first.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// Value of x in lane L^32 combined with x: returns {x[L%32], x[L%32 + 32]} in some order.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte chunk swizzle of K and V tiles in LDS (both row-major, RB = 2*D bytes per
// row): chunk c of row r is stored at chunk c ^ swz(r).  It is chosen so that
//  * the 16 rows read at one logical chunk by a K-operand ds_read_b128 land in 16
//    distinct 16-byte slots of a 256-byte bank window, and
//  * the 4 consecutive rows x 64 bytes read by a V-operand ds_read_b64_tr_b16 lane
//    group cover the 256-byte window exactly once.
// D = 128 (16 chunks/row): swap the 2-bit halves of the row's low nibble.
// D = 64 (8 chunks/row, two rows per window): bit 2 from row bit 1, bits 0-1 from
// row bits 2-3.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    if constexpr (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ u32x4 lds_read16(const lds_u8* base, int off) {
    return *reinterpret_cast<const lds_u32x4*>(base + off);
}
// Transposing read: see the V operand notes in the kernel.
__device__ __forceinline__ u32x2 lds_read_tr(const lds_u8* base, int off) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
    return __builtin_bit_cast(u32x2, v);
}

}  // namespace fa
