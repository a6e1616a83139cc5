// mfma_bf16.hpp — vector types and small helpers shared by the bf16 attention kernels
// (forward and gradients): the operand types of v_mfma_f32_32x32x16_bf16, packing of
// two floats to bf16, the transposing LDS load and the raw buffer resource word.
#pragma once

#include <stdint.h>

namespace mi355 {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw (unformatted, byte-addressed) buffer resource on gfx9.
constexpr int kBufferWord3 = 0x00020000;

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Transposing LDS load: within each group of 16 lanes, lane i receives element i % 4
// of the 8-byte blocks addressed by lanes i / 4 + 4 k, k = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const lds_char*)(p));
}

// One A operand of a 32x32x16 product whose k index runs over 16 rows of a row-major
// bf16 tile in LDS: rows 4 h + t and 8 + 4 h + t (t = 0..3, h = lane / 32) of one
// output column, from two transposing loads at p_lo and p_hi.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const char* p_lo, const char* p_hi) {
    const i16x4 lo = lds_read_tr16(p_lo);
    const i16x4 hi = lds_read_tr16(p_hi);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The two 16-bit input formats of the attention kernels: the 8-element operand vector of
// v_mfma_f32_32x32x16_{bf16,f16}, the product itself, the 16x16x32 product with the same
// operand vectors, two 16-bit ones packed in a word, and float -> 16-bit packing (round
// to nearest even).
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct ElemBF16 {
    using v8 = bf16x8;
    static constexpr uint32_t kOnes2 = 0x3F803F80u;
    __device__ static __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
};

struct ElemF16 {
    using v8 = f16x8;
    static constexpr uint32_t kOnes2 = 0x3C003C00u;
    __device__ static __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
    }
};

}  // namespace mi355
