// mi_attn_device.hpp -- device helpers shared by the libmi_attn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// bf16 bits -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// fp16 bits -> fp32 (exact widening).
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Two fp32 -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
    f16x2 p;
    p[0] = (_Float16)lo;
    p[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

// The two 16-bit input formats of the matrix-core kernels.  Operands are handled as
// eight raw 16-bit values (bf16x8 bit patterns); Fmt16<F16> picks the MFMA that reads
// them and the rounding of fp32 results back to the format.
template <bool F16>
struct Fmt16 {
    __device__ static __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
        if constexpr (F16)
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                          c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        if constexpr (F16)
            return pack_f16x2(lo, hi);
        else
            return pack_bf16x2(lo, hi);
    }
    // the two values of a packed pair, widened exactly to fp32
    __device__ static __forceinline__ float lo(uint32_t w) { return F16 ? f16_lo(w) : bf16_lo(w); }
    __device__ static __forceinline__ float hi(uint32_t w) { return F16 ? f16_hi(w) : bf16_hi(w); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max over the 16 lanes of a DPP row, result in every lane of the row.
// quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int LANES>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16, "row reduction width");
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    if (LANES >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
    if (LANES >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
    return v;
}

// Value of lane (lane ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float v) {
    return __int_as_float(__shfl_xor(__float_as_int(v), 32));
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane l
// receives element r = the 16-bit value at (address of lane 4r + l/4) + (l % 4).
__device__ __forceinline__ s16x4 lds_read_tr16(void* lds_base, int byte_offset) {
    typedef __attribute__((address_space(3))) char lds_char;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_char*)lds_base + byte_offset));
}

}  // namespace mi_attn
