// fa2_device.h -- device helpers for the gfx950 attention kernels.
//
// * Global reads go through raw buffer loads whose descriptor carries the size
//   of the (b,h) slice: a read past the end returns zero instead of faulting,
//   which is how ragged tails are loaded (the kernels then mask those keys).
// * Cross-lane reductions use DPP within 16-lane rows and ds_bpermute beyond.
// * Dtype tags: 0 = float32, 1 = float16, 2 = bfloat16 (same values as fa2_dtype).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Word 3 of a gfx9-family buffer descriptor for untyped dword access.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kBufferFlags);
}

// 16 bytes at byte offset `off` (0 when past the descriptor's size).
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2f_fast(float x) { return __builtin_amdgcn_logf(x); }

// DPP controls (gfx9): quad permutes, row mirrors.
#define FA2_DPP_QUAD_XOR1 0xB1   // quad_perm [1,0,3,2]
#define FA2_DPP_QUAD_XOR2 0x4E   // quad_perm [2,3,0,1]
#define FA2_DPP_ROW_HALF_MIRROR 0x141
#define FA2_DPP_ROW_MIRROR 0x140

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum or max over groups of G consecutive lanes (G in {8, 16, 32}); every lane
// of a group receives the group's result.  After the two quad steps all four
// lanes of a quad agree, so the half-row mirror (lane i <- 7-i) pairs quads and
// the row mirror (i <- 15-i) pairs half-rows.
template <int G, bool MAX = false>
__device__ __forceinline__ float group_reduce(float x) {
    static_assert(G == 8 || G == 16 || G == 32, "group size");
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    x = op(x, dpp<FA2_DPP_QUAD_XOR1>(x));
    x = op(x, dpp<FA2_DPP_QUAD_XOR2>(x));
    x = op(x, dpp<FA2_DPP_ROW_HALF_MIRROR>(x));
    if (G >= 16) x = op(x, dpp<FA2_DPP_ROW_MIRROR>(x));
    if (G >= 32) x = op(x, __shfl_xor(x, 16));
    return x;
}

__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask); }

// Maximum that returns NaN when either operand is NaN (IEEE 754-2019
// maximum).  fmaxf's NaN-dropping rule makes the compiler quiet every operand
// it cannot prove is an arithmetic result (one extra v_max per operand for
// MFMA accumulators and lane shuffles); this one is a single v_maximum3_f32.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(x[lane], x[lane ^ 16]) and max(x[lane], x[lane ^ 32]) on the VALU
// (v_permlane16_swap / v_permlane32_swap exchange 16-lane rows of a register
// pair; with the same register twice, one output holds the lane's own value
// and the other its partner's).
__device__ __forceinline__ float max_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nan(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nan(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// f32 -> 16-bit storage, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (DT == 1) {
        half2v h = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, h);
    } else {
        bf16x2 h = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, h);
    }
}

// 16-bit storage word pair -> two floats.
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float &a, float &b) {
    if constexpr (DT == 1) {
        half2v h = __builtin_bit_cast(half2v, w);
        a = (float)h[0];
        b = (float)h[1];
    } else {
        a = __uint_as_float(w << 16);
        b = __uint_as_float(w & 0xFFFF0000u);
    }
}

// Dot product of two 16-bit pairs accumulated in f32.
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == 1) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b),
                                      c, false);
    } else {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                               __builtin_bit_cast(bf16x2, b), c, false);
    }
}

__device__ __forceinline__ uint32_t swap_bits23(uint32_t x) {
    return (x & ~12u) | ((x & 4u) << 1) | ((x & 8u) >> 1);
}

}  // namespace fa2
