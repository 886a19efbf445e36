// Device-side helpers shared by the libpoetx kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

// bf16 is carried as its raw 16 bits; arithmetic always happens in float.
struct bf16_t {
    uint16_t bits;
};

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bf16, round to nearest even; NaN stays NaN (quiet).  gfx950
// converts in hardware (v_cvt_pk_bf16_f32); its result equals the bit-level
// rounding (add 0x7fff plus the kept lsb, NaN: upper half | 0x40) for every
// float32 pattern, denormals and NaNs included.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two floats -> packed bf16 pair (lo in bits 0..15), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> {
    static constexpr int kVec = 4;  // elements per 16-byte vector
    __device__ static float to_f32(float v) { return v; }
    __device__ static float from_f32(float v) { return v; }
};
template <> struct ElemTraits<bf16_t> {
    static constexpr int kVec = 8;
    __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v.bits); }
    __device__ static bf16_t from_f32(float v) { return bf16_t{f32_to_bf16(v)}; }
};

template <typename T> __device__ __forceinline__ float load_f32(const T* p) {
    return ElemTraits<T>::to_f32(*p);
}
template <typename T> __device__ __forceinline__ void store_f32(T* p, float v) {
    *p = ElemTraits<T>::from_f32(v);
}

// One 32x32 MFMA tile update from one 16-byte A fragment and one 16-byte B
// fragment per lane.  Lane l holds row (l % 32) of A / column (l % 32) of B and
// 16 bytes of consecutive k starting at (l / 32) * kVec; both operands use the
// same k assignment, so the order in which the instruction sums over k does
// not matter.
template <typename T> struct Mfma32;
template <> struct Mfma32<bf16_t> {
    static constexpr int kStepK = 16;  // k covered by one fragment pair
    __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x16_t& acc) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};
template <> struct Mfma32<float> {
    static constexpr int kStepK = 8;   // four v_mfma_f32_32x32x2_f32, two k each
    __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x16_t& acc) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    }
};

}  // namespace poetx
