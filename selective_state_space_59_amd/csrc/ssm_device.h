// ssm_device.h -- device-side helpers shared by the library's HIP kernels
// (gfx950 only).  I/O element types, exact bf16 widening, round-to-nearest-
// even narrowing, and the few transcendental building blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// log2(e): exp(v) is evaluated as exp2(v * log2(e)) on the hardware exp unit.
constexpr float kLog2e = 1.4426950408889634f;

struct io_f32 {
    using storage = float;
    static constexpr int bytes = 4;
};
struct io_bf16 {
    using storage = uint16_t;
    static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.  gfx950
// converts in hardware (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 bits (lo in bits 0..15), one conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename IO>
__device__ __forceinline__ float load_io(const void *p, int64_t i);
template <>
__device__ __forceinline__ float load_io<io_f32>(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
}
template <>
__device__ __forceinline__ float load_io<io_bf16>(const void *p, int64_t i) {
    return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
}

template <typename IO>
__device__ __forceinline__ void store_io(void *p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_io<io_f32>(void *p, int64_t i, float v) {
    static_cast<float *>(p)[i] = v;
}
template <>
__device__ __forceinline__ void store_io<io_bf16>(void *p, int64_t i, float v) {
    static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(v);
}

// Hardware 2^v (v_exp_f32).  Results below the normal range flush to zero.
__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
// Hardware reciprocal (v_rcp_f32, 1 ulp).
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// SiLU(v) = v * sigmoid(v) = v / (1 + e^-v).
__device__ __forceinline__ float silu(float v) {
    return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e));
}

// softplus with the hardware exp2 / log2: max(v,0) + log(1 + w), w = e^-|v|;
// for tiny w, log(1+w) ~ w (1 - w/2) keeps the relative accuracy.
__device__ __forceinline__ float softplus_fast(float v) {
    const float w = hw_exp2(-fabsf(v) * kLog2e);
    const float lg = __builtin_amdgcn_logf(1.0f + w) * 0.69314718055994531f;
    const float small = w * (1.0f - 0.5f * w);
    return fmaxf(v, 0.0f) + (w < 0.0078125f ? small : lg);
}

// softplus(v) = max(v, 0) + log(1 + e^-|v|), the overflow-free form.
__device__ __forceinline__ float softplus(float v) {
    return fmaxf(v, 0.0f) + log1pf(__expf(-fabsf(v)));
}

}  // namespace ssm
