// m2_device.h -- device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

constexpr int kWave = 64;  // CDNA wavefront width

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Storage types of activations.  bf16 is kept as raw 16-bit patterns in memory.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
    // round to nearest even (gfx950 has a native conversion for this)
    __bf16 b = (__bf16)v;
    return bf16_t{__builtin_bit_cast(uint16_t, b)};
}

__device__ __forceinline__ float bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

constexpr float kLog2e = 1.4426950408889634f;

// e^v through the hardware base-2 exponential
__device__ __forceinline__ float fast_exp(float v) { return __builtin_amdgcn_exp2f(v * kLog2e); }

// SiLU(v) = v / (1 + e^-v)
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + fast_exp(-v)); }

// softplus(v) = log(1 + e^v); above 20 it equals v to within 2e-9 relative
__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// dt = softplus(raw + bias) clamped to [dt_min, dt_max] (NaN passes through)
__device__ __forceinline__ float dt_of(float raw, float bias, float dt_min, float dt_max) {
    float dt = softplus(raw + bias);
    dt = dt < dt_min ? dt_min : dt;
    return dt > dt_max ? dt_max : dt;
}

}  // namespace m2
