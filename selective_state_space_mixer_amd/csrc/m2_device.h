// m2_device.h -- device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

constexpr int kWave = 64;  // CDNA wavefront width

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one dword, low half first: a single
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// the two bf16 of a packed dword as floats
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

constexpr float kLog2e = 1.4426950408889634f;

// e^v through the hardware base-2 exponential
__device__ __forceinline__ float fast_exp(float v) { return __builtin_amdgcn_exp2f(v * kLog2e); }

// SiLU(v) = v / (1 + e^-v)
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + fast_exp(-v)); }

// softplus(v) = log(1 + e^v) from the hardware base-2 exp and log, with x = e^v:
//   v > 20        -> v                          (the remainder is below 2e-9 relative)
//   x < 1/64      -> x (1 - x/2 + x^2/3)        (log1p series; relative error below x^3/4 < 1e-6)
//   otherwise     -> ln2 * log2(1 + x)          (1+x >= 1+1/64: rounding costs < 4e-6 relative)
__device__ __forceinline__ float softplus(float v) {
    const float x = fast_exp(v);
    const float series = x * (1.0f - x * (0.5f - x * (1.0f / 3.0f)));
    const float direct = 0.6931471805599453f * __builtin_amdgcn_logf(1.0f + x);
    return v > 20.0f ? v : (x < 0.015625f ? series : direct);
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP shifts inside each 16-lane row, then
// the row totals are read back as scalars and added to the later rows.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    float x = v;
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
    const int row = (int)(threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? r0 : 0.0f) + (row >= 2 ? r1 : 0.0f) + (row >= 3 ? r2 : 0.0f);
}

// dt = softplus(raw + bias) clamped to [dt_min, dt_max] (NaN passes through)
__device__ __forceinline__ float dt_of(float raw, float bias, float dt_min, float dt_max) {
    float dt = softplus(raw + bias);
    dt = dt < dt_min ? dt_min : dt;
    return dt > dt_max ? dt_max : dt;
}

}  // namespace m2
