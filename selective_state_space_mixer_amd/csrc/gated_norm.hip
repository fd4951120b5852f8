// gated_norm.hip -- gated group RMSNorm after the scan (gfx950).
//
// Article "Transformers 中 Zamba2 混合架构模型解析", §三: after the scan, the mixer applies a
// group RMSNorm times SiLU of the gate z over intermediate_size, split into groups; §五 gives
// rms_norm_eps.  Both gate orders:
//   gate first (norm_before_gate = 0):  g = y * SiLU(z),  out = g / sqrt(mean_group(g^2) + eps) * w
//   norm first (norm_before_gate = 1):  out = y / sqrt(mean_group(y^2) + eps) * w * SiLU(z)
//
// A pure HBM stream (y and z in, out back: three rows per token).  One wave owns one (token,
// group): each lane brings NV 16-byte pieces of y and z into registers, the wave sums the squares
// (DPP scan), and the same lanes scale and write their pieces.  Loads and stores are range-checked
// buffer accesses over the group, so a group that is not a whole number of wave-wide rows needs
// no guards.  The group is read in full before anything is written, so out may alias y.
#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct NormK {
    const void* y; const void* z; const float* w; void* out;
    int64_t ys, zs, os;
    int64_t npairs;   // tokens * groups
    int ngroups, gs;  // groups per row, channels per group
    float eps;
    int nbg;          // norm before gate
};

constexpr int kNormThreads = 256;  // four waves, four (token, group) pairs per block

template <typename T> struct NormIO;
template <> struct NormIO<bf16_t> {
    static constexpr int EPV = 8;  // elements per 16-byte piece
    static __device__ __forceinline__ float get(const u32x4_t& v, int e) {
        const uint32_t wd = v[e >> 1];
        return __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
    }
    static __device__ __forceinline__ u32x4_t put(const float (&o)[8]) {
        return u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7])};
    }
};
template <> struct NormIO<float> {
    static constexpr int EPV = 4;
    static __device__ __forceinline__ float get(const u32x4_t& v, int e) { return __uint_as_float(v[e]); }
    static __device__ __forceinline__ u32x4_t put(const float (&o)[4]) {
        return u32x4_t{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t norm_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// cache policy of the y and z loads: streaming (non-temporal) -- each is read once, and the
// cache is better left to the output, which the next layer reads (5% faster on the 32k output)
constexpr int kStream = 2;

// The gate order is a template parameter so that each kernel keeps only what its second pass needs:
// gate first keeps g = y * SiLU(z) (one fp32 per element) and lets the raw pieces go; norm first keeps
// the raw y and z pieces and forms SiLU(z) in the second pass.  With the order a runtime choice the
// compiler kept the raw pieces and every SiLU(z) across the reduction (208 VGPRs at a 5120-channel
// group, two waves per SIMD; now 106 and 151).
template <typename T, int NV, bool NBG>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(NormK k)
{
    using IO = NormIO<T>;
    constexpr int EPV = IO::EPV;
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * (kNormThreads / 64) + (threadIdx.x >> 6);
    if (pair >= k.npairs) return;  // whole waves leave together
    const int64_t t = pair / k.ngroups;
    const int g = (int)(pair % k.ngroups);
    const uint32_t bytes = (uint32_t)k.gs * sizeof(T);
    const auto ry = norm_rsrc(reinterpret_cast<const T*>(k.y) + t * k.ys + (int64_t)g * k.gs, bytes);
    const auto rz = norm_rsrc(reinterpret_cast<const T*>(k.z) + t * k.zs + (int64_t)g * k.gs, bytes);
    const auto ro = norm_rsrc(reinterpret_cast<T*>(k.out) + t * k.os + (int64_t)g * k.gs, bytes);
    const float* wg = k.w + (int64_t)g * k.gs;

    u32x4_t yv[NV], zv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const uint32_t off = (uint32_t)(j * 64 + lane) * 16u;
        yv[j] = __builtin_amdgcn_raw_buffer_load_b128(ry, (int)off, 0, kStream);
        zv[j] = __builtin_amdgcn_raw_buffer_load_b128(rz, (int)off, 0, kStream);
    }
    // sum of squares of the normalised operand (pieces past the group read as zero)
    float ss = 0.0f;
    float gv[NBG ? 1 : NV][EPV];  // gate first: y * SiLU(z)
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float yy = IO::get(yv[j], e);
            if constexpr (NBG) {
                ss = fmaf(yy, yy, ss);
            } else {
                gv[j][e] = yy * silu(IO::get(zv[j], e));
                ss = fmaf(gv[j][e], gv[j][e], ss);
            }
        }
    const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_prefix_sum(ss)), 63));
    const float r = __builtin_amdgcn_rsqf(tot / (float)k.gs + k.eps);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c0 = (j * 64 + lane) * EPV;
        if (c0 >= k.gs) break;  // lanes past the end of the group stop (their w would lie outside it)
        float wv[EPV];
#pragma unroll
        for (int e = 0; e < EPV; e += 4) {
            const float4 w4 = *reinterpret_cast<const float4*>(wg + c0 + e);
            wv[e] = w4.x; wv[e + 1] = w4.y; wv[e + 2] = w4.z; wv[e + 3] = w4.w;
        }
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            if constexpr (NBG) o[e] = IO::get(yv[j], e) * r * wv[e] * silu(IO::get(zv[j], e));
            else o[e] = gv[j][e] * r * wv[e];
        }
        __builtin_amdgcn_raw_buffer_store_b128(IO::put(o), ro, (int)((uint32_t)(j * 64 + lane) * 16u), 0, 0);
    }
}

template <typename T>
static hipError_t launch_norm_t(const NormArgs& a, hipStream_t s) {
    NormK k;
    k.y = a.y; k.z = a.z; k.w = a.w; k.out = a.out;
    k.ys = a.ys; k.zs = a.zs; k.os = a.os;
    k.ngroups = a.d_inner / a.gs;
    k.gs = a.gs;
    k.npairs = a.ntok * k.ngroups;
    k.eps = a.eps;
    k.nbg = a.norm_before_gate ? 1 : 0;
    const int nv = (a.gs / NormIO<T>::EPV + 63) / 64;
    const dim3 grid((unsigned)((k.npairs + 3) / 4)), block(kNormThreads);
    switch (nv) {
#define M2_NV(n) case n: return k.nbg ? launch_kernel(gated_rmsnorm_kernel<T, n, true>, grid, block, 0, s, k) \
                                      : launch_kernel(gated_rmsnorm_kernel<T, n, false>, grid, block, 0, s, k);
        M2_NV(1) M2_NV(2) M2_NV(3) M2_NV(4) M2_NV(5) M2_NV(6) M2_NV(7) M2_NV(8)
        M2_NV(9) M2_NV(10) M2_NV(11) M2_NV(12) M2_NV(13) M2_NV(14) M2_NV(15) M2_NV(16)
#undef M2_NV
        default: return hipErrorInvalidValue;
    }
}

int gated_rmsnorm_max_group(bool bf16) { return 16 * 64 * (bf16 ? 8 : 4); }

hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s) {
    return a.bf16 ? launch_norm_t<bf16_t>(a, s) : launch_norm_t<float>(a, s);
}

}  // namespace m2
