// conv1d.hip -- causal depthwise conv1d + SiLU over a prompt (gfx950).
//
// The mixer's depthwise conv (article "Transformers 中 Zamba2 混合架构模型解析", §三:
// groups = conv_dim, kernel width mamba_d_conv, SiLU on the output):
//     out[b,t,c] = SiLU(bias[c] + sum_{k<W} w[c,k] * x[b, t-(W-1)+k, c])
//
// Pure HBM stream (3 flop per byte).  Each lane owns VEC adjacent channels (one
// 8-byte load per token for 4 bf16 channels) and walks TILE consecutive tokens (64;
// 8 when there are too few tiles to fill the chip), keeping the last W inputs in
// registers, so every input is read from HBM once (plus a W-1 token halo per tile).
// A wave covers 64*VEC contiguous channels of one token, so each load and store
// instruction moves one contiguous row segment; loads run one group of 8 tokens
// ahead of the arithmetic.
#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

template <typename T, int VEC> struct Vec;
template <> struct Vec<bf16_t, 8> {
    uint4 raw;
    __device__ __forceinline__ float get(int i) const {
        const uint32_t wd = (&raw.x)[i >> 1];
        return __uint_as_float((i & 1) ? (wd & 0xffff0000u) : (wd << 16));
    }
    __device__ __forceinline__ void set2(int i, float lo, float hi) {
        (&raw.x)[i >> 1] = pack_bf16x2(lo, hi);
    }
};
template <> struct Vec<float, 4> {
    float4 raw;
    __device__ __forceinline__ float get(int i) const { return (&raw.x)[i]; }
    __device__ __forceinline__ void set2(int i, float lo, float hi) { (&raw.x)[i] = lo; (&raw.x)[i + 1] = hi; }
};
template <> struct Vec<bf16_t, 4> {
    uint2 raw;
    __device__ __forceinline__ float get(int i) const {
        const uint32_t wd = (&raw.x)[i >> 1];
        return __uint_as_float((i & 1) ? (wd & 0xffff0000u) : (wd << 16));
    }
    __device__ __forceinline__ void set2(int i, float lo, float hi) {
        (&raw.x)[i >> 1] = pack_bf16x2(lo, hi);
    }
};
template <typename T> struct Vec<T, 1> {
    T raw;
    __device__ __forceinline__ float get(int) const { return to_f32(raw); }
};

template <typename T, int VEC>
__device__ __forceinline__ Vec<T, VEC> load_vec(const T* p) {
    Vec<T, VEC> v;
    v.raw = *reinterpret_cast<const decltype(v.raw)*>(p);
    return v;
}

template <typename T, int VEC>
__device__ __forceinline__ void store_vals(T* p, const float (&o)[VEC]) {
    if constexpr (VEC == 1) {
        *p = from_f32<T>(o[0]);
    } else {
        Vec<T, VEC> v;
#pragma unroll
        for (int i = 0; i < VEC; i += 2) v.set2(i, o[i], o[i + 1]);
        *reinterpret_cast<decltype(v.raw)*>(p) = v.raw;
    }
}

template <typename T, int VEC>
__device__ __forceinline__ void load_vals(const T* p, float (&o)[VEC]) {
    Vec<T, VEC> v = load_vec<T, VEC>(p);
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = v.get(i);
}

#ifndef M2_CONV_TILE
#define M2_CONV_TILE 64
#endif
#ifndef M2_CONV_GROUP
#define M2_CONV_GROUP 8
#endif
constexpr int kConvTileTokens = M2_CONV_TILE;  // tokens per lane
constexpr int kConvGroup = M2_CONV_GROUP;      // tokens per load group (one group in flight while the previous computes)
constexpr int kConvThreads = 256;

template <typename T, int VEC> struct Raw;
template <> struct Raw<bf16_t, 8> { using type = u32x4; };
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
template <> struct Raw<bf16_t, 4> { using type = u32x2v; };
template <> struct Raw<float, 4> { using type = u32x4; };
template <typename T> struct Raw<T, 1> { using type = T; };

template <typename T, int VEC>
__device__ __forceinline__ void unpack(const typename Raw<T, VEC>::type& r, float (&o)[VEC]) {
    if constexpr (VEC == 1) {
        o[0] = to_f32(r);
    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const uint32_t wd = r[i >> 1];
            o[i] = __uint_as_float((i & 1) ? (wd & 0xffff0000u) : (wd << 16));
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = __uint_as_float(r[i]);
    }
}

// Lane <-> (token tile, channel group): the channel group runs fastest, so a wave covers 64
// adjacent 16-byte channel groups of one token row (a contiguous 1 KiB) and every lane has work
// whatever conv_dim is.  Each lane walks TILE tokens of its VEC channels.
#ifndef M2_CONV_WPE
#define M2_CONV_WPE 1
#endif
template <typename T, int VEC, int W, int TILE>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, kConvThreads), amdgpu_waves_per_eu(M2_CONV_WPE)))
conv1d_silu_kernel(
    const T* __restrict__ xbc, int64_t xs, int64_t L, int Cd,
    const float* __restrict__ w, const float* __restrict__ bias,
    const T* __restrict__ ring_in, int ring_phase,
    T* __restrict__ ring_out, int64_t rs, T* __restrict__ out, int64_t os, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cu, int64_t total)
{
    using R = typename Raw<T, VEC>::type;
    const int CG = Cd / VEC;
    const int64_t ntiles = L > 0 ? (L + TILE - 1) / TILE : 1;
    const int64_t item = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (item >= ntiles * CG) return;
    const int c0 = (int)(item % CG) * VEC;
    const int64_t t0 = (item / CG) * TILE;
    const int64_t b = blockIdx.y;
    // Sequence b starts at row b*L, or at cu[b] in a packed batch, and ends at its own length
    // (clamped to the rows that exist and to L).  The tile that starts at token 0 always runs, so
    // that an empty sequence still writes its ring.
    int64_t row0 = b * L, Lb = L;
    if (cu) {
        const int64_t r0 = cu[b], r1 = cu[b + 1];
        row0 = r0 < 0 ? 0 : (r0 > total ? total : r0);
        const int64_t end = r1 < row0 ? row0 : (r1 > total ? total : r1);
        Lb = end - row0 < L ? end - row0 : L;
    } else if (lens) {
        const int64_t v = lens[b];
        Lb = v < 0 ? 0 : (v > L ? L : v);
    }
    if (t0 > 0 && t0 >= Lb) return;
    const T* xb = xbc + row0 * xs + c0;
    T* ob = out + row0 * os + c0;

    float wr[VEC][W], br[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
#pragma unroll
        for (int kk = 0; kk < W; ++kk) wr[i][kk] = w[(int64_t)(c0 + i) * W + kk];
        br[i] = bias ? bias[c0 + i] : 0.0f;
    }

    // win[kk] holds token (next - W + kk); win[W-1] is the newest
    float win[W][VEC];
#pragma unroll
    for (int kk = 0; kk < W; ++kk) {
        const int64_t tau = t0 - W + kk;
        if (tau >= 0 && kk > 0) {
            load_vals<T, VEC>(xb + tau * xs, win[kk]);
        } else if (tau < 0 && ring_in) {
            const int slot = (int)(((ring_phase + tau) % W + W) % W);
            load_vals<T, VEC>(ring_in + (b * W + slot) * rs + c0, win[kk]);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) win[kk][i] = 0.0f;  // no history, or never enters a sum
        }
    }

    const int64_t t_end = t0 + TILE < Lb ? t0 + TILE : Lb;
    const int n = (int)(t_end - t0);
    R cur[kConvGroup], nxt[kConvGroup];
    auto load_group = [&](R (&dst)[kConvGroup], int base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kConvGroup; ++u) {
            const int tt = base + u < n ? base + u : n - 1;  // clamped: rows past the end are never used
            // read once: streaming loads leave the cache to the output, which the scan reads next
            if constexpr (VEC > 1) dst[u] = __builtin_nontemporal_load(reinterpret_cast<const R*>(xb + (t0 + tt) * xs));
            else dst[u] = *reinterpret_cast<const R*>(xb + (t0 + tt) * xs);
        }
    };
    if (n > 0) load_group(cur, 0);
    for (int base = 0; base < n; base += kConvGroup) {
        if (base + kConvGroup < n) load_group(nxt, base + kConvGroup);
#pragma unroll
        for (int u = 0; u < kConvGroup; ++u) {
            if (base + u < n) {
#pragma unroll
                for (int kk = 0; kk < W - 1; ++kk)
#pragma unroll
                    for (int i = 0; i < VEC; ++i) win[kk][i] = win[kk + 1][i];
                unpack<T, VEC>(cur[u], win[W - 1]);
                float o[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    float v = br[i];
#pragma unroll
                    for (int kk = 0; kk < W; ++kk) v = fmaf(wr[i][kk], win[kk][i], v);
                    o[i] = silu(v);
                }
#if M2_CONV_NTSTORE
                if constexpr (VEC == 8 || (VEC == 4 && sizeof(T) == 4)) {
                    Vec<T, VEC> sv;
#pragma unroll
                    for (int i = 0; i < VEC; i += 2) sv.set2(i, o[i], o[i + 1]);
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sv.raw), reinterpret_cast<u32x4*>(ob + (t0 + base + u) * os));
                } else {
                    store_vals<T, VEC>(ob + (t0 + base + u) * os, o);
                }
#else
                store_vals<T, VEC>(ob + (t0 + base + u) * os, o);
#endif
            }
        }
#pragma unroll
        for (int u = 0; u < kConvGroup; ++u) cur[u] = nxt[u];
    }

    // the tile holding the last token writes the ring (phase 0: slot j = token Lb-W+j)
    if (ring_out && t_end == Lb) {
#pragma unroll
        for (int kk = 0; kk < W; ++kk) store_vals<T, VEC>(ring_out + (b * W + kk) * rs + c0, win[kk]);
    }
}

// Tokens per lane: kConvTileTokens, or fewer where the channels are too few for the grid to fill the
// chip (the B and C channels alone, in the fused prompt path): about 2048 blocks at least.
template <typename T, int VEC, int W, int TILE>
static hipError_t launch_conv_t(const ConvArgs& a, hipStream_t s) {
    const int64_t tiles = a.L > 0 ? (a.L + TILE - 1) / TILE : 1;
    const int64_t items = tiles * (a.Cd / VEC);
    dim3 grid((unsigned)((items + kConvThreads - 1) / kConvThreads), (unsigned)a.batch);
    return launch_kernel(conv1d_silu_kernel<T, VEC, W, TILE>, grid, dim3(kConvThreads), 0, s,
                         (const T*)a.xbc, a.xs, a.L, a.Cd, a.w, a.bias, (const T*)a.ring_in, a.ring_phase,
                         (T*)a.ring_out, a.rs, (T*)a.out, a.os, a.lens, a.cu, a.total);
}

template <typename T, int VEC, int W>
static hipError_t launch_conv(const ConvArgs& a, hipStream_t s) {
    const int64_t groups = (int64_t)(a.Cd / VEC) * a.batch * (a.L > 0 ? a.L : 1);  // lanes at one token per lane
    if (groups / kConvTileTokens >= 2048 * (int64_t)kConvThreads) return launch_conv_t<T, VEC, W, kConvTileTokens>(a, s);
    return launch_conv_t<T, VEC, W, 8>(a, s);
}

template <typename T, int VEC>
static hipError_t launch_conv_w(const ConvArgs& a, hipStream_t s) {
    switch (a.W) {
        case 2: return launch_conv<T, VEC, 2>(a, s);
        case 3: return launch_conv<T, VEC, 3>(a, s);
        default: return launch_conv<T, VEC, 4>(a, s);
    }
}

#ifndef M2_CONV_VEC
#define M2_CONV_VEC 4
#endif
hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s) {
    if (a.bf16) return a.vec ? launch_conv_w<bf16_t, M2_CONV_VEC>(a, s) : launch_conv_w<bf16_t, 1>(a, s);
    return a.vec ? launch_conv_w<float, 4>(a, s) : launch_conv_w<float, 1>(a, s);
}

}  // namespace m2
