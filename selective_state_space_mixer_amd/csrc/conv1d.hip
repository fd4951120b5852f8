// conv1d.hip -- causal depthwise conv1d + SiLU over a prompt (gfx950).
//
// The mixer's depthwise conv (article "Transformers 中 Zamba2 混合架构模型解析", §三:
// groups = conv_dim, kernel width mamba_d_conv, SiLU on the output):
//     out[b,t,c] = SiLU(bias[c] + sum_{k<W} w[c,k] * x[b, t-(W-1)+k, c])
//
// Pure HBM stream (3 flop per byte).  Each lane owns VEC adjacent channels (one 8-byte load per
// token for 4 bf16 channels) and walks a tile of consecutive tokens, keeping the last W inputs in
// registers, so every input is read from HBM once (plus a W-1 token halo per tile).  A wave covers
// 64*VEC contiguous channels of one token, so each load and store instruction moves one contiguous
// row segment.  Two kernels:
//   - conv1d_silu_ring_kernel (long prompts): buffer-resource addressing, a rolling ring of loads,
//     and a tile sized at launch so that the whole grid is resident at once;
//   - conv1d_silu_kernel (everything else: short or narrow launches, scalar channels, offsets past
//     2^31 bytes): fixed tiles of 64 tokens (8 for narrow launches), loads one 8-token group ahead.
#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

template <typename T, int VEC> struct Vec;
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

constexpr int kConvTileTokens = 64;  // tokens per lane (conv1d_silu_kernel)
constexpr int kConvGroup = 8;        // tokens per load group (one group in flight while the previous computes)
constexpr int kConvThreads = 256;

template <typename T, int VEC> struct Raw;
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

// Sequence b starts at row b*L, or at cu[b] in a packed batch, and ends at its own length (clamped
// to the rows that exist and to L).
struct SeqSpan { int64_t row0, len; };
__device__ __forceinline__ SeqSpan seq_span(int64_t b, int64_t L, const int32_t* lens, const int32_t* cu,
                                            int64_t total) {
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
    return SeqSpan{row0, Lb};
}

// Lane <-> (token tile, channel group): the channel group runs fastest, so a wave covers 64
// adjacent channel groups of one token row and every lane has work whatever conv_dim is.  Each lane
// walks TILE tokens of its VEC channels.  The tile that starts at token 0 always runs, so that an
// empty sequence still writes its ring.
template <typename T, int VEC, int W, int TILE>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, kConvThreads)))
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
    const SeqSpan sq = seq_span(b, L, lens, cu, total);
    const int64_t row0 = sq.row0, Lb = sq.len;
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
                store_vals<T, VEC>(ob + (t0 + base + u) * os, o);
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

// ----------------------------------------------------------------------------------------------
// The long-prompt kernel.  The same lane map and arithmetic, with three changes that matter on a
// 32k-token prompt:
//   - a rolling ring of DEPTH loads: token u+DEPTH is requested as soon as token u has been
//     consumed, so DEPTH loads stay in flight in DEPTH registers (not two groups' worth);
//   - buffer-resource addressing: a lane's offset is one 32-bit register and the token's row offset
//     is a scalar, instead of a 64-bit pointer per token of a group (110 -> 85 VGPRs, 4 -> 5 waves
//     per SIMD);
//   - a runtime tile, chosen by the launcher so that the grid is one resident round: every lane
//     starts together and pays its start-up (weights, halo, first ring of loads) once.
// Offsets past the sequence (the tail of the last tile, the ring's look-ahead past a tile) are
// pushed out of the resource's range, where loads return zero without touching memory and stores
// are dropped; so the loop has no branches, and the compiler's wait counts follow the ring exactly.
// The window runs on over that tail, so the ring written at the sequence's end is re-read from the
// rows.  Every offset a sequence forms stays below 2^31 bytes (checked by the launcher).

constexpr uint32_t kOutOfRange = 0x80000000u;  // past every resource range here (ranges are < 2^31)
constexpr int kStreamLoad = 2;                 // non-temporal: each input is read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t conv_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Loads and stores at a lane offset plus a scalar (row) offset.  When the lane offset is
// kOutOfRange the access is out of range whether or not the hardware counts the scalar part in its
// range check: the scalar part is below 2^31, so the sum neither wraps nor falls back into range.
template <typename T> struct BufIO;
template <> struct BufIO<bf16_t> {
    using R = u32x2v;
    static __device__ __forceinline__ R load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, kStreamLoad);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, const float (&o)[4]) {
        const u32x2v v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, (int)soff, 0);
    }
};
template <> struct BufIO<float> {
    using R = u32x4;
    static __device__ __forceinline__ R load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, kStreamLoad);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, const float (&o)[4]) {
        const u32x4 v = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, (int)soff, 0);
    }
};

// ring depth: 16 loads of 8 bytes for bf16, 8 of 16 bytes for fp32 (register budget)
template <typename T> constexpr int ring_depth() { return sizeof(T) == 2 ? 16 : 8; }

template <typename T, int W>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, kConvThreads)))
conv1d_silu_ring_kernel(
    const T* __restrict__ xbc, int64_t xs, int64_t L, int Cd,
    const float* __restrict__ w, const float* __restrict__ bias,
    const T* __restrict__ ring_in, int ring_phase,
    T* __restrict__ ring_out, int64_t rs, T* __restrict__ out, int64_t os, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cu, int64_t total, int tile)
{
    constexpr int VEC = 4, DEPTH = ring_depth<T>();
    using IO = BufIO<T>;
    using R = typename IO::R;
    const int CG = Cd / VEC;
    const int64_t ntiles = L > 0 ? (L + tile - 1) / tile : 1;
    const int64_t item = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (item >= ntiles * CG) return;
    const int c0 = (int)(item % CG) * VEC;
    const int64_t t0 = (item / CG) * tile;
    const int64_t b = blockIdx.y;
    const SeqSpan sq = seq_span(b, L, lens, cu, total);
    const int64_t row0 = sq.row0, Lb = sq.len;
    if (t0 > 0 && t0 >= Lb) return;
    const T* xb = xbc + row0 * xs + c0;
    // the sequence's rows; its last row ends at (Lb-1)*stride + Cd <= Lb*stride elements
    const auto rx = conv_rsrc(xbc + row0 * xs, (uint32_t)(Lb * xs * (int64_t)sizeof(T)));
    const auto ro = conv_rsrc(out + row0 * os, (uint32_t)(Lb * os * (int64_t)sizeof(T)));
    const uint32_t xstep = (uint32_t)(xs * (int64_t)sizeof(T)), ostep = (uint32_t)(os * (int64_t)sizeof(T));
    const uint32_t xoff = (uint32_t)t0 * xstep + (uint32_t)c0 * (uint32_t)sizeof(T);
    const uint32_t ooff = (uint32_t)t0 * ostep + (uint32_t)c0 * (uint32_t)sizeof(T);

    float wr[VEC][W], br[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
#pragma unroll
        for (int kk = 0; kk < W; ++kk) wr[i][kk] = w[(int64_t)(c0 + i) * W + kk];
        br[i] = bias ? bias[c0 + i] : 0.0f;
    }

    // token tau < Lb of the history: the row, or the caller's ring before the sequence, or zero
    auto history = [&](int64_t tau, float (&dst)[VEC]) __attribute__((always_inline)) {
        if (tau >= 0) {
            load_vals<T, VEC>(xb + tau * xs, dst);
        } else if (ring_in) {
            const int slot = (int)(((ring_phase + tau) % W + W) % W);
            load_vals<T, VEC>(ring_in + (b * W + slot) * rs + c0, dst);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) dst[i] = 0.0f;
        }
    };
    // win[kk] holds token (next - W + kk); win[0] is shifted out before it enters a sum
    float win[W][VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) win[0][i] = 0.0f;
#pragma unroll
    for (int kk = 1; kk < W; ++kk) history(t0 - W + kk, win[kk]);

    const int64_t t_end = t0 + tile < Lb ? t0 + tile : Lb;
    const int n = (int)(t_end - t0);
    R ring[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) ring[u] = IO::load(rx, u < n ? xoff : kOutOfRange, (uint32_t)u * xstep);
    for (int base = 0; base < n; base += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
#pragma unroll
            for (int kk = 0; kk < W - 1; ++kk)
#pragma unroll
                for (int i = 0; i < VEC; ++i) win[kk][i] = win[kk + 1][i];
            unpack<T, VEC>(ring[u], win[W - 1]);
            const int tn = base + DEPTH + u;
            ring[u] = IO::load(rx, tn < n ? xoff : kOutOfRange, (uint32_t)tn * xstep);
            float o[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                float v = br[i];
#pragma unroll
                for (int kk = 0; kk < W; ++kk) v = fmaf(wr[i][kk], win[kk][i], v);
                o[i] = silu(v);
            }
            const int tc = base + u;
            IO::store(ro, tc < n ? ooff : kOutOfRange, (uint32_t)tc * ostep, o);
            // keep the ring rolling: without this the scheduler gathers the loads at the end of the turn
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // the tile holding the last token writes the ring (phase 0: slot j = token Lb-W+j)
    if (ring_out && t_end == Lb) {
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            float v[VEC];
            history(Lb - W + kk, v);
            store_vals<T, VEC>(ring_out + (b * W + kk) * rs + c0, v);
        }
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

// The ring kernel's tile: as long as it can be while the whole grid is resident at once (every CU
// holding as many blocks as the kernel's registers allow).  Returns 0 where that tile would be
// shorter than two turns of the ring (a short or narrow launch, such as the B and C channels
// alone): there the fixed-tile kernel is faster, since the ring would mostly carry empty slots.
template <typename T, int W>
static int64_t ring_tile(const ConvArgs& a) {
    constexpr int VEC = 4, DEPTH = ring_depth<T>();
    static const int per_cu = [] {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)conv1d_silu_ring_kernel<T, W>,
                                                         kConvThreads, 0) != hipSuccess || nb < 1)
            nb = 4;
        return nb;
    }();
    // every offset of a sequence (rows up to L, plus the look-ahead of two ring turns) below 2^31
    constexpr int64_t lim = 0x7fffffff;
    const int64_t rows = a.L + 2 * DEPTH + 1;
    if (a.L <= 0 || rows * a.xs * (int64_t)sizeof(T) >= lim || rows * a.os * (int64_t)sizeof(T) >= lim) return 0;
    const int64_t lanes = (int64_t)(a.Cd / VEC) * a.batch;
    const int64_t slots = (int64_t)device_shape().cus * per_cu * kConvThreads;
    const int64_t tiles = slots / lanes;
    if (tiles < 1) return 0;
    const int64_t tile = (a.L + tiles - 1) / tiles;
    return tile >= 2 * DEPTH ? tile : 0;
}

template <typename T, int VEC, int W>
static hipError_t launch_conv(const ConvArgs& a, hipStream_t s) {
    if constexpr (VEC == 4) {
        const int64_t tile = ring_tile<T, W>(a);
        if (tile > 0) {
            const int64_t tiles = (a.L + tile - 1) / tile;
            dim3 grid((unsigned)((tiles * (a.Cd / VEC) + kConvThreads - 1) / kConvThreads), (unsigned)a.batch);
            return launch_kernel(conv1d_silu_ring_kernel<T, W>, grid, dim3(kConvThreads), 0, s, (const T*)a.xbc, a.xs,
                                 a.L, a.Cd, a.w, a.bias, (const T*)a.ring_in, a.ring_phase, (T*)a.ring_out, a.rs,
                                 (T*)a.out, a.os, a.lens, a.cu, a.total, (int)tile);
        }
    }
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

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s) {
    if (a.bf16) return a.vec ? launch_conv_w<bf16_t, 4>(a, s) : launch_conv_w<bf16_t, 1>(a, s);
    return a.vec ? launch_conv_w<float, 4>(a, s) : launch_conv_w<float, 1>(a, s);
}

}  // namespace m2
