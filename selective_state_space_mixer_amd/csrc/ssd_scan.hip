// ssd_scan.hip -- chunked selective state-space scan over a prompt (gfx950, MFMA).
//
// The Zamba2 mixer's prompt path (article "Transformers 中 Zamba2 混合架构模型解析",
// §三: the sequence is cut into chunks of chunk_size and scanned with an intra-chunk
// plus an inter-chunk pass).  For a chunk of Q tokens starting after state S_prev,
// with a_t = dt_t * A and Lam_t = the sum of a over the chunk up to and including t:
//
//   y_t   = exp(Lam_t) * (S_prev . C_t)                                   (state part)
//         + sum_{s<=t} exp(Lam_t - Lam_s) * dt_s * (C_t . B_s) * x_s       (intra-chunk part)
//         + D * x_t
//   S_new = exp(Lam_end) * S_prev + sum_s exp(Lam_end - Lam_s) * dt_s * x_s (outer) B_s
//
// which is the token recurrence S_t = exp(dt_t A) S_{t-1} + dt_t x_t B_t^T, y_t = S_t C_t + D x_t
// unrolled over the chunk (exactly, up to rounding).
//
// One workgroup walks the chunks of one (sequence, head, segment) in order and keeps
// the fp32 state in MFMA accumulator registers for the whole walk.  Per chunk, four
// contractions run on v_mfma_f32_16x16x32_bf16 (fp32 activations: v_mfma_f32_16x16x4f32):
//   G^T[s][t] = sum_n B[s][n] C[t][n]            -> masked and scaled -> M[t][s] in LDS
//                                                   (bf16: as a hi + lo pair, see below)
//   Y^T[p][t] = sum_n S[p][n] (e^Lam_t C[t][n])   (state part, state as the A operand)
//   Y^T[p][t]+= sum_s X[s][p] M[t][s]             (intra-chunk part)
//   S^T[n][p] = e^Lam_end S^T[n][p] + sum_s B[s][n] (w_s X[s][p]),  w_s = e^(Lam_end-Lam_s) dt_s
// The e^Lam_t factor of the state part is applied to the output tile, w_s scales the X fragments
// already in registers, and the D skip is folded into M's diagonal, so the per-element work
// outside the MFMAs is one pass over M.
// Wave w owns p-block(s) w of the state and of the output, so the state never leaves
// its registers; only M (the same for every p-block) goes through LDS.  Operands whose
// contraction index runs down the rows of a row-major LDS tile (X and B over tokens) are
// read with ds_read_b64_tr_b16, which hands each lane four consecutive rows of one column.
//
// M carries the whole intra-chunk weight of a token on itself and its neighbours; where the
// decay is strong those terms are large and cancel, so a single bf16 rounding of M costs
// several percent of y.  M is therefore stored as bf16 hi = rn(M) and lo = rn(M - hi) and the
// intra contraction runs twice, which leaves M's error near 2^-17.
//
// Long sequences with few (sequence, head) pairs are split into segments that run in
// parallel: a first pass computes each segment's end state from a zero start, a small
// pass chains those into each segment's true initial state, and the main pass then
// walks every segment from its initial state.
#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

#define M2_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // native vector: stays in registers

// ----------------------------------------------------------------------------------------------
// element types

template <typename T> struct Lds;
template <> struct Lds<bf16_t> { using E = uint16_t; static constexpr int PAD = 8; };
template <> struct Lds<float> { using E = float; static constexpr int PAD = 4; };

// Eight k-values of one lane for a K=32 MFMA step: chunk 0 holds k = kbase+4q+{0..3},
// chunk 1 holds k = kbase+16+4q+{0..3} (q = lane/16).  Both operands of a product use the
// same assignment, so the sum runs over every k exactly once.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
    uint32_t w[4];
    __device__ __forceinline__ void set(int c, float a0, float a1, float a2, float a3) {
        w[2 * c] = pack_bf16x2(a0, a1);
        w[2 * c + 1] = pack_bf16x2(a2, a3);
    }
    __device__ __forceinline__ float get(int c, int e) const {
        const uint32_t v = w[2 * c + (e >> 1)];
        return __uint_as_float((e & 1) ? (v & 0xffff0000u) : (v << 16));
    }
};
template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void set(int c, float a0, float a1, float a2, float a3) {
        v[4 * c] = a0; v[4 * c + 1] = a1; v[4 * c + 2] = a2; v[4 * c + 3] = a3;
    }
    __device__ __forceinline__ float get(int c, int e) const { return v[4 * c + e]; }
};

__device__ __forceinline__ void mfma(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.w),
                                                  __builtin_bit_cast(bf16x8_t, b.w), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// chunk c of a fragment from a row-major LDS tile whose k index runs along the row
__device__ __forceinline__ void chunk_row(Frag<bf16_t>& f, int c, const uint16_t* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    f.w[2 * c] = v.x;
    f.w[2 * c + 1] = v.y;
}
__device__ __forceinline__ void chunk_row(Frag<float>& f, int c, const float* p) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    f.set(c, v.x, v.y, v.z, v.w);
}

// Fragment with k along a row: the lane supplies `row`, k = kbase + 4q (+16); kext = k extent.
template <typename T>
__device__ __forceinline__ Frag<T> frag_row(const typename Lds<T>::E* tile, int stride, int row, int kbase,
                                            int kext, int q) {
    Frag<T> f;
    chunk_row(f, 0, tile + row * stride + kbase + 4 * q);
    if (kbase + 16 < kext) chunk_row(f, 1, tile + row * stride + kbase + 16 + 4 * q);
    else f.set(1, 0.f, 0.f, 0.f, 0.f);
    return f;
}

// Chunk c of a fragment whose k index runs down the rows: lane (q, i) gets rows r0+4q..r0+4q+3
// of column col0+i.  bf16: one ds_read_b64_tr_b16 (lane i addresses row i/4, columns 4(i%4)..+3
// of its 16-lane group's 4x16 block and receives column i of the block).
__device__ __forceinline__ void chunk_col(Frag<bf16_t>& f, int c, const uint16_t* tile, int stride, int r0, int col0,
                                          int q, int i) {
    const uint16_t* p = tile + (r0 + 4 * q + (i >> 2)) * stride + col0 + 4 * (i & 3);
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((M2_LDS i16x4_t*)(p));
    const uint2 u = __builtin_bit_cast(uint2, v);
    f.w[2 * c] = u.x;
    f.w[2 * c + 1] = u.y;
}
__device__ __forceinline__ void chunk_col(Frag<float>& f, int c, const float* tile, int stride, int r0, int col0,
                                          int q, int i) {
    const float* p = tile + (r0 + 4 * q) * stride + col0 + i;
    f.set(c, p[0], p[stride], p[2 * stride], p[3 * stride]);
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_col(const typename Lds<T>::E* tile, int stride, int kbase, int kext,
                                            int col0, int q, int i) {
    Frag<T> f;
    chunk_col(f, 0, tile, stride, kbase, col0, q, i);
    if (kbase + 16 < kext) chunk_col(f, 1, tile, stride, kbase + 16, col0, q, i);
    else f.set(1, 0.f, 0.f, 0.f, 0.f);
    return f;
}

// four consecutive elements of a row as fp32, and back
__device__ __forceinline__ void row4(const uint16_t* p, float (&o)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void row4(const float* p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void put4(uint16_t* p, float a0, float a1, float a2, float a3) {
    uint2 v;
    v.x = pack_bf16x2(a0, a1);
    v.y = pack_bf16x2(a2, a3);
    *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ void put4(float* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<float4*>(p) = make_float4(a0, a1, a2, a3);
}
__device__ __forceinline__ void put4g(bf16_t* p, float a0, float a1, float a2, float a3) {
    put4(reinterpret_cast<uint16_t*>(p), a0, a1, a2, a3);
}
__device__ __forceinline__ void put4g(float* p, float a0, float a1, float a2, float a3) { put4(p, a0, a1, a2, a3); }

// ----------------------------------------------------------------------------------------------
// kernel parameters

struct ScanK {
    const void* x; const void* B; const void* C; const void* dt;
    int64_t xs, bcs, dts, ys;
    const float* dt_bias; const float* A; const float* D;
    float dt_min, dt_max;
    const float* state_in; float* state_out;
    void* y;
    float* ws_state;   // [nseg][batch*H][P*N]: segment end states, then segment initial states
    float* ws_lam;     // [nseg][batch*H]: summed log-decay of each segment
    int64_t L;
    int batch, H, G;
    int nseg, cps;     // segments per sequence, chunks per segment
    int nblocks;       // blocks in this launch
};

// Block -> logical unit.  Consecutive blocks are dealt round-robin to the 8 XCDs; the remap
// gives each XCD a contiguous run of logical units (the head groups of one sequence and
// segment), so the B/C rows those heads share are fetched into one L2.  XCD x receives
// n/8 blocks, plus one if x < n%8; its run starts after those of XCDs 0..x-1.
__device__ __forceinline__ int logical_block(int nblocks) {
    const int i = blockIdx.x;
    const int x = i % 8, per = nblocks / 8, extra = nblocks % 8;
    return x * per + (x < extra ? x : extra) + i / 8;
}

constexpr int kScanThreads = 256;  // four waves
#ifndef M2_SCAN_STATE_TILES
#define M2_SCAN_STATE_TILES 16
#endif
constexpr int kStateTiles = M2_SCAN_STATE_TILES;  // 16x16 state tiles per wave (PW * NNB)

// Work split: each wave owns PW p-blocks of one head, so its share of the state (PW x NNB
// accumulator tiles) stays within kStateTiles tiles (64 registers at 16: a whole 64x64 head per
// wave, so the decay mask of a head is computed once); WPH waves cover a head and the
// block holds HPW = 4 / WPH heads of one B/C group, which share the B and C tiles and G = B C^T.
template <typename T, int Q, int P, int N>
struct Cfg {
    using E = typename Lds<T>::E;
    static constexpr int NPB = P / 16;
    static constexpr int NNB = N / 16;
    static constexpr int NTB = Q / 16;
    static constexpr int PW_CAP = kStateTiles / NNB > 0 ? kStateTiles / NNB : 1;
    static constexpr int PW0 = NPB < PW_CAP ? NPB : PW_CAP;
    static constexpr int PW = PW0 > NPB / 4 ? PW0 : NPB / 4;  // at most four waves per head
    static constexpr int WPH = NPB / PW;          // waves per head
    static constexpr int HPW = 4 / WPH;           // heads per block
    static_assert(WPH >= 1 && WPH <= 4 && HPW * WPH == 4, "work split");
    static constexpr int XST = P + Lds<T>::PAD;   // LDS row strides (elements)
    static constexpr int BST = N + Lds<T>::PAD;
    static constexpr int EPU = 16 / (int)sizeof(E);  // elements per 16-byte unit
    static constexpr int XU = P / EPU, BU = N / EPU;
    static constexpr int KS_N = (N + 31) / 32;    // K=32 steps over d_state
    static constexpr int KS_Q = (Q + 31) / 32;    // K=32 steps over tokens
    // s-blocks that t-block tb's K=32 steps over tokens read: sb < 2*(tb/2)+2 (and < NTB)
    static constexpr int tiles_in_row(int tb) { return 2 * (tb / 2) + 2 < NTB ? 2 * (tb / 2) + 2 : NTB; }
    static constexpr int row_base(int tb) {
        int n = 0;
        for (int r = 0; r < tb; ++r) n += tiles_in_row(r);
        return n;
    }
    static constexpr int NTILES = row_base(NTB);
};

// Loads of a tile in 16-byte units: U units per row, RPP rows per pass, NP passes over R rows.
template <int U, int R>
struct TilePlan {
    static constexpr int RPP = kScanThreads / U;
    static constexpr int NP = (R + RPP - 1) / RPP;
    static constexpr bool kGuard = (R % RPP) != 0;  // some passes run past the last row
};

// ----------------------------------------------------------------------------------------------
// chunk walk.  kStateOnly: segment end state from a zero start (no C, no output).

template <typename T, int Q, int P, int N, bool kStateOnly>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(2)))
void ssd_chunk_scan_kernel(ScanK k)
{
    using Cf = Cfg<T, Q, P, N>;
    using E = typename Cf::E;
    constexpr int XST = Cf::XST, BST = Cf::BST, EPU = Cf::EPU, HPW = Cf::HPW, PW = Cf::PW;
    using PX = TilePlan<Cf::XU * HPW, Q>;  // the block's heads are adjacent in a token row
    using PB = TilePlan<Cf::BU, Q>;
    constexpr bool kSplitM = sizeof(E) == 2;  // bf16 operands: M as hi + lo

    __shared__ __attribute__((aligned(16))) E Xs[HPW * Q * XST];
    __shared__ __attribute__((aligned(16))) E Bs[Q * BST];
    __shared__ __attribute__((aligned(16))) E Cs[kStateOnly ? 8 : Q * BST];
    __shared__ __attribute__((aligned(16))) float Gs[kStateOnly ? 4 : Cf::NTILES * 256];
    __shared__ __attribute__((aligned(16))) float sLam[HPW * Q];
    __shared__ __attribute__((aligned(16))) float sDt[HPW * Q];
    __shared__ __attribute__((aligned(16))) float sW[HPW * Q];
    __shared__ __attribute__((aligned(16))) float sExpL[HPW * Q];
    __shared__ __attribute__((aligned(16))) float sGs[HPW * Q];  // e^(Lam_e(s) - Lam_s) dt_s, e(s) = last token of s's 16-block
    __shared__ float sEnd[HPW];

    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, li = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = wave / Cf::WPH;                  // head slot of this wave
    const int pblk0 = (wave % Cf::WPH) * PW;        // first p-block of this wave
    const bool stats_writer = (wave % Cf::WPH) == 0;

    // logical unit -> (segment, sequence, head group)
    const int unit = logical_block(k.nblocks);
    const int hpg = k.H / k.G;
    const int upg = (hpg + HPW - 1) / HPW;          // head units per group
    const int nhu = k.G * upg;
    const int hu = unit % nhu;
    const int sb_ = unit / nhu;
    const int64_t b = sb_ % k.batch;
    const int seg = sb_ / k.batch;
    const int g = hu / upg;
    const int h0 = g * hpg + (hu % upg) * HPW;
    const int hcount = hpg - (hu % upg) * HPW < HPW ? hpg - (hu % upg) * HPW : HPW;  // heads present
    const int h = h0 + (hw < hcount ? hw : hcount - 1);  // waves past the last head repeat it (results unused)
    const bool hvalid = hw < hcount;
    const int bh = (int)b * k.H + h;
    const int BH = k.batch * k.H;
    const int64_t nchunks = (k.L + Q - 1) / Q;
    const int64_t c_begin = (int64_t)seg * k.cps;
    const int64_t c_end = c_begin + k.cps < nchunks ? c_begin + k.cps : nchunks;
    const float bias_h = k.dt_bias[h], A_h = k.A[h];
    const float D_h = k.D ? k.D[h] : 0.0f;

    // per-thread tile coordinates and global base pointers
    const int xr0 = tid / (Cf::XU * HPW), xu = tid % (Cf::XU * HPW);
    int xh = xu / Cf::XU;                                  // head slot of this thread's X unit
    xh = xh < hcount ? xh : hcount - 1;
    const int xc = (xu % Cf::XU) * EPU;
    const int br0 = tid / Cf::BU, bc = (tid % Cf::BU) * EPU;
    const T* xg = reinterpret_cast<const T*>(k.x) + b * k.L * k.xs + (int64_t)(h0 + xh) * P + xc;
    const T* bgp = reinterpret_cast<const T*>(k.B) + b * k.L * k.bcs + (int64_t)g * N + bc;
    const T* cgp = reinterpret_cast<const T*>(k.C) + b * k.L * k.bcs + (int64_t)g * N + bc;
    const T* dtg = reinterpret_cast<const T*>(k.dt) + b * k.L * k.dts + h;
    E* const xdst = Xs + (xu / Cf::XU) * Q * XST + xc;      // this thread's X column in its head's tile
    const E* const Xh = Xs + hw * Q * XST;                  // this wave's head tile
    float* const lamh = sLam + hw * Q;
    float* const dth = sDt + hw * Q;
    float* const wh = sW + hw * Q;
    float* const elh = sExpL + hw * Q;
    float* const gsh = sGs + hw * Q;

    // state tiles in accumulator layout: accS[pw][nb][j] = S[p = (pblk0+pw)*16 + li][n = nb*16 + 4q + j]
    f32x4 accS[PW][Cf::NNB];
    {
        const float* src = nullptr;
        if (!kStateOnly) {
            if (seg == 0) src = k.state_in ? k.state_in + (int64_t)bh * P * N : nullptr;
            else src = k.ws_state + ((int64_t)(seg - 1) * BH + bh) * P * N;
        }
#pragma unroll
        for (int pw = 0; pw < PW; ++pw) {
            const int p = (pblk0 + pw) * 16 + li;
#pragma unroll
            for (int nb = 0; nb < Cf::NNB; ++nb) {
                if (src) {
                    const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)p * N + nb * 16 + 4 * q);
                    accS[pw][nb] = f32x4{v.x, v.y, v.z, v.w};
                } else {
                    accS[pw][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }

    // Register prefetch of one chunk (+ raw dt, one token per lane of every wave).  Loads are
    // issued without divergent branches (rows clamped into the sequence on the last chunk) and
    // stay raw until commit(), so nothing waits on them before the next chunk starts.  Both
    // helpers are forced inline: a prefetch array left in scratch would make every load synchronous.
    u32x4_t px[PX::NP], pbv[PB::NP], pcv[kStateOnly ? 1 : PB::NP];
    T pre_dt;
    auto prefetch = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t t0 = c * Q;
        const int valid = (int)(k.L - t0 < Q ? k.L - t0 : Q);
        const bool full = valid == Q;
#pragma unroll
        for (int i = 0; i < PX::NP; ++i) {
            int r = xr0 + i * PX::RPP;
            if (PX::kGuard && r >= Q) r = Q - 1;
            if (!full) r = r < valid ? r : valid - 1;
            px[i] = *reinterpret_cast<const u32x4_t*>(xg + (t0 + r) * k.xs);
        }
#pragma unroll
        for (int i = 0; i < PB::NP; ++i) {
            int r = br0 + i * PB::RPP;
            if (PB::kGuard && r >= Q) r = Q - 1;
            if (!full) r = r < valid ? r : valid - 1;
            pbv[i] = *reinterpret_cast<const u32x4_t*>(bgp + (t0 + r) * k.bcs);
            if constexpr (!kStateOnly) pcv[i] = *reinterpret_cast<const u32x4_t*>(cgp + (t0 + r) * k.bcs);
        }
        pre_dt = dtg[(t0 + (lane < valid ? lane : valid - 1)) * k.dts];
    };
    auto commit = [&](int64_t c) __attribute__((always_inline)) {
        const int valid = (int)(k.L - c * Q < Q ? k.L - c * Q : Q);
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        if (valid < Q) {  // the last chunk of the sequence: zero the rows past its end
#pragma unroll
            for (int i = 0; i < PX::NP; ++i) px[i] = xr0 + i * PX::RPP < valid ? px[i] : zero;
#pragma unroll
            for (int i = 0; i < PB::NP; ++i) {
                pbv[i] = br0 + i * PB::RPP < valid ? pbv[i] : zero;
                if constexpr (!kStateOnly) pcv[i] = br0 + i * PB::RPP < valid ? pcv[i] : zero;
            }
        }
#pragma unroll
        for (int i = 0; i < PX::NP; ++i) {
            const int r = xr0 + i * PX::RPP;
            if (!PX::kGuard || r < Q) *reinterpret_cast<u32x4_t*>(xdst + r * XST) = px[i];
        }
#pragma unroll
        for (int i = 0; i < PB::NP; ++i) {
            const int r = br0 + i * PB::RPP;
            if (!PB::kGuard || r < Q) {
                *reinterpret_cast<u32x4_t*>(Bs + r * BST + bc) = pbv[i];
                if constexpr (!kStateOnly) *reinterpret_cast<u32x4_t*>(Cs + r * BST + bc) = pcv[i];
            }
        }
        // dt and the cumulative log-decay of this wave's head over the chunk
        const float dtv = lane < valid ? dt_of(to_f32(pre_dt), bias_h, k.dt_min, k.dt_max) : 0.0f;
        const float lam = wave_prefix_sum(dtv * A_h);
        const float lam_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), Q - 1));
        // log-decay at the last token of this lane's 16-token block
        const float lam_blk = __shfl(lam, lane | 15, 64);
        if (stats_writer) {
            if (lane < Q) {
                lamh[lane] = lam;
                dth[lane] = dtv;
                wh[lane] = fast_exp(lam_end - lam) * dtv;
                elh[lane] = fast_exp(lam);
                gsh[lane] = fast_exp(lam_blk - lam) * dtv;
            }
            if (lane == 0) sEnd[hw] = lam_end;
        }
    };

    float lam_seg = 0.0f;  // summed log-decay of the segment (state-only pass)
    if (c_begin < c_end) prefetch(c_begin);
    for (int64_t c = c_begin; c < c_end; ++c) {
        commit(c);
        __syncthreads();  // tiles and chunk statistics in LDS
        if (c + 1 < c_end) prefetch(c + 1);
        const int64_t t0 = c * Q;
        const int valid = (int)(k.L - t0 < Q ? k.L - t0 : Q);
        const float lam_end = sEnd[hw];
        lam_seg += lam_end;

        if constexpr (!kStateOnly) {
            // ---- G^T[s][t] = sum_n B[s][n] C[t][n] for the tiles the K=32 token steps read, shared by
            // the block's heads; stored in accumulator layout (lane l owns 4 consecutive floats).
            constexpr int TPW = (Cf::NTILES + 3) / 4;
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                int id = wave + 4 * i;
                id = id < Cf::NTILES ? id : Cf::NTILES - 1;
                int tb = 0;
#pragma unroll
                for (int tt = 1; tt < Cf::NTB; ++tt) tb += id >= Cf::row_base(tt) ? 1 : 0;
                int base = 0;
#pragma unroll
                for (int tt = 1; tt < Cf::NTB; ++tt) base = id >= Cf::row_base(tt) ? Cf::row_base(tt) : base;
                const int sb = id - base;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < Cf::KS_N; ++ks) {
                    const Frag<T> fa = frag_row<T>(Bs, BST, sb * 16 + li, 32 * ks, N, q);
                    const Frag<T> fb = frag_row<T>(Cs, BST, tb * 16 + li, 32 * ks, N, q);
                    mfma(acc, fa, fb);
                }
                *reinterpret_cast<f32x4*>(Gs + id * 256 + lane * 4) = acc;
            }
        }

        // X fragments of this wave's head (k = token s, column p): A operand of the intra part
        Frag<T> xf[PW][Cf::KS_Q];
#pragma unroll
        for (int pw = 0; pw < PW; ++pw)
#pragma unroll
            for (int ks = 0; ks < Cf::KS_Q; ++ks)
                xf[pw][ks] = frag_col<T>(Xh, XST, 32 * ks, Q, (pblk0 + pw) * 16, q, li);

        if constexpr (!kStateOnly) {
            __syncthreads();  // G complete
            // state as the A operand of the state part: sa[pw][ks] covers n = 32ks .. 32ks+31
            Frag<T> sa[PW][Cf::KS_N];
#pragma unroll
            for (int pw = 0; pw < PW; ++pw)
#pragma unroll
                for (int ks = 0; ks < Cf::KS_N; ++ks) {
                    const f32x4 s0v = accS[pw][2 * ks];
                    sa[pw][ks].set(0, s0v[0], s0v[1], s0v[2], s0v[3]);
                    if (2 * ks + 1 < Cf::NNB) {
                        const f32x4 s1v = accS[pw][2 * ks + 1];
                        sa[pw][ks].set(1, s1v[0], s1v[1], s1v[2], s1v[3]);
                    } else {
                        sa[pw][ks].set(1, 0.f, 0.f, 0.f, 0.f);
                    }
                }
            T* yb = reinterpret_cast<T*>(k.y) + (b * k.L + t0) * k.ys + (int64_t)h * P;
#pragma unroll
            for (int tb = 0; tb < Cf::NTB; ++tb) {
                const int t = tb * 16 + li;
                f32x4 accY[PW];
#pragma unroll
                for (int pw = 0; pw < PW; ++pw) accY[pw] = f32x4{0.f, 0.f, 0.f, 0.f};
                // state part: Y^T[p][t] = e^Lam_t * sum_n S[p][n] C[t][n]
#pragma unroll
                for (int ks = 0; ks < Cf::KS_N; ++ks) {
                    const Frag<T> cf = frag_row<T>(Cs, BST, t, 32 * ks, N, q);
#pragma unroll
                    for (int pw = 0; pw < PW; ++pw) mfma(accY[pw], sa[pw][ks], cf);
                }
                const float lt = lamh[t];
                const float el = elh[t];
#pragma unroll
                for (int pw = 0; pw < PW; ++pw) accY[pw] *= el;
                // intra part: M[t][s] = G[t][s] e^(Lam_t - Lam_s) dt_s for s <= t, + D on the diagonal
#pragma unroll
                for (int ks = 0; ks < Cf::KS_Q; ++ks) {
                    if (32 * ks > tb * 16 + 15) continue;
                    Frag<T> mh, ml;
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const int sb = 2 * ks + cc;
                        if (sb >= Cf::tiles_in_row(tb) || sb > tb) {  // above the diagonal (or absent): zero
                            mh.set(cc, 0.f, 0.f, 0.f, 0.f);
                            ml.set(cc, 0.f, 0.f, 0.f, 0.f);
                            continue;
                        }
                        const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + (Cf::row_base(tb) + sb) * 256 + lane * 4);
                        const int s0 = sb * 16 + 4 * q;
                        float m[4];
                        if (sb < tb) {
                            // below the diagonal: e^(Lam_t - Lam_s) = e^(Lam_t - Lam_e) e^(Lam_e - Lam_s), both
                            // factors <= 1 (e = last token of block sb), the second precomputed per token
                            const float f = fast_exp(lt - lamh[sb * 16 + 15]);
                            const float4 gs = *reinterpret_cast<const float4*>(gsh + s0);
                            m[0] = gv[0] * f * gs.x; m[1] = gv[1] * f * gs.y;
                            m[2] = gv[2] * f * gs.z; m[3] = gv[3] * f * gs.w;
                        } else {
                            const float4 ls = *reinterpret_cast<const float4*>(lamh + s0);
                            const float4 ds = *reinterpret_cast<const float4*>(dth + s0);
                            const float lsv[4] = {ls.x, ls.y, ls.z, ls.w}, dsv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float v = gv[j] * fast_exp(lt - lsv[j]) * dsv[j];
                                m[j] = (s0 + j <= t ? v : 0.0f) + (s0 + j == t ? D_h : 0.0f);
                            }
                        }
                        if constexpr (kSplitM) {
                            const uint32_t h01 = pack_bf16x2(m[0], m[1]), h23 = pack_bf16x2(m[2], m[3]);
                            mh.w[2 * cc] = h01;
                            mh.w[2 * cc + 1] = h23;
                            ml.w[2 * cc] = pack_bf16x2(m[0] - lo_bf16(h01), m[1] - hi_bf16(h01));
                            ml.w[2 * cc + 1] = pack_bf16x2(m[2] - lo_bf16(h23), m[3] - hi_bf16(h23));
                        } else {
                            mh.set(cc, m[0], m[1], m[2], m[3]);
                        }
                    }
#pragma unroll
                    for (int pw = 0; pw < PW; ++pw) {
                        mfma(accY[pw], xf[pw][ks], mh);
                        if constexpr (kSplitM) mfma(accY[pw], xf[pw][ks], ml);
                    }
                }
                // store: the lane holds y[t][p = (pblk0+pw)*16 + 4q .. +3]
                if (hvalid && t < valid) {
#pragma unroll
                    for (int pw = 0; pw < PW; ++pw) {
                        const f32x4 a = accY[pw];
                        put4g(yb + t * k.ys + (pblk0 + pw) * 16 + 4 * q, a[0], a[1], a[2], a[3]);
                    }
                }
            }
        }

        // ---- state update: S^T[n][p] = e^Lam_end S^T[n][p] + sum_s B[s][n] (w_s X[s][p])
        const float decay = fast_exp(lam_end);
#pragma unroll
        for (int pw = 0; pw < PW; ++pw)
#pragma unroll
            for (int nb = 0; nb < Cf::NNB; ++nb) accS[pw][nb] *= decay;
#pragma unroll
        for (int ks = 0; ks < Cf::KS_Q; ++ks) {
            Frag<T> xw[PW];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int s0 = 32 * ks + 16 * cc + 4 * q;
                const float4 wv = s0 < Q ? *reinterpret_cast<const float4*>(wh + s0) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int pw = 0; pw < PW; ++pw)
                    xw[pw].set(cc, xf[pw][ks].get(cc, 0) * wv.x, xf[pw][ks].get(cc, 1) * wv.y,
                               xf[pw][ks].get(cc, 2) * wv.z, xf[pw][ks].get(cc, 3) * wv.w);
            }
#pragma unroll
            for (int nb = 0; nb < Cf::NNB; ++nb) {
                const Frag<T> bf = frag_col<T>(Bs, BST, 32 * ks, Q, nb * 16, q, li);
#pragma unroll
                for (int pw = 0; pw < PW; ++pw) mfma(accS[pw][nb], bf, xw[pw]);
            }
        }
        __syncthreads();  // LDS tiles free for the next chunk
    }

    // ---- write the state: S[p][n..n+3] per lane
    float* dst = nullptr;
    if (kStateOnly) dst = k.ws_state + ((int64_t)seg * BH + bh) * P * N;
    else if (seg == k.nseg - 1) dst = k.state_out ? k.state_out + (int64_t)bh * P * N : nullptr;
    if (dst && hvalid) {
#pragma unroll
        for (int pw = 0; pw < PW; ++pw) {
            const int p = (pblk0 + pw) * 16 + li;
#pragma unroll
            for (int nb = 0; nb < Cf::NNB; ++nb) {
                const f32x4 v = accS[pw][nb];
                *reinterpret_cast<float4*>(dst + (int64_t)p * N + nb * 16 + 4 * q) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
    if (kStateOnly && hvalid && (wave % Cf::WPH) == 0 && lane == 0) k.ws_lam[(int64_t)seg * BH + bh] = lam_seg;
}

// Chain the segments: S_in[seg+1] = exp(lam[seg]) * S_in[seg] + S_end_local[seg], written over
// S_end_local[seg] (so that segment seg+1 finds its initial state at index seg).  Only the
// combine is sequential: the loads of a batch of segments are issued together.
__global__ __launch_bounds__(256) void ssd_segment_chain_kernel(const float* __restrict__ state_in,
                                                                float* __restrict__ ws_state,
                                                                const float* __restrict__ ws_lam, int BH, int nseg,
                                                                int PN)
{
    constexpr int kBatch = 16;
    const int bh = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= PN) return;
    float s = state_in ? state_in[(int64_t)bh * PN + i] : 0.0f;
    for (int seg0 = 0; seg0 + 1 < nseg; seg0 += kBatch) {
        float loc[kBatch], dec[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int seg = seg0 + j < nseg - 1 ? seg0 + j : nseg - 2;
            loc[j] = ws_state[((int64_t)seg * BH + bh) * PN + i];
            dec[j] = ws_lam[(int64_t)seg * BH + bh];
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (seg0 + j < nseg - 1) {
                s = fast_exp(dec[j]) * s + loc[j];
                ws_state[((int64_t)(seg0 + j) * BH + bh) * PN + i] = s;
            }
        }
    }
}

// ----------------------------------------------------------------------------------------------
// host side

struct Plan {
    int nseg, cps, nhu;
    size_t ws_bytes;
};

// Heads per block for the (P, N) work split (see Cfg).
static int heads_per_block(int P, int N) {
    const int npb = P / 16, nnb = N / 16;
    const int cap = kStateTiles / nnb > 0 ? kStateTiles / nnb : 1;
    int pw = npb < cap ? npb : cap;
    pw = pw > npb / 4 ? pw : npb / 4;
    return 4 / (npb / pw);
}

static Plan plan_for(int64_t batch, int64_t L, int H, int G, int P, int N, int Q) {
    Plan pl;
    const int64_t nchunks = (L + Q - 1) / Q;
    const int hpw = heads_per_block(P, N);
    const int hpg = H / G;
    pl.nhu = G * ((hpg + hpw - 1) / hpw);
    const int64_t units = batch * pl.nhu;
    // one round of resident blocks: two per compute unit on 256 CUs
    const int64_t target = 512;
    int64_t nseg = units > 0 ? target / units : 1;
    if (nseg > nchunks) nseg = nchunks;
    if (nseg < 1) nseg = 1;
    const int64_t cps = nchunks > 0 ? (nchunks + nseg - 1) / nseg : 1;
    nseg = nchunks > 0 ? (nchunks + cps - 1) / cps : 1;
    pl.nseg = (int)nseg;
    pl.cps = (int)cps;
    pl.ws_bytes = nseg > 1 ? (size_t)(nseg * batch * H) * ((size_t)P * N + 1) * sizeof(float) + 256 : 0;
    return pl;
}

template <typename T, int Q, int P, int N>
static hipError_t run_scan(const ScanArgs& a, hipStream_t s) {
    const Plan pl = plan_for(a.batch, a.L, a.H, a.G, a.P, a.N, Q);
    ScanK k;
    k.x = a.x; k.B = a.B; k.C = a.C; k.dt = a.dt;
    k.xs = a.xs; k.bcs = a.bcs; k.dts = a.dts; k.ys = a.ys;
    k.dt_bias = a.dt_bias; k.A = a.A; k.D = a.D; k.dt_min = a.dt_min; k.dt_max = a.dt_max;
    k.state_in = a.state_in; k.state_out = a.state_out; k.y = a.y;
    k.L = a.L; k.batch = (int)a.batch; k.H = a.H; k.G = a.G;
    k.nseg = pl.nseg; k.cps = pl.cps;
    const int BH = (int)(a.batch * a.H);
    k.ws_state = nullptr;
    k.ws_lam = nullptr;
    if (pl.nseg > 1) {
        k.ws_state = reinterpret_cast<float*>(a.ws);
        k.ws_lam = k.ws_state + (size_t)pl.nseg * BH * P * N;
    }
    hipError_t e;
    const int per_seg = (int)a.batch * pl.nhu;
    if (pl.nseg > 1) {
        k.nblocks = (pl.nseg - 1) * per_seg;
        e = launch_kernel(ssd_chunk_scan_kernel<T, Q, P, N, true>, dim3(k.nblocks), dim3(kScanThreads), 0, s, k);
        if (e != hipSuccess) return e;
        dim3 g2((unsigned)((P * N + 255) / 256), (unsigned)BH);
        e = launch_kernel(ssd_segment_chain_kernel, g2, dim3(256), 0, s, a.state_in, k.ws_state,
                          (const float*)k.ws_lam, BH, pl.nseg, P * N);
        if (e != hipSuccess) return e;
    }
    k.nblocks = pl.nseg * per_seg;
    return launch_kernel(ssd_chunk_scan_kernel<T, Q, P, N, false>, dim3(k.nblocks), dim3(kScanThreads), 0, s, k);
}

template <typename T, int Q>
static hipError_t dispatch_pn(const ScanArgs& a, hipStream_t s) {
#define M2_PN(PP, NN) if (a.P == PP && a.N == NN) return run_scan<T, Q, PP, NN>(a, s);
    M2_PN(16, 16) M2_PN(16, 32) M2_PN(16, 64) M2_PN(32, 16) M2_PN(32, 32) M2_PN(32, 64)
    M2_PN(64, 16) M2_PN(64, 32) M2_PN(64, 64) M2_PN(64, 128)
    if constexpr (sizeof(T) == 2) {
        M2_PN(128, 64) M2_PN(128, 128)
    }
#undef M2_PN
    return hipErrorInvalidValue;
}

bool ssd_scan_supported(int P, int N, int Q, bool bf16) {
    if (!(Q == 16 || Q == 32 || Q == 64)) return false;
    if (!bf16 && Q == 64) return false;  // fp32 tiles are kept to 32 tokens (LDS budget)
    const bool small = (P == 16 || P == 32 || P == 64) && (N == 16 || N == 32 || N == 64 || (N == 128 && P == 64));
    const bool large = bf16 && P == 128 && (N == 64 || N == 128);
    return small || large;
}

int ssd_scan_default_chunk(int, int, bool) { return 32; }

size_t ssd_scan_workspace_bytes(int64_t batch, int64_t L, int H, int P, int N, int G, int Q, bool) {
    return plan_for(batch, L, H, G, P, N, Q).ws_bytes;
}

hipError_t launch_ssd_scan(const ScanArgs& a, hipStream_t s) {
    if (a.bf16) {
        switch (a.Q) {
            case 16: return dispatch_pn<bf16_t, 16>(a, s);
            case 32: return dispatch_pn<bf16_t, 32>(a, s);
            default: return dispatch_pn<bf16_t, 64>(a, s);
        }
    }
    switch (a.Q) {
        case 16: return dispatch_pn<float, 16>(a, s);
        default: return dispatch_pn<float, 32>(a, s);
    }
}

}  // namespace m2
