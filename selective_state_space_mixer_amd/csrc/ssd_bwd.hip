// ssd_bwd.hip -- backward of the chunked selective state-space scan (gfx950, MFMA): headdim 64,
// d_state 64, bf16 activations, chunks of 64 tokens.
//
// The training path of the stateful mixer (article "Transformers 中 Zamba2 混合架构模型解析", §三: the
// Mamba2 mixer's chunked scan, whose gradients a training step needs).  For the recurrence
//   S_t = e^(dt_t A) S_{t-1} + dt_t x_t (outer) B_t,   y_t = S_t C_t + D x_t
// it returns the gradients of  L = sum_t dy_t . y_t + <dS, S_final>.  Over a chunk of Q tokens with
// true initial state S0, true adjoint Ge of its end state (everything later tokens and dS send back)
// and Lam_t the in-chunk inclusive sum of dt A, L_ts = e^(Lam_t - Lam_s) (t >= s):
//   dx_s = D dy_s + dt_s dxr_s,   dxr_s = sum_{t>=s} L_ts (C_t.B_s) dy_t + e^(LamQ - Lam_s) Ge B_s
//   dB_s = sum_{t>=s} L_ts dt_s (dy_t.x_s) C_t + dt_s e^(LamQ - Lam_s) Ge^T x_s
//   dC_t = sum_{s<=t} L_ts dt_s (dy_t.x_s) B_s + e^(Lam_t) S0^T dy_t
//   dD   = sum_t dy_t.x_t
// and, with dLam_t the gradient through the cumulative log-decay,
//   dLam = rowsum(M) - colsum(M) + m0 - q  (+ q0 + sum q on the chunk's last token),
//   M_ts = L_ts dt_s (C_t.B_s)(dy_t.x_s),  m0_t = e^(Lam_t) dy_t.(S0 C_t),
//   q_s = e^(LamQ - Lam_s) dt_s x_s.(Ge B_s),  q0 = e^(LamQ) <Ge, S0>,
//   d(dt)_s = x_s.dxr_s + A R_s,  R_s = sum_{t>=s} dLam_t,   dA = sum_s dt_s R_s,
// then through the clamp and softplus to dt_raw and dt_bias.  Across chunks the initial states
// and end adjoints chain exactly as in the forward direction:
//   S0_{c+1} = e^(LamQ_c) S0_c + E_c,   E_c = sum_s e^(LamQ - Lam_s) dt_s x_s (outer) B_s
//   Ge_{c-1} = e^(LamQ_c) Ge_c + F_c,   F_c = sum_t e^(Lam_t) dy_t (outer) C_t
// and dstate_in = e^(LamQ_0) Ge_0 + F_0.
//
// Four kernels: the per-chunk E_c and F_c (one block per (sequence, group, chunk), the group's heads
// in turn), the chain over chunks (elementwise, in place: E_c becomes S0_c and F_c becomes Ge_c), the
// gradients (one block per (sequence, group, chunk), four waves on one head at a time, dB and dC
// summed over the group's heads in registers), and a reduction of the per-chunk dA, dD and dt_bias
// sums.  States in the workspace are fp32 and stored transposed, [n][p], so an accumulator's four
// rows land as one 16-byte piece; they enter the products as bf16 hi + lo pairs (a single bf16
// rounding of the chained adjoint left 2e-2 of dx, in an emulation of these kernels' rounding points
// and on the GPU).
//
// Operands follow the fragment convention of ssd_common.h (chunk 0: k = kbase + 4q + 0..3, chunk 1:
// k = kbase + 16 + 4q + 0..3), read from row-major LDS tiles along a row (frag_row) or down the rows
// with transposing reads (frag_col).  The decay-masked matrices that multiply another operand
// (C.B with L_ts, and dt_s L_ts (dy.x)) go through LDS as bf16 hi + lo pairs, as the forward pass's
// masked matrix does; so do the scaled inputs of E_c and F_c and the chained states.
#include "ssd_common.h"

namespace m2 {

namespace bwd {
constexpr int Q = 64, P = 64, N = 64;
constexpr int U = 8;               // 16-byte units per tile row (64 bf16)
constexpr int RS = (U + 1) * 8;    // elements per LDS tile row (one unit of padding)
constexpr int TE = Q * RS;         // elements per tile
constexpr int THREADS = 256;     // the per-chunk kernel: four waves
constexpr int GTHREADS = 512;    // the gradient kernel: eight waves
constexpr int PN = P * N;
}  // namespace bwd

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
// sum over the four 16-lane groups (lanes with the same lane % 16)
__device__ __forceinline__ float sum_over_q(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
// sum over the 16 lanes of a lane group
__device__ __forceinline__ float sum_over_li(float v) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ float lane_value(float v, int src) { return __shfl(v, src, 64); }

// rows [0, 64) of a token-major bf16 array (`stride` elements between rows) starting at `base`,
// 64 columns, into registers of a block of NT threads; rows at or past `rows` read as zero.  Unit
// u = threadIdx.x + NT j is row u / 8, columns 8 (u % 8) .. +7.
template <int NT>
__device__ __forceinline__ void fetch_tile(uint4 (&v)[512 / NT], const uint16_t* base, int64_t stride, int rows) {
#pragma unroll
    for (int j = 0; j < 512 / NT; ++j) {
        const int u = (int)threadIdx.x + NT * j, r = u >> 3, c8 = u & 7;
        v[j] = r < rows ? *reinterpret_cast<const uint4*>(base + (int64_t)r * stride + 8 * c8)
                        : make_uint4(0u, 0u, 0u, 0u);
    }
}
template <int NT>
__device__ __forceinline__ void put_tile(uint16_t* tile, const uint4 (&v)[512 / NT]) {
#pragma unroll
    for (int j = 0; j < 512 / NT; ++j) {
        const int u = (int)threadIdx.x + NT * j, r = u >> 3, c8 = u & 7;
        *reinterpret_cast<uint4*>(tile + r * bwd::RS + 8 * c8) = v[j];
    }
}

// a 64 x 64 fp32 tile (contiguous rows of 64) into registers: unit u = threadIdx.x + NT j is row
// u / 16, columns 4 (u % 16) .. +3
template <int NT>
__device__ __forceinline__ void fetch_tile32(float4 (&v)[1024 / NT], const float* base) {
#pragma unroll
    for (int j = 0; j < 1024 / NT; ++j) v[j] = reinterpret_cast<const float4*>(base)[(int)threadIdx.x + NT * j];
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
// four values v as hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split4(uint2& hi, uint2& lo, const float (&v)[4]) {
    hi = pack4(v[0], v[1], v[2], v[3]);
    lo = pack4(v[0] - lo_bf16(hi.x), v[1] - hi_bf16(hi.x), v[2] - lo_bf16(hi.y), v[3] - hi_bf16(hi.y));
}
__device__ __forceinline__ void unpack4(float (&o)[4], uint2 v) {
    o[0] = lo_bf16(v.x); o[1] = hi_bf16(v.x); o[2] = lo_bf16(v.y); o[3] = hi_bf16(v.y);
}
// the fp32 tile of fetch_tile32 as bf16 hi and lo tiles
template <int NT>
__device__ __forceinline__ void put_tile_split(uint16_t* hi, uint16_t* lo, const float4 (&v)[1024 / NT]) {
#pragma unroll
    for (int j = 0; j < 1024 / NT; ++j) {
        const int u = (int)threadIdx.x + NT * j, r = u >> 4, c4 = u & 15;
        const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint2 h2, l2;
        split4(h2, l2, f);
        *reinterpret_cast<uint2*>(hi + r * bwd::RS + 4 * c4) = h2;
        *reinterpret_cast<uint2*>(lo + r * bwd::RS + 4 * c4) = l2;
    }
}

}  // namespace

// ----------------------------------------------------------------------------------------------
// 1. per chunk: E_c, F_c (stored [n][p] fp32) and the chunk's summed log-decay; a block takes every
// gridDim.z-th head of its group

__global__ __launch_bounds__(bwd::THREADS) void ssd_bwd_chunk_kernel(BwdArgs k)
{
    using namespace bwd;
    __shared__ __attribute__((aligned(16))) uint16_t sB[TE], sC[TE], sX[TE], sDY[TE];
    const int c = blockIdx.x, bg = blockIdx.y;
    const int64_t b = bg / k.G;
    const int g = bg % k.G;
    const int lane = threadIdx.x & 63, q = lane >> 4, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hpg = k.H / k.G;
    const int BH = (int)k.batch * k.H;
    const int64_t t0 = (int64_t)c * Q;
    const int rows = (int)(k.L - t0 < Q ? k.L - t0 : Q);
    const int64_t row0 = b * k.L + t0;
    {
        uint4 vb[2], vc[2];
        fetch_tile<THREADS>(vb, k.B + row0 * k.bcs + (int64_t)g * N, k.bcs, rows);
        fetch_tile<THREADS>(vc, k.C + row0 * k.bcs + (int64_t)g * N, k.bcs, rows);
        put_tile<THREADS>(sB, vb);
        put_tile<THREADS>(sC, vc);
    }
    uint4 vx[2], vy[2];
    auto fetch = [&](int h) __attribute__((always_inline)) {
        fetch_tile<THREADS>(vx, k.x + row0 * k.xs + (int64_t)h * P, k.xs, rows);
        fetch_tile<THREADS>(vy, k.dy + row0 * k.dys + (int64_t)h * P, k.dys, rows);
    };
    // the group's heads blockIdx.z, blockIdx.z + gridDim.z, ...
    const int hstep = gridDim.z;
    if ((int)blockIdx.z < hpg) fetch(g * hpg + blockIdx.z);
    for (int i = blockIdx.z; i < hpg; i += hstep) {
        const int h = g * hpg + i;
        __syncthreads();  // the previous head's tiles are no longer read
        put_tile<THREADS>(sX, vx);
        put_tile<THREADS>(sDY, vy);
        const bool valid = lane < rows;
        const float raw = valid ? bits_to_f32(k.dt[(row0 + lane) * k.dts + h]) : 0.0f;
        __syncthreads();
        if (i + hstep < hpg) fetch(h + hstep);
        const float dtv = valid ? dt_of(raw, k.dt_bias[h], k.dt_min, k.dt_max) : 0.0f;
        const float lam = wave_prefix_sum(dtv * k.A[h]);
        const float lamQ = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 63));
        const float wgt = fast_exp(lamQ - lam) * dtv;  // weight of token s in E
        const float fct = fast_exp(lam);               // weight of token t in F
        // E[p][n] and F[p][n] for rows p = 16w + 4q + r, columns n = 16 nb + li
        f32x4 aE[4], aF[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            aE[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            aF[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < Q; kb += 32) {
            // A operands: x and dy down the tokens (m = p = 16w + li, k = s), scaled per token
            const Frag<bf16_t> xa = frag_col<bf16_t, U>(sX, kb, Q, 16 * w, q, li);
            const Frag<bf16_t> ya = frag_col<bf16_t, U>(sDY, kb, Q, 16 * w, q, li);
            Frag<bf16_t> xh, xl, yh, yl;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                float vxs[4], vys[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = kb + 16 * cc + 4 * q + e;
                    vxs[e] = xa.get(cc, e) * lane_value(wgt, s);
                    vys[e] = ya.get(cc, e) * lane_value(fct, s);
                }
                uint2 h2, l2;
                split4(h2, l2, vxs);
                xh.w[2 * cc] = h2.x; xh.w[2 * cc + 1] = h2.y; xl.w[2 * cc] = l2.x; xl.w[2 * cc + 1] = l2.y;
                split4(h2, l2, vys);
                yh.w[2 * cc] = h2.x; yh.w[2 * cc + 1] = h2.y; yl.w[2 * cc] = l2.x; yl.w[2 * cc + 1] = l2.y;
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const Frag<bf16_t> bb = frag_col<bf16_t, U>(sB, kb, Q, 16 * nb, q, li);
                const Frag<bf16_t> cf = frag_col<bf16_t, U>(sC, kb, Q, 16 * nb, q, li);
                mfma(aE[nb], xh, bb);
                mfma(aE[nb], xl, bb);
                mfma(aF[nb], yh, cf);
                mfma(aF[nb], yl, cf);
            }
        }
        const int64_t base = ((int64_t)c * BH + b * k.H + h) * PN;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int64_t o = base + (int64_t)(16 * nb + li) * P + 16 * w + 4 * q;
            *reinterpret_cast<float4*>(k.ws_es + o) = make_float4(aE[nb][0], aE[nb][1], aE[nb][2], aE[nb][3]);
            *reinterpret_cast<float4*>(k.ws_fg + o) = make_float4(aF[nb][0], aF[nb][1], aF[nb][2], aF[nb][3]);
        }
        if (threadIdx.x == 0) k.ws_lam[(int64_t)c * BH + b * k.H + h] = lamQ;
    }
}

// ----------------------------------------------------------------------------------------------
// 2. the chain over chunks, four state entries ([n][p] order) per thread, in place: the first
// PN / 1024 blocks of a sequence-head run forward for the initial states, the others backward for the
// end adjoints; the loads of a batch of chunks are issued together

__global__ __launch_bounds__(256) void ssd_bwd_chain_kernel(BwdArgs k)
{
    using namespace bwd;
    constexpr int kBatch = 16;
    constexpr int kHalf = PN / 1024;
    const int bh = blockIdx.y;
    const bool fwd = (int)blockIdx.x < kHalf;
    const int i = (((int)blockIdx.x % kHalf) * 256 + threadIdx.x) * 4;
    const int n = i / P, p = i % P;
    const int BH = (int)k.batch * k.H;
    const int nch = k.nch;
    float* const arr = fwd ? k.ws_es : k.ws_fg;
    const float* const init = fwd ? k.state_in : k.dstate_out;
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = init ? init[(int64_t)bh * PN + (p + e) * N + n] : 0.0f;
    // chunk order: 0 .. nch-1 forward, nch-1 .. 0 backward
    for (int j0 = 0; j0 < nch; j0 += kBatch) {
        float4 v[kBatch];
        float lam[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int jj = j0 + j < nch ? j0 + j : nch - 1;
            const int c = fwd ? jj : nch - 1 - jj;
            v[j] = *reinterpret_cast<const float4*>(arr + ((int64_t)c * BH + bh) * PN + i);
            lam[j] = k.ws_lam[(int64_t)c * BH + bh];
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (j0 + j < nch) {
                const int c = fwd ? j0 + j : nch - 1 - (j0 + j);
                *reinterpret_cast<float4*>(arr + ((int64_t)c * BH + bh) * PN + i) = make_float4(s[0], s[1], s[2], s[3]);
                const float d = fast_exp(lam[j]);
                s[0] = d * s[0] + v[j].x;
                s[1] = d * s[1] + v[j].y;
                s[2] = d * s[2] + v[j].z;
                s[3] = d * s[3] + v[j].w;
            }
        }
    }
    if (!fwd && k.dstate_in) {
#pragma unroll
        for (int e = 0; e < 4; ++e) k.dstate_in[(int64_t)bh * PN + (p + e) * N + n] = s[e];
    }
}

// ----------------------------------------------------------------------------------------------
// 3. the gradients of one (sequence, group, chunk): eight waves on one head at a time; wave w owns
// output rows 16 rb .. 16 rb + 15 (rb = w % 4) and column tiles 2 ch, 2 ch + 1 (ch = w / 4) of every
// 64 x 64 product

__global__ __launch_bounds__(bwd::GTHREADS) void ssd_bwd_grad_kernel(BwdArgs k)
{
    using namespace bwd;
    constexpr int NT = GTHREADS;
    __shared__ __attribute__((aligned(16))) uint16_t sB[TE], sC[TE], sX[TE], sDY[TE];
    __shared__ __attribute__((aligned(16))) uint16_t sS0[TE], sS0l[TE], sGE[TE], sGEl[TE];  // [n][p] hi, lo
    __shared__ __attribute__((aligned(16))) uint16_t sWh[TE], sWl[TE], sVh[TE], sVl[TE];    // W^T, V^T: [s][t]
    // partial sums: row sums of M per column half, and per row band the column sums of M, m0, q and
    // x . dxr; <Ge, S0> and the diagonal of dy.x per wave
    __shared__ float rRow[2][Q], rCol[4][Q], rM0[4][Q], rQ[4][Q], rDd[4][Q], rQ0[8], rD[8];
    const int c = blockIdx.x, bg = blockIdx.y;
    const int64_t b = bg / k.G;
    const int g = bg % k.G;
    const int lane = threadIdx.x & 63, q = lane >> 4, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rb = w & 3, ch = w >> 2;
    const int hpg = k.H / k.G;
    const int BH = (int)k.batch * k.H;
    const int64_t t0 = (int64_t)c * Q;
    const int rows = (int)(k.L - t0 < Q ? k.L - t0 : Q);
    const int64_t row0 = b * k.L + t0;
    {
        uint4 vb[1], vc[1];
        fetch_tile<NT>(vb, k.B + row0 * k.bcs + (int64_t)g * N, k.bcs, rows);
        fetch_tile<NT>(vc, k.C + row0 * k.bcs + (int64_t)g * N, k.bcs, rows);
        put_tile<NT>(sB, vb);
        put_tile<NT>(sC, vc);
    }
    uint4 vx[1], vy[1];
    float4 vs[2], vg[2];
    auto fetch = [&](int h) __attribute__((always_inline)) {
        const int64_t so = ((int64_t)c * BH + b * k.H + h) * PN;
        fetch_tile<NT>(vx, k.x + row0 * k.xs + (int64_t)h * P, k.xs, rows);
        fetch_tile<NT>(vy, k.dy + row0 * k.dys + (int64_t)h * P, k.dys, rows);
        fetch_tile32<NT>(vs, k.ws_es + so);
        fetch_tile32<NT>(vg, k.ws_fg + so);
    };
    fetch(g * hpg);
    __syncthreads();
    // C.B of the chunk (every head of the group shares it): rows t = 16 rb + 4q + r, columns
    // s = 16 (2 ch + j) + li
    f32x4 cb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) cb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < N; kb += 32) {
        const Frag<bf16_t> a = frag_row<bf16_t, U>(sC, 16 * rb + li, kb, N, q);
#pragma unroll
        for (int j = 0; j < 2; ++j) mfma(cb[j], a, frag_row<bf16_t, U>(sB, 16 * (2 * ch + j) + li, kb, N, q));
    }
    // dB^T and dC^T of the chunk, summed over the group's heads: rows n = 16 rb + 4q + r, columns
    // s (t) = 16 (2 ch + j) + li
    f32x4 dBa[2], dCa[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        dBa[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        dCa[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int i = 0; i < hpg; ++i) {
        const int h = g * hpg + i;
        __syncthreads();  // the previous head is done with the tiles and the partial sums
        put_tile<NT>(sX, vx);
        put_tile<NT>(sDY, vy);
        put_tile_split<NT>(sS0, sS0l, vs);
        put_tile_split<NT>(sGE, sGEl, vg);
        const bool valid = lane < rows;
        const float raw = valid ? bits_to_f32(k.dt[(row0 + lane) * k.dts + h]) : 0.0f;
        __syncthreads();
        if (i + 1 < hpg) fetch(h + 1);
        const float A_h = k.A[h], bias_h = k.dt_bias[h];
        const float D_h = k.D ? k.D[h] : 0.0f;
        // statistics of token `lane`
        const float dtv = valid ? dt_of(raw, bias_h, k.dt_min, k.dt_max) : 0.0f;
        const float lam = wave_prefix_sum(dtv * A_h);
        const float lamQ = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 63));
        const float eQ = fast_exp(lamQ - lam);  // e^(LamQ - Lam_s)
        const float el = fast_exp(lam);         // e^(Lam_t)

        // ---- dy.x: rows t = 16 rb + 4q + r, columns s
        f32x4 dx_[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) dx_[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int kb = 0; kb < P; kb += 32) {
            const Frag<bf16_t> a = frag_row<bf16_t, U>(sDY, 16 * rb + li, kb, P, q);
#pragma unroll
            for (int j = 0; j < 2; ++j) mfma(dx_[j], a, frag_row<bf16_t, U>(sX, 16 * (2 * ch + j) + li, kb, P, q));
        }
        // ---- W = L (C.B), V = L dt_s (dy.x), M = W dt_s (dy.x); row and column sums of M
        float lt[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) lt[r] = lane_value(lam, 16 * rb + 4 * q + r);
        float rsum[4] = {0.f, 0.f, 0.f, 0.f};
        float dpart = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = 16 * (2 * ch + j) + li;
            const float ls = lane_value(lam, s), ds = lane_value(dtv, s);
            float wv[4], vv[4], csum = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * rb + 4 * q + r;
                const float L = t >= s ? fast_exp(lt[r] - ls) : 0.0f;
                wv[r] = cb[j][r] * L;
                vv[r] = dx_[j][r] * ds * L;
                const float m = wv[r] * ds * dx_[j][r];
                rsum[r] += m;
                csum += m;
                if (t == s) dpart += dx_[j][r];
            }
            uint2 hi, lo;
            split4(hi, lo, wv);
            *reinterpret_cast<uint2*>(sWh + s * RS + 16 * rb + 4 * q) = hi;
            *reinterpret_cast<uint2*>(sWl + s * RS + 16 * rb + 4 * q) = lo;
            split4(hi, lo, vv);
            *reinterpret_cast<uint2*>(sVh + s * RS + 16 * rb + 4 * q) = hi;
            *reinterpret_cast<uint2*>(sVl + s * RS + 16 * rb + 4 * q) = lo;
            csum = sum_over_q(csum);
            if (q == 0) rCol[rb][s] = csum;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = sum_over_li(rsum[r]);
            if (li == 0) rRow[ch][16 * rb + 4 * q + r] = v;
        }
        dpart = wave_sum(dpart);
        // <Ge, S0> over rows n = 8w .. 8w+7 of the transposed states, eight columns per lane
        float g0 = 0.0f;
        {
            const int o = (8 * w + (lane >> 3)) * RS + 8 * (lane & 7);
            const uint4 a = *reinterpret_cast<const uint4*>(sGE + o), al = *reinterpret_cast<const uint4*>(sGEl + o);
            const uint4 bb = *reinterpret_cast<const uint4*>(sS0 + o), bl = *reinterpret_cast<const uint4*>(sS0l + o);
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, alw[4] = {al.x, al.y, al.z, al.w};
            const uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w}, blw[4] = {bl.x, bl.y, bl.z, bl.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                g0 += (lo_bf16(aw[e]) + lo_bf16(alw[e])) * (lo_bf16(bw[e]) + lo_bf16(blw[e]));
                g0 += (hi_bf16(aw[e]) + hi_bf16(alw[e])) * (hi_bf16(bw[e]) + hi_bf16(blw[e]));
            }
        }
        g0 = wave_sum(g0);
        if (lane == 0) {
            rQ0[w] = g0;
            rD[w] = dpart;
        }
        __syncthreads();  // W^T and V^T are in LDS

        // ---- dxr^T[p][s]: rows p = 16 rb + 4q + r, columns s = 16 (2 ch + j) + li
        f32x4 xr[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) xr[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int kb = 0; kb < N; kb += 32) {  // Ge B_s (k = n)
            const Frag<bf16_t> a = frag_col<bf16_t, U>(sGE, kb, N, 16 * rb, q, li);
            const Frag<bf16_t> al = frag_col<bf16_t, U>(sGEl, kb, N, 16 * rb, q, li);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const Frag<bf16_t> bf = frag_row<bf16_t, U>(sB, 16 * (2 * ch + j) + li, kb, N, q);
                mfma(xr[j], a, bf);
                mfma(xr[j], al, bf);
            }
        }
        float xs4[2][4], dy4[2][4];  // x[s][p] and dy[s][p] at this lane's (p, s) positions
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = 16 * (2 * ch + j) + li;
            const float e = lane_value(eQ, s), ds = lane_value(dtv, s);
            unpack4(xs4[j], *reinterpret_cast<const uint2*>(sX + s * RS + 16 * rb + 4 * q));
            unpack4(dy4[j], *reinterpret_cast<const uint2*>(sDY + s * RS + 16 * rb + 4 * q));
            float qp = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                xr[j][r] *= e;
                qp += xs4[j][r] * xr[j][r];
            }
            qp = sum_over_q(qp);
            if (q == 0) rQ[rb][s] = qp * ds;
        }
#pragma unroll 1
        for (int kb = 0; kb < Q; kb += 32) {  // sum_t W_ts dy_t (k = t)
            const Frag<bf16_t> a = frag_col<bf16_t, U>(sDY, kb, Q, 16 * rb, q, li);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                mfma(xr[j], a, frag_row<bf16_t, U>(sWh, 16 * (2 * ch + j) + li, kb, Q, q));
                mfma(xr[j], a, frag_row<bf16_t, U>(sWl, 16 * (2 * ch + j) + li, kb, Q, q));
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = 16 * (2 * ch + j) + li;
            const float ds = lane_value(dtv, s);
            float dd = 0.0f, o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dd += xs4[j][r] * xr[j][r];
                o[r] = ds * xr[j][r] + D_h * dy4[j][r];
            }
            dd = sum_over_q(dd);
            if (q == 0) rDd[rb][s] = dd;
            if (s < rows)
                *reinterpret_cast<uint2*>(k.dx + (row0 + s) * k.dxs + (int64_t)h * P + 16 * rb + 4 * q) =
                    pack4(o[0], o[1], o[2], o[3]);
        }

        // ---- dB^T[n][s] of this head: dt_s e^(LamQ - Lam_s) Ge^T x_s + sum_t V_ts C_t
        f32x4 acc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int kb = 0; kb < P; kb += 32) {  // k = p
            const Frag<bf16_t> a = frag_row<bf16_t, U>(sGE, 16 * rb + li, kb, P, q);
            const Frag<bf16_t> al = frag_row<bf16_t, U>(sGEl, 16 * rb + li, kb, P, q);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const Frag<bf16_t> bx = frag_row<bf16_t, U>(sX, 16 * (2 * ch + j) + li, kb, P, q);
                mfma(acc[j], a, bx);
                mfma(acc[j], al, bx);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = 16 * (2 * ch + j) + li;
            const float f = lane_value(eQ, s) * lane_value(dtv, s);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] *= f;
        }
#pragma unroll 1
        for (int kb = 0; kb < Q; kb += 32) {  // k = t
            const Frag<bf16_t> a = frag_col<bf16_t, U>(sC, kb, Q, 16 * rb, q, li);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                mfma(acc[j], a, frag_row<bf16_t, U>(sVh, 16 * (2 * ch + j) + li, kb, Q, q));
                mfma(acc[j], a, frag_row<bf16_t, U>(sVl, 16 * (2 * ch + j) + li, kb, Q, q));
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) dBa[j] += acc[j];

        // ---- dC^T[n][t] of this head: e^(Lam_t) S0^T dy_t + sum_s V_ts B_s
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int kb = 0; kb < P; kb += 32) {  // k = p
            const Frag<bf16_t> a = frag_row<bf16_t, U>(sS0, 16 * rb + li, kb, P, q);
            const Frag<bf16_t> al = frag_row<bf16_t, U>(sS0l, 16 * rb + li, kb, P, q);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const Frag<bf16_t> bd = frag_row<bf16_t, U>(sDY, 16 * (2 * ch + j) + li, kb, P, q);
                mfma(acc[j], a, bd);
                mfma(acc[j], al, bd);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = 16 * (2 * ch + j) + li;
            const float f = lane_value(el, t);
            float c4[4], m0 = 0.0f;
            unpack4(c4, *reinterpret_cast<const uint2*>(sC + t * RS + 16 * rb + 4 * q));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[j][r] *= f;
                m0 += c4[r] * acc[j][r];
            }
            m0 = sum_over_q(m0);
            if (q == 0) rM0[rb][t] = m0;
        }
#pragma unroll 1
        for (int kb = 0; kb < Q; kb += 32) {  // k = s
            const Frag<bf16_t> a = frag_col<bf16_t, U>(sB, kb, Q, 16 * rb, q, li);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                mfma(acc[j], a, frag_col<bf16_t, U>(sVh, kb, Q, 16 * (2 * ch + j), q, li));
                mfma(acc[j], a, frag_col<bf16_t, U>(sVl, kb, Q, 16 * (2 * ch + j), q, li));
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) dCa[j] += acc[j];
        __syncthreads();  // the partial sums are in LDS

        // ---- d(Lam), d(dt), and the head's dA, dD, dt_bias sums (wave 0, token `lane`)
        if (w == 0) {
            const float colsum = rCol[0][lane] + rCol[1][lane] + rCol[2][lane] + rCol[3][lane];
            const float m0 = rM0[0][lane] + rM0[1][lane] + rM0[2][lane] + rM0[3][lane];
            const float qv = rQ[0][lane] + rQ[1][lane] + rQ[2][lane] + rQ[3][lane];
            const float dd = rDd[0][lane] + rDd[1][lane] + rDd[2][lane] + rDd[3][lane];
            float q0s = 0.0f, dsum = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                q0s += rQ0[j];
                dsum += rD[j];
            }
            const float qsum = wave_sum(qv);
            const float q0 = fast_exp(lamQ) * q0s;
            const float dlam = rRow[0][lane] + rRow[1][lane] - colsum + m0 - qv + (lane == Q - 1 ? q0 + qsum : 0.0f);
            const float pre = wave_prefix_sum(dlam);
            const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pre), 63));
            const float R = tot - pre + dlam;  // sum of dLam over tokens lane .. 63
            const float ddt = dd + A_h * R;
            const float dA_part = wave_sum(dtv * R);
            const float v = raw + bias_h;
            const float sp = softplus(v);
            const bool pass = valid && !(sp < k.dt_min || sp > k.dt_max);
            const float graw = pass ? ddt * __builtin_amdgcn_rcpf(1.0f + fast_exp(-v)) : 0.0f;
            if (valid) k.ddt[(row0 + lane) * k.ddts + h] = f32_to_bits(graw);
            const float db_part = wave_sum(graw);
            if (lane == 0) {
                const int64_t pr = (b * k.nch + c) * k.H + h;
                const int64_t stride = k.batch * k.nch * k.H;
                k.ws_part[pr] = dA_part;
                k.ws_part[stride + pr] = dsum;
                k.ws_part[2 * stride + pr] = db_part;
            }
        }
    }
    // dB, dC rows of the chunk: row s, columns n = 16 rb + 4q .. +3
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int s = 16 * (2 * ch + j) + li;
        if (s < rows) {
            const int64_t o = (row0 + s) * k.dbcs + (int64_t)g * N + 16 * rb + 4 * q;
            *reinterpret_cast<uint2*>(k.dB + o) = pack4(dBa[j][0], dBa[j][1], dBa[j][2], dBa[j][3]);
            *reinterpret_cast<uint2*>(k.dC + o) = pack4(dCa[j][0], dCa[j][1], dCa[j][2], dCa[j][3]);
        }
    }
}

// ----------------------------------------------------------------------------------------------
// 4. dA, dD and dt_bias: the per-(sequence, chunk) sums of one head (a block), added up

__global__ __launch_bounds__(256) void ssd_bwd_reduce_kernel(BwdArgs k)
{
    __shared__ float red[3][4];
    const int h = blockIdx.x;
    const int64_t rows = k.batch * k.nch, stride = rows * k.H;
    float a = 0.0f, d = 0.0f, bi = 0.0f;
    for (int64_t r = threadIdx.x; r < rows; r += 256) {
        a += k.ws_part[r * k.H + h];
        d += k.ws_part[stride + r * k.H + h];
        bi += k.ws_part[2 * stride + r * k.H + h];
    }
    a = wave_sum(a);
    d = wave_sum(d);
    bi = wave_sum(bi);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][w] = a;
        red[1][w] = d;
        red[2][w] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        k.dA[h] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        k.dD[h] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
        k.ddt_bias[h] = red[2][0] + red[2][1] + red[2][2] + red[2][3];
    }
}

// ----------------------------------------------------------------------------------------------
// host side

bool ssd_bwd_supported(int P, int N, bool bf16) { return bf16 && P == bwd::P && N == bwd::N; }

namespace {
struct BwdLayout {
    size_t es, fg, lam, part, total;
};
BwdLayout bwd_layout(int64_t batch, int64_t L, int H) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const int64_t nch = (L + bwd::Q - 1) / bwd::Q;
    BwdLayout w;
    w.es = 0;
    w.fg = up((size_t)(nch * batch * H * bwd::PN) * 4);
    w.lam = up(w.fg + (size_t)(nch * batch * H * bwd::PN) * 4);
    w.part = up(w.lam + (size_t)(nch * batch * H) * 4);
    w.total = w.part + (size_t)(3 * batch * nch * H) * 4;
    return w;
}
}  // namespace

size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t L, int H) { return bwd_layout(batch, L, H).total + 256; }

hipError_t launch_ssd_scan_bwd(const BwdArgs& a_in, hipStream_t s) {
    BwdArgs a = a_in;
    const BwdLayout lay = bwd_layout(a.batch, a.L, a.H);
    uint8_t* base = reinterpret_cast<uint8_t*>(((uintptr_t)a.ws + 255) & ~(uintptr_t)255);
    a.ws_es = reinterpret_cast<float*>(base + lay.es);
    a.ws_fg = reinterpret_cast<float*>(base + lay.fg);
    a.ws_lam = reinterpret_cast<float*>(base + lay.lam);
    a.ws_part = reinterpret_cast<float*>(base + lay.part);
    a.nch = (int)((a.L + bwd::Q - 1) / bwd::Q);
    hipError_t e = hipSuccess;
    if (a.nch > 0 && a.batch > 0) {
        // the group's heads over up to four blocks, so that the launch has several blocks per CU
        const int hpg = a.H / a.G;
        const int hsplit = hpg < 4 ? hpg : 4;
        const dim3 grid((unsigned)a.nch, (unsigned)(a.batch * a.G), (unsigned)hsplit);
        e = launch_kernel(ssd_bwd_chunk_kernel, grid, dim3(bwd::THREADS), 0, s, a);
        if (e != hipSuccess) return e;
    }
    if (a.batch > 0) {
        e = launch_kernel(ssd_bwd_chain_kernel, dim3(2 * bwd::PN / 1024, (unsigned)(a.batch * a.H)), dim3(256), 0, s, a);
        if (e != hipSuccess) return e;
    }
    if (a.nch > 0 && a.batch > 0) {
        const dim3 grid((unsigned)a.nch, (unsigned)(a.batch * a.G));
        e = launch_kernel(ssd_bwd_grad_kernel, grid, dim3(bwd::GTHREADS), 0, s, a);
        if (e != hipSuccess) return e;
    }
    return launch_kernel(ssd_bwd_reduce_kernel, dim3((unsigned)a.H), dim3(256), 0, s, a);
}

}  // namespace m2
