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
// Four kernels: walks over the chunks of segments of the sequence (four heads of one group per
// block, the state or adjoint in accumulator registers; forward, each chunk's initial state from the
// segment's start is stored before E_c is added; backward, each chunk's end adjoint from the
// segment's end before F_c is added), a chain over the segments for what crosses segment boundaries,
// the gradients (one block per (sequence, group, chunk), eight waves on one head at a time, the
// boundary terms added as the states are loaded, dB and dC summed over the group's heads in
// registers), and a reduction of the per-chunk dA, dD and dt_bias sums.  States in the workspace are
// fp32 and stored transposed, [n][p], so an accumulator's four rows land as one 16-byte piece; they
// enter the products as bf16 hi + lo pairs (a single bf16 rounding of the chained adjoint left 2e-2
// of dx, in an emulation of these kernels' rounding points and on the GPU).

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

// sum over the wave, the same value in every lane (DPP prefix sums, then the last lane)
__device__ __forceinline__ float wave_sum(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_prefix_sum(v)), 63));
}
// inclusive prefix sum inside each 16-lane row (DPP row shifts): lane 15 of a row holds the row's sum
__device__ __forceinline__ float row_prefix_sum(float v) {
    float x = v;
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
    return x;
}
// sum over the four 16-lane groups (lanes with the same lane % 16)
__device__ __forceinline__ float sum_over_q(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
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

// Sequence b: its first row (b * seqlen, or cu[b] in a packed batch) and its tokens (seqlen, its
// length in a right-padded batch, or the offset difference in a packed one; clamped to the rows that
// exist and to seqlen).  A token past the length reads as zero x, B, C, dy and dt, so it changes
// neither the state nor the adjoint, and its gradients are not stored.
__device__ __forceinline__ int64_t bwd_row0(const BwdArgs& k, int64_t b) {
    if (!k.cu) return b * k.L;
    const int64_t r0 = k.cu[b];
    return r0 < 0 ? 0 : (r0 > k.total ? k.total : r0);
}
__device__ __forceinline__ int64_t bwd_seq_len(const BwdArgs& k, int64_t b) {
    if (k.cu) {
        const int64_t row0 = bwd_row0(k, b), r1 = k.cu[b + 1];
        const int64_t end = r1 < row0 ? row0 : (r1 > k.total ? k.total : r1);
        return end - row0 < k.L ? end - row0 : k.L;
    }
    if (!k.lens) return k.L;
    const int64_t v = k.lens[b];
    return v < 0 ? 0 : (v > k.L ? k.L : v);
}
// rows of chunk c (from token t0) that belong to a sequence of Lb tokens: 0 .. Q
__device__ __forceinline__ int chunk_rows(int64_t Lb, int64_t t0) {
    const int64_t r = Lb - t0;
    return (int)(r < 0 ? 0 : (r < bwd::Q ? r : bwd::Q));
}

}  // namespace

// ----------------------------------------------------------------------------------------------
// 1. the walks over the chunks of a segment, four heads of one group per block (a wave each, the state
// or adjoint in 64 accumulator registers): blockIdx.z = 0 runs forward (the chunk's initial state,
// from the segment's start, is stored before the chunk's E_c is added), blockIdx.z = 1 backward (the
// adjoint of the chunk's end state, from the segment's end, before F_c is added).  The first
// segment's walk starts from the caller's state, the last segment's backward walk from dstate_out,
// the others from zero; the segment chain adds what comes from across segment boundaries.

__global__ __launch_bounds__(bwd::THREADS) void ssd_bwd_walk_kernel(BwdArgs k)
{
    using namespace bwd;
    __shared__ __attribute__((aligned(16))) uint16_t sT[4][TE];  // x (dy) of the four heads
    __shared__ __attribute__((aligned(16))) uint16_t sG[TE];     // B (C) of the group
    const int seg = blockIdx.x;
    const bool fwd = blockIdx.z == 0;
    const int lane = threadIdx.x & 63, q = lane >> 4, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hpg = k.H / k.G;
    const int upg = (hpg + 3) / 4;               // head quads per group
    const int64_t b = blockIdx.y / (k.G * upg);
    const int hu = blockIdx.y % (k.G * upg);
    const int g = hu / upg;
    const int h0 = g * hpg + (hu % upg) * 4;
    const int hcount = hpg - (hu % upg) * 4 < 4 ? hpg - (hu % upg) * 4 : 4;
    const bool hvalid = w < hcount;
    const int h = h0 + (hvalid ? w : hcount - 1);  // waves past the last head repeat it (results unused)
    const int BH = (int)k.batch * k.H;
    const int bh = (int)b * k.H + h;
    const int c0 = seg * k.cps;
    const int c1 = c0 + k.cps < k.nch ? c0 + k.cps : k.nch;
    const float A_h = k.A[h], bias_h = k.dt_bias[h];
    const uint16_t* const src = fwd ? k.x : k.dy;
    const int64_t srs = fwd ? k.xs : k.dys;
    const uint16_t* const gsrc = fwd ? k.B : k.C;
    float* const out = fwd ? k.ws_es : k.ws_fg;
    float* const lamrun = fwd ? k.ws_lamb : k.ws_lame;

    // the state (adjoint) in accumulator layout: acc[pb][nb] lane (q, li) = S[p = 16 pb + 4q + r][n = 16 nb + li]
    f32x4 acc[4][4];
    const float* init = fwd ? (seg == 0 ? k.state_in : nullptr) : (seg == k.nseg - 1 ? k.dstate_out : nullptr);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[pb][nb][r] = init ? init[(int64_t)bh * PN + (16 * pb + 4 * q + r) * N + 16 * nb + li] : 0.0f;
        }
    float run = 0.0f;  // summed log-decay of the segment's chunks walked so far
    // the next chunk's tiles and raw dt, fetched into registers while the current one is computed; the
    // wave's own tile: unit u = lane + 64 m is row u / 8, columns 8 (u % 8) .. +7
    uint4 vt[8], vg[2];
    float raw_n = 0.0f;
    const int64_t Lb = bwd_seq_len(k, b), srow = bwd_row0(k, b);
    auto fetch = [&](int c) __attribute__((always_inline)) {
        const int64_t t0 = (int64_t)c * Q;
        const int rows = chunk_rows(Lb, t0);
        const int64_t row0 = srow + t0;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int u = lane + 64 * m, r = u >> 3, c8 = u & 7;
            vt[m] = r < rows ? *reinterpret_cast<const uint4*>(src + (row0 + r) * srs + (int64_t)h * P + 8 * c8)
                             : make_uint4(0u, 0u, 0u, 0u);
        }
        fetch_tile<THREADS>(vg, gsrc + row0 * k.bcs + (int64_t)g * N, k.bcs, rows);
        raw_n = lane < rows ? bits_to_f32(k.dt[(row0 + lane) * k.dts + h]) : 0.0f;
    };
    if (c1 > c0) fetch(fwd ? c0 : c1 - 1);
    for (int j = 0; j < c1 - c0; ++j) {
        const int c = fwd ? c0 + j : c1 - 1 - j;
        const int64_t t0 = (int64_t)c * Q;
        const int rows = chunk_rows(Lb, t0);
        __syncthreads();  // the previous chunk's tiles are no longer read
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int u = lane + 64 * m, r = u >> 3, c8 = u & 7;
            *reinterpret_cast<uint4*>(sT[w] + r * RS + 8 * c8) = vt[m];
        }
        put_tile<THREADS>(sG, vg);
        const bool valid = lane < rows;
        const float raw = raw_n;
        __syncthreads();
        if (j + 1 < c1 - c0) fetch(fwd ? c + 1 : c - 1);
        // the chunk's state (adjoint) before its own contribution, as [n][p] fp32
        if (hvalid) {
            float* const o = out + ((int64_t)c * BH + bh) * PN;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    *reinterpret_cast<float4*>(o + (16 * nb + li) * P + 16 * pb + 4 * q) =
                        make_float4(acc[pb][nb][0], acc[pb][nb][1], acc[pb][nb][2], acc[pb][nb][3]);
            if (lane == 0) lamrun[(int64_t)c * BH + bh] = run;
        }
        const float dtv = valid ? dt_of(raw, bias_h, k.dt_min, k.dt_max) : 0.0f;
        const float lam = wave_prefix_sum(dtv * A_h);
        const float lamQ = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 63));
        // token weights: e^(LamQ - Lam_s) dt_s forward (E_c), e^(Lam_t) backward (F_c)
        const float wgt = fwd ? fast_exp(lamQ - lam) * dtv : fast_exp(lam);
        const float d = fast_exp(lamQ);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pb][nb][r] *= d;
#pragma unroll 1
        for (int kb = 0; kb < Q; kb += 32) {
            float ws8[2][4];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int e = 0; e < 4; ++e) ws8[cc][e] = lane_value(wgt, kb + 16 * cc + 4 * q + e);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                // A operand: the head's tile down the tokens (m = p, k = s), scaled per token, hi + lo
                Frag<bf16_t> th, tl;
                const Frag<bf16_t> ta = frag_col<bf16_t, U>(sT[w], kb, Q, 16 * pb, q, li);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const float v4[4] = {ta.get(cc, 0) * ws8[cc][0], ta.get(cc, 1) * ws8[cc][1],
                                         ta.get(cc, 2) * ws8[cc][2], ta.get(cc, 3) * ws8[cc][3]};
                    uint2 h2, l2;
                    split4(h2, l2, v4);
                    th.w[2 * cc] = h2.x; th.w[2 * cc + 1] = h2.y;
                    tl.w[2 * cc] = l2.x; tl.w[2 * cc + 1] = l2.y;
                }
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const Frag<bf16_t> gb = frag_col<bf16_t, U>(sG, kb, Q, 16 * nb, q, li);
                    mfma(acc[pb][nb], th, gb);
                    mfma(acc[pb][nb], tl, gb);
                }
            }
        }
        run += lamQ;
    }
    // the segment's end state (its adjoint at the segment's start) and summed log-decay
    if (hvalid) {
        float* const o = (fwd ? k.ws_sege : k.ws_segf) + ((int64_t)seg * BH + bh) * PN;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                *reinterpret_cast<float4*>(o + (16 * nb + li) * P + 16 * pb + 4 * q) =
                    make_float4(acc[pb][nb][0], acc[pb][nb][1], acc[pb][nb][2], acc[pb][nb][3]);
        if (fwd && lane == 0) k.ws_seglam[(int64_t)seg * BH + bh] = run;
    }
}

// ----------------------------------------------------------------------------------------------
// 2. the chain over segments, four entries ([n][p] order) per thread, in place: forward, T[s] = the
// true state at segment s's start (s >= 1) = e^lam[s-1] T[s-1] + E[s-1] with T[1] = E[0] (the first
// walk started from the caller's state); backward, U[s] = the true adjoint at segment s's end
// (s <= nseg-2) = e^lam[s+1] U[s+1] + F[s+1] with U[nseg-2] = F[nseg-1]; dstate_in = F[0] + e^lam[0] U[0].

__global__ __launch_bounds__(256) void ssd_bwd_segchain_kernel(BwdArgs k)
{
    using namespace bwd;
    constexpr int kHalf = PN / 1024;
    const int bh = blockIdx.y;
    const bool fwd = (int)blockIdx.x < kHalf;
    const int i = (((int)blockIdx.x % kHalf) * 256 + threadIdx.x) * 4;
    const int n = i / P, p = i % P;
    const int BH = (int)k.batch * k.H;
    const int nseg = k.nseg;
    float* const arr = fwd ? k.ws_sege : k.ws_segf;
    auto at = [&](int sg) __attribute__((always_inline)) { return arr + ((int64_t)sg * BH + bh) * PN + i; };
    auto lam = [&](int sg) __attribute__((always_inline)) { return k.ws_seglam[(int64_t)sg * BH + bh]; };
    if (fwd) {
        float4 cur = *reinterpret_cast<const float4*>(at(0));
        for (int sg = 1; sg < nseg; ++sg) {
            const float4 e = *reinterpret_cast<const float4*>(at(sg));
            *reinterpret_cast<float4*>(at(sg)) = cur;
            const float d = fast_exp(lam(sg));
            cur = make_float4(d * cur.x + e.x, d * cur.y + e.y, d * cur.z + e.z, d * cur.w + e.w);
        }
    } else {
        float4 cur = *reinterpret_cast<const float4*>(at(nseg - 1));
        for (int sg = nseg - 2; sg >= 0; --sg) {
            const float4 f = *reinterpret_cast<const float4*>(at(sg));
            *reinterpret_cast<float4*>(at(sg)) = cur;
            const float d = fast_exp(lam(sg));
            cur = make_float4(d * cur.x + f.x, d * cur.y + f.y, d * cur.z + f.z, d * cur.w + f.w);
        }
        if (k.dstate_in) {
            k.dstate_in[(int64_t)bh * PN + (p + 0) * N + n] = cur.x;
            k.dstate_in[(int64_t)bh * PN + (p + 1) * N + n] = cur.y;
            k.dstate_in[(int64_t)bh * PN + (p + 2) * N + n] = cur.z;
            k.dstate_in[(int64_t)bh * PN + (p + 3) * N + n] = cur.w;
        }
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
    // a chunk past its sequence's length still runs (its inputs read as zero) and records zero sums
    const int rows = chunk_rows(bwd_seq_len(k, b), t0);
    const int64_t row0 = bwd_row0(k, b) + t0;
    {
        uint4 vb[1], vc[1];
        fetch_tile<NT>(vb, k.B + row0 * k.bcs + (int64_t)g * N, k.bcs, rows);
        fetch_tile<NT>(vc, k.C + row0 * k.bcs + (int64_t)g * N, k.bcs, rows);
        put_tile<NT>(sB, vb);
        put_tile<NT>(sC, vc);
    }
    uint4 vx[1], vy[1];
    float4 vs[2], vg[2], ts[2], tg[2];
    float fs = 0.0f, fg = 0.0f, raw_n = 0.0f, A_n = 0.0f, bias_n = 0.0f, D_n = 0.0f;
    // The chunk's true initial state and end adjoint: the walks' in-segment values plus what crosses the
    // segment's boundaries, e^(log-decay from the segment's start) T[seg] and e^(log-decay to its end)
    // U[seg].  fetch(h) issues every load of head h and waits for none of them: the boundary tiles go to
    // ts / tg with their factors in fs / fg and are added when the head's tiles are put in LDS, and a
    // boundary term that is not needed reads through an empty buffer range (zeros, no memory access).
    // Its log-decays come in one head earlier (lb_n, le_n), so the choice waits for no load either.
    const int seg = c / k.cps;
    const int64_t lrow = (int64_t)c * BH + b * k.H;  // log-decays of head h at lrow + h
    auto fetch = [&](int h, float lb, float le) __attribute__((always_inline)) {
        const int64_t bh = b * k.H + h;
        const int64_t so = ((int64_t)c * BH + bh) * PN, sg = ((int64_t)seg * BH + bh) * PN;
        fetch_tile<NT>(vx, k.x + row0 * k.xs + (int64_t)h * P, k.xs, rows);
        fetch_tile<NT>(vy, k.dy + row0 * k.dys + (int64_t)h * P, k.dys, rows);
        fetch_tile32<NT>(vs, k.ws_es + so);
        fetch_tile32<NT>(vg, k.ws_fg + so);
        // a boundary term whose factor is below 2^-60 is below the fp32 resolution of any state it
        // is added to (the states are finite), and is skipped
        const float fb = fast_exp(lb), fe = fast_exp(le);
        const bool use_b = seg > 0 && fb >= 0x1p-60f, use_e = seg < k.nseg - 1 && fe >= 0x1p-60f;
        const auto rs = make_rsrc(k.ws_sege + (use_b ? sg : 0), use_b ? PN * 4u : 0u);
        const auto rg = make_rsrc(k.ws_segf + (use_e ? sg : 0), use_e ? PN * 4u : 0u);
#pragma unroll
        for (int j = 0; j < 1024 / NT; ++j) {
            const uint32_t off = (uint32_t)((int)threadIdx.x + NT * j) * 16u;
            ts[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
            tg[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rg, (int)off, 0, 0));
        }
        fs = use_b ? fb : 0.0f;
        fg = use_e ? fe : 0.0f;
        raw_n = lane < rows ? bits_to_f32(k.dt[(row0 + lane) * k.dts + h]) : 0.0f;
        A_n = k.A[h];
        bias_n = k.dt_bias[h];
        D_n = k.D ? k.D[h] : 0.0f;
    };
    fetch(g * hpg, k.ws_lamb[lrow + g * hpg], k.ws_lame[lrow + g * hpg]);
    float lb_n = hpg > 1 ? k.ws_lamb[lrow + g * hpg + 1] : 0.0f;
    float le_n = hpg > 1 ? k.ws_lame[lrow + g * hpg + 1] : 0.0f;
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
        // No barrier here: the previous head's last one (before its d(Lam) tail) already has every wave
        // past its reads of the tiles, and the tail reads only the partial sums, which this head writes
        // after the next barrier, the one that waits for the tail's wave.
#pragma unroll
        for (int j = 0; j < 1024 / NT; ++j) {
            vs[j] = make_float4(vs[j].x + fs * ts[j].x, vs[j].y + fs * ts[j].y, vs[j].z + fs * ts[j].z, vs[j].w + fs * ts[j].w);
            vg[j] = make_float4(vg[j].x + fg * tg[j].x, vg[j].y + fg * tg[j].y, vg[j].z + fg * tg[j].z, vg[j].w + fg * tg[j].w);
        }
        put_tile<NT>(sX, vx);
        put_tile<NT>(sDY, vy);
        put_tile_split<NT>(sS0, sS0l, vs);
        put_tile_split<NT>(sGE, sGEl, vg);
        // <Ge, S0> from the fp32 tiles (both [n][p], the same entries in every thread)
        float g0 = 0.0f;
#pragma unroll
        for (int j = 0; j < 1024 / NT; ++j)
            g0 += vs[j].x * vg[j].x + vs[j].y * vg[j].y + vs[j].z * vg[j].z + vs[j].w * vg[j].w;
        const bool valid = lane < rows;
        const float raw = raw_n, A_h = A_n, bias_h = bias_n, D_h = D_n;
        __syncthreads();
        if (i + 1 < hpg) fetch(h + 1, lb_n, le_n);
        if (i + 2 < hpg) {
            lb_n = k.ws_lamb[lrow + h + 2];
            le_n = k.ws_lame[lrow + h + 2];
        }
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
            const float v = row_prefix_sum(rsum[r]);  // lane 15 of the row: the sum over its 16 columns
            if (li == 15) rRow[ch][16 * rb + 4 * q + r] = v;
        }
        dpart = wave_sum(dpart);
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
// a prompt of no tokens: dstate_in = dstate_out (or zero), one block per sequence-head

__global__ __launch_bounds__(256) void ssd_bwd_copy_state_kernel(BwdArgs k)
{
    const int64_t o = (int64_t)blockIdx.x * bwd::PN;
    for (int i = threadIdx.x; i < bwd::PN; i += 256) k.dstate_in[o + i] = k.dstate_out ? k.dstate_out[o + i] : 0.0f;
}

// ----------------------------------------------------------------------------------------------
// host side

bool ssd_bwd_supported(int P, int N, bool bf16) { return bf16 && P == bwd::P && N == bwd::N; }

namespace {
// Segments of the walks: at most two walk blocks (forward and backward together) per CU, the number
// resident at once (46 KB of LDS, about 190 registers per lane), and at most one segment per chunk.
struct BwdPlan {
    int nch, nseg, cps;
};
BwdPlan bwd_plan(int64_t batch, int64_t L, int H, int G) {
    BwdPlan pl;
    pl.nch = (int)((L + bwd::Q - 1) / bwd::Q);
    const int64_t quads = batch * G * ((H / G + 3) / 4);
    const int64_t target = (int64_t)device_shape().cus * 2;
    int64_t nseg = quads > 0 ? target / (2 * quads) : 1;
    if (nseg > pl.nch) nseg = pl.nch;
    if (nseg < 1) nseg = 1;
    pl.cps = pl.nch > 0 ? (int)((pl.nch + nseg - 1) / nseg) : 1;
    pl.nseg = pl.nch > 0 ? (pl.nch + pl.cps - 1) / pl.cps : 1;
    return pl;
}
struct BwdLayout {
    size_t es, fg, lamb, lame, sege, segf, seglam, part, total;
};
BwdLayout bwd_layout(int64_t batch, int64_t L, int H, int G) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const BwdPlan pl = bwd_plan(batch, L, H, G);
    const size_t BH = (size_t)(batch * H), st = (size_t)bwd::PN * 4;
    BwdLayout w;
    w.es = 0;
    w.fg = up(pl.nch * BH * st);
    w.lamb = up(w.fg + pl.nch * BH * st);
    w.lame = up(w.lamb + pl.nch * BH * 4);
    w.sege = up(w.lame + pl.nch * BH * 4);
    w.segf = up(w.sege + pl.nseg * BH * st);
    w.seglam = up(w.segf + pl.nseg * BH * st);
    w.part = up(w.seglam + pl.nseg * BH * 4);
    w.total = w.part + (size_t)(3 * batch * pl.nch * H) * 4;
    return w;
}
}  // namespace

size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t L, int H, int G) { return bwd_layout(batch, L, H, G).total + 256; }

hipError_t launch_ssd_scan_bwd(const BwdArgs& a_in, hipStream_t s) {
    BwdArgs a = a_in;
    const BwdPlan pl = bwd_plan(a.batch, a.L, a.H, a.G);
    const BwdLayout lay = bwd_layout(a.batch, a.L, a.H, a.G);
    uint8_t* base = reinterpret_cast<uint8_t*>(((uintptr_t)a.ws + 255) & ~(uintptr_t)255);
    a.ws_es = reinterpret_cast<float*>(base + lay.es);
    a.ws_fg = reinterpret_cast<float*>(base + lay.fg);
    a.ws_lamb = reinterpret_cast<float*>(base + lay.lamb);
    a.ws_lame = reinterpret_cast<float*>(base + lay.lame);
    a.ws_sege = reinterpret_cast<float*>(base + lay.sege);
    a.ws_segf = reinterpret_cast<float*>(base + lay.segf);
    a.ws_seglam = reinterpret_cast<float*>(base + lay.seglam);
    a.ws_part = reinterpret_cast<float*>(base + lay.part);
    a.nch = pl.nch;
    a.nseg = pl.nseg;
    a.cps = pl.cps;
    hipError_t e = hipSuccess;
    if (a.nch > 0 && a.batch > 0) {
        const int quads = (int)a.batch * a.G * ((a.H / a.G + 3) / 4);
        e = launch_kernel(ssd_bwd_walk_kernel, dim3((unsigned)a.nseg, (unsigned)quads, 2), dim3(bwd::THREADS), 0, s, a);
        if (e != hipSuccess) return e;
        e = launch_kernel(ssd_bwd_segchain_kernel, dim3(2 * bwd::PN / 1024, (unsigned)(a.batch * a.H)), dim3(256), 0, s,
                          a);
        if (e != hipSuccess) return e;
        e = launch_kernel(ssd_bwd_grad_kernel, dim3((unsigned)a.nch, (unsigned)(a.batch * a.G)), dim3(bwd::GTHREADS), 0,
                          s, a);
        if (e != hipSuccess) return e;
    } else if (a.batch > 0 && a.dstate_in) {
        // no tokens: the final state's gradient reaches the initial state unchanged
        e = launch_kernel(ssd_bwd_copy_state_kernel, dim3((unsigned)(a.batch * a.H)), dim3(256), 0, s, a);
        if (e != hipSuccess) return e;
    }
    return launch_kernel(ssd_bwd_reduce_kernel, dim3((unsigned)a.H), dim3(256), 0, s, a);
}

}  // namespace m2
