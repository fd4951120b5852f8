// ssd_walk.hip -- main pass of the prompt scan at headdim 64, d_state 64, bf16 activations,
// chunks of 32 tokens (the Zamba2-2.7B mixer shape), gfx950: one wave walks one head.
//
// The chunk identities are those of ssd_scan.hip (article "Transformers 中 Zamba2 混合架构模型解析",
// §三: intra-chunk plus inter-chunk scan over chunks of chunk_size tokens):
//   y_t   = e^Lam_t (S_prev . C_t) + sum_{s<=t} e^(Lam_t - Lam_s) dt_s (C_t . B_s) x_s + D x_t
//   S_new = e^Lam_end S_prev + sum_s e^(Lam_end - Lam_s) dt_s x_s (outer) B_s
// and the segment contract is the same (segments after the first start from zero; their end
// states and the maxima of those, summed log-decays and per-chunk starting log-decays go to the
// workspace for the chain and fix-up kernels of ssd_scan.hip).
//
// What differs from the general kernel is the split of the work.  Each wave owns one head and
// keeps the whole 64x64 fp32 state of that head in 64 accumulator registers (two waves per
// SIMD), so nothing a head needs is computed twice: the G = C B^T tiles, the decay-masked
// matrix M, the chunk statistics and the state's bf16 operand copy all belong to one wave.  A
// block holds the four heads of one B/C group that share the B and C tiles.  Every wave brings
// in the same share of each chunk's tiles (its own head's X tile and a quarter of B and of C),
// so the loads need no per-wave branching.  Tiles are unpadded 128-byte rows whose 16-byte
// units are permuted per row (unit u of row r at u ^ rowperm(r)); with that permutation the row
// fragment reads, the transposing column reads and the output staging reach every LDS bank
// evenly.
#include "ssd_common.h"

namespace m2 {

namespace walk {
constexpr int Q = 32, P = 64, N = 64;
constexpr int HPB = 4;                      // heads (waves) per block
constexpr int THREADS = 64 * HPB;
constexpr int ROWB = 128;                   // bytes per tile row: 64 bf16
constexpr int TILEB = Q * ROWB;             // 4 KB per tile
constexpr int BOFF = HPB * TILEB;           // buffer: X tiles of the four heads, then B, then C,
constexpr int COFF = BOFF + TILEB;          // then the raw dt of the four heads ([token][head] bf16)
constexpr int DOFF = COFF + TILEB;
constexpr int BUFB = DOFF + Q * HPB * 2;    // 24.25 KB
constexpr int NBUF = 3;                     // chunks i, i+1 and i+2 are in LDS while i is computed
constexpr int NSTAT = 5;                    // per-token statistics (see stats below)
constexpr float kRescale = 40.0f;           // lazy state scale: multiply out below e^-40
}  // namespace walk

// Position of 16-byte unit u of tile row r: unit u ^ rowperm(r).  rowperm(r + 16) = rowperm(r) ^ 4.
__device__ __forceinline__ int rowperm(int r) { return ((r & 3) * 2 + (r >> 2)) & 7; }

__device__ __forceinline__ uint2 lds_read8(const uint8_t* base, int off) {
    return *reinterpret_cast<const uint2*>(base + off);
}
__device__ __forceinline__ uint2 lds_read8_tr(const uint8_t* base, int off) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((M2_LDS i16x4_t*)(base + off));
    return __builtin_bit_cast(uint2, v);
}

template <bool FUSED>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, walk::THREADS), amdgpu_waves_per_eu(2)))
ssd_walk_kernel(ScanK k, WalkConv cv)
{
    using namespace walk;
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[NBUF * BUFB];
    // per head and token: Lam*log2(e), dt, w = e^(Lam_end - Lam) dt / e^sig, e^(Lam + sig_prev), and
    // gs = e^(Lam_e - Lam) dt with e the last token of the token's 16-block
    __shared__ __attribute__((aligned(16))) float sSt[2][HPB][NSTAT][Q];
    __shared__ uint64_t sBase[HPB][5];                                 // x, B, C, dt, y at the segment's first row
    // fused: the last four raw x rows of the chunk before, per head, laid out as tile rows 28..31
    __shared__ __attribute__((aligned(16))) uint8_t sHalo[FUSED ? HPB : 1][FUSED ? 4 * ROWB : 16];

    const int lane = threadIdx.x & 63, q = lane >> 4, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // block -> (segment, sequence, head group)
    const int hpg = k.H / k.G;
    const int upg = (hpg + HPB - 1) / HPB;
    const int nhu = k.G * upg;
    int hu, seg;
    int64_t b;
    if (!block_unit(k, nhu, hu, b, seg)) return;
    const int g = hu / upg;
    const int h0 = g * hpg + (hu % upg) * HPB;
    const int hcount = hpg - (hu % upg) * HPB < HPB ? hpg - (hu % upg) * HPB : HPB;
    const int hslot = w < hcount ? w : hcount - 1;  // waves past the last head repeat it (results unused)
    const int h = h0 + hslot;
    const bool hvalid = w < hcount;
    const int bh = (int)b * k.H + h;
    const int BH = k.batch * k.H;
    const int64_t Lb = seq_len(k, b);
    const int64_t nchunks = (Lb + Q - 1) / Q;
    const int cps = seg_chunks(k);
    const int64_t c_begin = (int64_t)seg * cps;
    const int64_t c_stop = c_begin + cps < nchunks ? c_begin + cps : nchunks;
    const int nc = c_stop > c_begin ? (int)(c_stop - c_begin) : 0;
    const int64_t row_begin = c_begin * Q;
    const int64_t row_end = Lb < row_begin + (int64_t)nc * Q ? Lb : row_begin + (int64_t)nc * Q;
    const float bias_h = k.dt_bias[h], A_h = k.A[h];
    // the fused kernel's x operands carry a factor log2(e) (see the conv below); every factor that
    // multiplies x (D here, dt, w and gs in the statistics) carries ln 2 to cancel it
    constexpr float xs_inv = FUSED ? 0.6931471805599453f : 1.0f;
    const float D_h = (k.D ? k.D[h] : 0.0f) * xs_inv;

    // ---- tile loads: piece m (0..3) of this wave's X tile (rows 8m..8m+7), piece w of B and of C, and
    // the raw dt of tokens 8w..8w+7 for the block's four heads.
    // Lane l of a piece covering rows R..R+7 fills LDS unit l of the piece: row R + l/8, unit
    // position l%8, which holds logical unit (l%8) ^ rowperm(row).
    const int lrow = lane >> 3;
    uint32_t vx[4], vbc, vdt;
    {
        const int xs_b = (int)k.xs * 2, bcs_b = (int)k.bcs * 2;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 8 * m + lrow;
            vx[m] = (uint32_t)(r * xs_b + hslot * (P * 2) + (((lane & 7) ^ rowperm(r)) << 4));
        }
        const int r = 8 * w + lrow;
        vbc = (uint32_t)(r * bcs_b + (((lane & 7) ^ rowperm(r)) << 4));
        // dt: lanes 0..15 bring tokens 8w .. 8w+7, two heads (one dword) each
        vdt = (uint32_t)((8 * w + (lane >> 1)) * (int)k.dts * 2 + 4 * (lane & 1));
    }

    // ---- fragment addresses (bytes within a tile).  Row fragments: lane (q, li) reads row
    // 16 tb + li, k = 32 ks + 16 c + 4q .. +3; its unit is (4ks + 2c + q/2) ^ rowperm(row), so every
    // variant is the base below with (((ks ^ tb) << 2) | (c << 1)) XORed into the unit, plus 2048 tb.
    const int arow = li * ROWB + ((((q >> 1) ^ rowperm(li))) << 4) + 8 * (q & 1);
    // Column (transposing) fragments: lane (q, li) reads row 16 hf + 4q + li/4, columns
    // 16 cb + 4 (li%4) .. +3; the variants XOR ((2 cb) ^ 4 hf) into the unit, plus 2048 hf.
    const int tr0 = 4 * q + (li >> 2);
    const int acol = tr0 * ROWB + (((((li >> 1) & 1)) ^ rowperm(tr0)) << 4) + 8 * (li & 1);
    auto row_off = [&](int tb, int ks, int c) __attribute__((always_inline)) {
        return (arow ^ ((((ks ^ tb) << 2) | (c << 1)) << 4)) + 2048 * tb;
    };
    auto col_off = [&](int hf, int cb) __attribute__((always_inline)) {
        return (acol ^ (((2 * cb) ^ (4 * hf)) << 4)) + 2048 * hf;
    };

    // ---- fused: this lane's conv taps and bias for its four x channels p = 16 pb + li of head h, taps
    // right-aligned (tap 3 multiplies the current token; a narrower conv leaves the first taps zero).
    // The taps and the bias are scaled by log2(e), so the conv gives b = log2(e) a and SiLU needs no
    // scale before the base-2 exponential.
    // Transposing reads of raw rows 4g .. 4g+3 of column block cb sit at base(g) ^ (2 cb << 4); the
    // lanes of q-group q read row groups q-1, q (tokens 4q-4 .. 4q+3) and q+3, q+4 (16+4q-4 .. 16+4q+3).
    // Group -1 is the halo: the last raw rows of the chunk before, kept as rows 28..31 in sHalo.
    float cw[4][4], cb4[4];
    int offA = 0, offB = 0, offC = 0, offD = 0;
    if constexpr (FUSED) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            const int64_t c = (int64_t)h * P + 16 * pb + li;
#pragma unroll
            for (int t = 0; t < 4; ++t) cw[pb][t] = t >= 4 - cv.W ? cv.w[c * cv.W + (t - (4 - cv.W))] * kLog2e : 0.0f;
            cb4[pb] = cv.bias ? cv.bias[c] * kLog2e : 0.0f;
        }
        auto gbase = [&](int r) __attribute__((always_inline)) {
            return r * ROWB + ((((li >> 1) & 1) ^ rowperm(r)) << 4) + 8 * (li & 1);
        };
        offA = gbase(q == 0 ? 28 + (li >> 2) : 4 * (q - 1) + (li >> 2));
        offB = gbase(4 * q + (li >> 2));
        offC = gbase(4 * (q + 3) + (li >> 2));
        offD = gbase(4 * (q + 4) + (li >> 2));
    }

    // ---- the state, in accumulator layout: accS[pb][nb] lane (q, li) = S[p = 16 pb + li][n = 16 nb + 4q + j]
    f32x4 accS[4][4];
    {
        const float* src = (seg == 0 && k.state_in) ? k.state_in + (int64_t)bh * P * N : nullptr;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                if (src) {
                    const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)(16 * pb + li) * N + 16 * nb + 4 * q);
                    accS[pb][nb] = f32x4{v.x, v.y, v.z, v.w};
                } else {
                    accS[pb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
    }

    // ---- buffer resources over a window of the segment's rows (as in the general kernel)
    const int xs = (int)k.xs, bcs = (int)k.bcs, dts = (int)k.dts, ys = (int)k.ys;
    const int nrows = nc > 0 ? (int)(row_end - row_begin) : 0;
    if (lane == 0) {
        const int64_t base = seq_row0(k, b) + row_begin;
        sBase[w][0] = (uint64_t)(reinterpret_cast<const bf16_t*>(k.x) + base * k.xs + (int64_t)h0 * P);
        sBase[w][1] = (uint64_t)(reinterpret_cast<const bf16_t*>(k.B) + base * k.bcs + (int64_t)g * N);
        sBase[w][2] = (uint64_t)(reinterpret_cast<const bf16_t*>(k.C) + base * k.bcs + (int64_t)g * N);
        sBase[w][3] = (uint64_t)(reinterpret_cast<const bf16_t*>(k.dt) + base * k.dts + h0);
        sBase[w][4] = (uint64_t)(reinterpret_cast<bf16_t*>(k.y) + base * k.ys + (int64_t)h * P);
    }
    i32x4_t rx, rb, rc, rd;
    __amdgpu_buffer_rsrc_t ry;
    int wbase = 0;
    auto rebase = [&](int i0) __attribute__((always_inline)) {
        wbase = i0;
        const int r0 = i0 * Q;
        const int left = nrows - r0;
        const int rows = (left < (k.win + 3) * Q ? left : (k.win + 3) * Q) - 1;
        auto at = [&](int j, int stride) __attribute__((always_inline)) {
            const uint64_t v = sBase[w][j];
            const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
            return reinterpret_cast<const bf16_t*>(u) + (int64_t)r0 * stride;
        };
        rx = make_desc(at(0, xs), (uint32_t)(rows * xs + HPB * P) * 2u);
        const uint32_t bc_bytes = (uint32_t)(rows * bcs + N) * 2u;
        rb = make_desc(at(1, bcs), bc_bytes);
        rc = make_desc(at(2, bcs), bc_bytes);
        rd = make_desc(at(3, dts), (uint32_t)(rows * dts + HPB) * 2u);
        ry = make_rsrc(at(4, ys), (uint32_t)(rows * ys + P) * 2u);
    };
    // Chunk i's tiles into LDS buffer `buf`, dt first (the end-of-iteration wait counts on that order).
    // Seven loads per wave; the dt load runs on lanes 0..15 only.
    auto stream = [&](int i, int buf) __attribute__((always_inline)) {
        const uint32_t rel = (uint32_t)((i - wbase) * Q);
        uint8_t* dst = &tiles[buf * BUFB];
        if (lane < 16) load_lds4(rd, dst + DOFF + 64 * w, vdt + rel * (uint32_t)dts * 2u);
        const uint32_t dx = rel * (uint32_t)xs * 2u, db = rel * (uint32_t)bcs * 2u;
#pragma unroll
        for (int m = 0; m < 4; ++m) load_lds16(rx, dst + w * TILEB + 1024 * m, vx[m] + dx);
        load_lds16(rb, dst + BOFF + 1024 * w, vbc + db);
        load_lds16(rc, dst + COFF + 1024 * w, vbc + db);
    };

    // ---- chunk statistics of this wave's head, one token per lane, from the raw dt in tile buffer
    // `tbuf` into sSt[sbuf][w]; the chunk's wave-uniform values come back through dec_o (factor on
    // the stored state after the chunk's output) and lamend_o (its summed log-decay)
    float sig = 0.0f, lam_seg = 0.0f;
    auto stats = [&](int i, int tbuf, int sbuf, float& dec_o, float& lamend_o) __attribute__((always_inline)) {
        const int left = nrows - i * Q;
        const int valid = left < Q ? left : Q;
        const uint16_t raw = *reinterpret_cast<const uint16_t*>(&tiles[tbuf * BUFB + DOFF + 8 * (lane & 31) + 2 * hslot]);
        const float dtv = lane < valid ? dt_of(bits_to_f32(raw), bias_h, k.dt_min, k.dt_max) : 0.0f;
        const float lam = wave_prefix_sum(dtv * A_h);
        const float lam_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), Q - 1));
        const float l15 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 15));
        const float lam_blk = lane < 16 ? l15 : lam_end;
        const float sig_prev = sig;
        const bool rescale = sig_prev + lam_end < -kRescale;
        const float wexp = rescale ? lam_end - lam : -(sig_prev + lam);
        sig = rescale ? 0.0f : sig_prev + lam_end;
        const float lam_before = lam_seg;
        lam_seg += lam_end;
        if (lane < Q) {
            float* st = &sSt[sbuf][w][0][lane];
            st[0 * Q] = lam * kLog2e;
            const float dtx = dtv * xs_inv;
            st[1 * Q] = dtx;
            st[2 * Q] = fast_exp(wexp) * dtx;
            st[3 * Q] = fast_exp(lam + sig_prev);
            st[4 * Q] = fast_exp(lam_blk - lam) * dtx;
        }
        if (lane == 0 && k.ws_lamc && hvalid) k.ws_lamc[(c_begin + i) * BH + bh] = lam_before;
        dec_o = rescale ? fast_exp(sig_prev + lam_end) : 1.0f;
        lamend_o = lam_end;
    };

    float dec_n = 1.0f, lamend_n = 0.0f;
    if constexpr (FUSED) {
        // the raw x rows just before the segment (tokens row_begin-4 .. row_begin-1 of this head) into
        // the halo, where chunk 0's conv looks for the chunk before; before the sequence they come from
        // the conv history (or are zero)
        if (nc > 0 && lane < 32) {
            const int r = lane >> 3, u = lane & 7;
            const int64_t tau = row_begin - 4 + r;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (tau >= 0) {
                v = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(k.x) + (seq_row0(k, b) + tau) * k.xs +
                                                    (int64_t)h * P + 8 * u);
            } else if (cv.ring_in && tau >= -(int64_t)(cv.W - 1)) {
                const int slot = (int)(((cv.phase + tau) % cv.W + cv.W) % cv.W);
                v = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(cv.ring_in) +
                                                    (b * cv.W + slot) * cv.rs + (int64_t)h * P + 8 * u);
            }
            *reinterpret_cast<uint4*>(&sHalo[w][r * ROWB + ((u ^ rowperm(28 + r)) << 4)]) = v;
        }
    }
    if (nc > 0) {
        rebase(0);
        stream(0, 0);
        if (1 < nc) {
            stream(1, 1);
            wait_vmem<6>();  // chunk 0 and chunk 1's dt are in (six tile loads of chunk 1 may still run)
        } else {
            wait_vmem<0>();
        }
    }
    __syncthreads();
    if (nc > 0) stats(0, 0, 0, dec_n, lamend_n);

    int tcur = 0;  // tile buffer of chunk i (i mod 3)
    for (int i = 0; i < nc; ++i) {
        const int tnext = tcur == NBUF - 1 ? 0 : tcur + 1;
        const int tnext2 = tnext == NBUF - 1 ? 0 : tnext + 1;
        const int sbuf = i & 1;
        if (i - wbase == k.win) rebase(i);  // chunks i .. i+2 are addressed from here on
        const float dec = dec_n;
        const bool split_diag = lamend_n > -60.0f;  // every e^(Lam_t - Lam_s) splits into two finite factors
        if (i + 2 < nc) stream(i + 2, tnext2);
        uint8_t* const T = &tiles[tcur * BUFB];
        uint8_t* const Xt = T + w * TILEB;
        const uint8_t* const Bt = T + BOFF;
        const uint8_t* const Ct = T + COFF;
        const float* const lamh = sSt[sbuf][w][0];
        const float* const dth = sSt[sbuf][w][1];
        const float* const wh = sSt[sbuf][w][2];
        const float* const elh = sSt[sbuf][w][3];
        const float* const gsh = sSt[sbuf][w][4];
        // C rows (k = n): B operand of the state part and of the G tiles
        Frag<bf16_t> cf[2][2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint2 a = lds_read8(Ct, row_off(tb, ks, 0)), c = lds_read8(Ct, row_off(tb, ks, 1));
                cf[tb][ks].w[0] = a.x; cf[tb][ks].w[1] = a.y; cf[tb][ks].w[2] = c.x; cf[tb][ks].w[3] = c.y;
            }
        // Raised wave priority around the MFMA bursts (1 for the state part and G, 2 for the intra part
        // and the state update): of the two waves on a SIMD, the one with matrix products to issue goes
        // first, and the other's VALU work fills in beside them.
        __builtin_amdgcn_s_setprio(1);
        // state part: Y^T[p][t] = sum_n S[p][n] C[t][n], the state's bf16 copy as the A operand
        f32x4 accY[2][4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            Frag<bf16_t> sa[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 s0 = accS[pb][2 * ks], s1 = accS[pb][2 * ks + 1];
                sa[ks].set(0, s0[0], s0[1], s0[2], s0[3]);
                sa[ks].set(1, s1[0], s1[1], s1[2], s1[3]);
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                accY[tb][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
                mfma(accY[tb][pb], sa[0], cf[tb][0]);
                mfma(accY[tb][pb], sa[1], cf[tb][1]);
            }
        }
        // G^T[s][t] = sum_n B[s][n] C[t][n] for the tiles at or below the diagonal: g[sb][tb]
        f32x4 g00 = {0.f, 0.f, 0.f, 0.f}, g01 = g00, g11 = g00;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                Frag<bf16_t> bf;
                const uint2 a = lds_read8(Bt, row_off(sb, ks, 0)), c = lds_read8(Bt, row_off(sb, ks, 1));
                bf.w[0] = a.x; bf.w[1] = a.y; bf.w[2] = c.x; bf.w[3] = c.y;
                if (sb == 0) {
                    mfma(g00, bf, cf[0][ks]);
                    mfma(g01, bf, cf[1][ks]);
                } else {
                    mfma(g11, bf, cf[1][ks]);
                }
            }
        __builtin_amdgcn_s_setprio(0);
        // X columns (k = token s): A operand of the intra part, and the source of w_s x_s
        Frag<bf16_t> xf[4];
        Frag<bf16_t> xwh[4], xwl[4];  // w_s x_s as bf16 hi + lo (fused: from the fp32 conv output)
        if constexpr (FUSED) {
            // conv + SiLU of the raw x rows, straight into fragment order: lane (q, li) computes
            // x[s][p = 16 pb + li] for s = 4q .. 4q+3 and 16+4q .. 16+4q+3
            // group -1 reads the halo, addressed as rows 28..31
            const uint8_t* const XA = q == 0 ? &sHalo[w][0] : Xt;
            const int offA_ = q == 0 ? offA - 28 * ROWB : offA;
            const float4 w0 = *reinterpret_cast<const float4*>(wh + 4 * q);
            const float4 w1 = *reinterpret_cast<const float4*>(wh + 16 + 4 * q);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int m = (2 * pb) << 4;
                const uint2 ra = lds_read8_tr(XA, offA_ ^ m), rb = lds_read8_tr(Xt, offB ^ m);
                const uint2 rc = lds_read8_tr(Xt, offC ^ m), rd = lds_read8_tr(Xt, offD ^ m);
                float v[2][8];  // raw rows 4g .. 4g+7 of the two halves
                v[0][0] = lo_bf16(ra.x); v[0][1] = hi_bf16(ra.x); v[0][2] = lo_bf16(ra.y); v[0][3] = hi_bf16(ra.y);
                v[0][4] = lo_bf16(rb.x); v[0][5] = hi_bf16(rb.x); v[0][6] = lo_bf16(rb.y); v[0][7] = hi_bf16(rb.y);
                v[1][0] = lo_bf16(rc.x); v[1][1] = hi_bf16(rc.x); v[1][2] = lo_bf16(rc.y); v[1][3] = hi_bf16(rc.y);
                v[1][4] = lo_bf16(rd.x); v[1][5] = hi_bf16(rd.x); v[1][6] = lo_bf16(rd.y); v[1][7] = hi_bf16(rd.y);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float xo[4];  // log2(e) SiLU(conv) of tokens 4q+j (c = 0) or 16+4q+j (c = 1)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float bv = cb4[pb];
#pragma unroll
                        for (int t = 0; t < 4; ++t) bv = fmaf(cw[pb][t], v[c][j + 1 + t], bv);
                        // log2(e) a / (1 + e^-a) with bv = log2(e) a
                        xo[j] = bv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-bv));
                    }
                    xf[pb].set(c, xo[0], xo[1], xo[2], xo[3]);
                    const float4 wv = c == 0 ? w0 : w1;
                    const float p0 = xo[0] * wv.x, p1 = xo[1] * wv.y, p2 = xo[2] * wv.z, p3 = xo[3] * wv.w;
                    xwh[pb].set(c, p0, p1, p2, p3);
                    xwl[pb].set(c, p0 - xwh[pb].get(c, 0), p1 - xwh[pb].get(c, 1), p2 - xwh[pb].get(c, 2),
                                p3 - xwh[pb].get(c, 3));
                }
            }
            // this chunk's last four raw rows become the halo of the next (read before the output
            // staging below overwrites this tile; LDS operations of one wave run in order)
            if (lane < 32) {
                const int o = (lane >> 3) * ROWB + 16 * (lane & 7);
                const uint4 hv = *reinterpret_cast<const uint4*>(Xt + 28 * ROWB + o);
                *reinterpret_cast<uint4*>(&sHalo[w][o]) = hv;
            }
        } else {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const uint2 a = lds_read8_tr(Xt, col_off(0, pb)), c = lds_read8_tr(Xt, col_off(1, pb));
                xf[pb].w[0] = a.x; xf[pb].w[1] = a.y; xf[pb].w[2] = c.x; xf[pb].w[3] = c.y;
            }
        }
        // e^(Lam_t + sig) on the state part
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const float el = elh[16 * tb + li];
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) accY[tb][pb] *= el;
        }
        // M[t][s] = G[t][s] e^(Lam_t - Lam_s) dt_s for s <= t, + D on the diagonal, as bf16 hi + lo
        Frag<bf16_t> mh[2], ml[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int t = 16 * tb + li;
            const float lt = lamh[t];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                float m[4];
                if (sb > tb) {
                    m[0] = m[1] = m[2] = m[3] = 0.0f;
                } else {
                    const f32x4 gv = sb == 0 ? (tb == 0 ? g00 : g01) : g11;
                    const int s0 = 16 * sb + 4 * q;
                    if (sb < tb || split_diag) {
                        const float f = __builtin_amdgcn_exp2f(lt - lamh[16 * sb + 15]);
                        const float4 gs = *reinterpret_cast<const float4*>(gsh + s0);
                        m[0] = gv[0] * f * gs.x; m[1] = gv[1] * f * gs.y;
                        m[2] = gv[2] * f * gs.z; m[3] = gv[3] * f * gs.w;
                    } else {
                        const float4 ls = *reinterpret_cast<const float4*>(lamh + s0);
                        const float4 ds = *reinterpret_cast<const float4*>(dth + s0);
                        m[0] = gv[0] * __builtin_amdgcn_exp2f(lt - ls.x) * ds.x;
                        m[1] = gv[1] * __builtin_amdgcn_exp2f(lt - ls.y) * ds.y;
                        m[2] = gv[2] * __builtin_amdgcn_exp2f(lt - ls.z) * ds.z;
                        m[3] = gv[3] * __builtin_amdgcn_exp2f(lt - ls.w) * ds.w;
                    }
                    if (sb == tb) {  // causal mask (s <= t), D on the diagonal
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float v = 4 * q + j == li ? m[j] + D_h : m[j];
                            m[j] = 4 * q + j <= li ? v : 0.0f;
                        }
                    }
                }
                const uint32_t h01 = pack_bf16x2(m[0], m[1]), h23 = pack_bf16x2(m[2], m[3]);
                mh[tb].w[2 * sb] = h01;
                mh[tb].w[2 * sb + 1] = h23;
                ml[tb].w[2 * sb] = pack_bf16x2(m[0] - lo_bf16(h01), m[1] - hi_bf16(h01));
                ml[tb].w[2 * sb + 1] = pack_bf16x2(m[2] - lo_bf16(h23), m[3] - hi_bf16(h23));
            }
        }
        __builtin_amdgcn_s_setprio(2);
        // intra part: Y^T[p][t] += sum_s X[s][p] M[t][s]
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                mfma(accY[tb][pb], xf[pb], mh[tb]);
                mfma(accY[tb][pb], xf[pb], ml[tb]);
            }
        // ---- state update: S^T[n][p] = dec S^T[n][p] + sum_s B[s][n] (w_s X[s][p]), w_s x_s as bf16 hi + lo.
        // One channel block of w_s x_s is split at a time and its products issued before the next block
        // is split, so the split's VALU work runs beside the matrix cores; the y tile is staged and
        // stored after all of them are issued.
        if (dec != 1.0f) {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) accS[pb][nb] *= dec;
        }
        Frag<bf16_t> bt[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const uint2 a = lds_read8_tr(Bt, col_off(0, nb)), c = lds_read8_tr(Bt, col_off(1, nb));
            bt[nb].w[0] = a.x; bt[nb].w[1] = a.y; bt[nb].w[2] = c.x; bt[nb].w[3] = c.y;
        }
        const float4 w0 = *reinterpret_cast<const float4*>(wh + 4 * q);
        const float4 w1 = *reinterpret_cast<const float4*>(wh + 16 + 4 * q);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            if constexpr (!FUSED) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const float4 wv = c == 0 ? w0 : w1;
                    const float v0 = xf[pb].get(c, 0) * wv.x, v1 = xf[pb].get(c, 1) * wv.y;
                    const float v2 = xf[pb].get(c, 2) * wv.z, v3 = xf[pb].get(c, 3) * wv.w;
                    xwh[pb].set(c, v0, v1, v2, v3);
                    xwl[pb].set(c, v0 - xwh[pb].get(c, 0), v1 - xwh[pb].get(c, 1), v2 - xwh[pb].get(c, 2),
                                v3 - xwh[pb].get(c, 3));
                }
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                mfma(accS[pb][nb], bt[nb], xwh[pb]);
                mfma(accS[pb][nb], bt[nb], xwl[pb]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // the next chunk's statistics, issued behind the state-update products (they write the other
        // statistics buffer, which this chunk does not read)
        if (i + 1 < nc) stats(i + 1, tnext, sbuf ^ 1, dec_n, lamend_n);
        // y out: lane (q, li) holds y[t = 16 tb + li][p = 16 pb + 4q .. +3]; staged (in this wave's own
        // X tile, whose reads are done) so that each store instruction writes eight whole 128-byte rows
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const f32x4 a = accY[tb][pb];
                *reinterpret_cast<u32x2_t*>(Xt + ((arow ^ (((2 * pb) ^ (4 * tb)) << 4)) + 2048 * tb)) =
                    u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
            }
        const uint32_t yrow = (uint32_t)((i - wbase) * Q);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 8 * j + lrow;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Xt + r * ROWB + 16 * (lane & 7));
            const uint32_t off = (yrow + r) * (uint32_t)ys * 2u + (uint32_t)((((lane & 7) ^ rowperm(r))) << 4);
            __builtin_amdgcn_raw_buffer_store_b128(v, ry, (int)off, 0, 0);
        }

        // Chunk i+1's tiles and chunk i+2's dt must be in LDS before the barrier: the dt load is the first
        // of chunk i+2's seven, so at most its six tile loads and this chunk's four y stores may still run.
        if (i + 2 < nc) wait_vmem<10>();
        else wait_vmem<4>();
        __syncthreads();
        tcur = tnext;
    }

    // ---- the state S = e^sig S_hat: the final state (one segment) or this segment's end state
    const float escale = fast_exp(sig);
    float* dst = nullptr;
    if (k.nseg > 1) dst = k.ws_state + ((int64_t)seg * BH + bh) * P * N;
    else dst = k.state_out ? k.state_out + (int64_t)bh * P * N : nullptr;
    float emax = 0.0f;  // max |state entry|: the segment's state scale for the fix-up test
    if (dst && hvalid) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const f32x4 v = accS[pb][nb] * escale;
                *reinterpret_cast<float4*>(dst + (int64_t)(16 * pb + li) * N + 16 * nb + 4 * q) =
                    make_float4(v[0], v[1], v[2], v[3]);
                emax = fmaxf(emax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
            }
    }
    if (k.nseg > 1) {
        emax = wave_max(emax);
        if (hvalid && lane == 0) {
            k.ws_emax[(int64_t)seg * BH + bh] = emax;
            k.ws_lam[(int64_t)seg * BH + bh] = lam_seg;
        }
    }
    if constexpr (FUSED) {
        // the conv ring of the block's x channels: the last W raw tokens before the sequence's end,
        // written by the block that holds its last chunk (the first segment's, for an empty sequence)
        const bool last = nc > 0 ? c_stop == nchunks : (nchunks == 0 && seg == 0);
        if (last && cv.ring_out) {
            const int64_t c = (int64_t)h0 * P + threadIdx.x;  // 256 threads: the four heads' x channels
            const bf16_t* X = reinterpret_cast<const bf16_t*>(k.x);
            const bf16_t* R = reinterpret_cast<const bf16_t*>(cv.ring_in);
            bf16_t* O = reinterpret_cast<bf16_t*>(cv.ring_out);
            const int64_t row0 = seq_row0(k, b);
            for (int j = 0; j < cv.W; ++j) {
                const int64_t tau = Lb - cv.W + j;
                bf16_t v{0};
                if (tau >= 0) v = X[(row0 + tau) * k.xs + c];
                else if (R) v = R[(b * cv.W + (((cv.phase + tau) % cv.W + cv.W) % cv.W)) * cv.rs + c];
                O[(b * cv.W + j) * cv.rs + c] = v;
            }
        }
    }
}

hipError_t launch_ssd_walk(const ScanK& k, const WalkConv* conv, hipStream_t s) {
    if (conv) return launch_kernel(ssd_walk_kernel<true>, dim3(k.nblocks), dim3(walk::THREADS), 0, s, k, *conv);
    return launch_kernel(ssd_walk_kernel<false>, dim3(k.nblocks), dim3(walk::THREADS), 0, s, k, WalkConv{});
}

}  // namespace m2
