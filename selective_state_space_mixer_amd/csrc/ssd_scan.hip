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
// One workgroup walks the chunks of a few heads of one (sequence, segment) in order; each wave
// keeps its share of a head's fp32 state in MFMA accumulator registers for the whole walk.
// Per chunk, four contractions run on v_mfma_f32_16x16x32_bf16 (fp32 activations:
// v_mfma_f32_16x16x4f32):
//   G^T[s][t] = sum_n B[s][n] C[t][n]            -> masked and scaled in registers -> M[t][s]
//                                                   (bf16: as a hi + lo pair, see below)
//   Y^T[p][t] = sum_n S[p][n] C[t][n]             (state part, state as the A operand)
//   Y^T[p][t]+= sum_s X[s][p] M[t][s]             (intra-chunk part)
//   S^T[n][p] = e^Lam_end S^T[n][p] + sum_s B[s][n] (w_s X[s][p]),  w_s = e^(Lam_end-Lam_s) dt_s
// The e^Lam_t factor of the state part is applied to the output tile, w_s scales the X fragments
// already in registers, and the D skip is folded into M's diagonal.  G comes out of the MFMA in
// exactly the register layout M needs as a B operand, so M never leaves the wave that uses it.
//
// The X, B and C tiles of a chunk move from HBM straight into LDS (buffer loads with the LDS
// destination), double-buffered: chunk c+1 streams in while chunk c is computed, and one
// barrier per chunk publishes c+1 and frees c's buffer.  Rows past the end of the sequence
// fall outside the buffer range and read as zero.
//
// M carries the whole intra-chunk weight of a token on itself and its neighbours; where the
// decay is strong those terms are large and cancel, so a single bf16 rounding of M costs
// several percent of y.  M is therefore stored as bf16 hi = rn(M) and lo = rn(M - hi) and the
// intra contraction runs twice, which leaves M's error near 2^-17.
//
// Long sequences with few (sequence, head) pairs are split into segments that run in
// parallel: the main pass walks every segment at once (the first from the caller's state,
// the others from zero), a small pass chains the segments' end states into each segment's
// true initial state and the final state, and a fix-up adds the initial state's share of
// the later segments' outputs where it has not yet decayed away.
//
// Sequence b's rows start at b*L (or, in a packed batch, at cu_seqlens[b]) and it has L tokens
// (or its padded or packed length); chunks are counted from each sequence's own first row, so
// a chunk never holds two sequences, and chunks past a sequence's end are not run.
#include "ssd_common.h"

#include <mutex>
#include <numeric>

namespace m2 {

// Workspace for callers that cannot allocate (m2_ssd_scan_fwd_noalloc): a static array each GPU the
// library runs on holds until the process ends.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device, with that device
// current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t static_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

// Work split.  A wave owns PW p-blocks of one head, so its share of the state is at most
// kMaxStateTiles 16x16 accumulator tiles (32 registers); WPH waves cover a head.  A block holds
// HPW heads of one B/C group, which share the B and C tiles in LDS, and WAVES = HPW * WPH waves
// (eight where the LDS budget allows: two such blocks fill a compute unit at four waves per SIMD).
// Every wave forms the decay-masked matrix M of its own head from G = C B^T tiles it computes
// itself, so the only data exchanged between waves are the tiles and the chunk statistics.
constexpr int kMaxStateTiles = 8;
constexpr int kScanWaves = 8;  // waves per block, when the heads allow

template <typename T, int Q, int P, int N>
struct Cfg {
    using E = typename Lds<T>::E;
    static constexpr int NPB = P / 16;
    static constexpr int NNB = N / 16;
    static constexpr int NTB = Q / 16;
    static constexpr int PW0 = kMaxStateTiles / NNB > 0 ? kMaxStateTiles / NNB : 1;
    static constexpr int PW = NPB < PW0 ? NPB : PW0;
    static constexpr int WPH = NPB / PW;          // waves per head
    static constexpr int EPU = 16 / (int)sizeof(E);  // elements per 16-byte unit
    static constexpr int UX = P / EPU, UB = N / EPU;  // units per X row and per B/C row
    static constexpr int KS_N = (N + 31) / 32;    // K=32 steps over d_state
    static constexpr int KS_Q = (Q + 31) / 32;    // K=32 steps over tokens
    static constexpr int kStats = 5;              // per-token chunk statistics (see the kernel)
    static constexpr int round_kb(int units) { return (units + 63) / 64 * 64; }  // whole 1 KB pieces
    // LDS units (16 bytes) of one buffer: X tiles of hpw heads, then B and C (rows padded by a unit)
    static constexpr int x_units(int hpw) { return round_kb(hpw * Q * (UX + 1)); }
    static constexpr int b_units() { return round_kb(Q * (UB + 1)); }
    // a wave's y tile on its way out: Q rows of PW*16 elements
    static constexpr int YRB = PW * 16 * (int)sizeof(E);  // bytes per row
    static constexpr int lds_bytes(int hpw) {
        return 2 * (16 * (x_units(hpw) + 2 * b_units()) + (kStats * Q + 1) * hpw * 4) + hpw * WPH * Q * YRB;
    }
    static constexpr int kLdsBudget = sizeof(E) == 2 ? 80 * 1024 : 150 * 1024;
    static constexpr int hpw_fit() {
        int hpw = kScanWaves / WPH > 0 ? kScanWaves / WPH : 1;
        while (hpw > 1 && lds_bytes(hpw) > kLdsBudget) hpw /= 2;
        return hpw;
    }
    static constexpr int HPW = hpw_fit();         // heads per block
    static constexpr int WAVES = HPW * WPH;
    static constexpr int THREADS = 64 * WAVES;
    // blocks resident on one compute unit (the occupancy the register budget is set for): up to
    // four waves per SIMD, as far as the 160 KB of LDS allow
    static constexpr int BPC_LDS = 160 * 1024 / lds_bytes(HPW);
    static constexpr int BPC = 16 / WAVES < BPC_LDS ? 16 / WAVES : BPC_LDS;
    static constexpr int WPE = BPC * WAVES / 4 > 0 ? BPC * WAVES / 4 : 1;  // waves per SIMD
    static_assert(NPB % PW == 0 && WAVES <= 16, "work split");
};

// ----------------------------------------------------------------------------------------------
// chunk walk

template <typename T, int Q, int P, int N>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, Cfg<T, Q, P, N>::THREADS),
                               amdgpu_waves_per_eu(Cfg<T, Q, P, N>::WPE)))
ssd_chunk_scan_kernel(ScanK k)
{
    using Cf = Cfg<T, Q, P, N>;
    using E = typename Cf::E;
    constexpr int HPW = Cf::HPW, PW = Cf::PW, UX = Cf::UX, UB = Cf::UB, EPU = Cf::EPU;
    constexpr int XUN = Cf::x_units(HPW), BUN = Cf::b_units();
    constexpr int NXP = XUN / 64, NBP = BUN / 64;        // 1 KB pieces of the X tiles and of B (C)
    constexpr int NPIECE = NXP + 2 * NBP;
    constexpr int PPW = (NPIECE + Cf::WAVES - 1) / Cf::WAVES;  // pieces per wave (at most)
    constexpr bool kSplitM = sizeof(E) == 2;  // bf16 operands: M as hi + lo
    constexpr int QS = HPW * Q;               // one statistic of every head of the block
    constexpr uint32_t SZ = sizeof(T);

    // one buffer: X tiles [HPW][Q rows][UX units], B [Q][UB], C [Q][UB] (each rounded to 1 KB)
    __shared__ __attribute__((aligned(1024))) E tiles[2][(XUN + 2 * BUN) * EPU];
    // per head and token, in order: Lam*log2(e), dt, w = e^(Lam_end - Lam) dt, e^Lam, and
    // gs = e^(Lam_e - Lam) dt with e the last token of the token's 16-block
    __shared__ __attribute__((aligned(16))) float sSt[2][Cf::kStats * QS];
    __shared__ float sDec[2][HPW];    // factor applied to the stored state after the chunk's output
    __shared__ float sLamEnd[2][HPW]; // summed log-decay of the chunk
    __shared__ float sSig[HPW];       // log-scale of the stored state at the end of the walk
    __shared__ uint64_t sBase[Cf::WAVES][5];  // x, B, C, dt, y addresses at the segment's first row
    // Each wave's y tile is staged here so that it leaves in 16-byte pieces, consecutive lanes
    // covering consecutive bytes of a row (the accumulator layout gives each lane 4 elements of
    // one row, with the lanes of a row 16 apart).  16-byte unit u of row r sits at u ^ (r % YU).
    constexpr int YRB = Cf::YRB, YU = YRB / 16;         // bytes and 16-byte units per staged row
    constexpr int YRPS = 64 / YU;                       // rows per store instruction
    constexpr int NYS = (Q + YRPS - 1) / YRPS;  // store instructions per chunk
    __shared__ __attribute__((aligned(16))) uint8_t sY[Cf::WAVES * Q * YRB];

    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, li = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Waves w, w + HPW, w + 2 HPW, ... share head slot w % HPW, so the heads' statistics writers
    // (waves 0 .. HPW-1) sit on different SIMDs.
    const int hw = wave % HPW;                      // head slot of this wave
    const int pblk0 = (wave / HPW) * PW;            // first p-block of this wave
    const bool stats_writer = wave < HPW;

    // block -> (segment, sequence, head group)
    // Uniform sequences: each XCD takes a contiguous run of units (head groups sharing B/C rows in
    // one L2).  Right-padded lengths: which units have work is known only here, and the units of the
    // first segments (nearly all busy) come first; dealt round-robin as launched, they spread
    // evenly over the XCDs, where contiguous runs would pile them onto the first few.  A packed
    // batch's plan lists the units with work (block_unit).
    const int hpg = k.H / k.G;
    const int upg = (hpg + HPW - 1) / HPW;          // head units per group
    const int nhu = k.G * upg;
    int hu, seg;
    int64_t b;
    if (!block_unit(k, nhu, hu, b, seg)) return;
    const int g = hu / upg;
    const int h0 = g * hpg + (hu % upg) * HPW;
    const int hcount = hpg - (hu % upg) * HPW < HPW ? hpg - (hu % upg) * HPW : HPW;  // heads present
    const int h = h0 + (hw < hcount ? hw : hcount - 1);  // waves past the last head repeat it (results unused)
    const bool hvalid = hw < hcount;
    const int bh = (int)b * k.H + h;
    const int BH = k.batch * k.H;
    // a right-padded sequence ends at its own length: chunks past it are not run, a segment that
    // starts past it runs none (end state = start state, log-decay 0)
    const int64_t Lb = seq_len(k, b);
    const int64_t nchunks = (Lb + Q - 1) / Q;
    const int cps = seg_chunks(k);
    const int64_t c_begin = (int64_t)seg * cps;
    const int64_t c_stop = c_begin + cps < nchunks ? c_begin + cps : nchunks;
    const int nc = c_stop > c_begin ? (int)(c_stop - c_begin) : 0;  // chunks here
    const int64_t row_begin = c_begin * Q;                       // first token of the segment
    const int64_t row_end = Lb < row_begin + (int64_t)nc * Q ? Lb : row_begin + (int64_t)nc * Q;
    const float bias_h = k.dt_bias[h], A_h = k.A[h];
    const float D_h = k.D ? k.D[h] : 0.0f;

    // Byte offset, within a chunk's rows, of the 16-byte unit this lane brings into each of its
    // wave's LDS pieces (piece i = wave + WAVES * j), and which tile the piece belongs to.
    uint32_t voff[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int piece = wave + Cf::WAVES * j;
        const int u = piece * 64 + lane;  // unit index in the buffer
        uint32_t o = 0;
        // row padding and the rounding past the last row point outside every range (ranges stay
        // below 2^31 and so do chunk offsets): zero-filled
        if (piece < NXP) {
            const int hh = u / (Q * (UX + 1)), rem = u % (Q * (UX + 1)), r = rem / (UX + 1), pos = rem % (UX + 1);
            o = (u < HPW * Q * (UX + 1) && pos < UX) ? (uint32_t)(r * k.xs + hh * P + pos * EPU) * SZ : 0x80000000u;
        } else {
            const int ub = (u - XUN) % BUN;
            const int r = ub / (UB + 1), pos = ub % (UB + 1);
            o = (ub < Q * (UB + 1) && pos < UB) ? (uint32_t)(r * k.bcs + pos * EPU) * SZ : 0x80000000u;
        }
        voff[j] = o;
    }

    // state tiles in accumulator layout: accS[pw][nb][j] = S[p = (pblk0+pw)*16 + li][n = nb*16 + 4q + j]
    f32x4 accS[PW][Cf::NNB];
    {
        // the first segment starts from the caller's state; later ones from zero (their true
        // initial state is added to their output afterwards, see ssd_segment_fix_kernel)
        const float* src = nullptr;
        if (seg == 0) src = k.state_in ? k.state_in + (int64_t)bh * P * N : nullptr;
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

    // Buffer resources over a window of the segment's rows, starting at local chunk wbase; each
    // range ends with the last row of the window (the sequence, unless the window is cut short
    // to keep offsets below 2^31, and then only rows the window never serves are cut).  The
    // window bases are kept in LDS rather than in scalar registers: a rebase is rare.
    const int xs = (int)k.xs, bcs = (int)k.bcs, dts = (int)k.dts, ys = (int)k.ys;  // < 2^31 / (3 Q SZ)
    const int nrows = nc > 0 ? (int)(row_end - row_begin) : 0;
    if (lane == 0) {
        const int64_t base = seq_row0(k, b) + row_begin;
        sBase[wave][0] = (uint64_t)(reinterpret_cast<const T*>(k.x) + base * k.xs + (int64_t)h0 * P);
        sBase[wave][1] = (uint64_t)(reinterpret_cast<const T*>(k.B) + base * k.bcs + (int64_t)g * N);
        sBase[wave][2] = (uint64_t)(reinterpret_cast<const T*>(k.C) + base * k.bcs + (int64_t)g * N);
        sBase[wave][3] = (uint64_t)(reinterpret_cast<const T*>(k.dt) + base * k.dts + h);
        sBase[wave][4] = (uint64_t)(reinterpret_cast<T*>(k.y) + base * k.ys + (int64_t)h * P);
    }
    i32x4_t rx, rb, rc;
    __amdgpu_buffer_rsrc_t rd, ry;
    int wbase = 0;
    auto rebase = [&](int i0) __attribute__((always_inline)) {
        wbase = i0;
        const int r0 = i0 * Q;
        const int left = nrows - r0;
        const int rows = (left < (k.win + 2) * Q ? left : (k.win + 2) * Q) - 1;
        auto at = [&](int j, int stride) __attribute__((always_inline)) {
            const uint64_t v = sBase[wave][j];
            const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
            return reinterpret_cast<const T*>(u) + (int64_t)r0 * stride;
        };
        rx = make_desc(at(0, xs), (uint32_t)(rows * xs + hcount * P) * SZ);
        const uint32_t bc_bytes = (uint32_t)(rows * bcs + N) * SZ;
        rb = make_desc(at(1, bcs), bc_bytes);
        rc = make_desc(at(2, bcs), bc_bytes);
        rd = make_rsrc(at(3, dts), (uint32_t)(rows * dts + 1) * SZ);
        ry = make_rsrc(at(4, ys), hvalid ? (uint32_t)(rows * ys + P) * SZ : 0u);
    };
    auto valid_of = [&](int i) __attribute__((always_inline)) {
        const int left = nrows - i * Q;
        return left < Q ? left : Q;
    };
    // Stream local chunk i's tiles into LDS buffer `buf`: each wave issues its pieces.
    auto stream = [&](int i, int buf) __attribute__((always_inline)) {
        const uint32_t rel = (uint32_t)((i - wbase) * Q);
        const uint32_t dx = rel * (uint32_t)xs * SZ, db = rel * (uint32_t)bcs * SZ;
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
            const int piece = wave + Cf::WAVES * j;
            if (piece >= NPIECE) break;
            E* dst = &tiles[buf][piece * 64 * EPU];
            if (piece < NXP) load_lds16(rx, dst, voff[j] + dx);
            else if (piece < NXP + NBP) load_lds16(rb, dst, voff[j] + db);
            else load_lds16(rc, dst, voff[j] + db);
        }
    };
    // raw dt of this wave's head, one token per lane (zero past the sequence)
    auto load_dt = [&](int i) __attribute__((always_inline)) {
        const uint32_t row = (uint32_t)((i - wbase) * Q + lane);
        return load_raw(rd, row * (uint32_t)dts * SZ, (T*)nullptr);
    };
    // The state is kept as S = e^sig * S_hat: a chunk whose decay keeps sig above -kRescale only
    // adds to S_hat (its token weights carry e^-sig, at most e^kRescale), and the stored state is
    // multiplied out only when sig would drop below that.  The statistics writer of each head
    // tracks sig (and the segment's summed log-decay) as it prepares the chunks in order.
    constexpr float kRescale = 40.0f;
    float sig = 0.0f, lam_seg = 0.0f;
    // dt and the cumulative log-decay of this wave's head over chunk i, into statistics buffer buf
    auto stats = [&](int i, int buf, uint32_t raw) __attribute__((always_inline)) {
        if (!stats_writer) return;
        const int valid = valid_of(i);
        const float dtv = lane < valid ? dt_of(raw_to_f32(raw, (T*)nullptr), bias_h, k.dt_min, k.dt_max) : 0.0f;
        const float lam = wave_prefix_sum(dtv * A_h);
        const float lam_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), Q - 1));
        // log-decay at the last token of this lane's 16-block
        const float l15 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 15));
        const float l31 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 31));
        const float l47 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 47));
        const float l63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam), 63));
        const float lam_blk = lane < 16 ? l15 : lane < 32 ? l31 : lane < 48 ? l47 : l63;
        const float sig_prev = sig;
        const bool rescale = sig_prev + lam_end < -kRescale;
        // token weight e^(Lam_end - Lam_s) dt_s / e^sig_new, sig_new = 0 (rescale) or sig_prev + Lam_end
        const float wexp = rescale ? lam_end - lam : -(sig_prev + lam);
        sig = rescale ? 0.0f : sig_prev + lam_end;
        const float lam_before = lam_seg;  // summed log-decay of the segment before chunk i
        lam_seg += lam_end;
        if (lane < Q) {
            float* st = &sSt[buf][hw * Q + lane];
            st[0 * QS] = lam * kLog2e;
            st[1 * QS] = dtv;
            st[2 * QS] = fast_exp(wexp) * dtv;
            st[3 * QS] = fast_exp(lam + sig_prev);
            st[4 * QS] = fast_exp(lam_blk - lam) * dtv;
        }
        if (lane == 0) {
            sDec[buf][hw] = rescale ? fast_exp(sig_prev + lam_end) : 1.0f;
            sLamEnd[buf][hw] = lam_end;
            if (k.ws_lamc && hvalid) k.ws_lamc[(c_begin + i) * BH + bh] = lam_before;
        }
    };

    uint32_t dt_next = 0;  // raw dt of the chunk after the one being computed
    if (nc > 0) {
        rebase(0);
        const uint32_t dt0 = load_dt(0);
        if (1 < nc) dt_next = load_dt(1);
        stream(0, 0);
        stats(0, 0, dt0);
    }
    wait_vmem<0>();
    __syncthreads();
    // y stores issued per chunk: the end-of-chunk wait lets them drain in the background
    constexpr int kStores = NYS;
    for (int i = 0; i < nc; ++i) {
        const int buf = i & 1;
        if (i - wbase == k.win) rebase(i);  // chunks i .. i+2 are addressed from here on
        if (i + 1 < nc) {
            const uint32_t raw = dt_next;
            if (i + 2 < nc) dt_next = load_dt(i + 2);
            stream(i + 1, buf ^ 1);
            stats(i + 1, buf ^ 1, raw);
        }
        // wave-uniform chunk values: the stored state's factor, and whether every intra-chunk decay
        // factor e^(Lam_t - Lam_s) splits into two that stay finite
        const float dec = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sDec[buf][hw])));
        const bool split_diag =
            __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sLamEnd[buf][hw]))) > -60.0f;
        const E* const Xh = &tiles[buf][hw * Q * (UX + 1) * EPU];  // this wave's head tile
        const E* const Bs = &tiles[buf][XUN * EPU];
        const float* const lamh = &sSt[buf][0 * QS + hw * Q];
        const float* const dth = &sSt[buf][1 * QS + hw * Q];
        const float* const wh = &sSt[buf][2 * QS + hw * Q];
        const float* const elh = &sSt[buf][3 * QS + hw * Q];
        const float* const gsh = &sSt[buf][4 * QS + hw * Q];

        // X fragments of this wave's head (k = token s, column p): A operand of the intra part
        Frag<T> xf[PW][Cf::KS_Q];
#pragma unroll
        for (int pw = 0; pw < PW; ++pw)
#pragma unroll
            for (int ks = 0; ks < Cf::KS_Q; ++ks) xf[pw][ks] = frag_col<T, UX>(Xh, 32 * ks, Q, (pblk0 + pw) * 16, q, li);

        {
            const E* const Cs = Bs + BUN * EPU;
            // state part for every t-block first, so the bf16 copy of the state is dead before the
            // intra part: Y^T[p][t] = sum_n S[p][n] C[t][n] (the e^Lam_t factor comes later)
            f32x4 accY[Cf::NTB][PW];
            {
                // state as the A operand: sa[pw][ks] covers n = 32ks .. 32ks+31
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
#pragma unroll
                for (int tb = 0; tb < Cf::NTB; ++tb) {
#pragma unroll
                    for (int pw = 0; pw < PW; ++pw) accY[tb][pw] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < Cf::KS_N; ++ks) {
                        const Frag<T> cf = frag_row<T, UB>(Cs, tb * 16 + li, 32 * ks, N, q);
#pragma unroll
                        for (int pw = 0; pw < PW; ++pw) mfma(accY[tb][pw], sa[pw][ks], cf);
                    }
                }
            }
            // output rows of this chunk and head; rows past the sequence (and waves without a
            // head) fall outside the range of ry and are not written
            const uint32_t yrow = (uint32_t)((i - wbase) * Q);
            uint8_t* const ystage = &sY[wave * Q * YRB];
#pragma unroll
            for (int tb = 0; tb < Cf::NTB; ++tb) {
                const int t = tb * 16 + li;
                // C rows of this t-block: B operand of the G tiles
                Frag<T> cf[Cf::KS_N];
#pragma unroll
                for (int ks = 0; ks < Cf::KS_N; ++ks) cf[ks] = frag_row<T, UB>(Cs, t, 32 * ks, N, q);
                // G^T[s][t] = sum_n B[s][n] C[t][n] for the s-blocks at or below the diagonal, in
                // accumulator layout: gacc[sb][j] = G[t][s = sb*16 + 4q + j]
                f32x4 gacc[Cf::NTB];
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb) {
                    gacc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < Cf::KS_N; ++ks)
                        mfma(gacc[sb], frag_row<T, UB>(Bs, sb * 16 + li, 32 * ks, N, q), cf[ks]);
                }
                const float lt = lamh[t];
                const float el = elh[t];
#pragma unroll
                for (int pw = 0; pw < PW; ++pw) accY[tb][pw] *= el;
                // intra part: M[t][s] = G[t][s] e^(Lam_t - Lam_s) dt_s for s <= t, + D on the diagonal
#pragma unroll
                for (int ks = 0; ks < Cf::KS_Q; ++ks) {
                    if (32 * ks > tb * 16 + 15) continue;
                    Frag<T> mh, ml;
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const int sb = 2 * ks + cc;
                        if (sb > tb) {  // above the diagonal: zero
                            mh.set(cc, 0.f, 0.f, 0.f, 0.f);
                            ml.set(cc, 0.f, 0.f, 0.f, 0.f);
                            continue;
                        }
                        const f32x4 gv = gacc[sb];
                        const int s0 = sb * 16 + 4 * q;
                        float m[4];
                        if (sb < tb || split_diag) {
                            // e^(Lam_t - Lam_s) = e^(Lam_t - Lam_e) e^(Lam_e - Lam_s), e = last token of
                            // block sb, the second factor precomputed per token.  Below the diagonal
                            // both are <= 1; on it the first is at most e^60.
                            const float f = __builtin_amdgcn_exp2f(lt - lamh[sb * 16 + 15]);
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
                        if (sb == tb) {  // diagonal tile: causal mask (s <= t), D on the diagonal
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float v = 4 * q + j == li ? m[j] + D_h : m[j];
                                m[j] = 4 * q + j <= li ? v : 0.0f;
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
                        mfma(accY[tb][pw], xf[pw][ks], mh);
                        if constexpr (kSplitM) mfma(accY[tb][pw], xf[pw][ks], ml);
                    }
                }
                // stage: the lane holds y[t][p = (pblk0+pw)*16 + 4q .. +3]
#pragma unroll
                for (int pw = 0; pw < PW; ++pw) {
                    const int b = (pw * 16 + 4 * q) * (int)SZ;  // byte offset in this wave's row share
                    uint8_t* const dst = ystage + t * YRB + ((b >> 4) ^ (t % YU)) * 16 + (b & 15);
                    const f32x4 a = accY[tb][pw];
                    if constexpr (sizeof(E) == 2)
                        *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
                    else
                        *reinterpret_cast<f32x4*>(dst) = a;
                }
            }
            // out to HBM: lane L takes 16-byte unit L % YU of row j*YRPS + L / YU
#pragma unroll
            for (int j = 0; j < NYS; ++j) {
                const int r = j * YRPS + lane / YU, u = lane % YU;
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ystage + (r < Q ? r : 0) * YRB + (u ^ (r % YU)) * 16);
                const uint32_t off = r < Q ? ((yrow + r) * (uint32_t)ys + pblk0 * 16) * SZ + u * 16 : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b128(v, ry, (int)off, 0, 0);
            }
        }

        // ---- state update: S_hat^T[n][p] = dec S_hat^T[n][p] + sum_s B[s][n] (w_s X[s][p])
        if (dec != 1.0f) {
#pragma unroll
            for (int pw = 0; pw < PW; ++pw)
#pragma unroll
                for (int nb = 0; nb < Cf::NNB; ++nb) accS[pw][nb] *= dec;
        }
#pragma unroll
        for (int ks = 0; ks < Cf::KS_Q; ++ks) {
            // w_s X[s][p]: bf16 operands carry it as hi = rn(v) and lo = rn(v - hi) (two products),
            // so the state does not take a 2^-9 rounding of every token's contribution
            Frag<T> xw[PW], xl[PW];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int s0 = 32 * ks + 16 * cc + 4 * q;
                const float4 wv = s0 < Q ? *reinterpret_cast<const float4*>(wh + s0) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int pw = 0; pw < PW; ++pw) {
                    const float v0 = xf[pw][ks].get(cc, 0) * wv.x, v1 = xf[pw][ks].get(cc, 1) * wv.y;
                    const float v2 = xf[pw][ks].get(cc, 2) * wv.z, v3 = xf[pw][ks].get(cc, 3) * wv.w;
                    xw[pw].set(cc, v0, v1, v2, v3);
                    if constexpr (kSplitM)
                        xl[pw].set(cc, v0 - xw[pw].get(cc, 0), v1 - xw[pw].get(cc, 1), v2 - xw[pw].get(cc, 2),
                                   v3 - xw[pw].get(cc, 3));
                }
            }
#pragma unroll
            for (int nb = 0; nb < Cf::NNB; ++nb) {
                const Frag<T> bf = frag_col<T, UB>(Bs, 32 * ks, Q, nb * 16, q, li);
#pragma unroll
                for (int pw = 0; pw < PW; ++pw) {
                    mfma(accS[pw][nb], bf, xw[pw]);
                    if constexpr (kSplitM) mfma(accS[pw][nb], bf, xl[pw]);
                }
            }
        }
        wait_vmem<kStores>();  // this wave's pieces of chunk i+1 are in LDS (the y stores may still drain)
        __syncthreads();       // chunk i+1 published, chunk i's buffer free
    }

    // ---- write the state S = e^sig S_hat: S[p][n..n+3] per lane
    if (stats_writer && lane == 0) sSig[hw] = sig;
    __syncthreads();
    const float escale = fast_exp(sSig[hw]);
    // one segment: the final state; several: this segment's end state from its own start, for the chain
    float* dst = nullptr;
    if (k.nseg > 1) dst = k.ws_state + ((int64_t)seg * BH + bh) * P * N;
    else dst = k.state_out ? k.state_out + (int64_t)bh * P * N : nullptr;
    float emax = 0.0f;  // max |state entry| of this wave's share
    if (dst && hvalid) {
#pragma unroll
        for (int pw = 0; pw < PW; ++pw) {
            const int p = (pblk0 + pw) * 16 + li;
#pragma unroll
            for (int nb = 0; nb < Cf::NNB; ++nb) {
                const f32x4 v = accS[pw][nb] * escale;
                *reinterpret_cast<float4*>(dst + (int64_t)p * N + nb * 16 + 4 * q) =
                    make_float4(v[0], v[1], v[2], v[3]);
                emax = fmaxf(emax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
            }
        }
    }
    if (k.nseg > 1) {
        // the segment's state scale for the fix-up test: max over the head's waves
        __shared__ float sEmax[Cf::WAVES];
        emax = wave_max(emax);
        if (lane == 0) sEmax[wave] = emax;
        __syncthreads();
        if (hvalid && stats_writer && lane == 0) {
            float m = 0.0f;
            for (int j = hw; j < Cf::WAVES; j += HPW) m = fmaxf(m, sEmax[j]);
            k.ws_emax[(int64_t)seg * BH + bh] = m;
            k.ws_lam[(int64_t)seg * BH + bh] = lam_seg;
        }
    }
}

// Chain the segments.  E[seg] is segment seg's end state from its own start (segment 0 starts from
// the caller's state), lam[seg] its summed log-decay.  The true end states follow
//   T[0] = E[0],  T[seg] = e^lam[seg] T[seg-1] + E[seg];
// T[seg] (the initial state of segment seg+1) is written over E[seg] (or, for bf16 outputs, to a
// bf16 copy), and T of the sequence's last segment is the final state.  A sequence's segments past
// its last chunk hold nothing (end state = start state, log-decay 0), so the chain stops at its last
// segment with work.  Only the combine is sequential: the loads of a batch of segments are issued
// together (kBatch of them: 8 for the few segments of a packed batch's plan, whose registers then
// leave room for more waves, else 32), and only segments that exist are loaded.  The first block of
// each sequence-head also chains the bounds Tb[seg] on max|T[seg]| from the segments' recorded
// maxima (see fix_cut).
template <int kBatch>
__global__ __launch_bounds__(256) void ssd_segment_chain_kernel(ScanK k, int BH, int PN, int Q)
{
    const int bh = blockIdx.y;
    const int cps = seg_chunks(k);
    const int64_t cb = (seq_len(k, bh / k.H) + Q - 1) / Q;
    const int64_t sb = (cb + cps - 1) / cps;
    const int nseg = sb < 1 ? 1 : (sb < k.nseg ? (int)sb : k.nseg);
    float* __restrict__ ws_state = k.ws_state;
    const float* __restrict__ ws_lam = k.ws_lam;
    const float* __restrict__ ws_emax = k.ws_emax;
    uint16_t* __restrict__ tin = k.ws_tin;
    // four consecutive state entries per thread (PN is a multiple of 16)
    const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= PN) return;
    // the first block of each sequence-head also chains the bounds on the end states' maxima
    const bool bound = blockIdx.x == 0 && threadIdx.x == 0;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    float tb = 0.0f;
    for (int seg0 = 0; seg0 < nseg; seg0 += kBatch) {
        float4 loc[kBatch];
        float dec[kBatch], em[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int seg = seg0 + j;
            if (seg < nseg) {
                loc[j] = *reinterpret_cast<const float4*>(ws_state + ((int64_t)seg * BH + bh) * PN + i);
                dec[j] = ws_lam[(int64_t)seg * BH + bh];
                em[j] = ws_emax[(int64_t)seg * BH + bh];
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int seg = seg0 + j;
            if (seg < nseg) {
                const float d = seg == 0 ? 0.0f : fast_exp(dec[j]);
                s = make_float4(d * s.x + loc[j].x, d * s.y + loc[j].y, d * s.z + loc[j].z, d * s.w + loc[j].w);
                tb = d * tb + em[j];
                if (bound) k.ws_tb[(int64_t)seg * BH + bh] = tb;
                const int64_t o = ((int64_t)seg * BH + bh) * PN + i;
                if (seg < nseg - 1) {
                    // the initial state of segment seg+1, for the fix-up: in bf16 when that is the
                    // precision it enters the fix-up's product in
                    if (tin) *reinterpret_cast<uint2*>(tin + o) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
                    else *reinterpret_cast<float4*>(ws_state + o) = s;
                } else if (k.state_out) {
                    *reinterpret_cast<float4*>(k.state_out + (int64_t)bh * PN + i) = s;
                }
            }
        }
    }
}

// Add the part of each later segment's output that comes from its true initial state S_in (the
// main pass ran it from zero):  y[t] += e^Lam_t (S_in . C_t),  Lam_t = the summed log-decay from the
// segment's first token through t.  The factor only falls along the segment, so only a leading run of
// its chunks needs the term (the test of fix_cut, on the main pass's and the chain kernel's figures).
// A wave takes one such chunk at a time: S_in, dt, C and y are loaded together, then the term is
// added and y stored.
constexpr int kFixThreads = 256;
constexpr int kFixBlocksPerCU = 4;

// Eight consecutive k-values of one lane, k = kbase + 8q .. +7, for a K = 32 MFMA step.  The fix-up
// gives both operands this assignment (any assignment the two operands share gives the same sum),
// so each lane reads 16 (bf16) or 32 (fp32) contiguous bytes of a row.
__device__ __forceinline__ void load8(Frag<bf16_t>& f, const void* src) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    f.w[0] = v.x; f.w[1] = v.y; f.w[2] = v.z; f.w[3] = v.w;
}
__device__ __forceinline__ void load8(Frag<float>& f, const void* src) {
    const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
template <typename T> __device__ __forceinline__ void zero8(Frag<T>& f) {
    f.set(0, 0.f, 0.f, 0.f, 0.f);
    f.set(1, 0.f, 0.f, 0.f, 0.f);
}

template <typename T, int Q, int P, int N>
__global__ __launch_bounds__(kFixThreads) void ssd_segment_fix_kernel(ScanK k)
{
    constexpr int NPB = P / 16, KS_N = (N + 31) / 32, NTB = Q / 16;
    constexpr int EB = (int)sizeof(T);
    // The term comes out of the MFMA as 4 consecutive p of one row per lane; it goes through LDS
    // (fp32, 16 rows at a time) so that y is read and written as 16 contiguous bytes per lane, whole
    // rows of the head per group of lanes.
    constexpr int EPL = 16 / EB;                  // y elements per lane and row piece
    constexpr int LPR = P / EPL;                  // lanes per row
    constexpr int RPP = 64 / LPR;                 // rows per pass
    constexpr int NPASS = (16 + RPP - 1) / RPP;   // passes per 16 rows
    constexpr int RS = P + 4;                     // LDS row stride in floats
    static_assert(64 % LPR == 0 && LPR >= 1, "y row pieces must tile a wave");
    __shared__ __attribute__((aligned(16))) float sAcc[kFixThreads / 64][16 * RS];
    const int lane = threadIdx.x & 63, q = lane >> 4, li = lane & 15;
    float* acc_lds = sAcc[threadIdx.x >> 6];
    const int prow = lane / LPR, pcol = (lane % LPR) * EPL;  // this lane's row in a pass, first column
    const int BH = k.batch * k.H;
    // Candidates: chunk j of pair = (later segment - 1) * BH + bh is cand = pair * cps + j.  Block b
    // tests b, b + nblocks, ..., a thread each, lists in LDS the ones that pass, and its waves share
    // the list.  A block count sharing a factor f with cps would give each block only chunks
    // j = b (mod f) of their segments, and the blocks holding the leading chunks (the ones that need
    // the term) would carry f times their share: the blocks past the largest count coprime to cps
    // sit out (the host makes its own count coprime to its cps; a packed plan may pick another).
    __shared__ int sItem[kFixThreads];
    __shared__ int sCount;
    const int npairs = (k.nseg - 1) * BH;
    const int cps = seg_chunks(k);
    const int64_t ncand = (int64_t)npairs * cps;
    auto gcd = [](int a, int b) {
        while (b) {
            const int t = a % b;
            a = b;
            b = t;
        }
        return a;
    };
    int nb = (int)gridDim.x;
    while (nb > 1 && gcd(nb, cps) > 1) --nb;
    if ((int)blockIdx.x >= nb) return;
    const int64_t nblk = nb;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t base = blockIdx.x; base < ncand; base += nblk * kFixThreads) {
        bool act = false;
        {
            const int64_t cand = base + (int64_t)threadIdx.x * nblk;
            const int pair = (int)(cand / cps), j = (int)(cand % cps);
            if (cand < ncand && pair < npairs) {
                const int seg = 1 + pair / BH, bh = pair % BH;
                const int64_t c = (int64_t)seg * cps + j;
                // chunks past the sequence have no recorded log-decay and nothing to fix
                if (c * Q < seq_len(k, bh / k.H)) {
                    const float tb = k.ws_tb[pair], em = k.ws_emax[pair + BH], lb = k.ws_lamc[c * BH + bh];
                    // e^lb tb >= e^cut em, in nats (a zero tb needs nothing, a zero em everything, NaN keeps it)
                    constexpr float kLn2 = 0.6931471805599453f;
                    act = tb != 0.0f &&
                          !(lb + kLn2 * __builtin_amdgcn_logf(tb) < fix_cut<T>() + kLn2 * __builtin_amdgcn_logf(em));
                }
            }
        }
        if (threadIdx.x == 0) sCount = 0;
        __syncthreads();
        const uint64_t mask = __ballot(act);
        int pos = 0;
        if (lane == 0 && mask) pos = atomicAdd(&sCount, (int)__popcll(mask));
        pos = __shfl(pos, 0, 64);
        if (act) sItem[pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u))] = threadIdx.x;
        __syncthreads();
        const int nitems = sCount;
        for (int it = wave; it < nitems; it += kFixThreads / 64) {
            const int64_t cand = base + (int64_t)sItem[it] * nblk;
            const int pair = (int)(cand / cps), j = (int)(cand % cps);
            const int seg = 1 + pair / BH, bh = pair % BH;
            const int64_t b = bh / k.H;
            const int h = bh % k.H, g = h / (k.H / k.G);
            const int64_t c = (int64_t)seg * cps + j;
            const int64_t t0 = c * Q;
            const int64_t left = seq_len(k, b) - t0;
            const int valid = (int)(left < Q ? left : Q);  // >= 1: tested chunks lie inside the sequence

            // S_in as the A operand of Y^T[p][t] = sum_n S[p][n] C[t][n] (rows p), from the chain's bf16
            // copy for bf16 outputs, else from its fp32 states
            Frag<T> sa[NPB][KS_N];
            const int64_t soff = ((int64_t)(seg - 1) * BH + bh) * P * N;
            const void* sbase = EB == 2 ? (const void*)(k.ws_tin + soff) : (const void*)(k.ws_state + soff);
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
                for (int ks = 0; ks < KS_N; ++ks) {
                    const int n0 = 32 * ks + 8 * q;
                    if (n0 < N) load8(sa[pb][ks], (const uint8_t*)sbase + ((int64_t)(pb * 16 + li) * N + n0) * EB);
                    else zero8(sa[pb][ks]);
                }
            // the chunk: starting log-decay, dt of token `lane`, C rows (B operand, rows t) and y (rows
            // past the sequence clamped to its last token; their stores are skipped)
            const float lam0 = k.ws_lamc[c * BH + bh];
            const int64_t row0 = seq_row0(k, b);
            const T* dtp = reinterpret_cast<const T*>(k.dt) + row0 * k.dts + h;
            const T dtr = dtp[(t0 + (lane < valid ? lane : valid - 1)) * k.dts];
            const uint8_t* cp =
                reinterpret_cast<const uint8_t*>(reinterpret_cast<const T*>(k.C) + row0 * k.bcs + (int64_t)g * N);
            uint8_t* yp = reinterpret_cast<uint8_t*>(reinterpret_cast<T*>(k.y) + row0 * k.ys + (int64_t)h * P);
            Frag<T> cf[NTB][KS_N];
            uint4 yv[NTB][NPASS];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const int t = tb * 16 + li;
                const int tr = t < valid ? t : valid - 1;
#pragma unroll
                for (int ks = 0; ks < KS_N; ++ks) {
                    const int n0 = 32 * ks + 8 * q;
                    if (n0 < N) load8(cf[tb][ks], cp + ((t0 + tr) * k.bcs + n0) * EB);
                    else zero8(cf[tb][ks]);
                }
#pragma unroll
                for (int ps = 0; ps < NPASS; ++ps) {
                    const int row = tb * 16 + ps * RPP + prow;
                    const int rr = row < valid ? row : valid - 1;
                    yv[tb][ps] = *reinterpret_cast<const uint4*>(yp + ((t0 + rr) * k.ys + pcol) * EB);
                }
            }
            const float dtv = lane < valid ? dt_of(to_f32(dtr), k.dt_bias[h], k.dt_min, k.dt_max) : 0.0f;
            const float lam = lam0 + wave_prefix_sum(dtv * k.A[h]);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                // e^Lam_t (S_in . C_t) for the 16 rows t = tb*16 + li, into LDS as [row][p]
                const float el = fast_exp(__shfl(lam, tb * 16 + li, 64));
#pragma unroll
                for (int pb = 0; pb < NPB; ++pb) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS_N; ++ks) mfma(acc, sa[pb][ks], cf[tb][ks]);
                    *reinterpret_cast<float4*>(acc_lds + li * RS + pb * 16 + 4 * q) =
                        make_float4(el * acc[0], el * acc[1], el * acc[2], el * acc[3]);
                }
                // back in row pieces (LDS operations of one wave complete in order): y += term
#pragma unroll
                for (int ps = 0; ps < NPASS; ++ps) {
                    const int rloc = ps * RPP + prow;
                    const int row = tb * 16 + rloc;
                    if (rloc < 16 && row < valid) {
                        const float* src = acc_lds + rloc * RS + pcol;
                        uint8_t* dst = yp + ((t0 + row) * k.ys + pcol) * EB;
                        const uint4 v = yv[tb][ps];
                        if constexpr (EB == 2) {
                            const float4 a = reinterpret_cast<const float4*>(src)[0];
                            const float4 e = reinterpret_cast<const float4*>(src)[1];
                            *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(lo_bf16(v.x) + a.x, hi_bf16(v.x) + a.y),
                                                                        pack_bf16x2(lo_bf16(v.y) + a.z, hi_bf16(v.y) + a.w),
                                                                        pack_bf16x2(lo_bf16(v.z) + e.x, hi_bf16(v.z) + e.y),
                                                                        pack_bf16x2(lo_bf16(v.w) + e.z, hi_bf16(v.w) + e.w));
                        } else {
                            const float4 a = *reinterpret_cast<const float4*>(src);
                            *reinterpret_cast<float4*>(dst) =
                                make_float4(__uint_as_float(v.x) + a.x, __uint_as_float(v.y) + a.y,
                                            __uint_as_float(v.z) + a.z, __uint_as_float(v.w) + a.w);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

// The plan of a packed batch, from its lengths (which only the device holds).  Chunks per segment:
// the least cps in [lo, hi] for which the (sequence, segment) pairs, sum_b max(1, ceil(c_b / cps)),
// fit the `pairs` that one round of resident blocks holds.  hi always fits (the host's bound for any
// lengths), and lo is the least any lengths of the batch's total could call for, so the host's grid
// and workspace, sized for lo, cover the choice.  Then the pairs themselves, sequence by sequence
// (an empty sequence keeps one, which passes its initial state on).  One block; uniform over it.
__global__ __launch_bounds__(256) void ssd_packed_plan_kernel(ScanK k, int Q, int pairs, int lo, int hi, int* plan)
{
    __shared__ int sRed[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    auto chunks = [&](int64_t b) { return (seq_len(k, b) + Q - 1) / Q; };
    auto segs_of = [](int64_t c, int cps) {
        const int64_t n = (c + cps - 1) / cps;
        return (int)(n < 1 ? 1 : n);
    };
    auto segs = [&](int64_t b, int cps) { return segs_of(chunks(b), cps); };
    // a batch of at most one block's threads: each thread's sequence is read once
    const bool one = k.batch <= 256;
    const int64_t cmine = one && (int)threadIdx.x < k.batch ? chunks(threadIdx.x) : 0;
    while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        int n = 0;
        if (one) n = (int)threadIdx.x < k.batch ? segs_of(cmine, mid) : 0;
        else
            for (int b = threadIdx.x; b < k.batch; b += 256) n += segs(b, mid);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) n += __shfl_xor(n, o, 64);
        if (lane == 0) sRed[wave] = n;
        __syncthreads();
        const int tot = sRed[0] + sRed[1] + sRed[2] + sRed[3];
        __syncthreads();
        if (tot <= pairs) hi = mid;
        else lo = mid + 1;
    }
    int2* table = reinterpret_cast<int2*>(plan + 2);
    int base = 0;
    for (int b0 = 0; b0 < k.batch; b0 += 256) {
        const int b = b0 + (int)threadIdx.x;
        const int n = b < k.batch ? segs(b, hi) : 0;
        int x = n;  // inclusive prefix sum over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) sRed[wave] = x;
        __syncthreads();
        int off = base + x - n;
        for (int j = 0; j < wave; ++j) off += sRed[j];
        const int tot = sRed[0] + sRed[1] + sRed[2] + sRed[3];
        __syncthreads();
        for (int j = 0; j < n; ++j) table[off + j] = make_int2(b, j);
        base += tot;
    }
    if (threadIdx.x == 0) {
        plan[0] = hi;
        plan[1] = base;
    }
}

// ----------------------------------------------------------------------------------------------
// host side

struct Plan {
    int nseg, cps, nhu;
    int cps_lo, pairs;  // packed batch: the device picks cps in [cps_lo, cps] (equal: no pick)
    size_t ws_bytes;
};

// Byte offsets of the workspace parts, from a 256-byte aligned base (the caller's pointer rounded up):
// segment states [nseg][B*H][P*N] f32, segment log-decays [nseg][B*H] f32, per-chunk starting
// log-decays [nchunks][B*H] f32, the segments' own end-state maxima and the bounds on their true ones
// [nseg][B*H] f32 each, for bf16 outputs the segments' initial states in bf16 [nseg-1][B*H][P*N],
// and a packed batch's plan: two ints and up to nseg * batch (sequence, segment) pairs.
struct WsLayout {
    size_t lam, emax, tb, lamc, tin, plan, total;
};
static WsLayout ws_layout(int64_t nseg, int64_t batch, int64_t BH, int64_t PN, int64_t nchunks, bool bf16) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    WsLayout w;
    w.lam = up((size_t)(nseg * BH * PN) * sizeof(float));
    w.emax = up(w.lam + (size_t)(nseg * BH) * sizeof(float));
    w.tb = up(w.emax + (size_t)(nseg * BH) * sizeof(float));
    w.lamc = up(w.tb + (size_t)(nseg * BH) * sizeof(float));
    w.tin = up(w.lamc + (size_t)(nchunks * BH) * sizeof(float));
    w.plan = up(w.tin + (bf16 ? (size_t)((nseg - 1) * BH * PN) * sizeof(uint16_t) : 0));
    w.total = w.plan + 2 * sizeof(int) + (size_t)(nseg * batch) * 2 * sizeof(int);
    return w;
}

// Segments: enough (sequence, head group, segment) units for one round of resident blocks.
// A packed batch (total >= 0 tokens, L the longest sequence): every (sequence, segment) pair with
// work should fit in one round of resident blocks.  For any lengths, sum_b ceil(c_b / cps) <=
// (total chunks + batch) / cps + batch bounds their number, which gives the upper bound cps; no
// lengths can fit fewer than cps_lo = ceil(total chunks / pairs).  The lengths are device memory, so
// the plan kernel picks the least that fits between the two, and the grid and the workspace are
// sized for cps_lo.
static Plan plan_for(int64_t batch, int64_t L, int H, int G, int N_P_N, int Q, int hpw, int bpc, bool bf16,
                     int64_t total) {
    Plan pl;
    const int cus = device_shape().cus;
    const int64_t nchunks = (L + Q - 1) / Q;
    const int hpg = H / G;
    pl.nhu = G * ((hpg + hpw - 1) / hpw);
    const int64_t units = batch * pl.nhu;
    const int64_t target = (int64_t)cus * bpc;  // blocks resident at once
    int64_t cps, cps_lo = 0;
    pl.pairs = 0;
    if (total >= 0) {
        const int64_t pairs = target / pl.nhu;                  // (sequence, segment) pairs per round
        const int64_t rchunks = (total + Q - 1) / Q;
        const int64_t tchunks = rchunks + batch;
        cps = pairs > batch ? (tchunks + (pairs - batch) - 1) / (pairs - batch) : nchunks;
        cps_lo = pairs > batch ? (rchunks + pairs - 1) / pairs : cps;
        pl.pairs = (int)(pairs < INT32_MAX ? pairs : INT32_MAX);
    } else {
        int64_t nseg = units > 0 ? target / units : 1;
        if (nseg > nchunks) nseg = nchunks;
        if (nseg < 1) nseg = 1;
        cps = nchunks > 0 ? (nchunks + nseg - 1) / nseg : 1;
    }
    if (cps > nchunks) cps = nchunks;
    if (cps < 1) cps = 1;
    if (total < 0 || cps_lo > cps) cps_lo = cps;
    if (cps_lo < 1) cps_lo = 1;
    const int64_t nseg = nchunks > 0 ? (nchunks + cps_lo - 1) / cps_lo : 1;
    pl.nseg = (int)nseg;
    pl.cps = (int)cps;
    pl.cps_lo = (int)cps_lo;
    pl.ws_bytes = nseg > 1 ? ws_layout(nseg, batch, batch * H, N_P_N, nchunks, bf16).total + 256 : 0;
    return pl;
}

template <typename T, int Q, int P, int N>
static Plan plan_of(int64_t batch, int64_t L, int H, int G, int64_t total) {
    using Cf = Cfg<T, Q, P, N>;
    return plan_for(batch, L, H, G, P * N, Q, Cf::HPW, Cf::BPC, sizeof(T) == 2, total);
}

template <typename T, int Q, int P, int N>
static hipError_t run_scan(const ScanArgs& a, hipStream_t s, const WalkConv* conv = nullptr) {
    using Cf = Cfg<T, Q, P, N>;
    const Plan pl = plan_of<T, Q, P, N>(a.batch, a.L, a.H, a.G, a.cu ? a.total : -1);
    ScanK k;
    k.x = a.x; k.B = a.B; k.C = a.C; k.dt = a.dt;
    k.xs = a.xs; k.bcs = a.bcs; k.dts = a.dts; k.ys = a.ys;
    k.dt_bias = a.dt_bias; k.A = a.A; k.D = a.D; k.dt_min = a.dt_min; k.dt_max = a.dt_max;
    k.state_in = a.state_in; k.state_out = a.state_out; k.y = a.y;
    k.L = a.L; k.batch = (int)a.batch; k.H = a.H; k.G = a.G; k.lens = a.lens; k.cu = a.cu; k.total = a.total;
    k.nseg = pl.nseg; k.cps = pl.cps;
    // buffer-resource windows: every byte offset inside one must stay below 2^31
    int64_t row_bytes = a.xs > a.bcs ? a.xs : a.bcs;
    row_bytes = row_bytes > a.dts ? row_bytes : a.dts;
    row_bytes = (row_bytes > a.ys ? row_bytes : a.ys) * (int64_t)sizeof(T);
    const int64_t win = (((int64_t)1 << 31) - 1) / ((int64_t)Q * row_bytes) - 3;
    if (win < 1) return hipErrorInvalidValue;
    k.win = (int)(win < pl.cps ? win : pl.cps);
    const int BH = (int)(a.batch * a.H);
    k.ws_state = nullptr;
    k.ws_lam = nullptr;
    k.ws_lamc = nullptr;
    k.ws_tin = nullptr;
    k.ws_emax = nullptr;
    k.ws_tb = nullptr;
    k.plan = nullptr;
    if (pl.nseg > 1) {
        const WsLayout w = ws_layout(pl.nseg, a.batch, BH, P * N, (a.L + Q - 1) / Q, sizeof(T) == 2);
        uint8_t* base = reinterpret_cast<uint8_t*>(((uintptr_t)a.ws + 255) & ~(uintptr_t)255);
        k.ws_state = reinterpret_cast<float*>(base);
        k.ws_lam = reinterpret_cast<float*>(base + w.lam);
        k.ws_emax = reinterpret_cast<float*>(base + w.emax);
        k.ws_tb = reinterpret_cast<float*>(base + w.tb);
        k.ws_lamc = reinterpret_cast<float*>(base + w.lamc);
        if (sizeof(T) == 2) k.ws_tin = reinterpret_cast<uint16_t*>(base + w.tin);
        if (pl.cps_lo < pl.cps) k.plan = reinterpret_cast<int*>(base + w.plan);
    }
    // every segment at once (later ones from a zero state), then, with several segments, the chain
    // of their end states and the fix-up of the later segments' leading chunks
    k.nblocks = pl.nseg * (int)a.batch * pl.nhu;
    k.nxcd = device_shape().xcds;
    hipError_t e;
    bool walk = false;
    if constexpr (sizeof(T) == 2 && Q == 32 && P == 64 && N == 64) {
        static_assert(Cf::HPW == 4, "the walk kernel's block covers four heads");
        // its blocks hold four heads of one group each, and it reads dt two heads per dword
        walk = (a.H / a.G) % 4 == 0 && ((uintptr_t)a.dt & 3u) == 0 && (a.dts & 1) == 0;
    }
    if (conv && !walk) return hipErrorInvalidValue;  // the fused path needs the walk kernel
    if (k.plan) {
        e = launch_kernel(ssd_packed_plan_kernel, dim3(1), dim3(256), 0, s, k, Q, pl.pairs, pl.cps_lo, pl.cps,
                          const_cast<int*>(k.plan));
        if (e != hipSuccess) return e;
    }
    if (walk) e = launch_ssd_walk(k, conv, s);
    else e = launch_kernel(ssd_chunk_scan_kernel<T, Q, P, N>, dim3(k.nblocks), dim3(Cf::THREADS), 0, s, k);
    if (e != hipSuccess || pl.nseg == 1) return e;
    dim3 g2((unsigned)((P * N / 4 + 255) / 256), (unsigned)BH);
    e = pl.nseg <= 8 ? launch_kernel(ssd_segment_chain_kernel<8>, g2, dim3(256), 0, s, k, BH, P * N, Q)
                     : launch_kernel(ssd_segment_chain_kernel<32>, g2, dim3(256), 0, s, k, BH, P * N, Q);
    if (e != hipSuccess) return e;
    // about one chunk to fix per wave on the 32k prompt's figures; at most one round of resident
    // blocks (the candidates are counted with the upper bound on the chunks per segment); the count
    // coprime to cps (see the kernel)
    const int64_t ncand = (int64_t)(pl.nseg - 1) * BH * pl.cps;
    int64_t nfb = (ncand + 63) / 64;
    const int64_t cap = (int64_t)device_shape().cus * kFixBlocksPerCU;
    nfb = nfb < cap ? nfb : cap;
    while (nfb > 1 && std::gcd(nfb, (int64_t)pl.cps) > 1) --nfb;
    return launch_kernel(ssd_segment_fix_kernel<T, Q, P, N>, dim3((unsigned)nfb), dim3(kFixThreads), 0, s, k);
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

template <typename T, int Q>
static size_t workspace_pn(int64_t batch, int64_t L, int H, int P, int N, int G, int64_t total) {
#define M2_PN(PP, NN) if (P == PP && N == NN) return plan_of<T, Q, PP, NN>(batch, L, H, G, total).ws_bytes;
    M2_PN(16, 16) M2_PN(16, 32) M2_PN(16, 64) M2_PN(32, 16) M2_PN(32, 32) M2_PN(32, 64)
    M2_PN(64, 16) M2_PN(64, 32) M2_PN(64, 64) M2_PN(64, 128)
    if constexpr (sizeof(T) == 2) {
        M2_PN(128, 64) M2_PN(128, 128)
    }
#undef M2_PN
    return 0;
}

size_t ssd_scan_workspace_bytes(int64_t batch, int64_t L, int H, int P, int N, int G, int Q, bool bf16,
                                int64_t total) {
    if (bf16) {
        switch (Q) {
            case 16: return workspace_pn<bf16_t, 16>(batch, L, H, P, N, G, total);
            case 32: return workspace_pn<bf16_t, 32>(batch, L, H, P, N, G, total);
            default: return workspace_pn<bf16_t, 64>(batch, L, H, P, N, G, total);
        }
    }
    switch (Q) {
        case 16: return workspace_pn<float, 16>(batch, L, H, P, N, G, total);
        default: return workspace_pn<float, 32>(batch, L, H, P, N, G, total);
    }
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

// ----------------------------------------------------------------------------------------------
// the fused prompt path

bool mixer_fusable(int P, int N, int H, int G, bool bf16) {
    return bf16 && P == 64 && N == 64 && G > 0 && (H / G) % 4 == 0;
}

bool mixer_dt_fusable(const void* dt, int64_t dts) { return ((uintptr_t)dt & 3u) == 0 && (dts & 1) == 0; }

size_t mixer_act_bytes(int64_t batch, int64_t L, int G, int N) {
    return ((size_t)(batch * L * 2 * G * N) * sizeof(uint16_t) + 255) & ~(size_t)255;
}

hipError_t launch_mixer_prefill(const ConvArgs& c, const ScanArgs& a, void* act, hipStream_t s) {
    const int GN = a.G * a.N, Di = a.H * a.P;
    // 1. conv + SiLU of the B and C channels into act (the scan's main pass reads them as tiles)
    ConvArgs bc = c;
    bc.xbc = c.xbc ? reinterpret_cast<const uint16_t*>(c.xbc) + Di : nullptr;
    bc.Cd = 2 * GN;
    bc.w = c.w + (int64_t)Di * c.W;
    bc.bias = c.bias ? c.bias + Di : nullptr;
    bc.ring_in = c.ring_in ? reinterpret_cast<const uint16_t*>(c.ring_in) + Di : nullptr;
    bc.ring_out = c.ring_out ? reinterpret_cast<uint16_t*>(c.ring_out) + Di : nullptr;
    bc.rs = c.Cd;
    bc.out = c.xbc ? act : nullptr;
    bc.os = 2 * GN;
    bc.vec = c.vec && GN % 4 == 0 && Di % 8 == 0;
    hipError_t e = launch_conv1d(bc, s);
    if (e != hipSuccess) return e;
    // 2. the scan, whose main pass convolves the x channels of the raw rows itself
    ScanArgs sa = a;
    sa.x = c.xbc;
    sa.xs = c.xs;
    sa.B = act;
    sa.C = reinterpret_cast<uint16_t*>(act) + GN;
    sa.bcs = 2 * GN;
    WalkConv cv;
    cv.w = c.w; cv.bias = c.bias; cv.ring_in = c.ring_in; cv.ring_out = c.ring_out;
    cv.rs = c.Cd; cv.W = c.W; cv.phase = c.ring_phase;
    return run_scan<bf16_t, 32, 64, 64>(sa, s, &cv);
}

}  // namespace m2
