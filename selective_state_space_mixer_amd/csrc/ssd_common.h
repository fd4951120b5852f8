// ssd_common.h -- pieces shared by the chunked scan kernels (gfx950): MFMA fragments, buffer
// resources, LDS-destination loads, the kernel parameter block and the per-sequence extents.
#pragma once

#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

#define M2_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------------------------
// element types

template <typename T> struct Lds;
template <> struct Lds<bf16_t> { using E = uint16_t; };
template <> struct Lds<float> { using E = float; };

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

// ----------------------------------------------------------------------------------------------
// LDS tiles: rows of U 16-byte units followed by one unit of padding, so that the 16 rows a
// fragment read touches at one column start in different banks.

// element offset of (row, col) in a tile of E elements with U units per row
template <typename E, int U>
__device__ __forceinline__ int tidx(int r, int c) {
    constexpr int EPU = 16 / (int)sizeof(E);
    return r * ((U + 1) * EPU) + c;
}

// chunk c of a fragment from a tile whose k index runs along the row (lane: `row`, k = k0..k0+3)
template <int U>
__device__ __forceinline__ void chunk_row(Frag<bf16_t>& f, int c, const uint16_t* tile, int row, int k0) {
    const uint2 v = *reinterpret_cast<const uint2*>(tile + tidx<uint16_t, U>(row, k0));
    f.w[2 * c] = v.x;
    f.w[2 * c + 1] = v.y;
}
template <int U>
__device__ __forceinline__ void chunk_row(Frag<float>& f, int c, const float* tile, int row, int k0) {
    const float4 v = *reinterpret_cast<const float4*>(tile + tidx<float, U>(row, k0));
    f.set(c, v.x, v.y, v.z, v.w);
}

// Fragment with k along a row: the lane supplies `row`, k = kbase + 4q (+16); kext = k extent.
template <typename T, int U>
__device__ __forceinline__ Frag<T> frag_row(const typename Lds<T>::E* tile, int row, int kbase, int kext, int q) {
    Frag<T> f;
    chunk_row<U>(f, 0, tile, row, kbase + 4 * q);
    if (kbase + 16 < kext) chunk_row<U>(f, 1, tile, row, kbase + 16 + 4 * q);
    else f.set(1, 0.f, 0.f, 0.f, 0.f);
    return f;
}

// Chunk c of a fragment whose k index runs down the rows: lane (q, i) gets rows r0+4q..r0+4q+3
// of column col0+i.  bf16: one ds_read_b64_tr_b16 (lane i addresses row i/4, columns 4(i%4)..+3
// of its 16-lane group's 4x16 block and receives column i of the block).
template <int U>
__device__ __forceinline__ void chunk_col(Frag<bf16_t>& f, int c, const uint16_t* tile, int r0, int col0, int q,
                                          int i) {
    const uint16_t* p = tile + tidx<uint16_t, U>(r0 + 4 * q + (i >> 2), col0 + 4 * (i & 3));
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((M2_LDS i16x4_t*)(p));
    const uint2 u = __builtin_bit_cast(uint2, v);
    f.w[2 * c] = u.x;
    f.w[2 * c + 1] = u.y;
}
template <int U>
__device__ __forceinline__ void chunk_col(Frag<float>& f, int c, const float* tile, int r0, int col0, int q, int i) {
    const int r = r0 + 4 * q, col = col0 + i;
    f.set(c, tile[tidx<float, U>(r, col)], tile[tidx<float, U>(r + 1, col)], tile[tidx<float, U>(r + 2, col)],
          tile[tidx<float, U>(r + 3, col)]);
}

template <typename T, int U>
__device__ __forceinline__ Frag<T> frag_col(const typename Lds<T>::E* tile, int kbase, int kext, int col0, int q,
                                            int i) {
    Frag<T> f;
    chunk_col<U>(f, 0, tile, kbase, col0, q, i);
    if (kbase + 16 < kext) chunk_col<U>(f, 1, tile, kbase + 16, col0, q, i);
    else f.set(1, 0.f, 0.f, 0.f, 0.f);
    return f;
}

// ----------------------------------------------------------------------------------------------
// buffer resources: a base address and a byte range; loads outside the range return zero and
// stores outside it are dropped

constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit dword access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// The same resource as four dwords, for the LDS-destination load below.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_desc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, kRsrcWord3};
}

// 64 lanes x 16 bytes from the buffer into 1 KB of LDS at `dst` (lane l -> dst + 16 l).
// Written out (M0 = LDS address, one wait state after M0 is set) rather than through
// the builtin: the compiler cannot tell which LDS bytes the builtin's load writes, and so holds
// every later LDS read until all such loads are done, which would serialise the prefetch.  The
// caller orders these loads with s_waitcnt and barriers; the load has no register result.
__device__ __forceinline__ void load_lds16(const i32x4_t& desc, void* dst, uint32_t voff) {
    const uint32_t m = (uint32_t)(uintptr_t)(M2_LDS void*)dst;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(desc), "{m0}"(m)
                 : "memory");
}

// One dword per active lane from the buffer into LDS at `dst` + 4 (lane id); otherwise as load_lds16.
__device__ __forceinline__ void load_lds4(const i32x4_t& desc, void* dst, uint32_t voff) {
    const uint32_t m = (uint32_t)(uintptr_t)(M2_LDS void*)dst;
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(desc), "{m0}"(m)
                 : "memory");
}

__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, bf16_t*, const f32x4& a) {
    const u32x2_t v = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, 0, 0);
}
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, float*, const f32x4& a) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, a), r, (int)voff, 0, 0);
}

// one element as raw bits, converted only where it is used (so nothing waits on the load early)
__device__ __forceinline__ uint32_t load_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff, bf16_t*) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0);
}
__device__ __forceinline__ uint32_t load_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff, float*) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
}
__device__ __forceinline__ float raw_to_f32(uint32_t v, bf16_t*) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float raw_to_f32(uint32_t v, float*) { return __uint_as_float(v); }

// wait until at most N of this wave's vector memory operations are outstanding (gfx9 s_waitcnt:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).  Operations complete in
// issue order, so this waits for everything issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// ----------------------------------------------------------------------------------------------
// kernel parameters

struct ScanK {
    const void* x; const void* B; const void* C; const void* dt;
    int64_t xs, bcs, dts, ys;
    const float* dt_bias; const float* A; const float* D;
    float dt_min, dt_max;
    const float* state_in; float* state_out;
    void* y;
    float* ws_state;   // [nseg][batch*H][P*N]: segment end states (fp32 outputs: then initial states)
    float* ws_lam;     // [nseg][batch*H]: summed log-decay of each segment
    float* ws_lamc;    // [nchunks][batch*H]: summed log-decay of the chunk's segment before the chunk
    uint16_t* ws_tin;  // bf16 outputs: [nseg-1][batch*H][P*N] bf16 initial states of segments 1.. (else null)
    float* ws_emax;    // [nseg][batch*H]: max |E[seg]|, the segment's end state from its own start
    float* ws_tb;      // [nseg][batch*H]: a bound on max |T[seg]|, the true end state (chain kernel)
    const int32_t* lens;  // [batch] tokens of each right-padded sequence, or null (all L)
    const int32_t* cu;    // packed batch: [batch+1] first row of each sequence, or null
    int64_t total;        // packed batch: rows of the packed arrays
    int64_t L;
    int batch, H, G;
    int nseg, cps;     // segments per sequence, chunks per segment
    const int* plan;   // packed batch with a device plan (ssd_packed_plan_kernel), else null:
                       // [0] chunks per segment, [1] pairs with work, then those (sequence, segment)
                       // pairs as int2, sequence by sequence
    int win;           // chunks per buffer-resource window (byte offsets inside one stay below 2^31)
    int nblocks;       // blocks in this launch
    int nxcd;          // XCDs the launch's blocks are dealt over (round-robin in launch order)
};

// First row of sequence b: b*L, or cu[b] (clamped to the rows that exist) in a packed batch.
__device__ __forceinline__ int64_t seq_row0(const ScanK& k, int64_t b) {
    if (!k.cu) return b * k.L;
    const int64_t r0 = k.cu[b];
    return r0 < 0 ? 0 : (r0 > k.total ? k.total : r0);
}
// Chunks per segment: the host's figure, or for a packed batch the one its plan kernel picked.
__device__ __forceinline__ int seg_chunks(const ScanK& k) { return k.plan ? *k.plan : k.cps; }

// Tokens of sequence b: L; its length clamped to [0, L] in a right-padded batch; in a packed
// batch cu[b+1] - cu[b], clamped to the rows that exist and to L.
__device__ __forceinline__ int64_t seq_len(const ScanK& k, int64_t b) {
    if (k.cu) {
        const int64_t r0 = seq_row0(k, b), r1 = k.cu[b + 1];
        const int64_t end = r1 < r0 ? r0 : (r1 > k.total ? k.total : r1);
        return end - r0 < k.L ? end - r0 : k.L;
    }
    if (!k.lens) return k.L;
    const int64_t v = k.lens[b];
    return v < 0 ? 0 : (v > k.L ? k.L : v);
}

// A later segment starts from zero in the main pass; the part of its output that comes from its true
// initial state T decays with the segment's summed log-decay Lam and is added afterwards (the fix-up)
// to each chunk j whose starting factor still matters against the segment's own state:
//     e^Lam_before(j) * max|T|  >=  e^cut * max|E|,   E = the segment's end state from zero.
// The term left out beyond that is below e^cut of the segment's own state scale: e^-12 (6e-6, far
// under bf16's 2^-9) for bf16 outputs, e^-20.8 (1e-9) for fp32 outputs.  The main pass records
// Lam_before of every chunk and max|E| of every segment; the chain kernel bounds max|T| by the chain
// of maxima Tb[seg] = e^lam[seg] Tb[seg-1] + max|E[seg]|, and the fix-up applies the test with Tb,
// which keeps every chunk the rule asks for (adding the exact term to a chunk is never wrong).
template <typename T> constexpr float fix_cut() { return sizeof(T) == 2 ? -12.0f : -20.8f; }

// max over the 64 lanes of a wave
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Block -> logical unit.  Consecutive blocks are dealt round-robin to the device's nx XCDs; the
// remap gives each XCD a contiguous run of logical units (the head groups of one sequence and
// segment), so the B/C rows those heads share are fetched into one L2.  XCD x receives
// n/nx blocks, plus one if x < n%nx; its run starts after those of XCDs 0..x-1.
__device__ __forceinline__ int logical_block(int nblocks, int nx) {
    const int i = blockIdx.x;
    if (nx <= 1) return i;
    const int x = i % nx, per = nblocks / nx, extra = nblocks % nx;
    return x * per + (x < extra ? x : extra) + i / nx;
}

// Block -> (head unit, sequence, segment); false for a block with nothing to do.  With a packed plan
// the first plan[1] * nhu blocks hold the (sequence, segment) pairs with work: one round of resident
// blocks spread evenly over the XCDs, each XCD a contiguous run of them (the head units of a pair
// share its B/C rows in one L2).  Otherwise: uniform sequences as logical_block deals them, variable
// lengths round-robin in launch order (the busy first segments come first).
__device__ __forceinline__ bool block_unit(const ScanK& k, int nhu, int& hu, int64_t& b, int& seg) {
    if (k.plan) {
        const int nbusy = k.plan[1] * nhu;
        if ((int)blockIdx.x >= nbusy) return false;
        const int u = logical_block(nbusy, k.nxcd);
        hu = u % nhu;
        const int2 e = reinterpret_cast<const int2*>(k.plan + 2)[u / nhu];
        b = e.x;
        seg = e.y;
        return true;
    }
    const int unit = (k.lens || k.cu) ? (int)blockIdx.x : logical_block(k.nblocks, k.nxcd);
    hu = unit % nhu;
    const int sb = unit / nhu;
    b = sb % k.batch;
    seg = sb / k.batch;
    return true;
}

// The conv of the x channels when the main pass takes the raw conv input (the fused prompt path):
// k.x then points at the raw xBC rows (x channels first), and k.B / k.C at the already convolved
// B and C channels.
struct WalkConv {
    const float* w;       // [conv_dim, W] conv weights
    const float* bias;    // [conv_dim], or null
    const void* ring_in;  // [batch, W, rs] history (bf16) before each sequence's first token, or null
    void* ring_out;       // [batch, W, rs]: receives the last W raw tokens of the x channels, or null
    int64_t rs;           // elements between ring slots (conv_dim)
    int W;                // conv width, 2..4
    int phase;            // ring_in's phase: token -j sits in slot (phase - j) mod W
};

// The main pass at headdim 64, d_state 64, bf16, 32-token chunks (ssd_walk.hip): one wave per
// head, four heads per block, the same workspace contract as the general main pass.  With a
// WalkConv it convolves the raw x channels itself.
hipError_t launch_ssd_walk(const ScanK& k, const WalkConv* conv, hipStream_t s);

}  // namespace m2
