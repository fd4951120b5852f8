// m2_launch.h -- host-side launch descriptors passed from the C ABI layer to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m2 {

struct ConvArgs {
    const void* xbc; int64_t xs;      // [batch, L, Cd], token stride xs
    int64_t L; int Cd; int W; int64_t batch;
    const float* w; const float* bias;
    const void* ring_in; int ring_phase;
    void* ring_out;
    int64_t rs;                       // elements between ring slots (conv_dim of the full ring)
    void* out; int64_t os;
    const int32_t* lens;  // [batch] valid tokens per sequence (device), or null
    const int32_t* cu;    // packed batch: [batch+1] first row of each sequence (device), or null
    int64_t total;        // packed batch: rows of the packed arrays
    bool bf16;  // storage type of activations
    bool vec;   // 16-byte vector path (alignment checked by the caller)
};

struct ScanArgs {
    int64_t batch, L;
    int H, P, N, G, Q;
    const void* x; int64_t xs;
    const void* B; const void* C; int64_t bcs;
    const void* dt; int64_t dts;
    const float* dt_bias; const float* A; const float* D;
    float dt_min, dt_max;
    const float* state_in; float* state_out;
    void* y; int64_t ys;
    void* ws; size_t ws_bytes;
    const int32_t* lens;  // [batch] valid tokens per sequence (device), or null
    const int32_t* cu;    // packed batch: [batch+1] first row of each sequence (device), or null
    int64_t total;        // packed batch: rows of the packed arrays
    bool bf16;
};

struct StepArgs {
    int64_t batch;
    int H, P, N, G, W, Cd;
    const void* xbc; int64_t xbs;
    const void* dt; int64_t dts;
    const float* w; const float* bias;
    const float* dt_bias; const float* A; const float* D;
    float dt_min, dt_max;
    void* ring; int64_t step;
    float* state; void* y;
    bool bf16;
};

struct NormArgs {
    int64_t ntok;
    int d_inner, gs;
    const void* y; int64_t ys;
    const void* z; int64_t zs;
    const float* w;
    float eps;
    bool norm_before_gate;
    void* out; int64_t os;
    bool bf16;
};

// Compute units and XCDs of the calling thread's current device, read once per device with
// hipDeviceGetAttribute and cached (thread-safe).  Plans that spread work over the chip size
// themselves from it; if the query fails, 256 compute units in 8 XCDs are assumed.
struct DeviceShape { int cus; int xcds; };
DeviceShape device_shape();

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s);
hipError_t launch_ssd_scan(const ScanArgs& a, hipStream_t s);

// Backward of the scan (bf16 activations, headdim 64, d_state 64).  Arrays are bf16 bit patterns
// with token strides in elements; ddt_bias, dA and dD are [H] fp32 and overwritten.
struct BwdArgs {
    const uint16_t* x; int64_t xs;
    const uint16_t* B; const uint16_t* C; int64_t bcs;
    const uint16_t* dt; int64_t dts;
    const uint16_t* dy; int64_t dys;
    const float* dt_bias; const float* A; const float* D;
    float dt_min, dt_max;
    const float* state_in; const float* dstate_out;
    uint16_t* dx; int64_t dxs;
    uint16_t* dB; uint16_t* dC; int64_t dbcs;
    uint16_t* ddt; int64_t ddts;
    float* ddt_bias; float* dA; float* dD; float* dstate_in;
    int64_t batch, L;
    int H, G;
    const int32_t* lens;  // [batch] valid tokens per sequence (device), or null
    const int32_t* cu;    // packed batch: [batch+1] first row of each sequence (device), or null
    int64_t total;        // packed batch: rows of the packed arrays
    void* ws;
    // set by the launcher
    int nch, nseg, cps;  // 64-token chunks, segments of the walks, chunks per segment
    float* ws_es;      // [nch][batch*H][N][P] fp32: each chunk's initial state from its segment's start
    float* ws_fg;      // [nch][batch*H][N][P] fp32: the adjoint of each chunk's end state from its segment's end
    float* ws_lamb;    // [nch][batch*H] summed log-decay of the segment before the chunk
    float* ws_lame;    // [nch][batch*H] summed log-decay of the segment after the chunk
    float* ws_sege;    // [nseg][batch*H][N][P]: segment end states, then the true segment initial states
    float* ws_segf;    // [nseg][batch*H][N][P]: segment start adjoints, then the true segment end adjoints
    float* ws_seglam;  // [nseg][batch*H] summed log-decay of each segment
    float* ws_part;    // [3][batch*nch][H] per-chunk sums of dA, dD and dt_bias
};
bool ssd_bwd_supported(int P, int N, bool bf16);
size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t L, int H, int G);
hipError_t launch_ssd_scan_bwd(const BwdArgs& a, hipStream_t s);
// total: tokens of a packed batch (L its longest sequence), or -1 for a padded one
size_t ssd_scan_workspace_bytes(int64_t batch, int64_t L, int H, int P, int N, int G, int Q, bool bf16,
                                int64_t total);
bool ssd_scan_supported(int P, int N, int Q, bool bf16);
// The fused prompt path (conv1d + SiLU and the scan in one pass over the raw conv input): built for
// bf16, headdim 64, d_state 64, head groups of a multiple of four heads, a dword-aligned dt view and
// padded (not packed) batches.  The conv of the B and C channels runs first, into `act`
// ([batch*seqlen, 2*G*N] bf16); the x channels are convolved inside the scan's main pass.  `c` holds
// the conv of all channels (out unused), `a` the scan (x/B/C unused: the launcher points them).
bool mixer_fusable(int P, int N, int H, int G, bool bf16);
bool mixer_dt_fusable(const void* dt, int64_t dts);
size_t mixer_act_bytes(int64_t batch, int64_t L, int G, int N);
hipError_t launch_mixer_prefill(const ConvArgs& c, const ScanArgs& a, void* act, hipStream_t s);

// A plain copy of `bytes` (a multiple of 16, both pointers 16-byte aligned): the bandwidth reference.
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

// The library's static scratch buffer on the current device (address looked up once per device)
// and its size in bytes; for the entry point that must not allocate.
hipError_t static_scratch(void** ptr, size_t* bytes);
int ssd_scan_default_chunk(int P, int N, bool bf16);
hipError_t launch_ssd_step(const StepArgs& a, hipStream_t s);
bool ssd_step_supported(int P, int N);
hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t s);
int gated_rmsnorm_max_group(bool bf16);

}  // namespace m2

namespace m2 {

template <class T> struct ident { using type = T; };

// Launch through hipLaunchKernel so the returned status is this launch's own
// (hipGetLastError would also report an earlier, unrelated failure of the thread).
template <typename... Args>
inline hipError_t launch_kernel(void (*kernel)(Args...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                                typename ident<Args>::type... args) {
    void* argv[] = {(void*)&args...};
    return hipLaunchKernel((const void*)kernel, grid, block, argv, shmem, s);
}

// Name of the last HIP error a call of this thread saw ("hipSuccess" if none).
void note_hip_error(hipError_t e);

}  // namespace m2
