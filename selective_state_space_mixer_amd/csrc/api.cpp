// api.cpp -- the C ABI of include/m2ssd.h: argument validation and dispatch.
//
// Everything here runs on the host before any launch.  A call that fails
// validation enqueues nothing.  No allocation, no synchronisation, no state.
#include "m2ssd.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "m2_launch.h"

namespace {

struct Derived {
    int64_t batch, L;
    int d_inner, H, P, N, G, W, Cd, Q;
    bool bf16;
    int esize;
};

m2_status derive(const m2_dims* d, Derived& o) {
    if (!d) return M2_ERR_NULL;
    if (d->io != M2_F32 && d->io != M2_BF16) return M2_ERR_DTYPE;
    if (d->batch < 0 || d->seqlen < 0 || d->d_model < 1 || d->expand < 1 || d->headdim < 1 ||
        d->d_state < 1 || d->n_groups < 1 || d->chunk_size < 0)
        return M2_ERR_SHAPE;
    if (d->d_conv < 2 || d->d_conv > 4) return M2_ERR_UNSUPPORTED;
    const int64_t d_inner = (int64_t)d->expand * d->d_model;
    if (d_inner % d->headdim) return M2_ERR_SHAPE;
    const int64_t H = d_inner / d->headdim;
    if (H % d->n_groups) return M2_ERR_SHAPE;
    const int64_t Cd = d_inner + 2 * (int64_t)d->n_groups * d->d_state;
    if (Cd > (int64_t)1 << 30) return M2_ERR_SHAPE;
    o.batch = d->batch;
    o.L = d->seqlen;
    o.d_inner = (int)d_inner;
    o.H = (int)H;
    o.P = d->headdim;
    o.N = d->d_state;
    o.G = d->n_groups;
    o.W = d->d_conv;
    o.Cd = (int)Cd;
    o.Q = d->chunk_size;
    o.bf16 = d->io == M2_BF16;
    o.esize = o.bf16 ? 2 : 4;
    return M2_OK;
}

// The chunk length the scan runs with: dims.chunk_size when the kernels are built for it at this
// (headdim, d_state, dtype), else the library's choice.  Results do not depend on it beyond rounding,
// so a model configuration's own value (Zamba2 uses 256) is taken as a hint.
int scan_chunk(const Derived& d) {
    if (d.Q > 0 && m2::ssd_scan_supported(d.P, d.N, d.Q, d.bf16)) return d.Q;
    return m2::ssd_scan_default_chunk(d.P, d.N, d.bf16);
}

// Byte range of a [rows, row_elems] view with `stride` elements between rows.
struct Range { uintptr_t lo, hi; };
Range span(const void* p, int64_t rows, int64_t stride, int64_t row_elems, int esize) {
    if (!p || rows <= 0 || row_elems <= 0) return {0, 0};
    const uintptr_t lo = (uintptr_t)p;
    return {lo, lo + (uintptr_t)(((rows - 1) * stride + row_elems) * esize)};
}
bool overlap(Range a, Range b) { return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

thread_local hipError_t g_last_hip_error = hipSuccess;

m2_status launched(hipError_t e) {
    if (e == hipSuccess) return M2_OK;
    g_last_hip_error = e;
    return M2_ERR_LAUNCH;
}

}  // namespace

namespace m2 {
void note_hip_error(hipError_t e) { g_last_hip_error = e; }

DeviceShape device_shape() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static DeviceShape cache[kMaxDevices];
    static bool known[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DeviceShape{256, 8};
    std::lock_guard<std::mutex> lock(mu);
    if (!known[dev]) {
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1) xcds = 8;
        cache[dev] = DeviceShape{cus, xcds};
        known[dev] = true;
    }
    return cache[dev];
}
}  // namespace m2

extern "C" {

const char* m2_status_str(m2_status s) {
    switch (s) {
        case M2_OK: return "ok";
        case M2_ERR_NULL: return "a required pointer is NULL";
        case M2_ERR_SHAPE: return "invalid or inconsistent sizes or strides";
        case M2_ERR_DTYPE: return "unsupported activation storage type";
        case M2_ERR_ALIAS: return "an output overlaps an input";
        case M2_ERR_WORKSPACE: return "workspace missing or too small";
        case M2_ERR_UNSUPPORTED: return "shape, width or alignment not supported by the built kernels";
        case M2_ERR_LAUNCH: return "kernel launch failed";
        case M2_ERR_TOO_LARGE: return "the call needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}

int m2_abi_version(void) { return M2SSD_ABI_VERSION; }

const char* m2_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

}  // extern "C"

namespace {

// Shared by the padded and the packed conv entry points: rows = rows of xbc/out; a packed batch
// passes its row offsets cu (batch+1 entries) and rows = total tokens.
m2_status conv_run(const Derived& d, int64_t rows, const int32_t* cu, const void* xbc, int64_t xbc_tok_stride,
                   const float* w, const float* bias, const void* ring_in, int64_t ring_in_step, void* ring_out,
                   void* out, int64_t out_tok_stride, const int32_t* seq_lens, void* stream) {
    if (!w) return M2_ERR_NULL;
    if (rows > 0 && (!xbc || !out)) return M2_ERR_NULL;
    if (rows > 0 && (xbc_tok_stride < d.Cd || out_tok_stride < d.Cd)) return M2_ERR_SHAPE;
    if (d.batch == 0 || (d.L == 0 && !ring_out)) return M2_OK;
    const Range rx = span(xbc, rows, xbc_tok_stride, d.Cd, d.esize);
    const Range ro = span(out, rows, out_tok_stride, d.Cd, d.esize);
    const Range rri = span(ring_in, d.batch * d.W, d.Cd, d.Cd, d.esize);
    const Range rro = span(ring_out, d.batch * d.W, d.Cd, d.Cd, d.esize);
    const Range rl = cu ? span(cu, d.batch + 1, 1, 1, 4) : span(seq_lens, d.batch, 1, 1, 4);
    if (overlap(rx, ro) || overlap(rri, rro) || overlap(rro, rx) || overlap(rro, ro) || overlap(ro, rri) ||
        overlap(rl, ro) || overlap(rl, rro))
        return M2_ERR_ALIAS;
    if (((uintptr_t)seq_lens & 3u) || ((uintptr_t)cu & 3u)) return M2_ERR_UNSUPPORTED;
    m2::ConvArgs a;
    a.xbc = xbc; a.xs = xbc_tok_stride; a.L = d.L; a.Cd = d.Cd; a.W = d.W; a.batch = d.batch;
    a.w = w; a.bias = bias; a.ring_in = ring_in;
    a.ring_phase = (int)(((ring_in_step % d.W) + d.W) % d.W);
    a.ring_out = ring_out; a.rs = d.Cd; a.out = out; a.os = out_tok_stride; a.lens = seq_lens; a.bf16 = d.bf16;
    a.cu = cu; a.total = cu ? rows : 0;
    const int vec = d.bf16 ? 8 : 4;
    a.vec = (d.Cd % vec == 0) && (rows == 0 || (xbc_tok_stride % vec == 0 && out_tok_stride % vec == 0 &&
                                                 aligned16(xbc) && aligned16(out))) &&
            aligned16(ring_in) && aligned16(ring_out);
    if (d.L == 0 || rows == 0) { a.xbc = nullptr; a.out = nullptr; }
    return launched(m2::launch_conv1d(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

m2_status m2_conv1d_fwd(const m2_dims* dims, const void* xbc, int64_t xbc_tok_stride, const float* w,
                        const float* bias, const void* ring_in, int64_t ring_in_step, void* ring_out, void* out,
                        int64_t out_tok_stride, const int32_t* seq_lens, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    return conv_run(d, d.batch * d.L, nullptr, xbc, xbc_tok_stride, w, bias, ring_in, ring_in_step, ring_out, out,
                    out_tok_stride, seq_lens, stream);
}

m2_status m2_conv1d_fwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                               const void* xbc, int64_t xbc_tok_stride, const float* w, const float* bias,
                               const void* ring_in, int64_t ring_in_step, void* ring_out, void* out,
                               int64_t out_tok_stride, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    if (total_tokens < 0) return M2_ERR_SHAPE;
    if (d.batch > 0 && !cu_seqlens) return M2_ERR_NULL;
    return conv_run(d, total_tokens, cu_seqlens, xbc, xbc_tok_stride, w, bias, ring_in, ring_in_step, ring_out, out,
                    out_tok_stride, nullptr, stream);
}

size_t m2_ssd_scan_workspace(const m2_dims* dims) {
    Derived d;
    if (derive(dims, d) != M2_OK) return 0;
    return m2::ssd_scan_workspace_bytes(d.batch, d.L, d.H, d.P, d.N, d.G, scan_chunk(d), d.bf16, -1);
}

size_t m2_ssd_scan_workspace_packed(const m2_dims* dims, int64_t total_tokens) {
    Derived d;
    if (derive(dims, d) != M2_OK || total_tokens < 0) return 0;
    return m2::ssd_scan_workspace_bytes(d.batch, d.L, d.H, d.P, d.N, d.G, scan_chunk(d), d.bf16, total_tokens);
}

}  // extern "C"

namespace {

// Shared by the padded and the packed scan entry points (rows and cu as for conv_run).
m2_status scan_run(const Derived& d, int64_t rows, const int32_t* cu, const void* x, int64_t x_tok_stride,
                   const void* B, const void* C, int64_t bc_tok_stride, const void* dt, int64_t dt_tok_stride,
                   const float* dt_bias, const float* A, const float* D, float dt_min, float dt_max,
                   const float* state_in, float* state_out, void* y, int64_t y_tok_stride, void* workspace,
                   size_t workspace_bytes, const int32_t* seq_lens, void* stream) {
    if (!dt_bias || !A) return M2_ERR_NULL;
    if (rows > 0 && (!x || !B || !C || !dt || !y)) return M2_ERR_NULL;
    const int GN = d.G * d.N;
    if (rows > 0 && (x_tok_stride < d.d_inner || bc_tok_stride < GN || dt_tok_stride < d.H ||
                     y_tok_stride < d.d_inner))
        return M2_ERR_SHAPE;
    if (std::isnan(dt_min) || std::isnan(dt_max) || dt_min > dt_max) return M2_ERR_SHAPE;
    const int Q = scan_chunk(d);
    if (!m2::ssd_scan_supported(d.P, d.N, Q, d.bf16)) return M2_ERR_UNSUPPORTED;
    if (d.batch == 0) return M2_OK;
    const Range ry = span(y, rows, y_tok_stride, d.d_inner, d.esize);
    const Range rs_in = span(state_in, d.batch * d.H, (int64_t)d.P * d.N, (int64_t)d.P * d.N, 4);
    const Range rs_out = span(state_out, d.batch * d.H, (int64_t)d.P * d.N, (int64_t)d.P * d.N, 4);
    if (overlap(ry, span(x, rows, x_tok_stride, d.d_inner, d.esize)) ||
        overlap(ry, span(B, rows, bc_tok_stride, GN, d.esize)) ||
        overlap(ry, span(C, rows, bc_tok_stride, GN, d.esize)) ||
        overlap(ry, span(dt, rows, dt_tok_stride, d.H, d.esize)) || overlap(rs_in, rs_out) ||
        overlap(rs_out, ry))
        return M2_ERR_ALIAS;
    if (!aligned16(state_in) || !aligned16(state_out) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)cu & 3u))
        return M2_ERR_UNSUPPORTED;
    // x, B, C and y move in 16-byte pieces of rows
    if (rows > 0 && (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
                     (x_tok_stride * d.esize) % 16 || (bc_tok_stride * d.esize) % 16 || (y_tok_stride * d.esize) % 16))
        return M2_ERR_UNSUPPORTED;
    const size_t need = m2::ssd_scan_workspace_bytes(d.batch, d.L, d.H, d.P, d.N, d.G, Q, d.bf16, cu ? rows : -1);
    if (need > 0 && (!workspace || workspace_bytes < need)) return M2_ERR_WORKSPACE;
    const Range rl = cu ? span(cu, d.batch + 1, 1, 1, 4) : span(seq_lens, d.batch, 1, 1, 4);
    if (overlap(rl, ry) || overlap(rl, rs_out) || overlap(rl, span(workspace, 1, 0, (int64_t)need, 1)))
        return M2_ERR_ALIAS;
    m2::ScanArgs a;
    a.batch = d.batch; a.L = d.L; a.H = d.H; a.P = d.P; a.N = d.N; a.G = d.G; a.Q = Q;
    a.x = x; a.xs = x_tok_stride; a.B = B; a.C = C; a.bcs = bc_tok_stride; a.dt = dt; a.dts = dt_tok_stride;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.dt_min = dt_min; a.dt_max = dt_max;
    a.state_in = state_in; a.state_out = state_out; a.y = y; a.ys = y_tok_stride;
    a.ws = workspace; a.ws_bytes = workspace_bytes; a.lens = seq_lens; a.bf16 = d.bf16;
    a.cu = cu; a.total = cu ? rows : 0;
    return launched(m2::launch_ssd_scan(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

m2_status m2_ssd_scan_fwd(const m2_dims* dims, const void* x, int64_t x_tok_stride, const void* B, const void* C,
                          int64_t bc_tok_stride, const void* dt, int64_t dt_tok_stride, const float* dt_bias,
                          const float* A, const float* D, float dt_min, float dt_max, const float* state_in,
                          float* state_out, void* y, int64_t y_tok_stride, void* workspace,
                          size_t workspace_bytes, const int32_t* seq_lens, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    return scan_run(d, d.batch * d.L, nullptr, x, x_tok_stride, B, C, bc_tok_stride, dt, dt_tok_stride, dt_bias, A,
                    D, dt_min, dt_max, state_in, state_out, y, y_tok_stride, workspace, workspace_bytes, seq_lens,
                    stream);
}

m2_status m2_ssd_scan_fwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                                 const void* x, int64_t x_tok_stride, const void* B, const void* C,
                                 int64_t bc_tok_stride, const void* dt, int64_t dt_tok_stride, const float* dt_bias,
                                 const float* A, const float* D, float dt_min, float dt_max, const float* state_in,
                                 float* state_out, void* y, int64_t y_tok_stride, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    if (total_tokens < 0) return M2_ERR_SHAPE;
    if (d.batch > 0 && !cu_seqlens) return M2_ERR_NULL;
    return scan_run(d, total_tokens, cu_seqlens, x, x_tok_stride, B, C, bc_tok_stride, dt, dt_tok_stride, dt_bias,
                    A, D, dt_min, dt_max, state_in, state_out, y, y_tok_stride, workspace, workspace_bytes, nullptr,
                    stream);
}

m2_status m2_ssd_scan_fwd_noalloc(const m2_dims* dims, const void* x, int64_t x_tok_stride, const void* B,
                                  const void* C, int64_t bc_tok_stride, const void* dt, int64_t dt_tok_stride,
                                  const float* dt_bias, const float* A, const float* D, float dt_min, float dt_max,
                                  const float* state_in, float* state_out, void* y, int64_t y_tok_stride,
                                  const int32_t* seq_lens, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    // the workspace this call needs (0 if its plan has one segment); compared with the static size
    // before the buffer's address is looked up, so an oversize call touches nothing
    const size_t need = m2_ssd_scan_workspace(dims);
    if (need > M2_STATIC_SCRATCH_BYTES) return M2_ERR_TOO_LARGE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        const hipError_t e = m2::static_scratch(&ws, &ws_bytes);
        if (e != hipSuccess) return launched(e);
        if (ws_bytes < need) return M2_ERR_TOO_LARGE;
    }
    return scan_run(d, d.batch * d.L, nullptr, x, x_tok_stride, B, C, bc_tok_stride, dt, dt_tok_stride, dt_bias, A,
                    D, dt_min, dt_max, state_in, state_out, y, y_tok_stride, ws, ws_bytes, seq_lens, stream);
}

size_t m2_mixer_prefill_workspace(const m2_dims* dims) {
    Derived d;
    if (derive(dims, d) != M2_OK || !m2::mixer_fusable(d.P, d.N, d.H, d.G, d.bf16)) return 0;
    return m2::mixer_act_bytes(d.batch, d.L, d.G, d.N) +
           m2::ssd_scan_workspace_bytes(d.batch, d.L, d.H, d.P, d.N, d.G, 32, d.bf16, -1);
}

size_t m2_mixer_prefill_workspace_packed(const m2_dims* dims, int64_t total_tokens) {
    Derived d;
    if (derive(dims, d) != M2_OK || total_tokens < 0 || !m2::mixer_fusable(d.P, d.N, d.H, d.G, d.bf16)) return 0;
    return m2::mixer_act_bytes(1, total_tokens, d.G, d.N) +
           m2::ssd_scan_workspace_bytes(d.batch, d.L, d.H, d.P, d.N, d.G, 32, d.bf16, total_tokens);
}

}  // extern "C"

namespace {

// Shared by the padded and the packed one-pass entry points (rows and cu as for conv_run; need is the
// workspace the entry point reports for these dims).
m2_status mixer_run(const Derived& d, int64_t rows, const int32_t* cu, size_t need, const void* xbc,
                    int64_t xbc_tok_stride, const float* conv_w, const float* conv_b, const void* ring_in,
                    int64_t ring_in_step, void* ring_out, const void* dt, int64_t dt_tok_stride,
                    const float* dt_bias, const float* A, const float* D, float dt_min, float dt_max,
                    const float* state_in, float* state_out, void* y, int64_t y_tok_stride, void* workspace,
                    size_t workspace_bytes, const int32_t* seq_lens, void* stream) {
    if (!conv_w || !dt_bias || !A) return M2_ERR_NULL;
    if (rows > 0 && (!xbc || !dt || !y)) return M2_ERR_NULL;
    if (rows > 0 && (xbc_tok_stride < d.Cd || dt_tok_stride < d.H || y_tok_stride < d.d_inner)) return M2_ERR_SHAPE;
    if (std::isnan(dt_min) || std::isnan(dt_max) || dt_min > dt_max) return M2_ERR_SHAPE;
    if (!m2::mixer_fusable(d.P, d.N, d.H, d.G, d.bf16)) return M2_ERR_UNSUPPORTED;
    if (d.batch == 0) return M2_OK;
    const int GN = d.G * d.N;
    const Range rx = span(xbc, rows, xbc_tok_stride, d.Cd, d.esize);
    const Range ry = span(y, rows, y_tok_stride, d.d_inner, d.esize);
    const Range rdt = span(dt, rows, dt_tok_stride, d.H, d.esize);
    const Range rri = span(ring_in, d.batch * d.W, d.Cd, d.Cd, d.esize);
    const Range rro = span(ring_out, d.batch * d.W, d.Cd, d.Cd, d.esize);
    const Range rs_in = span(state_in, d.batch * d.H, (int64_t)d.P * d.N, (int64_t)d.P * d.N, 4);
    const Range rs_out = span(state_out, d.batch * d.H, (int64_t)d.P * d.N, (int64_t)d.P * d.N, 4);
    const Range rl = cu ? span(cu, d.batch + 1, 1, 1, 4) : span(seq_lens, d.batch, 1, 1, 4);
    const Range rws = span(workspace, 1, 0, (int64_t)need, 1);
    const Range outs[] = {ry, rro, rs_out, rws};
    const Range ins[] = {rx, rdt, rri, rs_in, rl};
    for (const Range& o : outs)
        for (const Range& i : ins)
            if (overlap(o, i)) return M2_ERR_ALIAS;
    if (overlap(ry, rro) || overlap(ry, rs_out) || overlap(ry, rws) || overlap(rro, rs_out) || overlap(rro, rws) ||
        overlap(rs_out, rws))
        return M2_ERR_ALIAS;
    if (!aligned16(state_in) || !aligned16(state_out) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)cu & 3u))
        return M2_ERR_UNSUPPORTED;
    // raw x rows and y move in 16-byte pieces; dt is read two heads per dword; rings in 16-byte pieces
    if (rows > 0 && (!aligned16(xbc) || !aligned16(y) || (xbc_tok_stride * d.esize) % 16 ||
                     (y_tok_stride * d.esize) % 16 || !m2::mixer_dt_fusable(dt, dt_tok_stride)))
        return M2_ERR_UNSUPPORTED;
    if (!aligned16(ring_in) || !aligned16(ring_out)) return M2_ERR_UNSUPPORTED;
    if (need > 0 && (!workspace || workspace_bytes < need)) return M2_ERR_WORKSPACE;
    // the workspace, from a 256-byte boundary: the B/C activation (one row per token), then the scan's
    // own part
    uint8_t* base = reinterpret_cast<uint8_t*>(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
    const size_t act_bytes = cu ? m2::mixer_act_bytes(1, rows, d.G, d.N) : m2::mixer_act_bytes(d.batch, d.L, d.G, d.N);
    m2::ConvArgs c;
    c.xbc = rows > 0 ? xbc : nullptr; c.xs = xbc_tok_stride; c.L = d.L; c.Cd = d.Cd; c.W = d.W; c.batch = d.batch;
    c.w = conv_w; c.bias = conv_b; c.ring_in = ring_in;
    c.ring_phase = (int)(((ring_in_step % d.W) + d.W) % d.W);
    c.ring_out = ring_out; c.rs = d.Cd; c.out = nullptr; c.os = 2 * GN; c.lens = seq_lens; c.bf16 = true;
    c.cu = cu; c.total = cu ? rows : 0;
    c.vec = (d.Cd % 8 == 0) && (rows == 0 || (xbc_tok_stride % 8 == 0 && aligned16(xbc)));
    m2::ScanArgs a;
    a.batch = d.batch; a.L = d.L; a.H = d.H; a.P = d.P; a.N = d.N; a.G = d.G; a.Q = 32;
    a.x = nullptr; a.xs = 0; a.B = nullptr; a.C = nullptr; a.bcs = 0;
    a.dt = dt; a.dts = dt_tok_stride;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.dt_min = dt_min; a.dt_max = dt_max;
    a.state_in = state_in; a.state_out = state_out; a.y = y; a.ys = y_tok_stride;
    a.ws = base + act_bytes; a.ws_bytes = workspace_bytes > act_bytes + 255 ? workspace_bytes - act_bytes - 255 : 0;
    a.lens = seq_lens; a.bf16 = true; a.cu = cu; a.total = cu ? rows : 0;
    return launched(m2::launch_mixer_prefill(c, a, base, (hipStream_t)stream));
}

}  // namespace

extern "C" {

m2_status m2_mixer_prefill_fwd(const m2_dims* dims, const void* xbc, int64_t xbc_tok_stride, const float* conv_w,
                               const float* conv_b, const void* ring_in, int64_t ring_in_step, void* ring_out,
                               const void* dt, int64_t dt_tok_stride, const float* dt_bias, const float* A,
                               const float* D, float dt_min, float dt_max, const float* state_in, float* state_out,
                               void* y, int64_t y_tok_stride, void* workspace, size_t workspace_bytes,
                               const int32_t* seq_lens, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    return mixer_run(d, d.batch * d.L, nullptr, m2_mixer_prefill_workspace(dims), xbc, xbc_tok_stride, conv_w, conv_b,
                     ring_in, ring_in_step, ring_out, dt, dt_tok_stride, dt_bias, A, D, dt_min, dt_max, state_in,
                     state_out, y, y_tok_stride, workspace, workspace_bytes, seq_lens, stream);
}

m2_status m2_mixer_prefill_fwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                                      const void* xbc, int64_t xbc_tok_stride, const float* conv_w,
                                      const float* conv_b, const void* ring_in, int64_t ring_in_step, void* ring_out,
                                      const void* dt, int64_t dt_tok_stride, const float* dt_bias, const float* A,
                                      const float* D, float dt_min, float dt_max, const float* state_in,
                                      float* state_out, void* y, int64_t y_tok_stride, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    if (total_tokens < 0) return M2_ERR_SHAPE;
    if (d.batch > 0 && !cu_seqlens) return M2_ERR_NULL;
    return mixer_run(d, total_tokens, cu_seqlens, m2_mixer_prefill_workspace_packed(dims, total_tokens), xbc,
                     xbc_tok_stride, conv_w, conv_b, ring_in, ring_in_step, ring_out, dt, dt_tok_stride, dt_bias, A, D,
                     dt_min, dt_max, state_in, state_out, y, y_tok_stride, workspace, workspace_bytes, nullptr, stream);
}

m2_status m2_ssd_step(const m2_dims* dims, const void* xbc_tok, int64_t xbc_stride, const void* dt_tok,
                      int64_t dt_stride, const float* w, const float* bias, const float* dt_bias, const float* A,
                      const float* D, float dt_min, float dt_max, void* ring, int64_t step, float* state, void* y,
                      void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    if (!w || !dt_bias || !A) return M2_ERR_NULL;
    if (d.batch > 0 && (!xbc_tok || !dt_tok || !ring || !state || !y)) return M2_ERR_NULL;
    if (step < 0) return M2_ERR_SHAPE;
    if (d.batch > 0 && (xbc_stride < d.Cd || dt_stride < d.H)) return M2_ERR_SHAPE;
    if (std::isnan(dt_min) || std::isnan(dt_max) || dt_min > dt_max) return M2_ERR_SHAPE;
    if (!m2::ssd_step_supported(d.P, d.N)) return M2_ERR_UNSUPPORTED;
    if (d.batch == 0) return M2_OK;
    const Range ry = span(y, d.batch, d.d_inner, d.d_inner, d.esize);
    const Range rr = span(ring, d.batch * d.W, d.Cd, d.Cd, d.esize);
    const Range rs = span(state, d.batch * d.H, (int64_t)d.P * d.N, (int64_t)d.P * d.N, 4);
    const Range rx = span(xbc_tok, d.batch, xbc_stride, d.Cd, d.esize);
    const Range rd = span(dt_tok, d.batch, dt_stride, d.H, d.esize);
    if (overlap(ry, rr) || overlap(ry, rs) || overlap(ry, rx) || overlap(ry, rd) || overlap(rr, rs) ||
        overlap(rr, rx) || overlap(rr, rd) || overlap(rs, rx) || overlap(rs, rd))
        return M2_ERR_ALIAS;
    if (!aligned16(state)) return M2_ERR_UNSUPPORTED;
    m2::StepArgs a;
    a.batch = d.batch; a.H = d.H; a.P = d.P; a.N = d.N; a.G = d.G; a.W = d.W; a.Cd = d.Cd;
    a.xbc = xbc_tok; a.xbs = xbc_stride; a.dt = dt_tok; a.dts = dt_stride;
    a.w = w; a.bias = bias; a.dt_bias = dt_bias; a.A = A; a.D = D; a.dt_min = dt_min; a.dt_max = dt_max;
    a.ring = ring; a.step = step; a.state = state; a.y = y; a.bf16 = d.bf16;
    return launched(m2::launch_ssd_step(a, (hipStream_t)stream));
}

size_t m2_ssd_scan_bwd_workspace(const m2_dims* dims) {
    Derived d;
    if (derive(dims, d) != M2_OK || !m2::ssd_bwd_supported(d.P, d.N, d.bf16)) return 0;
    return m2::ssd_bwd_workspace_bytes(d.batch, d.L, d.H, d.G);
}

}  // extern "C"

namespace {

// The backward for a right-padded batch (cu null, rows = batch * seqlen) or a packed one (rows = its
// token count): argument checks over `rows` rows, then the launches.
m2_status bwd_run(const Derived& d, int64_t rows, const int32_t* cu, const void* x, int64_t x_tok_stride,
                  const void* B, const void* C, int64_t bc_tok_stride, const void* dt, int64_t dt_tok_stride,
                  const float* dt_bias, const float* A, const float* D, float dt_min, float dt_max,
                  const float* state_in, const void* dy, int64_t dy_tok_stride, const float* dstate_out, void* dx,
                  int64_t dx_tok_stride, void* dB, void* dC, int64_t dbc_tok_stride, void* ddt,
                  int64_t ddt_tok_stride, float* ddt_bias, float* dA, float* dD, float* dstate_in,
                  void* workspace, size_t workspace_bytes, const int32_t* seq_lens, void* stream) {
    const int GN = d.G * d.N;
    if (!dt_bias || !A || !ddt_bias || !dA || !dD) return M2_ERR_NULL;
    if (rows > 0 && (!x || !B || !C || !dt || !dy || !dx || !dB || !dC || !ddt)) return M2_ERR_NULL;
    if (rows > 0 && (x_tok_stride < d.d_inner || bc_tok_stride < GN || dt_tok_stride < d.H ||
                     dy_tok_stride < d.d_inner || dx_tok_stride < d.d_inner || dbc_tok_stride < GN ||
                     ddt_tok_stride < d.H))
        return M2_ERR_SHAPE;
    if (std::isnan(dt_min) || std::isnan(dt_max) || dt_min > dt_max) return M2_ERR_SHAPE;
    if (!m2::ssd_bwd_supported(d.P, d.N, d.bf16)) return M2_ERR_UNSUPPORTED;
    // grid rows: (sequence, group) and (sequence, head) pairs
    if (d.batch * d.H > 65535) return M2_ERR_UNSUPPORTED;
    if (rows > 0 && (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(dy) || !aligned16(dx) ||
                     !aligned16(dB) || !aligned16(dC) || (x_tok_stride * 2) % 16 || (bc_tok_stride * 2) % 16 ||
                     (dy_tok_stride * 2) % 16 || (dx_tok_stride * 2) % 16 || (dbc_tok_stride * 2) % 16 ||
                     ((uintptr_t)dt & 1u) || ((uintptr_t)ddt & 1u)))
        return M2_ERR_UNSUPPORTED;
    if (((uintptr_t)state_in & 3u) || ((uintptr_t)dstate_out & 3u) || ((uintptr_t)dstate_in & 3u) ||
        ((uintptr_t)seq_lens & 3u) || ((uintptr_t)cu & 3u))
        return M2_ERR_UNSUPPORTED;
    const size_t need = m2::ssd_bwd_workspace_bytes(d.batch, d.L, d.H, d.G);
    if (!workspace || workspace_bytes < need) return M2_ERR_WORKSPACE;
    const int64_t SS = (int64_t)d.P * d.N;
    const Range ins[] = {span(x, rows, x_tok_stride, d.d_inner, 2), span(B, rows, bc_tok_stride, GN, 2),
                         span(C, rows, bc_tok_stride, GN, 2), span(dt, rows, dt_tok_stride, d.H, 2),
                         span(dy, rows, dy_tok_stride, d.d_inner, 2), span(dt_bias, 1, 0, d.H, 4),
                         span(A, 1, 0, d.H, 4), span(D, 1, 0, d.H, 4), span(state_in, d.batch * d.H, SS, SS, 4),
                         span(dstate_out, d.batch * d.H, SS, SS, 4), span(seq_lens, d.batch, 1, 1, 4),
                         span(cu, d.batch + 1, 1, 1, 4)};
    const Range outs[] = {span(dx, rows, dx_tok_stride, d.d_inner, 2), span(dB, rows, dbc_tok_stride, GN, 2),
                          span(dC, rows, dbc_tok_stride, GN, 2), span(ddt, rows, ddt_tok_stride, d.H, 2),
                          span(ddt_bias, 1, 0, d.H, 4), span(dA, 1, 0, d.H, 4), span(dD, 1, 0, d.H, 4),
                          span(dstate_in, d.batch * d.H, SS, SS, 4), span(workspace, 1, 0, (int64_t)need, 1)};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return M2_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(outs[i], outs[j])) return M2_ERR_ALIAS;
    }
    m2::BwdArgs a{};
    a.x = (const uint16_t*)x; a.xs = x_tok_stride;
    a.B = (const uint16_t*)B; a.C = (const uint16_t*)C; a.bcs = bc_tok_stride;
    a.dt = (const uint16_t*)dt; a.dts = dt_tok_stride;
    a.dy = (const uint16_t*)dy; a.dys = dy_tok_stride;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.dt_min = dt_min; a.dt_max = dt_max;
    a.state_in = state_in; a.dstate_out = dstate_out;
    a.dx = (uint16_t*)dx; a.dxs = dx_tok_stride;
    a.dB = (uint16_t*)dB; a.dC = (uint16_t*)dC; a.dbcs = dbc_tok_stride;
    a.ddt = (uint16_t*)ddt; a.ddts = ddt_tok_stride;
    a.ddt_bias = ddt_bias; a.dA = dA; a.dD = dD; a.dstate_in = dstate_in;
    a.batch = d.batch; a.L = d.L; a.H = d.H; a.G = d.G;
    a.lens = seq_lens;
    a.cu = cu;
    a.total = cu ? rows : 0;
    a.ws = workspace;
    return launched(m2::launch_ssd_scan_bwd(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

m2_status m2_ssd_scan_bwd(const m2_dims* dims, const void* x, int64_t x_tok_stride, const void* B, const void* C,
                          int64_t bc_tok_stride, const void* dt, int64_t dt_tok_stride, const float* dt_bias,
                          const float* A, const float* D, float dt_min, float dt_max, const float* state_in,
                          const void* dy, int64_t dy_tok_stride, const float* dstate_out, void* dx,
                          int64_t dx_tok_stride, void* dB, void* dC, int64_t dbc_tok_stride, void* ddt,
                          int64_t ddt_tok_stride, float* ddt_bias, float* dA, float* dD, float* dstate_in,
                          void* workspace, size_t workspace_bytes, const int32_t* seq_lens, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    return bwd_run(d, d.batch * d.L, nullptr, x, x_tok_stride, B, C, bc_tok_stride, dt, dt_tok_stride, dt_bias, A, D,
                   dt_min, dt_max, state_in, dy, dy_tok_stride, dstate_out, dx, dx_tok_stride, dB, dC, dbc_tok_stride,
                   ddt, ddt_tok_stride, ddt_bias, dA, dD, dstate_in, workspace, workspace_bytes, seq_lens, stream);
}

m2_status m2_ssd_scan_bwd_packed(const m2_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens,
                                 const void* x, int64_t x_tok_stride, const void* B, const void* C,
                                 int64_t bc_tok_stride, const void* dt, int64_t dt_tok_stride, const float* dt_bias,
                                 const float* A, const float* D, float dt_min, float dt_max, const float* state_in,
                                 const void* dy, int64_t dy_tok_stride, const float* dstate_out, void* dx,
                                 int64_t dx_tok_stride, void* dB, void* dC, int64_t dbc_tok_stride, void* ddt,
                                 int64_t ddt_tok_stride, float* ddt_bias, float* dA, float* dD, float* dstate_in,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    Derived d;
    m2_status st = derive(dims, d);
    if (st != M2_OK) return st;
    if (total_tokens < 0) return M2_ERR_SHAPE;
    if (d.batch > 0 && !cu_seqlens) return M2_ERR_NULL;
    return bwd_run(d, total_tokens, cu_seqlens, x, x_tok_stride, B, C, bc_tok_stride, dt, dt_tok_stride, dt_bias, A,
                   D, dt_min, dt_max, state_in, dy, dy_tok_stride, dstate_out, dx, dx_tok_stride, dB, dC,
                   dbc_tok_stride, ddt, ddt_tok_stride, ddt_bias, dA, dD, dstate_in, workspace, workspace_bytes,
                   nullptr, stream);
}

m2_status m2_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (bytes == 0) return M2_OK;
    if (!dst || !src) return M2_ERR_NULL;
    if (bytes % 16 || !aligned16(dst) || !aligned16(src)) return M2_ERR_UNSUPPORTED;
    if (overlap(Range{(uintptr_t)dst, (uintptr_t)dst + bytes}, Range{(uintptr_t)src, (uintptr_t)src + bytes}))
        return M2_ERR_ALIAS;
    return launched(m2::launch_stream_copy(dst, src, bytes, (hipStream_t)stream));
}

m2_status m2_gated_rmsnorm(int64_t ntok, int32_t d_inner, int32_t group_size, int32_t io, const void* y,
                           int64_t y_tok_stride, const void* z, int64_t z_tok_stride, const float* w, float eps,
                           int32_t norm_before_gate, void* out, int64_t out_tok_stride, void* stream) {
    if (io != M2_F32 && io != M2_BF16) return M2_ERR_DTYPE;
    if (ntok < 0 || d_inner < 1 || group_size < 1 || d_inner % group_size) return M2_ERR_SHAPE;
    if (!w) return M2_ERR_NULL;
    if (std::isnan(eps) || eps < 0.0f) return M2_ERR_SHAPE;
    const bool bf16 = io == M2_BF16;
    const int esize = bf16 ? 2 : 4, epv = 16 / esize;
    if (group_size % epv || group_size > m2::gated_rmsnorm_max_group(bf16)) return M2_ERR_UNSUPPORTED;
    if (ntok == 0) return M2_OK;
    if (!y || !z || !out) return M2_ERR_NULL;
    if (y_tok_stride < d_inner || z_tok_stride < d_inner || out_tok_stride < d_inner) return M2_ERR_SHAPE;
    const Range ry = span(y, ntok, y_tok_stride, d_inner, esize);
    const Range rz = span(z, ntok, z_tok_stride, d_inner, esize);
    const Range ro = span(out, ntok, out_tok_stride, d_inner, esize);
    const bool in_place = out == y && out_tok_stride == y_tok_stride;
    if (overlap(ro, rz) || (!in_place && overlap(ro, ry))) return M2_ERR_ALIAS;
    if (!aligned16(y) || !aligned16(z) || !aligned16(out) || !aligned16(w) || (y_tok_stride * esize) % 16 ||
        (z_tok_stride * esize) % 16 || (out_tok_stride * esize) % 16)
        return M2_ERR_UNSUPPORTED;
    m2::NormArgs a;
    a.ntok = ntok; a.d_inner = d_inner; a.gs = group_size;
    a.y = y; a.ys = y_tok_stride; a.z = z; a.zs = z_tok_stride; a.w = w; a.eps = eps;
    a.norm_before_gate = norm_before_gate != 0; a.out = out; a.os = out_tok_stride; a.bf16 = bf16;
    return launched(m2::launch_gated_rmsnorm(a, (hipStream_t)stream));
}

}  // extern "C"
