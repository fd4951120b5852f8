// ssd_scan.hip -- selective state-space scan over a prompt (gfx950).
//
// First version: one block per (sequence, head) walks the tokens in order with the
// P x N fp32 state held in registers (16-byte slices per lane), exactly the
// recurrence S_t = exp(dt_t A) S_{t-1} + dt_t x_t B_t^T, y_t = S_t C_t + D x_t.
// Inputs of token t+1 are prefetched while token t is applied.
#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

constexpr int kScanThreads = 256;

template <typename T, int N, int K>
__global__ __launch_bounds__(kScanThreads) void ssd_scan_seq_kernel(
    const T* __restrict__ x, int64_t xs, const T* __restrict__ Bm, const T* __restrict__ Cm, int64_t bcs,
    const T* __restrict__ dtr, int64_t dts, const float* __restrict__ dt_bias, const float* __restrict__ Aa,
    const float* __restrict__ Dd, float dt_min, float dt_max, const float* __restrict__ state_in,
    float* __restrict__ state_out, T* __restrict__ y, int64_t ys, int64_t L, int H, int P, int G)
{
    constexpr int TPR = N / 4;
    __shared__ float buf[2][512 + 2 * 256];
    const int h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x;
    const int g = h / (H / G);
    const int nvec = P * TPR;
    const int nld = P + 2 * N;  // elements loaded per token

    float4 s[K];
    const int64_t soff = ((b * H + h) * (int64_t)P) * N;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = tid + k * kScanThreads;
        s[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (state_in && i < nvec) s[k] = reinterpret_cast<const float4*>(state_in + soff)[i];
    }
    const float bias_h = dt_bias[h], A_h = Aa[h], D_h = Dd ? Dd[h] : 0.0f;

    // element j of a token: x[p] (j < P), B[n], C[n]
    auto src = [&](int64_t t, int j) -> float {
        const int64_t bt = b * L + t;
        if (j < P) return to_f32(x[bt * xs + (int64_t)h * P + j]);
        if (j < P + N) return to_f32(Bm[bt * bcs + (int64_t)g * N + (j - P)]);
        return to_f32(Cm[bt * bcs + (int64_t)g * N + (j - P - N)]);
    };
    float pre0 = 0.f, pre1 = 0.f, pdt = 0.f;
    if (L > 0) {
        if (tid < nld) pre0 = src(0, tid);
        if (tid + kScanThreads < nld) pre1 = src(0, tid + kScanThreads);
        pdt = to_f32(dtr[(b * L) * dts + h]);
    }
    for (int64_t t = 0; t < L; ++t) {
        float* cur = buf[t & 1];
        if (tid < nld) cur[tid] = pre0;
        if (tid + kScanThreads < nld) cur[tid + kScanThreads] = pre1;
        const float dt = dt_of(pdt, bias_h, dt_min, dt_max);
        if (t + 1 < L) {
            if (tid < nld) pre0 = src(t + 1, tid);
            if (tid + kScanThreads < nld) pre1 = src(t + 1, tid + kScanThreads);
            pdt = to_f32(dtr[(b * L + t + 1) * dts + h]);
        }
        __syncthreads();
        const float decay = fast_exp(dt * A_h);
        const float* xv = cur;
        const float* Bv = cur + P;
        const float* Cv = cur + P + N;
        T* yt = y + (b * L + t) * ys + (int64_t)h * P;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int i = tid + k * kScanThreads;
            const int p = i / TPR, n0 = (i % TPR) * 4;
            float part = 0.0f;
            if (i < nvec) {
                const float dx = dt * xv[p];
                float4 v = s[k];
                v.x = fmaf(decay, v.x, dx * Bv[n0 + 0]);
                v.y = fmaf(decay, v.y, dx * Bv[n0 + 1]);
                v.z = fmaf(decay, v.z, dx * Bv[n0 + 2]);
                v.w = fmaf(decay, v.w, dx * Bv[n0 + 3]);
                s[k] = v;
                part = v.x * Cv[n0] + v.y * Cv[n0 + 1] + v.z * Cv[n0 + 2] + v.w * Cv[n0 + 3];
            }
#pragma unroll
            for (int off = 1; off < TPR; off <<= 1) part += __shfl_xor(part, off, kWave);
            if (i < nvec && (i % TPR) == 0) yt[p] = from_f32<T>(part + D_h * xv[p]);
        }
    }
    if (state_out) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int i = tid + k * kScanThreads;
            if (i < nvec) reinterpret_cast<float4*>(state_out + soff)[i] = s[k];
        }
    }
}

template <typename T, int N, int K>
static hipError_t launch_scan_nk(const ScanArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.H, (unsigned)a.batch);
    return launch_kernel(ssd_scan_seq_kernel<T, N, K>, grid, dim3(kScanThreads), 0, s,
                       (const T*)a.x, a.xs, (const T*)a.B, (const T*)a.C, a.bcs, (const T*)a.dt, a.dts,
                       a.dt_bias, a.A, a.D, a.dt_min, a.dt_max, a.state_in, a.state_out, (T*)a.y, a.ys, a.L,
                       a.H, a.P, a.G);
}

template <typename T, int N>
static hipError_t launch_scan_n(const ScanArgs& a, hipStream_t s) {
    const int K = (a.P * (N / 4) + kScanThreads - 1) / kScanThreads;
    switch (K) {
        case 1: return launch_scan_nk<T, N, 1>(a, s);
        case 2: return launch_scan_nk<T, N, 2>(a, s);
        case 3: case 4: return launch_scan_nk<T, N, 4>(a, s);
        default: return launch_scan_nk<T, N, 8>(a, s);
    }
}

template <typename T>
static hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
    switch (a.N) {
        case 16: return launch_scan_n<T, 16>(a, s);
        case 32: return launch_scan_n<T, 32>(a, s);
        case 64: return launch_scan_n<T, 64>(a, s);
        default: return launch_scan_n<T, 128>(a, s);
    }
}

bool ssd_scan_supported(int P, int N, int Q, bool) {
    (void)Q;
    if (!(N == 16 || N == 32 || N == 64 || N == 128)) return false;
    if (P + 2 * N > 512) return false;
    return (int64_t)P * (N / 4) <= 8 * kScanThreads;
}

int ssd_scan_default_chunk(int, int, bool) { return 64; }

size_t ssd_scan_workspace_bytes(int64_t, int64_t, int, int, int, int, int, bool) { return 0; }

hipError_t launch_ssd_scan(const ScanArgs& a, hipStream_t s) {
    return a.bf16 ? launch_scan_t<bf16_t>(a, s) : launch_scan_t<float>(a, s);
}

}  // namespace m2
