// ssd_step.hip -- fused single-token decode step (gfx950).
//
// The mixer's recurrent single-step path (article "Transformers 中 Zamba2 混合架构模型解析",
// §三: with a cached state and a new sequence length of 1 the scan is replaced by a
// recurrent state update; the cache holds each layer's conv state and recurrent state).
// One block per (sequence b, head h):
//   1. conv window = W-1 cached tokens from the ring + the new token, 4-tap dot + SiLU
//      for the head's P x-channels and its group's N B-channels and N C-channels
//      (kept in fp32 in LDS, never rounded);
//   2. dt = softplus(dt_raw + dt_bias), decay = exp(dt * A);
//   3. S[p,n] <- decay * S[p,n] + dt * x[p] * B[n];  y[p] = sum_n S[p,n] C[n] + D x[p].
// The state (P*N fp32) dominates the traffic: it is read and written once, as 16-byte
// vectors, and its loads are issued before the conv so their latency overlaps it.
// The new token goes into ring slot step mod W, the slot that left the window; no
// block reads that slot in this step, so the heads sharing B/C channels do not race.
// The x-channels of a head are written by that head's block, the B/C channels by the
// first head of the group.
#include "m2_device.h"
#include "m2_launch.h"

namespace m2 {

constexpr int kStepThreads = 256;

template <typename T, int N, int K>
__global__ __launch_bounds__(kStepThreads) void ssd_step_kernel(
    const T* __restrict__ xbc, int64_t xbs, const T* __restrict__ dtr, int64_t dts,
    const float* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ dt_bias, const float* __restrict__ Aa, const float* __restrict__ Dd,
    float dt_min, float dt_max, T* __restrict__ ring, int phase, int W,
    float* __restrict__ state, T* __restrict__ y, int H, int P, int G, int Cd)
{
    constexpr int TPR = N / 4;  // lanes per state row (float4 each)
    __shared__ float act[1024];
    const int h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x;
    const int hpg = H / G, g = h / hpg;
    const int Di = H * P;
    const int nvec = P * TPR;  // float4 chunks of the state

    f32x4* Sb = reinterpret_cast<f32x4*>(state + ((b * H + h) * (int64_t)P) * N);
    f32x4 s[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = tid + k * kStepThreads;
        if (i < nvec) s[k] = __builtin_nontemporal_load(Sb + i);
    }

    // conv + SiLU for the channels this head reads: x (P), then B (N), then C (N)
    const int nch = P + 2 * N;
    const T* tok = xbc + b * xbs;
    T* rb = ring + b * (int64_t)W * Cd;
    for (int j = tid; j < nch; j += kStepThreads) {
        int c;
        bool writer;
        if (j < P) { c = h * P + j; writer = true; }
        else if (j < P + N) { c = Di + g * N + (j - P); writer = (h % hpg) == 0; }
        else { c = Di + G * N + g * N + (j - P - N); writer = (h % hpg) == 0; }
        const T xin = tok[c];
        float v = bias ? bias[c] : 0.0f;
        for (int k = 0; k < W - 1; ++k) {
            int slot = phase - (W - 1) + k;   // token -(W-1-k) relative to the new one
            slot += slot < 0 ? W : 0;
            v = fmaf(w[(int64_t)c * W + k], to_f32(rb[(int64_t)slot * Cd + c]), v);
        }
        v = fmaf(w[(int64_t)c * W + W - 1], to_f32(xin), v);
        act[j] = silu(v);
        if (writer) rb[(int64_t)phase * Cd + c] = xin;
    }
    const float dt = dt_of(to_f32(dtr[b * dts + h]), dt_bias[h], dt_min, dt_max);
    const float decay = fast_exp(dt * Aa[h]);
    const float Dh = Dd ? Dd[h] : 0.0f;
    __syncthreads();

    const float* xs = act;
    const float* Bs = act + P;
    const float* Cs = act + P + N;
    T* yb = y + (b * H + h) * (int64_t)P;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = tid + k * kStepThreads;
        const int p = i / TPR, n0 = (i % TPR) * 4;
        float part = 0.0f;
        if (i < nvec) {
            const float dx = dt * xs[p];
            f32x4 v = s[k];
            v.x = fmaf(decay, v.x, dx * Bs[n0 + 0]);
            v.y = fmaf(decay, v.y, dx * Bs[n0 + 1]);
            v.z = fmaf(decay, v.z, dx * Bs[n0 + 2]);
            v.w = fmaf(decay, v.w, dx * Bs[n0 + 3]);
            __builtin_nontemporal_store(v, Sb + i);
            part = v.x * Cs[n0] + v.y * Cs[n0 + 1] + v.z * Cs[n0 + 2] + v.w * Cs[n0 + 3];
        }
        // sum over the TPR lanes of this row (they are adjacent lanes of one wave)
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) part += __shfl_xor(part, off, kWave);
        if (i < nvec && (i % TPR) == 0) yb[p] = from_f32<T>(part + Dh * xs[p]);
    }
}

template <typename T, int N, int K>
static hipError_t launch_step_nk(const StepArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.H, (unsigned)a.batch);
    const int phase = (int)(a.step % a.W);
    return launch_kernel(ssd_step_kernel<T, N, K>, grid, dim3(kStepThreads), 0, s,
                       (const T*)a.xbc, a.xbs, (const T*)a.dt, a.dts, a.w, a.bias, a.dt_bias, a.A, a.D,
                       a.dt_min, a.dt_max, (T*)a.ring, phase, a.W, a.state, (T*)a.y, a.H, a.P, a.G, a.Cd);
}

template <typename T, int N>
static hipError_t launch_step_n(const StepArgs& a, hipStream_t s) {
    const int nvec = a.P * (N / 4);
    const int K = (nvec + kStepThreads - 1) / kStepThreads;
    switch (K) {
        case 1: return launch_step_nk<T, N, 1>(a, s);
        case 2: return launch_step_nk<T, N, 2>(a, s);
        case 3: case 4: return launch_step_nk<T, N, 4>(a, s);
        default: return launch_step_nk<T, N, 8>(a, s);
    }
}

template <typename T>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t s) {
    switch (a.N) {
        case 16: return launch_step_n<T, 16>(a, s);
        case 32: return launch_step_n<T, 32>(a, s);
        case 64: return launch_step_n<T, 64>(a, s);
        case 128: return launch_step_n<T, 128>(a, s);
        default: return launch_step_n<T, 256>(a, s);
    }
}

bool ssd_step_supported(int P, int N) {
    if (!(N == 16 || N == 32 || N == 64 || N == 128 || N == 256)) return false;
    if (P + 2 * N > 1024) return false;            // LDS act buffer
    return (int64_t)P * (N / 4) <= 8 * kStepThreads;
}

hipError_t launch_ssd_step(const StepArgs& a, hipStream_t s) {
    return a.bf16 ? launch_step_t<bf16_t>(a, s) : launch_step_t<float>(a, s);
}

}  // namespace m2
