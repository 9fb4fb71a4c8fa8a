// Single-token (decode) step of the selective scan for gfx950.
//
// The recurrent use of the model (note "상태공간 모델(SSM)과 Mamba 아키텍처", §2: the
// recurrence carries the state from token to token; page "3.2 선택적 스캔(Selective Scan)
// 알고리즘과 정보의 압축 및 선별", §1.2 softplus step, §2.1 exp discretisation, §1.1
// readout, §3 of the note for the SiLU gate): for one token per (batch row, channel),
//   δ = softplus(dt_bias + dt_raw);  h_n ← exp(δ A_n) h_n + δ B_n x;  y = (Σ_n C_n h_n + D x)·silu(z)
// with the state read and written in place.  Δraw is per (row, channel) [B, D] or one
// value per token [B] shared by the channels.  Per channel the state is N floats, and it is
// the whole of the traffic that grows with N: the step is bound by HBM bandwidth.
//
// Layout: S = min(N, 4) states per lane, G = N / S lanes per channel, so a wave reads and
// writes 64·S contiguous floats of the state (1 KB at N >= 4) and every lane moves 16 bytes.
// B and C of a batch row are shared by all its channels and stay in cache.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

namespace {

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace

// four floats as a native vector (the nontemporal builtins take no struct types)
typedef float ntf4 __attribute__((ext_vector_type(4)));

// one thread per (batch row, channel, lane of the channel's group); grid = ceil(B·D·G / 256)
template <typename Tin, int S, int G, bool kGate, bool kZoh>
__global__ __launch_bounds__(256) void step_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ A, const Tin* __restrict__ Bm,
    const Tin* __restrict__ Cm, const float* __restrict__ Dskip, const float* h_in, float* h_out,
    float* __restrict__ y, int64_t BD, int64_t D, int dt_shared) {
    constexpr int N = S * G;
    const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t ch = gid / G;                  // b * D + d
    if (ch >= BD) return;                        // whole groups only: G divides 64
    const int l = int(gid % G);
    const int64_t b = ch / D, d = ch - b * D;
    const int n0 = l * S;

    const float xv = to_f32(x[ch]);
    const float delta = softplus(dt_bias[d] + to_f32(dt_raw[dt_shared ? b : ch]));
    const float dx = delta * xv;
    float h[S];
    const float* hp = h_in + ch * N + n0;
    // the state streams through once per step: nontemporal load and store (cache hint only)
    if constexpr (S == 4) {
        const ntf4 v = __builtin_nontemporal_load(reinterpret_cast<const ntf4*>(hp));
        h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) h[s] = hp[s];
    }
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = n0 + s;
        const float a = A[d * N + n];
        const float t2 = delta * (a * kLog2e);
        const float abar = exp2_hw(t2);
        float bx = (kZoh ? xv : dx) * to_f32(Bm[b * N + n]);
        if (kZoh) bx *= zoh_gain(t2, abar, delta, 1.0f / a);
        h[s] = fmaf(abar, h[s], bx);
        acc = fmaf(to_f32(Cm[b * N + n]), h[s], acc);
    }
    float* ho = h_out + ch * N + n0;             // may be h_in: this lane read its states above
    if constexpr (S == 4) {
        __builtin_nontemporal_store(ntf4{h[0], h[1], h[2], h[3]}, reinterpret_cast<ntf4*>(ho));
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) ho[s] = h[s];
    }
    acc = group_sum<G>(acc);
    if (l == 0) {
        float out = fmaf(Dskip[d], xv, acc);
        if (kGate) out *= silu(to_f32(z[ch]));
        y[ch] = out;
    }
}

template <typename Tin, int S, int G>
static hipError_t launch_step_t(const StepLaunch& p, hipStream_t s) {
    const int64_t threads = p.B * p.D * G;
    dim3 grid(unsigned((threads + 255) / 256));
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
    const Tin* Bm = static_cast<const Tin*>(p.Bm);
    const Tin* Cm = static_cast<const Tin*>(p.Cm);
#define SS_STEP_ARGS x, dr, z, p.dt_bias, p.A, Bm, Cm, p.Dskip, p.h_in, p.h_out, p.y, p.B * p.D, p.D, \
                     p.dt_shared
    if (p.zoh) {
        if (z) hipLaunchKernelGGL((step_kernel<Tin, S, G, true, true>), grid, dim3(256), 0, s, SS_STEP_ARGS);
        else hipLaunchKernelGGL((step_kernel<Tin, S, G, false, true>), grid, dim3(256), 0, s, SS_STEP_ARGS);
    } else {
        if (z) hipLaunchKernelGGL((step_kernel<Tin, S, G, true, false>), grid, dim3(256), 0, s, SS_STEP_ARGS);
        else hipLaunchKernelGGL((step_kernel<Tin, S, G, false, false>), grid, dim3(256), 0, s, SS_STEP_ARGS);
    }
#undef SS_STEP_ARGS
    return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_step_dt(const StepLaunch& p, hipStream_t s) {
    switch (p.N) {
        case 1: return launch_step_t<Tin, 1, 1>(p, s);
        case 2: return launch_step_t<Tin, 2, 1>(p, s);
        case 4: return launch_step_t<Tin, 4, 1>(p, s);
        case 8: return launch_step_t<Tin, 4, 2>(p, s);
        case 16: return launch_step_t<Tin, 4, 4>(p, s);
        case 32: return launch_step_t<Tin, 4, 8>(p, s);
        case 64: return launch_step_t<Tin, 4, 16>(p, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step(int bf16, const StepLaunch& p, hipStream_t s) {
    return bf16 ? launch_step_dt<bf16_t>(p, s) : launch_step_dt<float>(p, s);
}

}  // namespace ss
