// Device helpers shared by the gfx950 selective-scan kernels.
//
// Numerics of the per-token step (page "3.2 선택적 스캔(Selective Scan) 알고리즘과
// 정보의 압축 및 선별", §1.2 softplus step size, §2.1 exp discretisation) and of
// the SiLU gate (note "상태공간 모델(SSM)과 Mamba 아키텍처", §3), written for the
// CDNA4 transcendental unit: exp and log are the hardware base-2 instructions,
// with natural-base constants folded into their operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware 2^x (v_exp_f32).  Arguments here are <= 0 or moderate, results normal or 0.
__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
// Hardware log2 (v_log_f32), used for arguments in (1, 2].
__device__ __forceinline__ float log2_hw(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float rcp_hw(float v) { return __builtin_amdgcn_rcpf(v); }

// softplus(u) = log(1 + e^u) = max(u, 0) + log1p(w), w = e^{-|u|} in (0, 1].
// log1p(w) = log(v) + (w - (v - 1)) with v = fl(1 + w): the hardware log2 of v (measured
// on gfx950 at <= 1.2e-7 relative error for every v in (1, 2], including v -> 1) plus
// the first-order correction for the rounding of v (v - 1 is exact for v in [1, 2]).
__device__ __forceinline__ float softplus(float u) {
    const float w = exp2_hw(-fabsf(u) * kLog2e);
    const float v = 1.0f + w;
    return fmaxf(u, 0.0f) + fmaf(log2_hw(v), kLn2, w - (v - 1.0f));
}

// Exact zero-order hold (page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및
// 선별", §2.1): B̄x = g·B x with the gain g = (e^{δA} - 1)/A = δ·φ(u), u = δA,
// φ(u) = (e^u - 1)/u.  For |u| < 1/8, δ times the degree-4 series of φ (truncation below
// u^5/6! < 4.3e-8), written in t2 = u·log2(e) so the caller's exponent argument serves;
// elsewhere (Ā - 1)·(1/A) in one fused rounding, whose relative error is at most
// |Ā/(Ā - 1)| < 7.6 times that of Ā.  t2 and abar = 2^t2 as the caller computed them,
// inv_a = 1/A (a per-channel constant; A = 0 gives t2 = 0, the series side).
constexpr float kZohC1 = 0.34657359027997264f;    // ln2^k / (k+1)!
constexpr float kZohC2 = 0.08007550231970023f;
constexpr float kZohC3 = 0.013876027166205394f;
constexpr float kZohC4 = 0.0019236258215256953f;
constexpr float kZohSwitch2 = 0.18033688011112042f;  // |u| = 1/8 in units of t2
__device__ __forceinline__ float zoh_gain(float t2, float abar, float delta, float inv_a) {
    float p = fmaf(t2, kZohC4, kZohC3);
    p = fmaf(t2, p, kZohC2);
    p = fmaf(t2, p, kZohC1);
    p = fmaf(t2, p, 1.0f);
    const float q = fmaf(abar, inv_a, -inv_a);
    return fabsf(t2) < kZohSwitch2 ? delta * p : q;
}

// ∂g/∂A of the same gain, for the backward: δ²·ψ(u) with ψ(u) = Σ_k (k+1)u^k/(k+2)!, the
// term-by-term derivative of φ.  For |u| < 1/8, the degree-4 series in t2 (truncation below
// 7.3e-8 relative); elsewhere the closed form (δĀ - g)·(1/A), g the caller's zoh_gain value,
// whose cancellation costs at most a factor 16 over the error of g (at |u| = 1/8).
constexpr float kZohD1 = 0.23104906018664842f;    // (k+1) ln2^k / (k+2)!
constexpr float kZohD2 = 0.06005662673977517f;
constexpr float kZohD3 = 0.011100821732964315f;
constexpr float kZohD4 = 0.0016030215179380794f;
__device__ __forceinline__ float zoh_gain_da(float t2, float abar, float delta, float inv_a,
                                             float gain) {
    float p = fmaf(t2, kZohD4, kZohD3);
    p = fmaf(t2, p, kZohD2);
    p = fmaf(t2, p, kZohD1);
    p = fmaf(t2, p, 0.5f);
    const float q = fmaf(delta, abar, -gain) * inv_a;
    return fabsf(t2) < kZohSwitch2 ? (delta * delta) * p : q;
}

// sigmoid(z) = 1 / (1 + e^{-z}); e^{-z} = inf for z << 0 gives exactly 0.
__device__ __forceinline__ float sigmoid(float z) { return rcp_hw(1.0f + exp2_hw(-z * kLog2e)); }

// silu(z) = z * sigmoid(z): the gate of the output branch.
__device__ __forceinline__ float silu(float z) { return z * sigmoid(z); }

// ---- input element types -------------------------------------------------------------
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(uint32_t(v.bits) << 16); }

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for f32) as float.
__device__ __forceinline__ void load8(const float* __restrict__ p, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* __restrict__ p, float (&o)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void store8(float* __restrict__ p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

}  // namespace ss
