// Forward selective-scan kernels for gfx950.
//
// Page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별":
//   §2.1  Ā_t = exp(Δ_t A) with diagonal A, so the discretisation is elementwise;
//   §2.2  h_t = Ā_t h_{t-1} + B̄_t x_t, an associative scan over affine pairs;
//   §3.1/§3.2  the (B, L, D, N) state and Ā, B̄ are never written to HBM: inputs are
//         read once, the state lives on chip, only y leaves.
// Here "on chip" means VGPRs: one lane owns one (b, d) channel and keeps its N
// states in registers for the whole time range it covers.  B_t and C_t are the
// same for every channel of a batch row, so all lanes of a workgroup read them
// at the same address: they come through the scalar cache into SGPRs (one
// 2N-float row per step from a [B, L, 2N] float32 staging copy made by
// bc_stage_kernel), never through VGPRs or LDS.
//
// Two modes of one kernel body:
//   OUT — full step with readout and gate, writes y (and h_final on the last chunk);
//   AGG — chunk aggregate for the sequence-parallel plan: the chunk's local scan
//         from a zero state (h_end) and Σδ over the chunk, whose exp gives the
//         chunk's product of Ā (Π_t exp(δ_t A) = exp(A Σ_t δ_t)).
#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

// ---------------------------------------------------------------------------------------
// B, C [B, N, L] (or token-major [B, L, N]; in dtype) -> BC [B, L, 2N] float32: row t
// holds B[:, t] then C[:, t].  A 256-thread block stages a 64-step tile through LDS so both
// sides are coalesced.
// ---------------------------------------------------------------------------------------
template <typename Tin, int N>
__global__ __launch_bounds__(256) void bc_stage_kernel(const Tin* __restrict__ Bm,
                                                       const Tin* __restrict__ Cm,
                                                       float* __restrict__ BC, int64_t L, int tok) {
    constexpr int TT = 64;
    constexpr int R = 2 * N;  // rows of the tile
    __shared__ float tile[R][TT + 1];
    const int b = blockIdx.y;
    const int64_t t0 = int64_t(blockIdx.x) * TT;
    const int tid = threadIdx.x;
    for (int e = tid; e < R * TT; e += 256) {
        // channel-major: steps fastest across threads; token-major: states fastest
        const int r = tok ? e % R : e / TT, c = tok ? e / R : e % TT;
        const int64_t t = t0 + c;
        float v = 0.0f;
        if (t < L) {
            const Tin* src = (r < N) ? Bm : Cm;
            const int n = (r < N) ? r : r - N;
            v = to_f32(src[tok ? (int64_t(b) * L + t) * N + n : (int64_t(b) * N + n) * L + t]);
        }
        tile[r][c] = v;
    }
    __syncthreads();
    const int64_t nt = (L - t0 < TT) ? (L - t0) : TT;
    float* dst = BC + (int64_t(b) * L + t0) * R;
    for (int e = tid; e < nt * R; e += 256) dst[e] = tile[e % R][e / R];
}

// ---------------------------------------------------------------------------------------
// Channel-parallel scan over one chunk [k*chunk, min(L, (k+1)*chunk)) of each channel.
// grid = (ceil(D / blockDim), K, B); lane = channel d.
// h_init: nullable, [B, D, K, N] (K = 1 holds h0).  OUT: y [B, D, L]; h_last (nullable)
// = h_final [B, D, N], written by chunk K-1.  AGG: h_last = h_end [B, D, K, N],
// dsum [B, D, K].
// ---------------------------------------------------------------------------------------
template <typename Tin, int N, bool kGate, bool kAgg, bool kZoh>
__global__ __launch_bounds__(256) void scan_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ BC,
    const float* __restrict__ h_init, float* __restrict__ y, float* __restrict__ h_last,
    float* __restrict__ h_ckpt, float* __restrict__ dsum_out, int64_t L, int64_t D,
    int64_t chunk, int K, int vec, int tok, DtRows dtr) {
    const int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int k = blockIdx.y;
    const int b = blockIdx.z;
    if (d >= D) return;   // the vote below is over the remaining (active) lanes
    const int64_t t_begin = int64_t(k) * chunk;
    const int64_t t_end = (t_begin + chunk < L) ? t_begin + chunk : L;

    float A2[N], iA[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float a = A[d * N + n];
        A2[n] = a * kLog2e;
        if (kZoh) iA[n] = 1.0f / a;
    }
    const int64_t hidx = ((int64_t(b) * D + d) * K + k) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = h_init ? h_init[hidx + n] : 0.0f;

    const float bias = dt_bias[d];
    const float Dd = kAgg ? 0.0f : Dskip[d];
    // element t of x, z, y at row[t·ts] (channel-major rows, or token-major with a wave's
    // 64 channels side by side); Δraw at its own rows
    const int64_t row = tok ? int64_t(b) * L * D + d : (int64_t(b) * D + d) * L;
    const int64_t ts = tok ? D : 1;
    const Tin* xr = x + row;
    const Tin* dr = dt_raw + int64_t(b) * dtr.sb + d * dtr.sd;
    const int64_t dts = dtr.ts;
    const Tin* zr = kGate ? z + row : nullptr;
    float* yr = kAgg ? nullptr : y + row;
    // 8-step vector loads where a tensor's steps are contiguous and 16-byte aligned
    const bool xvec = vec && ts == 1, dvec = vec && dts == 1;
    const float* bcb = BC + int64_t(b) * L * (2 * N);
    float dsum = 0.0f;
    // checkpoints: the state entering step t for every t % kCkptSteps == 0
    const int64_t nck = (L + kCkptSteps - 1) / kCkptSteps;
    float* ckr = (!kAgg && h_ckpt) ? h_ckpt + (int64_t(b) * D + d) * nck * N : nullptr;

    // One step.  Bq/Cq hold this step's B and C (uniform across the wave: SGPRs).  The
    // state update reads only Bq and the readout only Cq, so the next step's B row is
    // loaded right after the update and its C row right after the readout: each scalar
    // load is covered by about half a step without a second register set.
    // kS4D: A[d, n] = -(n+1) exactly (S4D-real): Ā_n = exp(-(n+1)δ) = r^(n+1) with
    // r = exp(-δ) = 1 / (1 + e^u) (δ = softplus(u)), so one reciprocal and a chain of
    // multiplies replace the N exponentials; r^(n+1) by repeated multiplication carries
    // about (n+1) ulp of relative error.
    float Bq[N], Cq[N];
    auto load_B = [&](int64_t tt) {
#pragma unroll
        for (int n = 0; n < N; ++n) Bq[n] = bcb[tt * (2 * N) + n];
    };
    auto load_C = [&](int64_t tt) {
#pragma unroll
        for (int n = 0; n < N; ++n) Cq[n] = bcb[tt * (2 * N) + N + n];
    };
    auto step = [&](auto s4d_tag, float xv, float dv, float zv, int64_t tt) -> float {
        constexpr bool kS4D = decltype(s4d_tag)::value;
        if (ckr && tt % kCkptSteps == 0) {      // uniform: every lane is at step tt
#pragma unroll
            for (int n = 0; n < N; ++n) ckr[(tt / kCkptSteps) * N + n] = h[n];
        }
        float delta, r = 1.0f;
        if constexpr (kS4D) {
            const float u = bias + dv;
            const float w = exp2_hw(-fabsf(u) * kLog2e);            // e^{-|u|}
            const float v = 1.0f + w;
            delta = fmaxf(u, 0.0f) + fmaf(log2_hw(v), kLn2, w - (v - 1.0f));
            r = (u > 0.0f ? w : 1.0f) * rcp_hw(v);                   // e^{-δ}
        } else {
            delta = softplus(bias + dv);
        }
        if (kAgg) dsum += delta;
        const float dx = delta * xv;
        float a = r;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float t2 = delta * A2[n];
            const float abar = kS4D ? a : exp2_hw(t2);
            float bx = (kZoh ? xv : dx) * Bq[n];
            if (kZoh) bx *= zoh_gain(t2, abar, delta, iA[n]);
            h[n] = fmaf(abar, h[n], bx);
            if (kS4D) a *= r;
        }
        const bool more = tt + 1 < t_end;
        if (more) load_B(tt + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (kAgg) return 0.0f;
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) acc = fmaf(Cq[n], h[n], acc);
        if (more) load_C(tt + 1);
        __builtin_amdgcn_sched_barrier(0);
        float s = fmaf(Dd, xv, acc);
        if (kGate) s *= silu(zv);
        return s;
    };

    bool s4d = true;
#pragma unroll
    for (int n = 0; n < N; ++n) s4d = s4d && (A[d * N + n] == -float(n + 1));
    const bool fast = __all(s4d);   // uniform across the (active lanes of the) wave

    using Tag1 = std::integral_constant<bool, true>;
    using Tag0 = std::integral_constant<bool, false>;
    auto run = [&](auto s4d_tag) {
        int64_t t = t_begin;
        if (t < t_end) {
            load_B(t);
            if (!kAgg) load_C(t);
        }
        if ((vec || tok) && t + 8 <= t_end) {
            Tin xr8[8], dr8[8], zr8[8];
            auto load_group = [&](int64_t tt) {
                constexpr int V = int(8 * sizeof(Tin) / 16);   // uint4 per 8 elements
                if (xvec) {
#pragma unroll
                    for (int q = 0; q < V; ++q) {
                        reinterpret_cast<uint4*>(xr8)[q] = reinterpret_cast<const uint4*>(xr + tt)[q];
                        if (kGate && !kAgg)
                            reinterpret_cast<uint4*>(zr8)[q] = reinterpret_cast<const uint4*>(zr + tt)[q];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        xr8[i] = xr[(tt + i) * ts];
                        if (kGate && !kAgg) zr8[i] = zr[(tt + i) * ts];
                    }
                }
                if (dvec) {
#pragma unroll
                    for (int q = 0; q < V; ++q)
                        reinterpret_cast<uint4*>(dr8)[q] = reinterpret_cast<const uint4*>(dr + tt)[q];
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) dr8[i] = dr[(tt + i) * dts];
                }
            };
            load_group(t);
            for (; t + 8 <= t_end; t += 8) {
                float xv[8], dv[8], zv[8], yv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    xv[i] = to_f32(xr8[i]);
                    dv[i] = to_f32(dr8[i]);
                    zv[i] = (kGate && !kAgg) ? to_f32(zr8[i]) : 0.0f;
                }
                if (t + 16 <= t_end) load_group(t + 8);
                // rolled: an unrolled body keeps several B/C rows live and spills SGPRs
#pragma unroll 1
                for (int i = 0; i < 8; ++i) yv[i] = step(s4d_tag, xv[i], dv[i], zv[i], t + i);
                if (!kAgg) {
                    if (xvec) {
                        store8(yr + t, yv);
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) yr[(t + i) * ts] = yv[i];
                    }
                }
            }
        }
        for (; t < t_end; ++t) {
            const float zv = (kGate && !kAgg) ? to_f32(zr[t * ts]) : 0.0f;
            const float r = step(s4d_tag, to_f32(xr[t * ts]), to_f32(dr[t * dts]), zv, t);
            if (!kAgg) yr[t * ts] = r;
        }
    };
    if (fast) run(Tag1{});
    else run(Tag0{});

    if (kAgg) {
        const int64_t aidx = (int64_t(b) * D + d) * K + k;
#pragma unroll
        for (int n = 0; n < N; ++n) h_last[aidx * N + n] = h[n];
        dsum_out[aidx] = dsum;
    } else if (h_last && k == K - 1) {
        const int64_t fidx = (int64_t(b) * D + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) h_last[fidx + n] = h[n];
    }
}

// ---------------------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------------------
template <typename Tin, int N>
static hipError_t launch_bc_stage_t(const void* Bm, const void* Cm, float* BC, int64_t B,
                                    int64_t L, int tok, hipStream_t s) {
    dim3 grid(unsigned((L + 63) / 64), unsigned(B));
    hipLaunchKernelGGL((bc_stage_kernel<Tin, N>), grid, dim3(256), 0, s,
                       static_cast<const Tin*>(Bm), static_cast<const Tin*>(Cm), BC, L, tok);
    return hipGetLastError();
}

template <typename Tin, int N>
static hipError_t launch_scan_t(const ScanLaunch& p, hipStream_t s) {
    const int wg = p.D >= 256 ? 256 : int((p.D + 63) / 64) * 64;
    // the last chunk's aggregate has no successor: the carry reads it only into values it
    // never stores (the final state comes from the output pass), so it is not computed
    const unsigned kg = unsigned((p.agg && p.K > 1) ? p.K - 1 : p.K);
    dim3 grid(unsigned((p.D + wg - 1) / wg), kg, unsigned(p.B));
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
#define SS_SCAN_ARGS x, dr, z, p.dt_bias, p.A, p.Dskip, p.BC, p.h_init, p.y, p.h_last, p.h_ckpt, \
                     p.dsum, p.L, p.D, p.chunk, p.K, p.vec, p.tok, p.dtr
    if (p.zoh) {
        if (p.agg)
            hipLaunchKernelGGL((scan_kernel<Tin, N, false, true, true>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
        else if (p.z)
            hipLaunchKernelGGL((scan_kernel<Tin, N, true, false, true>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
        else
            hipLaunchKernelGGL((scan_kernel<Tin, N, false, false, true>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
    } else {
        if (p.agg)
            hipLaunchKernelGGL((scan_kernel<Tin, N, false, true, false>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
        else if (p.z)
            hipLaunchKernelGGL((scan_kernel<Tin, N, true, false, false>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
        else
            hipLaunchKernelGGL((scan_kernel<Tin, N, false, false, false>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
    }
#undef SS_SCAN_ARGS
    return hipGetLastError();
}

#define SS_DISPATCH_N(FN, TIN, ...)                        \
    switch (N) {                                           \
        case 1: return FN<TIN, 1>(__VA_ARGS__);            \
        case 2: return FN<TIN, 2>(__VA_ARGS__);            \
        case 4: return FN<TIN, 4>(__VA_ARGS__);            \
        case 8: return FN<TIN, 8>(__VA_ARGS__);            \
        case 16: return FN<TIN, 16>(__VA_ARGS__);          \
        case 32: return FN<TIN, 32>(__VA_ARGS__);          \
        default: return hipErrorInvalidValue;              \
    }

hipError_t launch_bc_stage(int bf16, int N, const void* Bm, const void* Cm, float* BC, int64_t B,
                           int64_t L, int tok, hipStream_t s) {
    if (bf16) { SS_DISPATCH_N(launch_bc_stage_t, bf16_t, Bm, Cm, BC, B, L, tok, s) }
    SS_DISPATCH_N(launch_bc_stage_t, float, Bm, Cm, BC, B, L, tok, s)
}

hipError_t launch_scan(int bf16, int N, const ScanLaunch& p, hipStream_t s) {
    if (bf16) { SS_DISPATCH_N(launch_scan_t, bf16_t, p, s) }
    SS_DISPATCH_N(launch_scan_t, float, p, s)
}

}  // namespace ss
