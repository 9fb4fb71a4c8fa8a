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
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

// ---------------------------------------------------------------------------------------
// B, C [B, N, L] (in dtype) -> BC [B, L, 2N] float32: row t holds B[:, t] then C[:, t].
// A 256-thread block stages a 64-step tile through LDS so both sides are coalesced.
// ---------------------------------------------------------------------------------------
template <typename Tin, int N>
__global__ __launch_bounds__(256) void bc_stage_kernel(const Tin* __restrict__ Bm,
                                                       const Tin* __restrict__ Cm,
                                                       float* __restrict__ BC, int64_t L) {
    constexpr int TT = 64;
    constexpr int R = 2 * N;  // rows of the tile
    __shared__ float tile[R][TT + 1];
    const int b = blockIdx.y;
    const int64_t t0 = int64_t(blockIdx.x) * TT;
    const int tid = threadIdx.x;
    for (int e = tid; e < R * TT; e += 256) {
        const int r = e / TT, c = e % TT;
        const int64_t t = t0 + c;
        float v = 0.0f;
        if (t < L) {
            const Tin* src = (r < N) ? Bm : Cm;
            const int n = (r < N) ? r : r - N;
            v = to_f32(src[(int64_t(b) * N + n) * L + t]);
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
template <typename Tin, int N, bool kGate, bool kAgg>
__global__ __launch_bounds__(256) void scan_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ BC,
    const float* __restrict__ h_init, float* __restrict__ y, float* __restrict__ h_last,
    float* __restrict__ dsum_out, int64_t L, int64_t D, int64_t chunk, int K, int vec) {
    const int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int k = blockIdx.y;
    const int b = blockIdx.z;
    if (d >= D) return;
    const int64_t t_begin = int64_t(k) * chunk;
    const int64_t t_end = (t_begin + chunk < L) ? t_begin + chunk : L;

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = A[d * N + n] * kLog2e;
    const int64_t hidx = ((int64_t(b) * D + d) * K + k) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = h_init ? h_init[hidx + n] : 0.0f;

    const float bias = dt_bias[d];
    const float Dd = kAgg ? 0.0f : Dskip[d];
    const int64_t row = (int64_t(b) * D + d) * L;
    const Tin* xr = x + row;
    const Tin* dr = dt_raw + row;
    const Tin* zr = kGate ? z + row : nullptr;
    float* yr = kAgg ? nullptr : y + row;
    const float* bcb = BC + int64_t(b) * L * (2 * N);
    float dsum = 0.0f;

    auto step = [&](float xv, float dv, float zv, const float* __restrict__ bct) -> float {
        const float delta = softplus(bias + dv);
        if (kAgg) dsum += delta;
        const float dx = delta * xv;
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float abar = exp2_hw(delta * A2[n]);
            h[n] = fmaf(abar, h[n], dx * bct[n]);
            if (!kAgg) acc = fmaf(bct[N + n], h[n], acc);
        }
        if (kAgg) return 0.0f;
        float s = fmaf(Dd, xv, acc);
        if (kGate) s *= silu(zv);
        return s;
    };

    int64_t t = t_begin;
    if (vec) {
        for (; t + 8 <= t_end; t += 8) {
            float xv[8], dv[8], zv[8], yv[8];
            load8(xr + t, xv);
            load8(dr + t, dv);
            if (kGate && !kAgg) load8(zr + t, zv);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                yv[i] = step(xv[i], dv[i], (kGate && !kAgg) ? zv[i] : 0.0f, bcb + (t + i) * (2 * N));
            if (!kAgg) store8(yr + t, yv);
        }
    }
    for (; t < t_end; ++t) {
        const float zv = (kGate && !kAgg) ? to_f32(zr[t]) : 0.0f;
        const float r = step(to_f32(xr[t]), to_f32(dr[t]), zv, bcb + t * (2 * N));
        if (!kAgg) yr[t] = r;
    }

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
                                    int64_t L, hipStream_t s) {
    dim3 grid(unsigned((L + 63) / 64), unsigned(B));
    hipLaunchKernelGGL((bc_stage_kernel<Tin, N>), grid, dim3(256), 0, s,
                       static_cast<const Tin*>(Bm), static_cast<const Tin*>(Cm), BC, L);
    return hipGetLastError();
}

template <typename Tin, int N>
static hipError_t launch_scan_t(const ScanLaunch& p, hipStream_t s) {
    const int wg = p.D >= 256 ? 256 : int((p.D + 63) / 64) * 64;
    dim3 grid(unsigned((p.D + wg - 1) / wg), unsigned(p.K), unsigned(p.B));
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
#define SS_SCAN_ARGS x, dr, z, p.dt_bias, p.A, p.Dskip, p.BC, p.h_init, p.y, p.h_last, p.dsum, \
                     p.L, p.D, p.chunk, p.K, p.vec
    if (p.agg)
        hipLaunchKernelGGL((scan_kernel<Tin, N, false, true>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
    else if (p.z)
        hipLaunchKernelGGL((scan_kernel<Tin, N, true, false>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
    else
        hipLaunchKernelGGL((scan_kernel<Tin, N, false, false>), grid, dim3(wg), 0, s, SS_SCAN_ARGS);
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
                           int64_t L, hipStream_t s) {
    if (bf16) { SS_DISPATCH_N(launch_bc_stage_t, bf16_t, Bm, Cm, BC, B, L, s) }
    SS_DISPATCH_N(launch_bc_stage_t, float, Bm, Cm, BC, B, L, s)
}

hipError_t launch_scan(int bf16, int N, const ScanLaunch& p, hipStream_t s) {
    if (bf16) { SS_DISPATCH_N(launch_scan_t, bf16_t, p, s) }
    SS_DISPATCH_N(launch_scan_t, float, p, s)
}

}  // namespace ss
