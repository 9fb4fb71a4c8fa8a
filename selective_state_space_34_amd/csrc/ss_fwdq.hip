// Quad-split forward selective-scan kernel for gfx950.
//
// Same computation as scan_kernel (page "3.2 선택적 스캔(Selective Scan) 알고리즘과
// 정보의 압축 및 선별": §1.2 softplus step, §2.1 exp discretisation of diagonal A,
// §2.2 recurrence, §1.1 readout; SiLU gate of the note "상태공간 모델(SSM)과 Mamba
// 아키텍처", §3), laid out for CDNA4 occupancy: the N states of a channel are split
// over a quad of four adjacent lanes (S = N/4 states per lane), so a 64-lane wave
// covers 16 channels and a batch of B*D channels yields B*D/16 waves.
//
// Per 32-step tile:
//   - lane j of a quad loads and prepares steps [8j, 8j+8) of its channel: widening,
//     δ = softplus(dt_bias + dt_raw), δ·x.  No element is prepared twice.
//   - the workgroup copies the tile's B and C ([B, N, L] inputs, N rows of 32 steps
//     each) into LDS transposed to [step][B row | C row] as float32.
//   - the recurrence walks the 32 steps; step t's δ and δ·x come from lane t/8 of
//     the quad through a DPP quad_perm broadcast; B_t, C_t for the lane's S states
//     come from the LDS tile (one 16-byte broadcast read each).
//   - each lane's partial readouts (its S states) go to a per-wave LDS area; lane j
//     sums the four partials of its own 8 steps, adds D·x, applies the gate and
//     stores 8 outputs.
// All global loads of the next tile (x, dt_raw, z, and the B/C tile) are issued
// before the current tile's arithmetic.  The state never leaves VGPRs (§3.2).
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

namespace {

constexpr int kTile = 32;      // steps per tile
constexpr int kPer = 8;        // steps prepared per lane (kTile / 4)
// lane stride (floats) of the partial-readout area: 36 = 4 mod 32 puts the 16-byte
// writes of 8 consecutive lanes on 8 disjoint groups of 4 banks
constexpr int kPS = kTile + 4;
constexpr int kChanPerBlock = 64;
constexpr int kThreads = 256;  // 4 waves x 16 quads

template <int K>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), K * 0x55, 0xf, 0xf, false));
}
// quad all-reduce (sum over the 4 lanes of a quad)
__device__ __forceinline__ float quad_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));  // [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));  // [2,3,0,1]
    return v;
}

// B or C values of the lane's S states at one step (LDS -> VGPR)
template <int S>
struct Row {
    float v[S];
    __device__ __forceinline__ void load(const float* p) {
        if constexpr (S % 4 == 0) {
#pragma unroll
            for (int q = 0; q < S; q += 4) {
                const float4 a = *reinterpret_cast<const float4*>(p + q);
                v[q] = a.x; v[q + 1] = a.y; v[q + 2] = a.z; v[q + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < S; ++q) v[q] = p[q];
        }
    }
};

// raw (undecoded) storage of 8 input elements
template <typename Tin> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void decode(float (&o)[8]) const {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
// raw storage of 4 consecutive input elements (one B or C row segment)
template <typename Tin> struct Raw4;
template <> struct Raw4<bf16_t> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t w = (i < 2) ? v.x : v.y;
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct Raw4<float> {
    float4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ float get(int i) const {
        return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
    }
};

template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void decode(float (&o)[8]) const {
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

}  // namespace

// grid = (ceil(D / 64), K, B), block = 256.  Requires L % 8 == 0 and chunk % 32 == 0
// (or K == 1) for the tiled part; the last < 32 steps of a chunk run a per-step tail.
template <typename Tin, int S, bool kGate, bool kAgg>
__global__ __launch_bounds__(kThreads) void scanq_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const Tin* __restrict__ Bm, const Tin* __restrict__ Cm,
    const float* __restrict__ h_init, float* __restrict__ y, float* __restrict__ h_last,
    float* __restrict__ dsum_out, int64_t L, int64_t D, int64_t chunk, int K) {
    constexpr int N = 4 * S;
    // LDS tile row per step: B_t (N floats) then C_t (N floats), padded by 4 floats so
    // the transposing writes of a wave fall on at most two lanes per bank
    constexpr int R = 2 * N + 4;
    constexpr int TILE_F = kTile * R;             // floats per B/C tile
    __shared__ __align__(16) float bc_lds[2][TILE_F];
    __shared__ __align__(16) float part_lds[kAgg ? 1 : kThreads * kPS];

    const int tid = threadIdx.x;
    const int j = tid & 3;                        // state group / step block within the quad
    const int64_t d_raw = int64_t(blockIdx.x) * kChanPerBlock + (tid >> 2);
    const bool valid = d_raw < D;
    const int64_t d = valid ? d_raw : D - 1;      // clamped for loads
    const int k = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = int64_t(k) * chunk;
    const int64_t t_end = (t_begin + chunk < L) ? t_begin + chunk : L;
    const int64_t n_tiles = (t_end - t_begin) / kTile;
    const int64_t t_tiles_end = t_begin + n_tiles * kTile;
    const int n0 = j * S;

    float A2[S], h[S];
#pragma unroll
    for (int s = 0; s < S; ++s) A2[s] = A[d * N + n0 + s] * kLog2e;
    const int64_t hidx = ((int64_t(b) * D + d) * K + k) * N + n0;
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] = h_init ? h_init[hidx + s] : 0.0f;
    const float bias = dt_bias[d];
    const float Dd = kAgg ? 0.0f : Dskip[d];
    const int64_t row = (int64_t(b) * D + d) * L;
    const Tin* xr = x + row;
    const Tin* dr = dt_raw + row;
    const Tin* zr = kGate ? z + row : nullptr;
    float* yr = kAgg ? nullptr : y + row;
    const Tin* Bb = Bm + int64_t(b) * N * L;
    const Tin* Cb = Cm + int64_t(b) * N * L;
    float dsum = 0.0f;

    // B/C tile copy: 2·N rows of 32 steps; unit e covers steps 4q..4q+3 of state n of
    // B (m = 0) or C (m = 1), with n fastest across lanes
    constexpr int BC_UNITS = 2 * N * (kTile / 4);
    constexpr int BC_PASSES = (BC_UNITS + kThreads - 1) / kThreads;
    Raw4<Tin> bc_next[BC_PASSES];
    Raw8<Tin> xn, dn, zn;

    auto issue_loads = [&](int64_t t0) {
#pragma unroll
        for (int p = 0; p < BC_PASSES; ++p) {
            const int e = tid + p * kThreads;
            if (BC_UNITS % kThreads == 0 || e < BC_UNITS) {
                const int n = e % N, q = (e / N) % (kTile / 4), m = e / (N * (kTile / 4));
                bc_next[p].load((m ? Cb : Bb) + int64_t(n) * L + t0 + 4 * q);
            }
        }
        const int64_t te = t0 + kPer * j;
        xn.load(xr + te);
        dn.load(dr + te);
        if (kGate && !kAgg) zn.load(zr + te);
    };

    if (n_tiles > 0) issue_loads(t_begin);
    float* my_part = part_lds + (kAgg ? 0 : (tid & ~63) * kPS);  // wave-private area
    const int lane = tid & 63;

    for (int64_t it = 0; it < n_tiles; ++it) {
        const int64_t t0 = t_begin + it * kTile;
        float* buf = bc_lds[it & 1];
#pragma unroll
        for (int p = 0; p < BC_PASSES; ++p) {
            const int e = tid + p * kThreads;
            if (BC_UNITS % kThreads == 0 || e < BC_UNITS) {
                const int n = e % N, q = (e / N) % (kTile / 4), m = e / (N * (kTile / 4));
                float* dst = buf + 4 * q * R + m * N + n;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * R] = bc_next[p].get(i);
            }
        }
        float xv[kPer], dv[kPer], zv[kPer];
        xn.decode(xv);
        dn.decode(dv);
        if (kGate && !kAgg) zn.decode(zv);
        if (it + 1 < n_tiles) issue_loads(t0 + kTile);
        __syncthreads();

        // per-element preparation of this lane's 8 steps
        float dl[kPer], dx[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            dl[i] = softplus(bias + dv[i]);
            dx[i] = dl[i] * xv[i];
            if (kAgg) dsum += dl[i];
        }

        // recurrence over the 32 steps; B/C of step t+1 are read from LDS during step t
        float part[kTile];
        Row<S> bcur, ccur, bnxt, cnxt;
        bnxt.load(buf + n0);
        cnxt.load(buf + N + n0);
#define SS_QSTEP(KK)                                                                        \
        _Pragma("unroll") for (int i = 0; i < kPer; ++i) {                                  \
            const int t = KK * kPer + i;                                                    \
            bcur = bnxt;                                                                    \
            ccur = cnxt;                                                                    \
            if (t + 1 < kTile) {                                                            \
                bnxt.load(buf + (t + 1) * R + n0);                                          \
                cnxt.load(buf + (t + 1) * R + N + n0);                                      \
            }                                                                               \
            __builtin_amdgcn_sched_barrier(0); /* keep the next step's reads issued here */ \
            const float db = quad_bcast<KK>(dl[i]);                                         \
            const float xb = quad_bcast<KK>(dx[i]);                                         \
            float acc = 0.0f;                                                               \
            _Pragma("unroll") for (int s = 0; s < S; ++s) {                                 \
                const float abar = exp2_hw(db * A2[s]);                                     \
                h[s] = fmaf(abar, h[s], xb * bcur.v[s]);                                    \
                if (!kAgg) acc = fmaf(ccur.v[s], h[s], acc);                                \
            }                                                                               \
            part[t] = acc;                                                                  \
        }
        SS_QSTEP(0)
        SS_QSTEP(1)
        SS_QSTEP(2)
        SS_QSTEP(3)
#undef SS_QSTEP

        if (!kAgg) {
            // partial readouts through the wave's LDS area: lane writes its 32, then
            // gathers the four partials of its own 8 steps
            float* mine = my_part + lane * kPS;
#pragma unroll
            for (int q = 0; q < kTile; q += 4)
                *reinterpret_cast<float4*>(mine + q) = make_float4(part[q], part[q + 1], part[q + 2], part[q + 3]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float sum[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) sum[i] = 0.0f;
            const int qbase = lane & ~3;
            // lane j starts at source j (rotation): the 8 lanes served together then read
            // 8 disjoint groups of 4 banks
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int src = (j + r) & 3;
                const float* p = my_part + (qbase + src) * kPS + kPer * j;
                const float4 a = *reinterpret_cast<const float4*>(p);
                const float4 c = *reinterpret_cast<const float4*>(p + 4);
                sum[0] += a.x; sum[1] += a.y; sum[2] += a.z; sum[3] += a.w;
                sum[4] += c.x; sum[5] += c.y; sum[6] += c.z; sum[7] += c.w;
            }
            float out[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                float s = fmaf(Dd, xv[i], sum[i]);
                if (kGate) s *= silu(zv[i]);
                out[i] = s;
            }
            if (valid) store8(yr + t0 + kPer * j, out);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

    // tail: the last (t_end - t_tiles_end) < 32 steps, one step at a time; every lane
    // prepares the step itself and reads its B/C straight from the inputs
    for (int64_t t = t_tiles_end; t < t_end; ++t) {
        const float xt = to_f32(xr[t]);
        const float delta = softplus(bias + to_f32(dr[t]));
        const float dxt = delta * xt;
        if (kAgg) dsum += (j == 0) ? delta : 0.0f;
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const float abar = exp2_hw(delta * A2[s]);
            h[s] = fmaf(abar, h[s], dxt * to_f32(Bb[int64_t(n0 + s) * L + t]));
            if (!kAgg) acc = fmaf(to_f32(Cb[int64_t(n0 + s) * L + t]), h[s], acc);
        }
        if (!kAgg) {
            acc = quad_sum(acc);
            float sv = fmaf(Dd, xt, acc);
            if (kGate) sv *= silu(to_f32(zr[t]));
            if (valid && j == 0) yr[t] = sv;
        }
    }

    if (kAgg) {
        dsum = quad_sum(dsum);
        const int64_t aidx = (int64_t(b) * D + d) * K + k;
        if (valid) {
#pragma unroll
            for (int s = 0; s < S; ++s) h_last[aidx * N + n0 + s] = h[s];
            if (j == 0) dsum_out[aidx] = dsum;
        }
    } else if (h_last && k == K - 1 && valid) {
        const int64_t fidx = (int64_t(b) * D + d) * N + n0;
#pragma unroll
        for (int s = 0; s < S; ++s) h_last[fidx + s] = h[s];
    }
}

template <typename Tin, int S>
static hipError_t launch_scanq_t(const ScanLaunch& p, hipStream_t s) {
    dim3 grid(unsigned((p.D + kChanPerBlock - 1) / kChanPerBlock), unsigned(p.K), unsigned(p.B));
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
    const Tin* Bm = static_cast<const Tin*>(p.Bm);
    const Tin* Cm = static_cast<const Tin*>(p.Cm);
#define SS_ARGS x, dr, z, p.dt_bias, p.A, p.Dskip, Bm, Cm, p.h_init, p.y, p.h_last, p.dsum, p.L, \
                p.D, p.chunk, p.K
    if (p.agg)
        hipLaunchKernelGGL((scanq_kernel<Tin, S, false, true>), grid, dim3(kThreads), 0, s, SS_ARGS);
    else if (p.z)
        hipLaunchKernelGGL((scanq_kernel<Tin, S, true, false>), grid, dim3(kThreads), 0, s, SS_ARGS);
    else
        hipLaunchKernelGGL((scanq_kernel<Tin, S, false, false>), grid, dim3(kThreads), 0, s, SS_ARGS);
#undef SS_ARGS
    return hipGetLastError();
}

hipError_t launch_scanq(int bf16, int N, const ScanLaunch& p, hipStream_t s) {
    if (bf16) {
        switch (N) {
            case 4: return launch_scanq_t<bf16_t, 1>(p, s);
            case 8: return launch_scanq_t<bf16_t, 2>(p, s);
            case 16: return launch_scanq_t<bf16_t, 4>(p, s);
            case 32: return launch_scanq_t<bf16_t, 8>(p, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (N) {
        case 4: return launch_scanq_t<float, 1>(p, s);
        case 8: return launch_scanq_t<float, 2>(p, s);
        case 16: return launch_scanq_t<float, 4>(p, s);
        case 32: return launch_scanq_t<float, 8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ss
