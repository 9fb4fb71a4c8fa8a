// Backward selective-scan kernels for gfx950, recomputing states instead of storing them.
//
// Page "3.3 재계산(Recomputation) 전략" of "3.2 선택적 스캔(Selective Scan) 알고리즘과
// 정보의 압축 및 선별": the backward needs the forward states, which the fused forward
// never writes out, so they are recomputed from the inputs on chip.  The gradients
// are the exact adjoint of the recurrence of §2.1/§2.2 with the §1.1 readout, the D
// skip term and the SiLU gate; with g = ∂/∂h_t swept from t = L-1 to 0:
//   ds = dy·z·σ(z) (dy without gate); dz = dy·s·σ(z)(1 + z(1 - σ(z)))
//   g += ds·C_t;  dC_t += ds·h_t;  dB_t += g·δ·x;  dx = ds·D + δ Σ_n g B_t
//   dδ = Σ_n g (A Ā h_{t-1}) + x Σ_n g B_t;  dA += g δ Ā h_{t-1};  ddt_raw = dδ σ(u)
//   g ← Ā_t g  (after t = 0 this is dh0)
//
// Plan (sequence split into chunks of 16..64 steps, quad layout as the forward: the
// N states of a channel on four lanes, 16 channels per wave):
//   1. bwd_agg_kernel: per chunk, the forward pair (Π Ā, local state from zero) and the
//      reverse pair (Π Ā, Σ_t (Π_{s<=t} Ā_s) ds_t C_t), both from one forward sweep (the
//      cumulative product only shrinks, so no division ever appears);
//   2. the carry kernel scans the forward pairs (chunk start states, from h0) and the
//      reverse pairs from the last chunk down (the adjoint entering each chunk from the
//      right, from dh_final; its final value is dh0);
//   3. bwd_chunk_kernel: per chunk, one forward sweep keeps the state at each 16-step
//      tile start in LDS, then tile by tile from the last: recompute the tile's 16
//      states, sweep the adjoint backwards through them, reduce the Σ_n terms over the
//      quad through LDS, and reduce the dB/dC terms over the wave's 16 channels by an
//      LDS transpose into per-wave partials;
//   4. reduce kernels sum the partials into dB, dC, dA, dD, ddt_bias.
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_plan.h"

namespace ss {

namespace {

constexpr int kBT = 16;          // steps per tile
constexpr int kBPer = 4;         // steps prepared per lane per tile
constexpr int kBMaxTiles = 4;    // chunk <= 64 steps
constexpr int kBThreads = 256;   // 4 waves x 16 quads = 64 channels
constexpr int kBChan = 64;

template <int K>
__device__ __forceinline__ float qbc(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), K * 0x55, 0xf, 0xf, false));
}
__device__ __forceinline__ float qsum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));
    return v;
}

// 4 consecutive elements [t, t+4) of a row, zero past t_end; vector load when full and aligned
__device__ __forceinline__ void load4(const float* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                      float (&o)[4]) {
    if (vec && t + 4 <= t_end) {
        const float4 v = *reinterpret_cast<const float4*>(p + t);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (t + i < t_end) ? p[t + i] : 0.0f;
    }
}
__device__ __forceinline__ void load4(const bf16_t* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                      float (&o)[4]) {
    if (vec && t + 4 <= t_end) {
        const uint2 v = *reinterpret_cast<const uint2*>(p + t);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (t + i < t_end) ? to_f32(p[t + i]) : 0.0f;
    }
}
__device__ __forceinline__ void store4(float* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                       const float (&v)[4]) {
    if (vec && t + 4 <= t_end) {
        *reinterpret_cast<float4*>(p + t) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (t + i < t_end) p[t + i] = v[i];
    }
}

// Stage the B/C rows of steps [t0, t0 + n) from the [B, L, 2N] staging copy into LDS.
__device__ __forceinline__ void stage_bc(float* __restrict__ lds, const float* __restrict__ src,
                                         int nfloats, int tid) {
    // float4 copies only when the source rows are 16-byte aligned (not so for N = 1, odd L)
    const int nv = (reinterpret_cast<uintptr_t>(src) & 15u) ? 0 : nfloats / 4;
    for (int e = tid; e < nv; e += kBThreads)
        reinterpret_cast<float4*>(lds)[e] = reinterpret_cast<const float4*>(src)[e];
    for (int e = nv * 4 + tid; e < nfloats; e += kBThreads) lds[e] = src[e];
}

}  // namespace

// ---------------------------------------------------------------------------------------
// 1. chunk aggregates.  grid (ceil(D/64), K, B), 256 threads.
// ---------------------------------------------------------------------------------------
template <typename Tin, int S, bool kGate>
__global__ __launch_bounds__(kBThreads) void bwd_agg_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dy, const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ BC, float* __restrict__ h_end, float* __restrict__ rev_end,
    float* __restrict__ dsum_out, int64_t L, int64_t D, int Nr, int64_t chunk, int K, int vec) {
    constexpr int SQ = 4 * S;
    __shared__ __align__(16) float bc_lds[kBMaxTiles * kBT * 2 * SQ];
    const int tid = threadIdx.x;
    const int j = tid & 3;
    const int64_t d_raw = int64_t(blockIdx.x) * kBChan + (tid >> 2);
    const bool valid = d_raw < D;
    const int64_t d = valid ? d_raw : D - 1;
    const int k = blockIdx.y, b = blockIdx.z;
    const int64_t t0c = int64_t(k) * chunk;
    const int64_t t1c = (t0c + chunk < L) ? t0c + chunk : L;
    const int nsteps = int(t1c - t0c);
    const int R = 2 * Nr;
    stage_bc(bc_lds, BC + (int64_t(b) * L + t0c) * R, nsteps * R, tid);

    float A2[S], h[S], P[S], Rv[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = j * S + s;
        A2[s] = (n < Nr) ? A[d * Nr + n] * kLog2e : 0.0f;
        h[s] = 0.0f; P[s] = 1.0f; Rv[s] = 0.0f;
    }
    const float bias = dt_bias[d];
    const int64_t row = (int64_t(b) * D + d) * L;
    float dsum = 0.0f;
    __syncthreads();

    for (int t0 = 0; t0 < nsteps; t0 += kBT) {
        const int64_t te = t0c + t0 + kBPer * j;
        float xv[4], dv[4], zv[4], gv[4];
        load4(x + row, te, t1c, vec, xv);
        load4(dt_raw + row, te, t1c, vec, dv);
        load4(dy + row, te, t1c, vec, gv);
        if (kGate) load4(z + row, te, t1c, vec, zv);
        else zv[0] = zv[1] = zv[2] = zv[3] = 0.0f;
        float dl[4], dx[4], ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = te + i < t1c;
            dl[i] = ok ? softplus(bias + dv[i]) : 0.0f;
            dx[i] = dl[i] * xv[i];
            ds[i] = kGate ? gv[i] * silu(zv[i]) : gv[i];
            dsum += dl[i];
        }
        const int nt = (nsteps - t0 < kBT) ? nsteps - t0 : kBT;
#define SS_AGG_STEP(KK)                                                              \
        _Pragma("unroll") for (int i = 0; i < kBPer; ++i) {                          \
            const int tl = KK * kBPer + i;                                           \
            const float db = qbc<KK>(dl[i]);                                         \
            const float xb = qbc<KK>(dx[i]);                                         \
            const float sb = qbc<KK>(ds[i]);                                         \
            if (tl < nt) {                                                           \
                const float* bt = bc_lds + (t0 + tl) * R;                            \
                _Pragma("unroll") for (int s = 0; s < S; ++s) {                      \
                    const int n = j * S + s;                                         \
                    const float Bn = (S > 1 || n < Nr) ? bt[n] : 0.0f;               \
                    const float Cn = (S > 1 || n < Nr) ? bt[Nr + n] : 0.0f;          \
                    const float a = exp2_hw(db * A2[s]);                             \
                    h[s] = fmaf(a, h[s], xb * Bn);                                   \
                    P[s] *= a;                                                       \
                    Rv[s] = fmaf(P[s], sb * Cn, Rv[s]);                              \
                }                                                                    \
            }                                                                        \
        }
        SS_AGG_STEP(0)
        SS_AGG_STEP(1)
        SS_AGG_STEP(2)
        SS_AGG_STEP(3)
#undef SS_AGG_STEP
    }
    dsum = qsum(dsum);
    if (valid) {
        const int64_t aidx = (int64_t(b) * D + d) * K + k;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int n = j * S + s;
            if (n < Nr) {
                h_end[aidx * Nr + n] = h[s];
                rev_end[aidx * Nr + n] = Rv[s];
            }
        }
        if (j == 0) dsum_out[aidx] = dsum;
    }
}

// ---------------------------------------------------------------------------------------
// 3. final pass.  grid (ceil(D/64), K, B), 256 threads.
//   h_start [B,D,K,N]: state entering each chunk; overwritten with dA partials.
//   q       [B,D,K,N]: adjoint entering each chunk from the right.
//   dbc_part [B, NB, L, 2N] (NB = ceil(D/64)): per-block sums over 64 channels of dB | dC.
//   ddt_part [B, D, K, 2]: per-chunk dD and ddt_bias partials.
// ---------------------------------------------------------------------------------------
template <typename Tin, int S, bool kGate>
__global__ __launch_bounds__(kBThreads) void bwd_chunk_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dy, const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ BC, float* h_start,
    const float* __restrict__ q, float* __restrict__ dxo, float* __restrict__ ddto,
    float* __restrict__ dzo, float* __restrict__ dbc_part, float* __restrict__ ddt_part,
    int64_t L, int64_t D, int Nr, int64_t chunk, int K, int vec) {
    constexpr int SQ = 4 * S;
    __shared__ __align__(16) float bc_lds[kBMaxTiles * kBT * 2 * SQ];
    // per-wave scratch, LS floats per lane (quad reduce-scatter, then dB/dC transpose);
    // LS = 4 mod 32 keeps the 16-byte writes of 8 consecutive lanes on disjoint banks
    constexpr int LS = ((8 * S > 32) ? 8 * S : 32) + 4;
    __shared__ __align__(16) float scr[kBThreads * LS];
    __shared__ float comb[4 * 8 * SQ];   // wave totals of one 4-step batch
    // state at each 16-step tile start, [tile][s][thread]
    __shared__ float ck_lds[kBMaxTiles * S * kBThreads];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = tid & 3;
    const int64_t d_raw = int64_t(blockIdx.x) * kBChan + (tid >> 2);
    const bool valid = d_raw < D;
    const int64_t d = valid ? d_raw : D - 1;
    const int k = blockIdx.y, b = blockIdx.z;
    const int64_t t0c = int64_t(k) * chunk;
    const int64_t t1c = (t0c + chunk < L) ? t0c + chunk : L;
    const int nsteps = int(t1c - t0c);
    const int ntiles = (nsteps + kBT - 1) / kBT;
    const int R = 2 * Nr;
    stage_bc(bc_lds, BC + (int64_t(b) * L + t0c) * R, nsteps * R, tid);
    float* wscr = scr + wave * 64 * LS;
    const int64_t NB = (D + kBChan - 1) / kBChan;        // channel blocks

    const int64_t sidx = ((int64_t(b) * D + d) * K + k) * Nr;
    float A2[S], An[S], h[S], g[S], dA[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = j * S + s;
        const bool ok = n < Nr;
        An[s] = ok ? A[d * Nr + n] : 0.0f;
        A2[s] = An[s] * kLog2e;
        h[s] = ok ? h_start[sidx + n] : 0.0f;
        g[s] = ok ? q[sidx + n] : 0.0f;
        dA[s] = 0.0f;
    }
    const float bias = dt_bias[d];
    const float Dd = Dskip[d];
    const int64_t row = (int64_t(b) * D + d) * L;
    float accD = 0.0f, accT = 0.0f;
    __syncthreads();

    auto BCn = [&](const float* bt, int s, float& Bn, float& Cn) {
        const int n = j * S + s;
        const bool ok = (S > 1) || n < Nr;
        Bn = ok ? bt[n] : 0.0f;
        Cn = ok ? bt[Nr + n] : 0.0f;
    };

    // ---- forward sweep: state at every tile start ----
    auto CK = [&](int tile, int s) -> float& { return ck_lds[(tile * S + s) * kBThreads + tid]; };
    for (int tile = 0; tile < ntiles; ++tile) {
#pragma unroll
        for (int s = 0; s < S; ++s) CK(tile, s) = h[s];
        if (tile == ntiles - 1) break;     // the last tile's end state is not needed
        const int t0 = tile * kBT;
        const int64_t te = t0c + t0 + kBPer * j;
        float xv[4], dv[4];
        load4(x + row, te, t1c, vec, xv);
        load4(dt_raw + row, te, t1c, vec, dv);
        float dl[4], dx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dl[i] = softplus(bias + dv[i]);
            dx[i] = dl[i] * xv[i];
        }
#define SS_FW_STEP(KK)                                                                \
        _Pragma("unroll") for (int i = 0; i < kBPer; ++i) {                           \
            const float db = qbc<KK>(dl[i]);                                          \
            const float xb = qbc<KK>(dx[i]);                                          \
            const float* bt = bc_lds + (t0 + KK * kBPer + i) * R;                     \
            _Pragma("unroll") for (int s = 0; s < S; ++s) {                           \
                float Bn, Cn;                                                         \
                BCn(bt, s, Bn, Cn);                                                   \
                h[s] = fmaf(exp2_hw(db * A2[s]), h[s], xb * Bn);                      \
            }                                                                         \
        }
        SS_FW_STEP(0)
        SS_FW_STEP(1)
        SS_FW_STEP(2)
        SS_FW_STEP(3)
#undef SS_FW_STEP
    }

    // ---- tiles from the last to the first ----
    for (int tile = ntiles - 1; tile >= 0; --tile) {
        const int t0 = tile * kBT;
        const int nt = (nsteps - t0 < kBT) ? nsteps - t0 : kBT;
        const int64_t te = t0c + t0 + kBPer * j;
        float xv[4], dv[4], zv[4], gv[4];
        load4(x + row, te, t1c, vec, xv);
        load4(dt_raw + row, te, t1c, vec, dv);
        load4(dy + row, te, t1c, vec, gv);
        if (kGate) load4(z + row, te, t1c, vec, zv);
        float dl[4], dx[4], ds[4], su[4], sz[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = te + i < t1c;
            const float u = bias + dv[i];
            dl[i] = ok ? softplus(u) : 0.0f;
            su[i] = sigmoid(u);
            dx[i] = dl[i] * xv[i];
            if (kGate) {
                sz[i] = sigmoid(zv[i]);
                ds[i] = ok ? gv[i] * zv[i] * sz[i] : 0.0f;
            } else {
                ds[i] = ok ? gv[i] : 0.0f;
            }
            if (!valid) { ds[i] = 0.0f; dx[i] = 0.0f; }
        }

        // recompute the tile's states (and the readout for dz)
        float hs[kBT][S];
        float sp[kBT];
        float hc[S];
#pragma unroll
        for (int s = 0; s < S; ++s) { hc[s] = CK(tile, s); h[s] = hc[s]; }
#define SS_RC_STEP(KK)                                                                \
        _Pragma("unroll") for (int i = 0; i < kBPer; ++i) {                           \
            const int tl = KK * kBPer + i;                                            \
            const float db = qbc<KK>(dl[i]);                                          \
            const float xb = qbc<KK>(dx[i]);                                          \
            const float* bt = bc_lds + (t0 + tl) * R;                                 \
            float acc = 0.0f;                                                         \
            _Pragma("unroll") for (int s = 0; s < S; ++s) {                           \
                float Bn, Cn;                                                         \
                BCn(bt, s, Bn, Cn);                                                   \
                h[s] = fmaf(exp2_hw(db * A2[s]), h[s], xb * Bn);                      \
                hs[tl][s] = h[s];                                                     \
                if (kGate) acc = fmaf(Cn, h[s], acc);                                 \
            }                                                                         \
            sp[tl] = acc;                                                             \
        }
        SS_RC_STEP(0)
        SS_RC_STEP(1)
        SS_RC_STEP(2)
        SS_RC_STEP(3)
#undef SS_RC_STEP

        float dzv[4];
        if (kGate) {
            // readout partials -> owner lanes (steps 4j..4j+3 of lane j)
            float* mine = wscr + lane * LS;
#pragma unroll
            for (int q4 = 0; q4 < kBT; q4 += 4)
                *reinterpret_cast<float4*>(mine + q4) = make_float4(sp[q4], sp[q4 + 1], sp[q4 + 2], sp[q4 + 3]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float stot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            const int qb = lane & ~3;
#pragma unroll
            for (int src = 0; src < 4; ++src) {
                const float4 v = *reinterpret_cast<const float4*>(wscr + (qb + src) * LS + kBPer * j);
                stot[0] += v.x; stot[1] += v.y; stot[2] += v.z; stot[3] += v.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sv = fmaf(Dd, xv[i], stot[i]);
                dzv[i] = gv[i] * sv * sz[i] * fmaf(zv[i], 1.0f - sz[i], 1.0f);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }

        // reverse sweep over the tile, in batches of 4 steps (one prepared block each)
        float pdx[kBT], pdd[kBT];
    #define SS_RV_BATCH(KK)                                                                    \
        {                                                                                  \
            float cB[kBPer][S], cC[kBPer][S];                                              \
            _Pragma("unroll") for (int i = kBPer - 1; i >= 0; --i) {                       \
                const int tl = KK * kBPer + i;                                             \
                const float db = qbc<KK>(ds[i]);                                           \
                const float lb = qbc<KK>(dl[i]);                                           \
                const float xb = qbc<KK>(dx[i]);                                           \
                float px = 0.0f, pd = 0.0f;                                                \
                if (tl < nt) {                                                             \
                    const float* bt = bc_lds + (t0 + tl) * R;                              \
                    _Pragma("unroll") for (int s = 0; s < S; ++s) {                        \
                        float Bn, Cn;                                                      \
                        BCn(bt, s, Bn, Cn);                                                \
                        const float hp = (tl > 0) ? hs[tl > 0 ? tl - 1 : 0][s] : hc[s];  \
                        g[s] = fmaf(db, Cn, g[s]);                                         \
                        cC[i][s] = db * hs[tl][s];                                         \
                        cB[i][s] = g[s] * xb;                                              \
                        px = fmaf(g[s], Bn, px);                                           \
                        const float a = exp2_hw(lb * A2[s]);                               \
                        const float wa = g[s] * (a * hp);                                  \
                        dA[s] = fmaf(wa, lb, dA[s]);                                       \
                        pd = fmaf(wa, An[s], pd);                                          \
                        g[s] *= a;                                                         \
                    }                                                                      \
                } else {                                                                   \
                    _Pragma("unroll") for (int s = 0; s < S; ++s) { cB[i][s] = 0.0f; cC[i][s] = 0.0f; } \
                }                                                                          \
                pdx[tl] = px;                                                              \
                pdd[tl] = pd;                                                              \
            }                                                                              \
            /* dB | dC over the block's 64 channels: each wave transposes its 16 channels  \
               through its LDS area (per lane [type][step][state], lane stride LS), the    \
               wave totals meet in `comb`, and one block partial per (b, t, n) is written  \
               (fixed order: deterministic).                                              */ \
            float* mine = wscr + lane * LS;                                                \
            _Pragma("unroll") for (int i = 0; i < kBPer; ++i) {                            \
                _Pragma("unroll") for (int s = 0; s < S; ++s) {                            \
                    mine[i * S + s] = cB[i][s];                                            \
                    mine[4 * S + i * S + s] = cC[i][s];                                    \
                }                                                                          \
            }                                                                              \
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");                         \
            __builtin_amdgcn_wave_barrier();                                               \
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");                         \
            /* e = lane + 64r -> (state sp_, lane group jp, type ty, step st): each       \
               32-lane half reads 32 distinct banks (LS = 4 mod 32)                       */ \
            _Pragma("unroll") for (int r = 0; r < (8 * SQ + 63) / 64; ++r) {               \
                const int e = lane + 64 * r;                                               \
                if (e < 8 * SQ) {                                                          \
                    const int sp_ = e % S;                                                 \
                    const int jp = (e / S) % 4;                                            \
                    const int ty = (e / (4 * S)) % 2;                                      \
                    const int st = e / (8 * S);                                            \
                    const float* col = wscr + jp * LS + ty * 4 * S + st * S + sp_;         \
                    float tot = 0.0f;                                                      \
                    _Pragma("unroll") for (int c = 0; c < 16; ++c) tot += col[c * 4 * LS]; \
                    comb[wave * 8 * SQ + e] = tot;                                         \
                }                                                                          \
            }                                                                              \
            __syncthreads();                                                               \
            for (int e = tid; e < 8 * SQ; e += kBThreads) {                                \
                const int sp_ = e % S;                                                     \
                const int jp = (e / S) % 4;                                                \
                const int ty = (e / (4 * S)) % 2;                                          \
                const int st = e / (8 * S);                                                \
                const int n = jp * S + sp_;                                                \
                const float tot = (comb[e] + comb[8 * SQ + e]) +                           \
                                  (comb[16 * SQ + e] + comb[24 * SQ + e]);                 \
                const int64_t t = t0c + t0 + KK * kBPer + st;                              \
                if (n < Nr && t < t1c)                                                     \
                    dbc_part[((int64_t(b) * NB + blockIdx.x) * L + t) * R + ty * Nr + n] = tot; \
            }                                                                              \
            __syncthreads();                                                               \
        }
        SS_RV_BATCH(3)
        SS_RV_BATCH(2)
        SS_RV_BATCH(1)
        SS_RV_BATCH(0)
#undef SS_RV_BATCH

        // Σ_n partials -> owner lanes; per-element gradients
        {
            float* mine = wscr + lane * LS;
#pragma unroll
            for (int q4 = 0; q4 < kBT; q4 += 4) {
                *reinterpret_cast<float4*>(mine + q4) = make_float4(pdx[q4], pdx[q4 + 1], pdx[q4 + 2], pdx[q4 + 3]);
                *reinterpret_cast<float4*>(mine + 16 + q4) = make_float4(pdd[q4], pdd[q4 + 1], pdd[q4 + 2], pdd[q4 + 3]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float PX[4] = {0.0f, 0.0f, 0.0f, 0.0f}, PD[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            const int qb = lane & ~3;
#pragma unroll
            for (int src = 0; src < 4; ++src) {
                const float4 a = *reinterpret_cast<const float4*>(wscr + (qb + src) * LS + kBPer * j);
                const float4 c = *reinterpret_cast<const float4*>(wscr + (qb + src) * LS + 16 + kBPer * j);
                PX[0] += a.x; PX[1] += a.y; PX[2] += a.z; PX[3] += a.w;
                PD[0] += c.x; PD[1] += c.y; PD[2] += c.z; PD[3] += c.w;
            }
            float ox[4], od[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ox[i] = fmaf(ds[i], Dd, dl[i] * PX[i]);
                const float ddel = fmaf(xv[i], PX[i], PD[i]);
                od[i] = ddel * su[i];
                const bool ok = te + i < t1c;
                accD += ok ? ds[i] * xv[i] : 0.0f;
                accT += ok ? od[i] : 0.0f;
            }
            if (valid) {
                store4(dxo + row, te, t1c, vec, ox);
                store4(ddto + row, te, t1c, vec, od);
                if (kGate) store4(dzo + row, te, t1c, vec, dzv);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

    accD = qsum(accD);
    accT = qsum(accT);
    if (valid) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int n = j * S + s;
            if (n < Nr) h_start[sidx + n] = dA[s];   // dA partial of this (b, chunk, d)
        }
        if (j == 0) {
            const int64_t pidx = ((int64_t(b) * D + d) * K + k) * 2;
            ddt_part[pidx] = accD;
            ddt_part[pidx + 1] = accT;
        }
    }
}

// ---------------------------------------------------------------------------------------
// 4. reductions
// ---------------------------------------------------------------------------------------
// dB | dC: part [B, NB, L, 2N] summed over NB -> dB, dC [B, N, L].  One thread per (t, v)
// of a batch row: reads are coalesced across threads, the sum runs over the channel blocks.
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part,
                                                            float* __restrict__ dB,
                                                            float* __restrict__ dC, int64_t L,
                                                            int NB, int Nr) {
    const int R = 2 * Nr;
    const int b = blockIdx.y;
    const int64_t f = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t LR = L * R;
    if (f >= LR) return;
    const float* p = part + int64_t(b) * NB * LR + f;
    float acc = 0.0f;
    for (int gi = 0; gi < NB; ++gi) acc += p[int64_t(gi) * LR];
    const int64_t t = f / R;
    const int v = int(f % R);
    float* out = (v < Nr) ? dB + (int64_t(b) * Nr + v) * L : dC + (int64_t(b) * Nr + v - Nr) * L;
    out[t] = acc;
}

// dA [D, N] = Σ_{b,k} part[b,d,k,n];  dD, ddt_bias [D] = Σ_{b,k} ddt_part[b,d,k,0|1].
// One block per channel d: for each b the K*N (and K*2) partials of (b, d) are
// contiguous, so the block reads them coalesced and folds over k through LDS.
__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(
    const float* __restrict__ dA_part, const float* __restrict__ ddt_part, float* __restrict__ dA,
    float* __restrict__ dD, float* __restrict__ ddt_bias, int64_t D, int Nr, int Bn, int K) {
    __shared__ float red[256];
    const int64_t d = blockIdx.x;
    const int tid = threadIdx.x;
    const int KN = K * Nr;
    // thread tid accumulates entries e = tid + 256 i of the K*N block; Nr divides 256,
    // so every entry a thread touches has state n = tid % Nr
    float acc = 0.0f;
    for (int b = 0; b < Bn; ++b) {
        const float* p = dA_part + (int64_t(b) * D + d) * KN;
        for (int e = tid; e < KN; e += 256) acc += p[e];
    }
    red[tid] = acc;
    __syncthreads();
    if (tid < Nr) {
        float t = 0.0f;
        for (int i = tid; i < 256; i += Nr) t += red[i];
        dA[d * Nr + tid] = t;
    }
    __syncthreads();
    float a0 = 0.0f, a1 = 0.0f;
    for (int b = 0; b < Bn; ++b) {
        const float* q = ddt_part + (int64_t(b) * D + d) * K * 2;
        for (int k = tid; k < K; k += 256) { a0 += q[2 * k]; a1 += q[2 * k + 1]; }
    }
    red[tid] = a0;
    __syncthreads();
    if (tid == 0) {
        float t = 0.0f;
        for (int i = 0; i < 256; ++i) t += red[i];
        dD[d] = t;
    }
    __syncthreads();
    red[tid] = a1;
    __syncthreads();
    if (tid == 0) {
        float t = 0.0f;
        for (int i = 0; i < 256; ++i) t += red[i];
        ddt_bias[d] = t;
    }
}

// ---------------------------------------------------------------------------------------
// plan helpers and launchers
// ---------------------------------------------------------------------------------------
int64_t bwd_reduce_blocks(const Plan& p) { return (p.D + kBChan - 1) / kBChan; }

size_t bwd_partial_bytes(const Plan& p) {
    // dB|dC per-block partials + dD/ddt_bias per-chunk partials
    const size_t bc = size_t(p.B) * size_t(bwd_reduce_blocks(p)) * size_t(p.L) * size_t(2 * p.N) * 4;
    const size_t dt = size_t(p.B) * size_t(p.K) * size_t(p.D) * 2 * 4;
    return align256(bc) + dt;
}

template <typename Tin, int S>
static hipError_t launch_bwd_t(const BwdLaunch& p, hipStream_t s) {
    dim3 grid(unsigned((p.D + kBChan - 1) / kBChan), unsigned(p.K), unsigned(p.B));
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
    if (p.stage == 0) {
        if (z)
            hipLaunchKernelGGL((bwd_agg_kernel<Tin, S, true>), grid, dim3(kBThreads), 0, s, x, dr, z,
                               p.dy, p.dt_bias, p.A, p.BC, p.h_end, p.rev_end, p.dsum, p.L, p.D,
                               int(p.N), p.chunk, p.K, p.vec);
        else
            hipLaunchKernelGGL((bwd_agg_kernel<Tin, S, false>), grid, dim3(kBThreads), 0, s, x, dr, z,
                               p.dy, p.dt_bias, p.A, p.BC, p.h_end, p.rev_end, p.dsum, p.L, p.D,
                               int(p.N), p.chunk, p.K, p.vec);
    } else {
        if (z)
            hipLaunchKernelGGL((bwd_chunk_kernel<Tin, S, true>), grid, dim3(kBThreads), 0, s, x, dr, z,
                               p.dy, p.dt_bias, p.A, p.Dskip, p.BC, p.h_end, p.rev_end, p.dx,
                               p.ddt_raw, p.dz, p.dbc_part, p.ddt_part, p.L, p.D, int(p.N), p.chunk,
                               p.K, p.vec);
        else
            hipLaunchKernelGGL((bwd_chunk_kernel<Tin, S, false>), grid, dim3(kBThreads), 0, s, x, dr, z,
                               p.dy, p.dt_bias, p.A, p.Dskip, p.BC, p.h_end, p.rev_end, p.dx,
                               p.ddt_raw, p.dz, p.dbc_part, p.ddt_part, p.L, p.D, int(p.N), p.chunk,
                               p.K, p.vec);
    }
    return hipGetLastError();
}

hipError_t launch_bwd(int bf16, const BwdLaunch& p, hipStream_t s) {
    const int S = p.N <= 4 ? 1 : int(p.N / 4);
    if (bf16) {
        switch (S) {
            case 1: return launch_bwd_t<bf16_t, 1>(p, s);
            case 2: return launch_bwd_t<bf16_t, 2>(p, s);
            case 4: return launch_bwd_t<bf16_t, 4>(p, s);
            case 8: return launch_bwd_t<bf16_t, 8>(p, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (S) {
        case 1: return launch_bwd_t<float, 1>(p, s);
        case 2: return launch_bwd_t<float, 2>(p, s);
        case 4: return launch_bwd_t<float, 4>(p, s);
        case 8: return launch_bwd_t<float, 8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_reduce(const BwdLaunch& p, hipStream_t s) {
    const int NB = int((p.D + kBChan - 1) / kBChan);
    const int64_t LR = p.L * 2 * p.N;
    hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(unsigned((LR + 255) / 256), unsigned(p.B)), dim3(256),
                       0, s, p.dbc_part, p.dB, p.dC, p.L, NB, int(p.N));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3(unsigned(p.D)), dim3(256), 0, s, p.h_end,
                       p.ddt_part, p.dA, p.dD, p.ddt_bias, p.D, int(p.N), int(p.B), p.K);
    return hipGetLastError();
}

}  // namespace ss

