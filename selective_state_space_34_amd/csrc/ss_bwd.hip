// Backward selective-scan kernels for gfx950, recomputing states instead of storing them.
//
// Page "3.3 재계산(Recomputation) 전략" of "3.2 선택적 스캔(Selective Scan) 알고리즘과
// 정보의 압축 및 선별": the backward needs the forward states, which the fused forward
// never writes out, so they are recomputed from the inputs on chip.  The gradients
// are the exact adjoint of the recurrence of §2.1/§2.2 with the §1.1 readout, the D
// skip term and the SiLU gate; with g = ∂/∂h_t swept from t = L-1 to 0:
//   ds = dy·z·σ(z) (dy without gate); dz = dy·s·σ(z)(1 + z(1 - σ(z)))
//   g += ds·C_t;  dC_t += ds·h_t;  dB_t += g·δ·x;  dx = ds·D + δ Σ_n g B_t
//   g ← Ā_t g;  w = g·h_{t-1};  dA += δ w;  dδ = Σ_n A w + x Σ_n g B_t (g before ← Ā_t g)
//   ddt_raw = dδ σ(u)   (after t = 0, g is dh0)
// With the exact zero-order hold of §2.1 (kZoh) the input term is f·B_t·x with the per-state
// gain f = (e^{δA} - 1)/A, whose partials are ∂f/∂δ = Ā and ∂f/∂A = (δĀ - f)/A:
//   dB_t += g·f·x;  dx = ds·D + Σ_n g f B_t;  dδ = Σ_n A w + x Σ_n (Ā g) B_t;
//   dA += δ w + (∂f/∂A)·g·B_t·x   (g before ← Ā_t g, w after)
//
// Plan (sequence split into chunks of 16..64 steps; the N states of a channel on four
// lanes, 16 channels per wave, 64 per workgroup):
//   1. bwd_agg_kernel: per chunk, the reverse pair (Π Ā, Σ_t (Π_{s<=t} Ā_s) ds_t C_t) and,
//      without checkpoints, the forward pair (Π Ā, local state from zero), from one
//      forward sweep (the cumulative product only shrinks: no division ever appears);
//   2. the carry kernel scans the reverse pairs from the last chunk down (the adjoint
//      entering each chunk from the right, from dh_final; its final value is dh0) and,
//      without checkpoints, the forward pairs (chunk start states, from h0);
//   3. bwd_chunk_kernel: per chunk, the state at each 16-step tile start comes from the
//      forward's checkpoints or, without them, from one forward sweep over the chunk;
//      then tile by tile from the last: recompute the tile's 16 states, sweep the adjoint backwards through them, sum the Σ_n terms over the four
//      lanes of a channel through LDS, and sum the dB/dC terms over the wave's 16
//      channels by an LDS transpose and over the workgroup's 4 waves once per tile;
//   4. reduce kernels sum the partials into dB, dC, dA, dD, ddt_bias.
// Both sweeping kernels copy the chunk's B and C from the [B, N, L] inputs into LDS
// (float32, zero past the chunk's end and past N).  Each lane of a channel forms the step
// values (δ, x or δ·x, ds) of its own steps, and the four lanes of the channel take each
// step's values from the lane that formed them by a DPP quad broadcast.  Steps past the end
// of the sequence run as identities (δ = 0, ds = 0), so the sweeps carry no per-step branches.
#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_plan.h"

namespace ss {

namespace {

constexpr int kBMaxSteps = 64;                // chunk <= 64 steps
constexpr int kBThreads = 256;                // 4 waves x 16 channels x 4 lanes
constexpr int kBChan = int(kBwdChan);
// 16-step tiles (the forward's checkpoint interval), 4 steps prepared per lane
constexpr int kBT = kCkptSteps;
constexpr int kBPer = 4;
constexpr int kBMaxTiles = kBMaxSteps / kBT;
// floats per channel in a wave's step rows of the final pass: steps x (δ, x, ds, σ(u)), +4 so
// that the rows of different channels start on different banks
constexpr int kRW = 4 * kBT + 4;

// DPP quad permutations.  Every lane of a quad is a valid source and every lane is active
// where these run, so bound_ctrl with a zero old value gives the same result as a plain move;
// that form lets the compiler fold the permutation into the VOP2 instruction that consumes it
// (v_mul_f32_dpp, v_add_f32_dpp) instead of issuing a separate v_mov_b32_dpp.
template <int Ctrl>
__device__ __forceinline__ float qperm(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xf, 0xf, true));
}

__device__ __forceinline__ float qsum(float v) {
    v += qperm<0xB1>(v);
    v += qperm<0x4E>(v);
    return v;
}

// v from lane O of this lane's quad
template <int O>
__device__ __forceinline__ float quad_bcast(float v) {
    return qperm<O * 0x55>(v);
}

// element t % 4 of v from quad lane t / 4 (t a constant after unrolling)
__device__ __forceinline__ float quad_bcast_i(const float (&v)[4], int t) {
    switch (t >> 2) {
        case 0: return quad_bcast<0>(v[t & 3]);
        case 1: return quad_bcast<1>(v[t & 3]);
        case 2: return quad_bcast<2>(v[t & 3]);
        default: return quad_bcast<3>(v[t & 3]);
    }
}

// Reduce-scatter over the quad: lane j of each quad gets Σ_q v_q[j], the sum over the quad's
// four lanes of their element j.  Two exchange stages (DPP quad permutations xor 1, xor 2, each
// folded into its add): at each, a lane keeps the half of its values whose index bit matches
// its lane bit and adds the partner's matching half.
__device__ __forceinline__ float quad_reduce_scatter(const float (&v)[4], int j) {
    const bool b0 = j & 1, b1 = j & 2;
    float r[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float keep = b0 ? v[2 * k + 1] : v[2 * k];
        const float send = b0 ? v[2 * k] : v[2 * k + 1];
        r[k] = keep + qperm<0xB1>(send);              // quad_perm [1, 0, 3, 2]
    }
    const float keep = b1 ? r[1] : r[0];
    const float send = b1 ? r[0] : r[1];
    return keep + qperm<0x4E>(send);                  // quad_perm [2, 3, 0, 1]
}

// The same over a tile's 16 per-step values, steps 4q..4q+3 owned by quad lane q: lane j gets
// Σ_q v_q[4j + i] for i < 4, the quad's totals of its own four steps.
__device__ __forceinline__ void quad_reduce_scatter16(const float (&v)[16], int j, float (&out)[4]) {
    const bool b0 = j & 1, b1 = j & 2;
    float r[8];                                       // [hi][i]: step 4 (2 hi + b0) + i
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = v[8 * hi + i], c = v[8 * hi + 4 + i];
            const float keep = b0 ? c : a;
            const float send = b0 ? a : c;
            r[4 * hi + i] = keep + qperm<0xB1>(send);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = b1 ? r[4 + i] : r[i];
        const float send = b1 ? r[i] : r[4 + i];
        out[i] = keep + qperm<0x4E>(send);
    }
}

// Sums across lanes for the dB|dC channel reduction.  gfx950's v_permlane32_swap exchanges
// the upper 32 lanes of its first operand with the lower 32 of its second, v_permlane16_swap
// the odd 16-lane rows of the first with the even rows of the second.  Applied to a pair (a, b)
// and summed, the lower lanes (rows) get a summed over lane bit 5 (bit 4) and the upper ones b
// summed over the same bit: one exchange and one add halve two values.
__device__ __forceinline__ float swap_sum32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// every lane gets the sum over the four lanes 4 apart in its 16-lane row (lane bits 2 and 3):
// DPP row rotations by 4 and by 8, each folded into its add
template <int Ctrl>
__device__ __forceinline__ float row_rot(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xf, 0xf, true));
}
__device__ __forceinline__ float row4_sum(float v) {
    v += row_rot<0x124>(v);   // row_ror:4
    v += row_rot<0x128>(v);   // row_ror:8
    return v;
}

// Σ over channels of the wave of one step's dB|dC terms of the lane's S states (cB, cC).
// Lane bit 5 picks the type (dB for 0, dC for 1); with S >= 2, bit 4 picks the half of the
// states, so a lane ends with W = max(S / 2, 1) sums: states j·S + (S / 2)·bit4 + [0, W) of the
// type bit5 (for S = 1 the same in both values of bit 4).  kRows = false: the sums cover the
// four channels that differ in lane bits 4 and 5, and the four lanes that differ in bits 2 and
// 3 hold the other channel groups' sums (they meet once per tile through LDS, for fewer
// instructions per step than two more lane exchanges); kRows = true: DPP row rotations add
// those too, so each sum covers all 16 channels, the same in the four lanes.
template <int S, bool kRows>
__device__ __forceinline__ void chan_sum(const float (&cB)[S], const float (&cC)[S],
                                         float (&w)[(S + 1) / 2]) {
    float u[S];
#pragma unroll
    for (int k = 0; k < S; ++k) u[k] = swap_sum32(cB[k], cC[k]);
    if constexpr (S >= 2) {
#pragma unroll
        for (int k = 0; k < S / 2; ++k) w[k] = swap_sum16(u[k], u[k + S / 2]);
    } else {
        w[0] = swap_sum16(u[0], u[0]);
    }
#pragma unroll
    for (int k = 0; k < (S + 1) / 2; ++k) {
        if constexpr (kRows) w[k] = row4_sum(w[k]);
        // formed here, for every lane: left alone, the compiler sinks the last add into the
        // caller's masked store, where the row rotation no longer folds into it
        asm volatile("" : "+v"(w[k]));
    }
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// S floats from LDS (16-byte aligned when S % 4 == 0)
template <int S>
struct Vec {
    float v[S];
    __device__ __forceinline__ void load(const float* p) {
        if constexpr (S % 4 == 0) {
#pragma unroll
            for (int q = 0; q < S; q += 4) {
                const float4 a = *reinterpret_cast<const float4*>(p + q);
                v[q] = a.x; v[q + 1] = a.y; v[q + 2] = a.z; v[q + 3] = a.w;
            }
        } else if constexpr (S % 2 == 0) {
#pragma unroll
            for (int q = 0; q < S; q += 2) {
                const float2 a = *reinterpret_cast<const float2*>(p + q);
                v[q] = a.x; v[q + 1] = a.y;
            }
        } else {
#pragma unroll
            for (int q = 0; q < S; ++q) v[q] = p[q];
        }
    }
};

// Elements [t, t+4) of a channel's row, element t at p[t·ts] (ts = 1: channel-major,
// ts = D: token-major), zero past t_end; one vector access when the four are contiguous,
// in range and aligned (vec: rows start on 8-element boundaries)
__device__ __forceinline__ void load4(const float* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                      int64_t ts, float (&o)[4]) {
    if (vec && ts == 1 && t + 4 <= t_end) {
        const float4 v = *reinterpret_cast<const float4*>(p + t);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (t + i < t_end) ? p[(t + i) * ts] : 0.0f;
    }
}
__device__ __forceinline__ void load4(const bf16_t* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                      int64_t ts, float (&o)[4]) {
    if (vec && ts == 1 && t + 4 <= t_end) {
        const uint2 v = *reinterpret_cast<const uint2*>(p + t);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (t + i < t_end) ? to_f32(p[(t + i) * ts]) : 0.0f;
    }
}
// 8 consecutive elements [t, t+8) of a row, zero past t_end: one 16-byte load of bf16 (two of
// float32) when the run is whole and aligned (vec: L % 8 == 0, so t % 8 == 0 rows start on
// 16 bytes), else two 4-element loads
__device__ __forceinline__ void load8(const bf16_t* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                      int64_t ts, float (&o)[8]) {
    if (vec && ts == 1 && t + 8 <= t_end) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + t);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        float a[4], b[4];
        load4(p, t, t_end, vec, ts, a);
        load4(p, t + 4, t_end, vec, ts, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
    }
}
__device__ __forceinline__ void load8(const float* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                      int64_t ts, float (&o)[8]) {
    float a[4], b[4];
    load4(p, t, t_end, vec, ts, a);
    load4(p, t + 4, t_end, vec, ts, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
}
__device__ __forceinline__ void store4(float* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                       int64_t ts, const float (&v)[4]) {
    if (vec && ts == 1 && t + 4 <= t_end) {
        *reinterpret_cast<float4*>(p + t) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (t + i < t_end) p[(t + i) * ts] = v[i];
    }
}

// 4 consecutive input elements [t, t+4) of a row in their storage type, zero past t_end
// (vector load when full and aligned); decoded to float32 when used
template <typename T> struct In4;
template <> struct In4<bf16_t> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                         int64_t ts) {
        if (vec && ts == 1 && t + 4 <= t_end) {
            v = *reinterpret_cast<const uint2*>(p + t);
        } else {
            uint32_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = (t + i < t_end) ? p[(t + i) * ts].bits : 0u;
            v = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
        }
    }
    __device__ __forceinline__ void decode(float (&o)[4]) const {
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
};
template <> struct In4<float> {
    float4 v;
    __device__ __forceinline__ void load(const float* __restrict__ p, int64_t t, int64_t t_end, int vec,
                                         int64_t ts) {
        if (vec && ts == 1 && t + 4 <= t_end) {
            v = *reinterpret_cast<const float4*>(p + t);
        } else {
            v.x = (t < t_end) ? p[t * ts] : 0.0f;
            v.y = (t + 1 < t_end) ? p[(t + 1) * ts] : 0.0f;
            v.z = (t + 2 < t_end) ? p[(t + 2) * ts] : 0.0f;
            v.w = (t + 3 < t_end) ? p[(t + 3) * ts] : 0.0f;
        }
    }
    __device__ __forceinline__ void decode(float (&o)[4]) const {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};

// B and C of steps [t0, t0 + nsteps) of batch row b, from the [B, Nr, L] (token-major:
// [B, L, Nr]) inputs into LDS as [step][B_0 .. B_{NP-1} | C_0 .. C_{NP-1}] float32 with row
// stride R; zero for steps past nsteps (up to kBMaxSteps) and states past Nr.  Lanes run
// along the contiguous dimension: coalesced reads.
template <typename Tin, int NP>
__device__ __forceinline__ void load_chunk_bc(float* __restrict__ lds, const Tin* __restrict__ Bm,
                                              const Tin* __restrict__ Cm, int b, int Nr, int64_t L,
                                              int64_t t0, int nsteps, int tid, int tok, int vec) {
    constexpr int R = 2 * NP + 4;
    constexpr int total = 2 * NP * kBMaxSteps;
    if (!tok && vec && Nr == NP) {
        // channel-major rows whose runs start on 16 bytes (L % 8 == 0 and t0 % 16 == 0): each
        // thread copies 16-byte pieces (PE steps of one B or C row), states fastest across lanes;
        // a piece reaching past the chunk's steps is read element by element, zero past them
        constexpr int PE = 16 / int(sizeof(Tin));
        constexpr int PPR = kBMaxSteps / PE;          // pieces per 64-step row
        constexpr int units = 2 * NP * PPR;
        for (int e = tid; e < units; e += kBThreads) {
            const int n = e % NP, q = (e / NP) % PPR, m = e / (NP * PPR);
            const Tin* src = (m ? Cm : Bm) + (int64_t(b) * NP + n) * L + t0 + PE * q;
            float v[PE];
            if (PE * q + PE <= nsteps) {
                const uint4 w = *reinterpret_cast<const uint4*>(src);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
                if constexpr (sizeof(Tin) == 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] = __uint_as_float(ww[i] << 16);
                        v[2 * i + 1] = __uint_as_float(ww[i] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(ww[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < PE; ++i) v[i] = (PE * q + i < nsteps) ? to_f32(src[i]) : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < PE; ++i) lds[(PE * q + i) * R + m * NP + n] = v[i];
        }
        return;
    }
    for (int e = tid; e < total; e += kBThreads) {
        const int t = tok ? (e / NP) % kBMaxSteps : e % kBMaxSteps;
        const int n = tok ? e % NP : (e / kBMaxSteps) % NP;
        const int m = e / (kBMaxSteps * NP);
        float v = 0.0f;
        if (n < Nr && t < nsteps) {
            const int64_t i = tok ? (int64_t(b) * L + t0 + t) * Nr + n : (int64_t(b) * Nr + n) * L + t0 + t;
            v = to_f32((m ? Cm : Bm)[i]);
        }
        lds[t * R + m * NP + n] = v;
    }
}

}  // namespace

// ---------------------------------------------------------------------------------------
// 1. chunk aggregates.  grid (ceil(D/64), K, B), 256 threads.
// ---------------------------------------------------------------------------------------
template <typename Tin, int S, bool kGate, bool kFwd, bool kZoh>
__global__ __launch_bounds__(kBThreads) void bwd_agg_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dy, const float* __restrict__ dt_bias, const float* __restrict__ A,
    const Tin* __restrict__ Bm, const Tin* __restrict__ Cm, float* __restrict__ h_end,
    float* __restrict__ rev_end, float* __restrict__ dsum_out, int64_t L, int64_t D, int Nr,
    int64_t chunk, int K, int vec, int tok, DtRows dtr) {
    constexpr int NP = 4 * S;
    constexpr int R = 2 * NP + 4;
    __shared__ __align__(16) float bc_lds[kBMaxSteps * R];
    const int tid = threadIdx.x;
    const int j = tid & 3;
    const int n0 = j * S;
    const int64_t d_raw = int64_t(blockIdx.x) * kBChan + (tid >> 2);
    const bool valid = d_raw < D;
    const int64_t d = valid ? d_raw : D - 1;
    const int k = blockIdx.y, b = blockIdx.z;
    const int64_t t0c = int64_t(k) * chunk;
    const int64_t t1c = (t0c + chunk < L) ? t0c + chunk : L;
    const int nsteps = int(t1c - t0c);
    const int ntiles = (nsteps + kBT - 1) / kBT;
    // element t of channel (b, d) at row[t·ts]; Δraw at its own rows
    const int64_t row = tok ? int64_t(b) * L * D + d : (int64_t(b) * D + d) * L;
    const int64_t ts = tok ? D : 1;
    const Tin* drr = dt_raw + int64_t(b) * dtr.sb + d * dtr.sd;
    const float bias = dt_bias[d];

    // Lane j of a channel owns the 16 steps [16 j, 16 j + 16) of the chunk: the four lanes
    // read the chunk's whole run of each input at once (a 64-step bf16 run is one 128-byte
    // line), before anything waits, and each lane forms δ, ds (and the input term) of its
    // own steps.  Steps past the chunk's end are identities (δ = 0, ds = 0).
    const int64_t tl = t0c + kBT * j;
    float dl[kBT], dsv[kBT], xin[kFwd ? kBT : 1];
    float dsum = 0.0f;
    {
        float xv[kBT], dv[kBT], gv[kBT], zv[kBT];
        // 16-byte loads: each instruction of a quad covers half of a bf16 line
#pragma unroll
        for (int q = 0; q < kBT / 8; ++q) {
            float t8[8];
            load8(drr, tl + 8 * q, t1c, vec, dtr.ts, t8);
#pragma unroll
            for (int i = 0; i < 8; ++i) dv[8 * q + i] = t8[i];
            load8(dy + row, tl + 8 * q, t1c, vec, ts, t8);
#pragma unroll
            for (int i = 0; i < 8; ++i) gv[8 * q + i] = t8[i];
            if (kGate) {
                load8(z + row, tl + 8 * q, t1c, vec, ts, t8);
#pragma unroll
                for (int i = 0; i < 8; ++i) zv[8 * q + i] = t8[i];
            }
            if (kFwd) {
                load8(x + row, tl + 8 * q, t1c, vec, ts, t8);
#pragma unroll
                for (int i = 0; i < 8; ++i) xv[8 * q + i] = t8[i];
            }
        }
        load_chunk_bc<Tin, NP>(bc_lds, Bm, Cm, b, Nr, L, t0c, nsteps, tid, tok, vec);
        const int rem = nsteps - kBT * j;             // this lane's steps inside the chunk
#pragma unroll
        for (int i = 0; i < kBT; ++i) {
            // past the chunk's end the loads gave zeros, so ds is zero there already; δ is
            // formed everywhere and selected (no branch around the transcendentals)
            const float sp = softplus(bias + dv[i]);
            dl[i] = (i < rem) ? sp : 0.0f;
            dsv[i] = kGate ? gv[i] * silu(zv[i]) : gv[i];
            dsum += dl[i];
            // δ·x, or x with the exact hold (its gain depends on the state)
            if (kFwd) xin[i] = kZoh ? xv[i] : dl[i] * xv[i];
        }
    }

    float A2[S], iA[S], h[S], P[S], Rv[S];
    bool pow_lane = true;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = n0 + s;
        const float a = (n < Nr) ? A[d * Nr + n] : 0.0f;
        A2[s] = a * kLog2e;
        if (kZoh && kFwd) iA[s] = 1.0f / a;
        h[s] = 0.0f; P[s] = 1.0f; Rv[s] = 0.0f;
        pow_lane = pow_lane && a == -float(n + 1);
    }
    // A[d, n] = -(n + 1) for every state of every channel of the wave: a lane's first Ā (or
    // cumulative product) takes one exponential and the next S - 1 are products with the
    // step's e^{-δ} (or e^{-Σδ})
    constexpr bool kMayPow = !kZoh && S >= 2;
    const bool pow_path = kMayPow && __builtin_amdgcn_readfirstlane(int(__all(pow_lane))) != 0;
    // Without the forward pair a step needs only Σδ up to it: dl[i] becomes that running sum
    // (this lane's prefix plus the totals of the quad's lower lanes, which own the earlier
    // steps of the chunk), and the lane that owns a step forms its e^{-Σδ} once for the quad
    // (the forward pair, which needs e^{-δ} and more registers, forms it per step)
    constexpr bool kRho = kMayPow && !kFwd;
    float rho[kRho ? kBT : 1];
    if constexpr (!kFwd) {
        float run = 0.0f;
#pragma unroll
        for (int i = 0; i < kBT; ++i) { run += dl[i]; dl[i] = run; }
        float incl = run;
        const float up1 = qperm<0x90>(incl);             // quad lane j - 1
        incl += j >= 1 ? up1 : 0.0f;
        const float up2 = qperm<0x40>(incl);             // quad lane j - 2
        incl += j >= 2 ? up2 : 0.0f;
        const float below = incl - run;
#pragma unroll
        for (int i = 0; i < kBT; ++i) dl[i] += below;
        if constexpr (kRho) {
            if (pow_path) {
#pragma unroll
                for (int i = 0; i < kBT; ++i) rho[i] = exp2_hw(-dl[i] * kLog2e);
            }
        }
    }
    __syncthreads();

    // tile T's steps sit in lane T of each quad: broadcast each step's values to the quad.
    // Without the forward pair no step needs its own Ā: the cumulative product is taken as
    // 2^(A·log2(e)·Σδ) from the running sum of δ, one exponential and no product per state.
    auto tile = [&](auto tc, auto pw) {
        constexpr int T = decltype(tc)::value;
        constexpr bool kPow = decltype(pw)::value && kMayPow;
        const float* bt = bc_lds + T * kBT * R;
#pragma unroll
        for (int i = 0; i < kBT; ++i) {
            // δ of the step (forward pair) or Σδ up to it (reverse pair only)
            const float arg = quad_bcast<T>(dl[i]);
            const float dst = quad_bcast<T>(dsv[i]);
            Vec<S> bc, cc;
            cc.load(bt + i * R + NP + n0);
            float xt = 0.0f;
            if (kFwd) {
                xt = quad_bcast<T>(xin[i]);
                bc.load(bt + i * R + n0);
            }
            // power path: the first state's factor and the ratio to the next state's
            float pp = 1.0f, rt = 1.0f;
            if constexpr (kPow) {
                pp = exp2_hw(arg * A2[0]);
                if constexpr (kRho) rt = quad_bcast<T>(rho[i]);
                else rt = exp2_hw(-arg * kLog2e);
            }
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if constexpr (kFwd) {
                    const float dlt = arg;
                    const float t2 = dlt * A2[s];
                    float a;
                    if constexpr (kPow) {
                        a = pp;
                        if (s + 1 < S) pp *= rt;
                    } else {
                        a = exp2_hw(t2);
                    }
                    float bx = xt * bc.v[s];
                    if (kZoh) bx *= zoh_gain(t2, a, dlt, iA[s]);
                    h[s] = fmaf(a, h[s], bx);
                    P[s] *= a;
                } else if constexpr (kPow) {
                    // pp carries the step's ds: one product per state for the chain, one FMA
                    if (s == 0) pp *= dst;
                    Rv[s] = fmaf(pp, cc.v[s], Rv[s]);
                    if (s + 1 < S) pp *= rt;
                    continue;
                } else {
                    P[s] = exp2_hw(arg * A2[s]);
                }
                Rv[s] = fmaf(P[s], dst * cc.v[s], Rv[s]);
            }
        }
    };
    static_assert(kBMaxSteps == 4 * kBT, "one tile per lane of a channel");
    auto tiles = [&](auto pw) {
        tile(std::integral_constant<int, 0>{}, pw);
        if (ntiles > 1) tile(std::integral_constant<int, 1>{}, pw);
        if (ntiles > 2) tile(std::integral_constant<int, 2>{}, pw);
        if (ntiles > 3) tile(std::integral_constant<int, 3>{}, pw);
    };
    if constexpr (kMayPow) {
        if (pow_path) tiles(std::true_type{});
        else tiles(std::false_type{});
    } else {
        tiles(std::false_type{});
    }
    dsum = qsum(dsum);
    if (valid) {
        const int64_t aidx = (int64_t(b) * D + d) * K + k;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int n = n0 + s;
            if (n < Nr) {
                if (kFwd) h_end[aidx * Nr + n] = h[s];
                rev_end[aidx * Nr + n] = Rv[s];
            }
        }
        if (j == 0) dsum_out[aidx] = dsum;
    }
}

// ---------------------------------------------------------------------------------------
// 3. final pass.  grid (ceil(D/64), K, B), 256 threads.
//   h_start [B,D,K,N]: state entering each chunk (kCk = false); overwritten with dA partials.
//   h_ckpt  [B,D,ceil(L/16),N]: the forward's state entering every 16th step (kCk = true).
//   q       [B,D,K,N]: adjoint entering each chunk from the right.
//   dbc_part [B, NB, L, 2N] (NB = ceil(D/64)): per-block sums over 64 channels of dB | dC.
//   ddt_part [B, D, K, 2]: per-chunk dD and ddt_bias partials.
// ---------------------------------------------------------------------------------------
// Two waves per SIMD: the tile's 16 recomputed states per lane and the per-step Σ_n
// partials take most of the 256 registers a wave then has.
template <typename Tin, int S, bool kGate, bool kCk, bool kZoh>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(S >= 8 ? 1 : 2, S >= 8 ? 1 : 2))) void bwd_chunk_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dy, const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const Tin* __restrict__ Bm, const Tin* __restrict__ Cm,
    const float* __restrict__ h_ckpt, float* h_start, const float* __restrict__ q,
    float* __restrict__ dxo, float* __restrict__ ddto, float* __restrict__ dzo,
    float* __restrict__ dbc_part, float* __restrict__ ddt_part, float* __restrict__ ddt_blk,
    int64_t L, int64_t D, int Nr, int64_t chunk, int K, int vec, int tok, DtRows dtr, DtRows gdr) {
    constexpr int NP = 4 * S;
    constexpr int R = 2 * NP + 4;
    // steps per reverse batch = steps a lane prepares: batch bi is lane bi's steps, so the
    // lane that owns a batch's elements finishes their gradients right after the batch
    constexpr int kBB = kBPer;
    constexpr int kNBat = kBT / kBB;
    constexpr int OUTW = kBT * 2 * NP;          // dB|dC sums of one tile for one partial plane
    constexpr int CW = (S + 1) / 2;             // channel sums a lane holds per step
    // planes sit PS floats apart (a multiple of 32) plus an offset of {0, CW, 16, 16 + CW} floats
    // for plane p = lane bits 2-3: the lanes of one store then hit disjoint LDS banks
    constexpr int PS = OUTW + 32;
    // partial planes per wave: with the gate, four (the channel sums skip lane bits 2 and 3);
    // without it the full butterfly, one plane (the ungated kernels, scheduled without the dz
    // section between the sweeps, spilled registers with four)
    constexpr int kPl = kGate ? 4 : 1;
    __shared__ __align__(16) float bc_lds[kBMaxSteps * R];
    __shared__ __align__(16) float rows[4 * 16 * kRW];
    // a shared Δraw's gradient of a tile: [wave][channel][step], summed over the block
    __shared__ __align__(16) float dtx[4 * 16 * kBT];
    // a tile's dB|dC partial sums, [wave][plane][step][type][state]
    __shared__ __align__(16) float comb[4 * kPl * PS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = tid & 3;
    const int n0 = j * S;
    const int64_t d_raw = int64_t(blockIdx.x) * kBChan + (tid >> 2);
    const bool valid = d_raw < D;
    const int64_t d = valid ? d_raw : D - 1;
    const int k = blockIdx.y, b = blockIdx.z;
    const int64_t t0c = int64_t(k) * chunk;
    const int64_t t1c = (t0c + chunk < L) ? t0c + chunk : L;
    const int nsteps = int(t1c - t0c);
    const int ntiles = (nsteps + kBT - 1) / kBT;
    const int64_t NB = (D + kBChan - 1) / kBChan;
    float* wdt = dtx + wave * 16 * kBT;         // this wave's shared-Δraw gradient rows
    float* myrow = rows + wave * 16 * kRW + (lane >> 2) * kRW;

    const int64_t sidx = ((int64_t(b) * D + d) * K + k) * Nr;
    const float bias = dt_bias[d];
    const float Dd = Dskip[d];
    // element t of channel (b, d) at row[t·ts] for x, z, dy, dx, dz; Δraw and its gradient
    // at their own rows (dtr, gdr)
    const int64_t row = tok ? int64_t(b) * L * D + d : (int64_t(b) * D + d) * L;
    const int64_t ts = tok ? D : 1;
    const Tin* xr = x + row;
    const Tin* drr = dt_raw + int64_t(b) * dtr.sb + d * dtr.sd;
    const int64_t dts = dtr.ts;
    float* ddr = ddto + int64_t(b) * gdr.sb + d * gdr.sd;
    const Tin* zr = kGate ? z + row : nullptr;
    const float* gr = dy + row;
    // checkpoints of this channel: tile tt of the chunk starts at checkpoint (t0c / 16) + tt
    const int64_t nck = (L + kBT - 1) / kBT;
    const float* ckr = kCk ? h_ckpt + (int64_t(b) * D + d) * nck * Nr + (t0c / kBT) * Nr : nullptr;
    // with checkpoints, the reverse sweep's global loads run one tile ahead (its first
    // tile is issued here); without, registers are short and each tile loads on entry
    In4<Tin> bx, bd, bz;
    In4<float> bg;
    float ckn[S];                               // next tile's start state (kCk)
    auto load_tile = [&](int tt) {
        const int64_t tl = t0c + tt * kBT + kBPer * j;
        bx.load(xr, tl, t1c, vec, ts);
        bd.load(drr, tl, t1c, vec, dts);
        bg.load(gr, tl, t1c, vec, ts);
        if (kGate) bz.load(zr, tl, t1c, vec, ts);
        if (kCk) {
#pragma unroll
            for (int s = 0; s < S; ++s) ckn[s] = (n0 + s < Nr) ? ckr[tt * Nr + n0 + s] : 0.0f;
        }
    };
    if (kCk) load_tile(ntiles - 1);
    load_chunk_bc<Tin, NP>(bc_lds, Bm, Cm, b, Nr, L, t0c, nsteps, tid, tok, vec);
    float A2[S], An[S], iA[S], g[S], dA[S];
    float ck[kCk ? 1 : kBMaxTiles][S];          // state entering each tile (uniform index)
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = n0 + s;
        const bool ok = n < Nr;
        An[s] = ok ? A[d * Nr + n] : 0.0f;
        A2[s] = An[s] * kLog2e;
        if (kZoh) iA[s] = 1.0f / An[s];
        g[s] = ok ? q[sidx + n] : 0.0f;
        dA[s] = 0.0f;
        if (!kCk) ck[0][s] = ok ? h_start[sidx + n] : 0.0f;
    }
    // A[d, n] = -(n + 1) for every state of every channel of the wave (the S4D-real A): both
    // sweeps form a lane's first Ā with one exponential and the next S - 1 as products with
    // r = e^{-δ}, which the lane that prepared the step broadcasts (first-order hold, S >= 2)
    constexpr bool kMayPow = !kZoh && S >= 2;
    bool pow_lane = true;
#pragma unroll
    for (int s = 0; s < S; ++s) pow_lane = pow_lane && An[s] == -float(n0 + s + 1);
    const bool pow_path = kMayPow && __builtin_amdgcn_readfirstlane(int(__all(pow_lane))) != 0;
    float accD = 0.0f, accT = 0.0f;
    __syncthreads();

    if constexpr (!kCk) {
        // ---- forward sweep: the state entering every tile but the first ----
        In4<Tin> ax, ad;
        ax.load(xr, t0c + kBPer * j, t1c, vec, ts);
        ad.load(drr, t0c + kBPer * j, t1c, vec, dts);
        float h[S];
#pragma unroll
        for (int s = 0; s < S; ++s) h[s] = ck[0][s];
#pragma unroll 1
        for (int tile = 0; tile + 1 < ntiles; ++tile) {
            const int tb = tile * kBT;
            float xv[4], dv[4];
            ax.decode(xv);
            ad.decode(dv);
            if (tile + 2 < ntiles) {
                const int64_t ta = t0c + tb + kBT + kBPer * j;
                ax.load(xr, ta, t1c, vec, ts);
                ad.load(drr, ta, t1c, vec, dts);
            }
            // (δ, δ·x) of this lane's steps (x with the exact hold), broadcast per step
            float fdl[kBPer], fxi[kBPer];
#pragma unroll
            for (int i = 0; i < kBPer; ++i) {
                fdl[i] = softplus(bias + dv[i]);  // every step of a non-last tile is real
                fxi[i] = kZoh ? xv[i] : fdl[i] * xv[i];
            }
            const float* bt = bc_lds + tb * R;
            Vec<S> bc, bn;
            bn.load(bt + n0);
#pragma unroll
            for (int t = 0; t < kBT; ++t) {
                float2 rc;
                rc.x = quad_bcast_i(fdl, t);
                rc.y = quad_bcast_i(fxi, t);
                bc = bn;
                if (t + 1 < kBT) bn.load(bt + (t + 1) * R + n0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float t2 = rc.x * A2[s];
                    const float ab = exp2_hw(t2);
                    float bx = rc.y * bc.v[s];
                    if (kZoh) bx *= zoh_gain(t2, ab, rc.x, iA[s]);
                    h[s] = fmaf(ab, h[s], bx);
                }
            }
#pragma unroll
            for (int s = 0; s < S; ++s) ck[tile + 1][s] = h[s];
        }
    }

    // the tile loop in two copies, the power path and the general one, chosen once per wave
    auto run_tiles = [&](auto pw) {
        constexpr bool kPow = decltype(pw)::value && kMayPow;
        // ---- tiles from the last to the first ----
#pragma unroll 1
        for (int tt = ntiles - 1; tt >= 0; --tt) {
            const int tb = tt * kBT;
            const int64_t te = t0c + tb + kBPer * j;
            const int rem = nsteps - (tb + kBPer * j);      // this lane's steps inside the chunk
            if (!kCk) load_tile(tt);
            float xv[4], dv[4], zv[4], gv[4];
            bx.decode(xv);
            bd.decode(dv);
            bg.decode(gv);
            if (kGate) bz.decode(zv);
            float hc[S];                            // state entering this tile
#pragma unroll
            for (int s = 0; s < S; ++s) hc[s] = kCk ? ckn[s] : ck[kCk ? 0 : tt][s];
            if (kCk && tt > 0) load_tile(tt - 1);
            float sz[4];
            // this lane's steps 4j..4j+3: (δ, x, ds) stay in registers, and the sweeps take each
            // step's values from the quad lane that formed them (DPP broadcast); the LDS row
            // (δ, x, ds, σ(u)) serves the per-step finishing below
            float rdl[kBPer], rx[kBPer], rds[kBPer], rr[kBPer];
#pragma unroll
            for (int i = 0; i < kBPer; ++i) {
                // past the sequence's end the loads gave zeros, so ds is zero there already; δ
                // is formed everywhere and selected (no branch around the transcendentals)
                const float u = bias + dv[i];
                const float sp = softplus(u);
                const float dl = (i < rem) ? sp : 0.0f;
                if constexpr (kPow) rr[i] = exp2_hw(-dl * kLog2e);   // e^{-δ}
                float ds;
                if (kGate) {
                    sz[i] = sigmoid(zv[i]);
                    ds = gv[i] * zv[i] * sz[i];
                } else {
                    ds = gv[i];
                }
                // channels past D compute on a clamped copy and must add nothing to dB, dC:
                // their x and ds are zero
                rdl[i] = dl;
                rx[i] = valid ? xv[i] : 0.0f;
                rds[i] = valid ? ds : 0.0f;
                *reinterpret_cast<float4*>(myrow + 4 * (kBPer * j + i)) =
                    make_float4(dl, rx[i], rds[i], sigmoid(u));
            }
            wave_sync();
            const float* bt = bc_lds + tb * R;

            // recompute the tile's states (and, with the gate, the readout for dz)
            float hs[kBT][S];
            Vec<S> rbn, rcn;                        // B, C of the reverse sweep's next step
            {
                float sp[kBT];
                float h[S];
                Vec<S> bc, cc, bn, cn;
                bn.load(bt + n0);
                if (kGate) cn.load(bt + NP + n0);
#pragma unroll
                for (int s = 0; s < S; ++s) h[s] = hc[s];
#pragma unroll
                for (int t = 0; t < kBT; ++t) {
                    float2 rc;
                    rc.x = quad_bcast_i(rdl, t);
                    rc.y = quad_bcast_i(rx, t);
                    // with the exact hold, keep these steps' values apart from the reverse sweep's:
                    // shared, the gains and exponentials of all 16 steps would stay live between
                    // the two sweeps and spill
                    if constexpr (kZoh) asm volatile("" : "+v"(rc.x));
                    bc = bn;
                    if (kGate) cc = cn;
                    if (t + 1 < kBT) {
                        bn.load(bt + (t + 1) * R + n0);
                        if (kGate) cn.load(bt + (t + 1) * R + NP + n0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    const float dxr = rc.x * rc.y;
                    float acc = 0.0f;
                    float abp = 1.0f, rt = 1.0f;
                    if constexpr (kPow) {
                        rt = quad_bcast_i(rr, t);
                        abp = exp2_hw(rc.x * A2[0]);
                    }
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        const float t2 = rc.x * A2[s];
                        float ab;
                        if constexpr (kPow) {
                            ab = abp;
                            if (s + 1 < S) abp *= rt;
                        } else {
                            ab = exp2_hw(t2);
                        }
                        const float bx = kZoh ? rc.y * bc.v[s] * zoh_gain(t2, ab, rc.x, iA[s]) : dxr * bc.v[s];
                        h[s] = fmaf(ab, h[s], bx);
                        hs[t][s] = h[s];
                        if (kGate) acc = fmaf(cc.v[s], h[s], acc);
                    }
                    sp[t] = acc;
                }
                // the reverse sweep's first step (the tile's last) reads in flight during the dz
                // section
                rbn.load(bt + (kBT - 1) * R + n0);
                rcn.load(bt + (kBT - 1) * R + NP + n0);
                if (kGate) {
                    // readout partials -> quad totals of the owner lane's steps (4j..4j+3 of
                    // lane j), by a reduce-scatter in registers; dz right away
                    float stot[4];
                    quad_reduce_scatter16(sp, j, stot);
                    float dzv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float sv = fmaf(Dd, xv[i], stot[i]);
                        dzv[i] = gv[i] * sv * sz[i] * fmaf(zv[i], 1.0f - sz[i], 1.0f);
                    }
                    if (valid) store4(dzo + row, te, t1c, vec, ts, dzv);
                }
            }

            // reverse sweep over the tile, in batches of kBB steps.  B and C of the step after
            // are read one step ahead (issued before this step's LDS stores of channel sums, which
            // the compiler cannot prove disjoint from them and would otherwise wait behind)
            const int cpl = kPl > 1 ? (lane >> 2) & 3 : 0;
            float* cbuf = comb + (wave * kPl + cpl) * PS + (cpl & 1) * CW + (cpl >> 1) * 16;
            // which channel sums this lane holds after chan_sum, and whether it stores them
            const int cs_type = (lane >> 5) & 1, cs_half = (lane >> 4) & 1;
            const int cs_off = cs_type * NP + n0 + (S >= 2 ? (S / 2) * cs_half : 0);
            const bool cs_store = (kPl > 1 || (lane & 12) == 0) && (S >= 2 || cs_half == 0);
#pragma unroll
            for (int bi = kNBat - 1; bi >= 0; --bi) {
                float pxb[kBB], pdb[kBB];
                // the row (δ, x, ds, σ(u)) of step 4 bi + j, which this lane finishes after the
                // batch: written before the recompute sweep, read now so it is in by then
                const int tj = bi * kBB + j;
                const float4 rw = *reinterpret_cast<const float4*>(myrow + 4 * tj);
#pragma unroll
                for (int i = kBB - 1; i >= 0; --i) {
                    const int t = bi * kBB + i;
                    float4 rc;
                    rc.x = quad_bcast_i(rdl, t);
                    rc.y = quad_bcast_i(rx, t);
                    rc.z = quad_bcast_i(rds, t);
                    const Vec<S> bc = rbn, cc = rcn;
                    if (t > 0) {
                        rbn.load(bt + (t - 1) * R + n0);
                        rcn.load(bt + (t - 1) * R + NP + n0);
                    }
                    // those reads stay issued at the step's start, ahead of its arithmetic
                    __builtin_amdgcn_sched_barrier(0);
                    const float dxr = rc.x * rc.y;
                    float pxa = 0.0f, pda = 0.0f;
                    float cB[S], cC[S];
                    float abp = 1.0f, rt = 1.0f;
                    if constexpr (kPow) {
                        rt = quad_bcast_i(rr, t);
                        abp = exp2_hw(rc.x * A2[0]);
                    }
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        const float hp = (t > 0) ? hs[t > 0 ? t - 1 : 0][s] : hc[s];
                        const float t2 = rc.x * A2[s];
                        float ab;
                        if constexpr (kPow) {
                            ab = abp;
                            if (s + 1 < S) abp *= rt;
                        } else {
                            ab = exp2_hw(t2);
                        }
                        g[s] = fmaf(rc.z, cc.v[s], g[s]);
                        cC[s] = rc.z * hs[t][s];
                        if (kZoh) {
                            // input term f·B·x, f the state's gain: dB += g f x, Σ_n g f B for dx,
                            // dA += g (∂f/∂A) B x, and ∂f/∂δ = Ā puts (Ā g) B x into dδ
                            const float f = zoh_gain(t2, ab, rc.x, iA[s]);
                            const float gB = g[s] * bc.v[s];
                            const float gBx = gB * rc.y;
                            cB[s] = g[s] * (rc.y * f);
                            pxa = fmaf(gB, f, pxa);
                            dA[s] = fmaf(zoh_gain_da(t2, ab, rc.x, iA[s], f), gBx, dA[s]);
                            // dA has no use inside the tile: without this empty register constraint
                            // the compiler sinks every step's ∂f/∂A term to the tile's end and holds
                            // all their operands live (it emits no instruction)
                            asm volatile("" : "+v"(dA[s]));
                            pda = fmaf(ab, gBx, pda);
                        } else {
                            cB[s] = g[s] * dxr;
                            pxa = fmaf(g[s], bc.v[s], pxa);
                        }
                        g[s] *= ab;
                        const float w = g[s] * hp;
                        dA[s] = fmaf(w, rc.x, dA[s]);
                        asm volatile("" : "+v"(dA[s]));
                        pda = fmaf(w, An[s], pda);
                    }
                    pxb[i] = pxa;
                    pdb[i] = pda;
                    // this step's dB|dC terms summed over channels in registers; the lanes store
                    // their sums in their plane as [step][type][state] (one lane of the four
                    // holding the same sums with a single plane)
                    float cs[CW];
                    chan_sum<S, kPl == 1>(cB, cC, cs);
                    if (cs_store) {
                        float* dst = cbuf + t * 2 * NP + cs_off;
                        if constexpr (CW == 4) {
                            *reinterpret_cast<float4*>(dst) = make_float4(cs[0], cs[1], cs[2], cs[3]);
                        } else if constexpr (CW == 2) {
                            *reinterpret_cast<float2*>(dst) = make_float2(cs[0], cs[1]);
                        } else {
                            dst[0] = cs[0];
                        }
                    }
                }
                {
                    // lane j finishes step 4 bi + j of its channel: Σ_n over the quad's partials
                    // of that step (a reduce-scatter in registers), then dx and dΔ from its row
                    const float PX = quad_reduce_scatter(pxb, j);
                    const float PD = quad_reduce_scatter(pdb, j);
                    const int64_t tg = t0c + tb + tj;
                    const bool ok = tg < t1c;
                    // exact hold: PX already carries the gain and PD the input term of dδ
                    const float ox = fmaf(rw.z, Dd, kZoh ? PX : rw.x * PX);
                    const float od = (kZoh ? PD : fmaf(rw.y, PX, PD)) * rw.w;
                    accD += ok ? rw.z * rw.y : 0.0f;
                    accT += ok ? od : 0.0f;
                    // park (dx, dΔraw) in the step's row, which no later batch reads: the tile's
                    // outputs leave in 16-byte runs per lane once the sweep is done
                    *reinterpret_cast<float2*>(myrow + 4 * tj) = make_float2(ox, od);
                }
            }
            wave_sync();   // every lane's parked (dx, dΔraw) visible to the lane that stores it

            // dx, dΔraw of the lane's own 4 steps, from the rows.  A Δraw shared by the channels
            // (ddt_blk) takes the sum over the block's channels instead: each wave parks its 16
            // channels' values in its own rows of dtx, summed below.
            {
                float ox[4], od[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float2 v = *reinterpret_cast<const float2*>(myrow + 4 * (kBPer * j + i));
                    ox[i] = v.x;
                    od[i] = v.y;
                }
                if (valid) store4(dxo + row, te, t1c, vec, ts, ox);
                if (ddt_blk) {
                    *reinterpret_cast<float4*>(wdt + (lane >> 2) * kBT + kBPer * j) =
                        valid ? make_float4(od[0], od[1], od[2], od[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
                } else if (valid) {
                    store4(ddr, te, t1c, vec, gdr.ts, od);
                }
            }

            // dB|dC of the tile: the waves' planes meet once per tile, summed in a fixed order
            __syncthreads();
            if (ddt_blk && tid < kBT) {
                // Σ over the block's 64 channels of dΔraw at step tb + tid
                float sdt = 0.0f;
                for (int w = 0; w < 4; ++w)
                    for (int cl = 0; cl < 16; ++cl) sdt += dtx[(w * 16 + cl) * kBT + tid];
                const int64_t t = t0c + tb + tid;
                if (t < t1c) ddt_blk[(int64_t(b) * NB + blockIdx.x) * L + t] = sdt;
            }
            for (int e = tid; e < OUTW; e += kBThreads) {
                const int st = e / (2 * NP);
                const int v = e % (2 * NP);
                const int ty = v / NP, n = v % NP;
                float tot = 0.0f;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const float* c = comb + w2 * kPl * PS + e;   // wave w2's planes
                    float tw = c[0];
#pragma unroll
                    for (int q = 1; q < kPl; ++q) tw += c[q * PS + (q & 1) * CW + (q >> 1) * 16];
                    tot = w2 ? tot + tw : tw;
                }
                const int64_t t = t0c + tb + st;
                if (n < Nr && t < t1c)
                    dbc_part[((int64_t(b) * NB + blockIdx.x) * L + t) * (2 * Nr) + ty * Nr + n] = tot;
            }
            __syncthreads();
        }
    };
    if constexpr (kMayPow) {
        if (pow_path) run_tiles(std::true_type{});
        else run_tiles(std::false_type{});
    } else {
        run_tiles(std::false_type{});
    }

    accD = qsum(accD);
    accT = qsum(accT);
    if (valid) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int n = n0 + s;
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
// dB | dC: part [B, NB, L, 2N] summed over NB -> dB, dC [B, N, L] (token-major: [B, L, N]).
// One thread per four consecutive (t, v) entries of a batch row (one per entry when L·2N is
// not a multiple of 4): reads are coalesced across threads, the sum runs over the channel
// blocks.
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part,
                                                            float* __restrict__ dB,
                                                            float* __restrict__ dC, int64_t L,
                                                            int NB, int Nr, int tok) {
    const int R = 2 * Nr;
    const int b = blockIdx.y;
    const int64_t LR = L * R;
    // four consecutive (t, v) entries per thread when LR % 4 == 0 (each block row then starts
    // on 16 bytes): 16-byte loads, sixteen blocks' loads in flight at a time
    const bool v4 = (LR & 3) == 0;
    const int64_t f0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * (v4 ? 4 : 1);
    if (f0 >= LR) return;
    const float* p = part + int64_t(b) * NB * LR + f0;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (v4) {
        float4 a[4] = {};
        int gi = 0;
        for (; gi + 16 <= NB; gi += 16) {
            float4 q[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) q[u] = *reinterpret_cast<const float4*>(p + int64_t(gi + u) * LR);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                a[u & 3].x += q[u].x; a[u & 3].y += q[u].y; a[u & 3].z += q[u].z; a[u & 3].w += q[u].w;
            }
        }
        for (; gi < NB; ++gi) {
            const float4 q = *reinterpret_cast<const float4*>(p + int64_t(gi) * LR);
            a[0].x += q.x; a[0].y += q.y; a[0].z += q.z; a[0].w += q.w;
        }
        acc[0] = (a[0].x + a[1].x) + (a[2].x + a[3].x);
        acc[1] = (a[0].y + a[1].y) + (a[2].y + a[3].y);
        acc[2] = (a[0].z + a[1].z) + (a[2].z + a[3].z);
        acc[3] = (a[0].w + a[1].w) + (a[2].w + a[3].w);
    } else {
        // eight independent partial sums: eight loads in flight instead of a chain
        float a[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        int gi = 0;
        for (; gi + 8 <= NB; gi += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] += p[int64_t(gi + u) * LR];
        }
        for (; gi < NB; ++gi) a[0] += p[int64_t(gi) * LR];
        acc[0] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    }
    const int nf = v4 ? 4 : 1;
    for (int i = 0; i < nf; ++i) {
        const int64_t f = f0 + i;
        const int64_t t = f / R;
        const int v = int(f % R);
        const int n = v < Nr ? v : v - Nr;
        float* out = v < Nr ? dB : dC;
        out[tok ? (int64_t(b) * L + t) * Nr + n : (int64_t(b) * Nr + n) * L + t] = acc[i];
    }
}

// Δraw shared by the channels (one value per token): its gradient [B, L] is the sum over
// channels of the per-channel gradients, which the final pass has already summed over each
// block of 64 channels: part [B, NB, L] summed over NB.  One thread per (b, t), coalesced
// across t.
__global__ __launch_bounds__(256) void bwd_reduce_dt_kernel(const float* __restrict__ part,
                                                            float* __restrict__ out, int NB,
                                                            int64_t L) {
    const int b = blockIdx.y;
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (t >= L) return;
    const float* p = part + int64_t(b) * NB * L + t;
    float acc = 0.0f;
    for (int gi = 0; gi < NB; ++gi) acc += p[int64_t(gi) * L];
    out[int64_t(b) * L + t] = acc;
}

// dA [D, N] = Σ_{b,k} part[b,d,k,n];  dD, ddt_bias [D] = Σ_{b,k} ddt_part[b,d,k,0|1].
// One block per channel d: for each b the K*N (and K*2) partials of (b, d) are
// contiguous, so the block reads them coalesced and folds over k through LDS.
__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(
    const float* __restrict__ dA_part, const float* __restrict__ ddt_part, float* __restrict__ dA,
    float* __restrict__ dD, float* __restrict__ ddt_bias, int64_t D, int Nr, int Bn, int K) {
    __shared__ float red[1024];
    __shared__ float wsum[2][4];
    const int64_t d = blockIdx.x;
    const int tid = threadIdx.x;
    const int KN = K * Nr;
    // dA: entry e of a (b, d) block of K*N partials has state e % Nr.  With Nr >= 4 (so
    // KN % 4 == 0 and every block starts on 16 bytes) thread tid reads 16-byte runs 4 tid + 1024 i,
    // whose four entries have states (4 tid + q) % Nr, since Nr divides 1024, and keeps its sum
    // q in red[4 tid + q]; otherwise it reads single entries tid + 256 i, state tid % Nr, and
    // keeps the sum in red[tid] (slots 256.. hold zeros).  Either way every red[f] belongs to
    // state f % Nr.
    float ac[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool vec4 = Nr >= 4;
    for (int b = 0; b < Bn; ++b) {
        const float* p = dA_part + (int64_t(b) * D + d) * KN;
        if (vec4) {
            const float4* p4 = reinterpret_cast<const float4*>(p);
            for (int e = tid; e < KN / 4; e += 256) {
                const float4 v = p4[e];
                ac[0] += v.x; ac[1] += v.y; ac[2] += v.z; ac[3] += v.w;
            }
        } else {
            for (int e = tid; e < KN; e += 256) ac[0] += p[e];
        }
    }
    if (vec4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) red[4 * tid + q] = ac[q];
    } else {
        red[tid] = ac[0];
#pragma unroll
        for (int q = 0; q < 3; ++q) red[256 + 3 * tid + q] = 0.0f;
    }
    __syncthreads();
    // fold the 1024 slots to 256 (f, f + 256, f + 512, f + 768 share a state), then each
    // state's 256 / Nr slots
    const float f4 = (red[tid] + red[tid + 256]) + (red[tid + 512] + red[tid + 768]);
    __syncthreads();
    red[tid] = f4;
    __syncthreads();
    if (tid < Nr) {
        float t = 0.0f;
        for (int i = tid; i < 256; i += Nr) t += red[i];
        dA[d * Nr + tid] = t;
    }
    // dD and ddt_bias: Σ over batch rows and chunks of the (dD, ddt) pairs
    float a0 = 0.0f, a1 = 0.0f;
    for (int b = 0; b < Bn; ++b) {
        const float2* q = reinterpret_cast<const float2*>(ddt_part + (int64_t(b) * D + d) * K * 2);
        for (int k = tid; k < K; k += 256) {
            const float2 v = q[k];
            a0 += v.x; a1 += v.y;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        a0 += __shfl_xor(a0, o);
        a1 += __shfl_xor(a1, o);
    }
    if ((tid & 63) == 0) { wsum[0][tid >> 6] = a0; wsum[1][tid >> 6] = a1; }
    __syncthreads();
    if (tid == 0) {
        dD[d] = (wsum[0][0] + wsum[0][1]) + (wsum[0][2] + wsum[0][3]);
        ddt_bias[d] = (wsum[1][0] + wsum[1][1]) + (wsum[1][2] + wsum[1][3]);
    }
}

// ---------------------------------------------------------------------------------------
// plan helpers and launchers
// ---------------------------------------------------------------------------------------
template <typename Tin, int S, bool kGate>
static void launch_bwd_g(const BwdLaunch& p, dim3 grid, hipStream_t s) {
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
    const Tin* Bm = static_cast<const Tin*>(p.Bm);
    const Tin* Cm = static_cast<const Tin*>(p.Cm);
    with_bool(p.h_ckpt != nullptr, [&](auto ck) {
      return with_bool(p.zoh != 0, [&](auto zoh) {
        if (p.stage == 0)
            hipLaunchKernelGGL((bwd_agg_kernel<Tin, S, kGate, !ck.value, zoh.value && !ck.value>),
                               grid, dim3(kBThreads), 0,
                               s, x, dr, z, p.dy, p.dt_bias, p.A, Bm, Cm, p.h_end, p.rev_end, p.dsum,
                               p.L, p.D, int(p.N), p.chunk, p.K, p.vec, p.tok, p.dtr);
        else
            hipLaunchKernelGGL((bwd_chunk_kernel<Tin, S, kGate, ck.value, zoh.value>), grid,
                               dim3(kBThreads), 0,
                               s, x, dr, z, p.dy, p.dt_bias, p.A, p.Dskip, Bm, Cm, p.h_ckpt, p.h_end,
                               p.rev_end, p.dx, p.ddt_raw, p.dz, p.dbc_part, p.ddt_part,
                               p.ddt_shared ? p.ddt_blk : nullptr, p.L, p.D, int(p.N), p.chunk,
                               p.K, p.vec, p.tok, p.dtr, p.gdr);
        return hipSuccess;
      });
    });
}

template <typename Tin, int S>
static hipError_t launch_bwd_t(const BwdLaunch& p, hipStream_t s) {
    dim3 grid(unsigned((p.D + kBChan - 1) / kBChan), unsigned(p.K), unsigned(p.B));
    if (p.z) launch_bwd_g<Tin, S, true>(p, grid, s);
    else launch_bwd_g<Tin, S, false>(p, grid, s);
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
    const int64_t per = (LR % 4 == 0) ? 4 : 1;   // entries per thread (bwd_reduce_bc_kernel)
    hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(unsigned((LR / per + 255) / 256), unsigned(p.B)), dim3(256),
                       0, s, p.dbc_part, p.dB, p.dC, p.L, NB, int(p.N), p.tok);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.ddt_shared) {
        hipLaunchKernelGGL(bwd_reduce_dt_kernel, dim3(unsigned((p.L + 255) / 256), unsigned(p.B)),
                           dim3(256), 0, s, p.ddt_blk, p.ddt_shared, NB, p.L);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3(unsigned(p.D)), dim3(256), 0, s, p.h_end,
                       p.ddt_part, p.dA, p.dD, p.ddt_bias, p.D, int(p.N), int(p.B), p.K);
    return hipGetLastError();
}

}  // namespace ss

