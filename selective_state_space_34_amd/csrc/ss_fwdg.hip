// Group-split forward selective-scan kernel for gfx950.
//
// Same computation as scan_kernel (page "3.2 선택적 스캔(Selective Scan) 알고리즘과
// 정보의 압축 및 선별": §1.2 softplus step, §2.1 exp discretisation of diagonal A,
// §2.2 recurrence, §1.1 readout; SiLU gate of the note "상태공간 모델(SSM)과 Mamba
// 아키텍처", §3), laid out for CDNA4 occupancy: the N states of a channel are split
// over a group of G adjacent lanes (G = 4 or 8, S = N/G states per lane), so a
// 64-lane wave covers 64/G channels and B*D channels yield B*D*G/64 waves.  G = 8
// gives five waves per SIMD at B*D = 40960, where G = 4 leaves the SIMDs unevenly
// loaded (2.5 waves each), but it moves more operand bytes through LDS per state-step
// and is LDS-issue bound on gfx950 (measured slower); G = 4 is the default.  A single pass
// whose last round of four-lane waves would be at most half full runs its remaining
// channels on eight lanes in the same launch (scang_mixed_kernel), which evens out the
// SIMDs; N = 64 runs on eight lanes of eight states.
//
// Per 32-step tile:
//   - the workgroup copies the tile's B and C ([B, N, L] inputs, N rows of 32 steps
//     each) into LDS transposed to [step][B row | C row] as float32;
//   - lane l of a group loads and prepares steps [16h + kH·l, 16h + kH·(l+1)) of both
//     halves h of the tile (kH = 16/G): widening, δ = softplus(dt_bias + dt_raw), δ·x.
//     No element is prepared twice.
// Per 16-step half:
//   - four lanes, first-order hold: step t's (δ, δ·x) stays in quad lane t / 4, which
//     formed it, and reaches the quad by a DPP broadcast folded into the multiplies that
//     use it; otherwise (eight lanes, or the exact zero-order hold, whose pair is (δ, x)
//     and whose per-state gain uses δ in fused multiply-adds) the lanes write their pairs
//     into a per-wave LDS row of their channel and each step reads its pair from there;
//   - the recurrence walks the 16 steps, reading B_t, C_t for the lane's S states from
//     the tile, one step ahead, as broadcast LDS reads;
//   - each lane's partial readouts (its S states, 16 steps) go to the same per-wave
//     area; lane l sums the G partials of its own kH steps, adds D·x, applies the
//     gate and stores kH outputs.
// All global loads of the next tile (x, dt_raw, z, B/C) are issued before the current
// tile's arithmetic.  The state never leaves VGPRs (§3.2).
#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

namespace {

constexpr int kTile = 32;      // steps per tile (B/C copy, global loads, one block barrier)
constexpr int kHalf = 16;      // steps per recurrence sweep (LDS exchange granularity)
constexpr int kThreads = 256;  // 4 waves
// lane stride (floats) of the partial-readout area: 20 floats = 80 bytes puts the
// 16-byte writes of 8 consecutive lanes on 8 disjoint groups of 4 banks
constexpr int kPS = kHalf + 4;
// channel stride (floats) of the (δ, δ·x) rows: 34 = 2 mod 32, so the 8-byte reads of
// up to 16 channels fall on distinct bank pairs
constexpr int kDS = 2 * kHalf + 2;

// S floats (B or C of the lane's states at one step), LDS -> VGPR
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

// K consecutive input elements in their storage type (K = 2, 4, 8)
template <typename Tin, int K> struct Raw;
template <int K> struct Raw<bf16_t, K> {
    uint32_t w[K / 2];
    __device__ __forceinline__ void load(const bf16_t* p) {
        if constexpr (K == 2) {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        } else if constexpr (K == 4) {
            const uint2 a = *reinterpret_cast<const uint2*>(p);
            w[0] = a.x; w[1] = a.y;
        } else {
            const uint4 a = *reinterpret_cast<const uint4*>(p);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        }
    }
    // elements base[off], base[off + st], ..., base[off + (K-1)·st] (token-major rows); 32-bit
    // offsets from a base shared by the wave, so each load takes one offset register
    __device__ __forceinline__ void load_strided(const bf16_t* base, uint32_t off, uint32_t st) {
#pragma unroll
        for (int i = 0; i < K / 2; ++i)
            w[i] = uint32_t(base[off + 2 * i * st].bits) | (uint32_t(base[off + (2 * i + 1) * st].bits) << 16);
    }
    __device__ __forceinline__ void decode(float (&o)[K]) const {
#pragma unroll
        for (int i = 0; i < K / 2; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <int K> struct Raw<float, K> {
    float v[K];
    __device__ __forceinline__ void load(const float* p) {
        if constexpr (K == 2) {
            const float2 a = *reinterpret_cast<const float2*>(p);
            v[0] = a.x; v[1] = a.y;
        } else {
#pragma unroll
            for (int q = 0; q < K; q += 4) {
                const float4 a = *reinterpret_cast<const float4*>(p + q);
                v[q] = a.x; v[q + 1] = a.y; v[q + 2] = a.z; v[q + 3] = a.w;
            }
        }
    }
    __device__ __forceinline__ void load_strided(const float* base, uint32_t off, uint32_t st) {
#pragma unroll
        for (int i = 0; i < K; ++i) v[i] = base[off + i * st];
    }
    __device__ __forceinline__ void decode(float (&o)[K]) const {
#pragma unroll
        for (int i = 0; i < K; ++i) o[i] = v[i];
    }
};

// raw storage of 4 consecutive elements of one B or C row
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

template <int K>
__device__ __forceinline__ void store_k(float* p, const float (&v)[K]) {
    if constexpr (K == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int q = 0; q < K; q += 4)
            *reinterpret_cast<float4*>(p + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
    }
}

// sum over the G lanes of a group (groups are aligned runs of G lanes)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// element t % 4 of v from lane t / 4 of this lane's quad (t a constant after unrolling).
// Every lane of the quad is a valid source and all lanes are active where this runs, so
// bound_ctrl with a zero old value equals a plain move, and in that form the compiler folds
// the permutation into the multiply that consumes it (v_mul_f32_dpp): no extra instruction.
template <int K>
__device__ __forceinline__ float quad_step(const float (&v)[K], int t) {
    static_assert(K == 4, "four steps per lane of a quad");
    const int i = __float_as_int(v[t & 3]);
    switch (t >> 2) {
        case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x00, 0xf, 0xf, true));
        case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x55, 0xf, 0xf, true));
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0xAA, 0xf, 0xf, true));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0xFF, 0xf, 0xf, true));
    }
}

// v from quad lane quad_perm(Ctrl) of this lane's quad (same folding form as quad_step)
template <int Ctrl>
__device__ __forceinline__ float qperm(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xf, 0xf, true));
}

// order LDS traffic of one wave: everything before is visible to the wave's lanes after
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

// Token-major staging of one 32-step tile of x, Δraw and z for the CW channels of a wave:
// the wave reads each step's CW elements as 16-byte pieces (one per lane per tensor for
// bf16 at G = 4) and stores them, in the element type, as rows of its exchange area; each
// lane then reads its own steps of its channel from there.  Rows are padded so that the
// lanes of one read (G lane groups, kH rows apart) fall on distinct banks.
template <int G, typename Tin>
struct TokStage {
    static constexpr int CW = 64 / G;
    static constexpr int ELEM = int(sizeof(Tin));
    static constexpr int PIECE = 16 / ELEM;              // elements per 16-byte piece
    static constexpr int ROWB = CW * ELEM;               // bytes of a step's CW elements
    static constexpr int PPR = ROWB / 16;                // pieces per step
    static constexpr int RSB = ROWB + (ROWB >= 32 ? 16 : 0);  // row stride, bytes
    static constexpr int PIECES = kTile * PPR;           // pieces per tensor per wave
    static constexpr int PL = (PIECES + 63) / 64;        // pieces per lane per tensor
    static constexpr int TBYTES = kTile * RSB;           // bytes per tensor
    static constexpr int FLOATS = 3 * TBYTES / 4;
};

// LDS floats the body of a G-lane workgroup needs: a double-buffered B/C tile, then the
// four waves' exchange areas (large enough for the token-major staging)
template <int G, int S, typename Tin = float, bool kTok = false>
struct GroupLds {
    static constexpr int N = G * S;
    static constexpr int CW = 64 / G;
    static constexpr int R = 2 * N + 4;           // B_t | C_t row, padded by 4 floats
    static constexpr int TILE_F = kTile * R;
    static constexpr int WAREA0 = (64 * kPS > CW * kDS) ? 64 * kPS : CW * kDS;
    static constexpr int WAREA = (kTok && TokStage<G, Tin>::FLOATS > WAREA0)
                                     ? TokStage<G, Tin>::FLOATS : WAREA0;
    static constexpr int FLOATS = 2 * TILE_F + 4 * WAREA;
};

// One workgroup's scan: channels d_lo + blk * (256 / G) + [0, 256 / G) of batch row b (those
// below d_hi), chunk k.  lds: GroupLds<G, S>::FLOATS floats, 16-byte aligned.  Requires
// L % 8 == 0 and chunk % 32 == 0 (or K == 1) for the tiled part; the last < 32 steps of a
// chunk run a per-step tail.
template <typename Tin, int G, int S, bool kGate, bool kAgg, bool kZoh, bool kTok, bool kMayPow = true,
          bool kWiden = false>
__device__ __forceinline__ void scang_body(
    float* __restrict__ lds, int64_t blk, int k, int b, int64_t d_lo, int64_t d_hi,
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const Tin* __restrict__ Bm, const Tin* __restrict__ Cm,
    const float* __restrict__ h_init, float* __restrict__ y, float* __restrict__ h_last,
    float* __restrict__ h_ckpt, float* __restrict__ dsum_out, int64_t L, int64_t D,
    int64_t chunk, int K, DtRows dtr) {
    using Lay = GroupLds<G, S, Tin, kTok>;
    using TS = TokStage<G, Tin>;
    constexpr int N = G * S;
    constexpr int CW = 64 / G;                    // channels per wave
    constexpr int CB = 4 * CW;                    // channels per block
    constexpr int kH = kHalf / G;                 // steps per lane per half
    // four lanes, first order: step t's (δ, δ·x) stay in quad lane t / 4, which formed them,
    // and reach the other three by DPP (folded into the multiplies that use them) instead of
    // through the channel's LDS row; the exact hold's gain uses δ in fused multiply-adds,
    // which take no DPP operand, so it keeps the row
    constexpr bool kDpp = (G == 4) && !kZoh;
    // LDS tile row per step: B_t (N floats) then C_t (N floats), padded by 4 floats so
    // the transposing writes of a wave fall on at most two lanes per bank
    constexpr int R = Lay::R;
    constexpr int TILE_F = Lay::TILE_F;
    // per-wave exchange area: the (δ, δ·x) rows during a sweep, the partial readouts after
    constexpr int WAREA = Lay::WAREA;
    float* const w_lds = lds + 2 * TILE_F;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l = lane & (G - 1);                 // lane within the group: states, steps
    const int c = lane / G;                       // channel within the wave
    const int64_t d_raw = d_lo + blk * CB + tid / G;
    const bool valid = d_raw < d_hi;
    const int64_t d = valid ? d_raw : d_hi - 1;   // clamped for loads
    const int64_t t_begin = int64_t(k) * chunk;
    const int64_t t_end = (t_begin + chunk < L) ? t_begin + chunk : L;
    const int64_t n_tiles = (t_end - t_begin) / kTile;
    const int64_t t_tiles_end = t_begin + n_tiles * kTile;
    const int n0 = l * S;

    float A2[S], iA[S], h[S];
    bool pow_lane = true;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float a = A[d * N + n0 + s];
        A2[s] = a * kLog2e;
        if (kZoh) iA[s] = 1.0f / a;
        pow_lane = pow_lane && (a == -float(n0 + s + 1));
    }
    // A[d, n] = -(n + 1) for every state of every channel of the wave (the S4D-real A): then
    // Ā_n = r^(n+1) with r = e^{-δ}, so a lane forms its first state's Ā = 2^(δ·A_{n0}·log2 e)
    // with one exponential and the next S - 1 by multiplying with r, which the lane that
    // prepared the step broadcasts with (δ, δ·x) (four lanes, first-order hold only).  The
    // chain carries at most S ulp of relative error.  The vote is uniform over the wave.
    const bool pow_path = kDpp && kMayPow && __builtin_amdgcn_readfirstlane(int(__all(pow_lane))) != 0;
    const int64_t hidx = ((int64_t(b) * D + d) * K + k) * N + n0;
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] = h_init ? h_init[hidx + s] : 0.0f;
    const float bias = dt_bias[d];
    const float Dd = kAgg ? 0.0f : Dskip[d];
    // channel (b, d): element t of x, z, y at row[t·ts]; Δraw at its own rows (dtr)
    const int64_t row = kTok ? int64_t(b) * L * D + d : (int64_t(b) * D + d) * L;
    const int64_t ts = kTok ? D : 1;
    const Tin* xr = x + row;
    const Tin* dr = dt_raw + int64_t(b) * dtr.sb + d * dtr.sd;
    const int64_t dts = dtr.ts;
    const Tin* zr = kGate ? z + row : nullptr;
    float* yr = kAgg ? nullptr : y + row;
    // token-major: the batch row's bases (uniform) and 32-bit element offsets (L·D < 2^31)
    const int64_t brow = int64_t(b) * L * D;
    const Tin* xb = x + brow;
    const Tin* zb = kGate ? z + brow : nullptr;
    float* yb = kAgg ? nullptr : y + brow;
    const Tin* db = dt_raw + int64_t(b) * dtr.sb;
    const uint32_t dofs = uint32_t(d * dtr.sd), d32 = uint32_t(d), D32 = uint32_t(D);
    const uint32_t dts32 = uint32_t(dtr.ts);
    // B, C of row b: [N, L] (channel-major) or [L, N] (token-major)
    const Tin* Bb = Bm + int64_t(b) * N * L;
    const Tin* Cb = Cm + int64_t(b) * N * L;
    float dsum = 0.0f;
    // checkpoints: the state entering step t for every t % kCkptSteps == 0
    const int64_t nck = (L + kCkptSteps - 1) / kCkptSteps;
    float* ckr = (!kAgg && h_ckpt && valid) ? h_ckpt + (int64_t(b) * D + d) * nck * N + n0 : nullptr;
    auto checkpoint = [&](int64_t t) {
#pragma unroll
        for (int s = 0; s < S; ++s) ckr[(t / kCkptSteps) * N + s] = h[s];
    };

    // B/C tile copy: 2·N rows of 32 steps.  Channel-major: unit e covers steps 4q..4q+3 of
    // state n of B (m = 0) or C (m = 1), with n fastest across lanes.  Token-major: unit e
    // covers states 4q..4q+3 of step tt, with q fastest (a step's N states are contiguous).
    constexpr int BC_UNITS = 2 * N * (kTile / 4);
    constexpr int NQ = N / 4;
    constexpr int BC_PASSES = (BC_UNITS + kThreads - 1) / kThreads;
    Raw4<Tin> bc_next[BC_PASSES];
    Raw<Tin, kH> xn[2], dn[2], zn[2];
    // token-major: the wave's 16-byte pieces of the next tile (x, Δraw, z).  A Δraw shared
    // by the channels is not staged: each lane reads its own steps of the row, both halves'
    // kH elements packed into the same registers (2·kH elements fit in TS::PL pieces)
    uint4 px[kTok ? TS::PL : 1], pd[kTok ? TS::PL : 1], pz[kTok ? TS::PL : 1];
    static_assert(!kTok || 2 * kH * int(sizeof(Tin)) <= 16 * TS::PL, "shared Δraw steps fit");
    const int64_t dw0 = d_lo + blk * CB + (tid >> 6) * CW;   // the wave's first channel
    const bool dt_full = dtr.sd != 0;
    // 16-byte pieces need every row's start on a piece boundary
    const bool pieces_aligned = (D % TS::PIECE) == 0;
    auto load_piece = [&](const Tin* base, uint32_t off, int64_t ch0) -> uint4 {
        // elements [off, off + PIECE) of a row (32-bit offset from the batch row's base):
        // channels ch0 .. ch0 + PIECE - 1, those at or past d_hi read as zero
        if (pieces_aligned && ch0 + TS::PIECE <= d_hi)
            return *reinterpret_cast<const uint4*>(base + off);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if constexpr (sizeof(Tin) == 2) {
#pragma unroll
            for (int e = 0; e < TS::PIECE; ++e)
                if (ch0 + e < d_hi)
                    w[e >> 1] |= uint32_t(reinterpret_cast<const uint16_t*>(base)[off + e]) << (16 * (e & 1));
        } else {
#pragma unroll
            for (int e = 0; e < TS::PIECE; ++e)
                if (ch0 + e < d_hi) w[e] = __float_as_uint(reinterpret_cast<const float*>(base)[off + e]);
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    };

    auto issue_loads = [&](int64_t t0) {
#pragma unroll
        for (int p = 0; p < BC_PASSES; ++p) {
            const int e = tid + p * kThreads;
            if (BC_UNITS % kThreads == 0 || e < BC_UNITS) {
                if constexpr (kTok) {
                    const int q = e % NQ, tt = (e / NQ) % kTile, m = e / (NQ * kTile);
                    bc_next[p].load((m ? Cb : Bb) + (t0 + tt) * N + 4 * q);
                } else {
                    const int n = e % N, q = (e / N) % (kTile / 4), m = e / (N * (kTile / 4));
                    bc_next[p].load((m ? Cb : Bb) + int64_t(n) * L + t0 + 4 * q);
                }
            }
        }
        if constexpr (kTok) {
#pragma unroll
            for (int j = 0; j < TS::PL; ++j) {
                const int q = lane + 64 * j;
                if (TS::PIECES % 64 == 0 || q < TS::PIECES) {
                    const int row = q / TS::PPR, pc = q % TS::PPR;
                    const int64_t ch0 = dw0 + pc * TS::PIECE;
                    const uint32_t off = uint32_t(t0 + row) * D32 + uint32_t(ch0);
                    px[j] = load_piece(xb, off, ch0);
                    if (dt_full) pd[j] = load_piece(db, off, ch0);
                    if (kGate && !kAgg) pz[j] = load_piece(zb, off, ch0);
                }
            }
            if (!dt_full) {
                uint32_t* w = reinterpret_cast<uint32_t*>(pd);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t o = uint32_t(t0 + kHalf * hh + kH * l) * dts32 + dofs;
#pragma unroll
                    for (int i = 0; i < kH; ++i) {
                        const int e = hh * kH + i;           // element of the packed run
                        if constexpr (sizeof(Tin) == 2) {
                            const uint32_t v = uint32_t(reinterpret_cast<const uint16_t*>(db)[o + i * dts32]);
                            w[e >> 1] = (e & 1) ? (w[e >> 1] | (v << 16)) : v;
                        } else {
                            w[e] = __float_as_uint(reinterpret_cast<const float*>(db)[o + i * dts32]);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int64_t te = t0 + kHalf * hh + kH * l;
                xn[hh].load(xr + te);
                dn[hh].load(dr + te);
                if (kGate && !kAgg) zn[hh].load(zr + te);
            }
        }
    };

    if (n_tiles > 0) issue_loads(t_begin);
    float* wa = w_lds + (tid >> 6) * WAREA;       // this wave's exchange area
    float* dd_row = wa + c * kDS;                 // (δ, δ·x) of this lane's channel
    float* mine = wa + lane * kPS;                // this lane's partial readouts

    // the tile loop in two copies, the power path and the general one, chosen once per wave
    // (separate copies keep either one's registers to what it needs alone)
    auto run_tiles = [&](auto pw) {
        constexpr bool kPow = decltype(pw)::value && kDpp;
        // the aggregate pass on the power path sums weighted inputs instead of running the
        // recurrence: over a 16-step half, h_n ← e^{-(n+1)Δ}·h_n + Σ_t e^{-(n+1)R_t}·δ_t x_t·B_{t,n},
        // Δ the half's Σδ and R_t the Σδ of the half's steps after t (the products of Ā over
        // the steps after t, §2.2's pair composed over the half): the weight of a lane's next
        // state is the previous one times e^{-R_t}, so a state costs one product and one FMA
        constexpr bool kRev = kPow && kAgg;
        for (int64_t it = 0; it < n_tiles; ++it) {
            const int64_t t0 = t_begin + it * kTile;
            float* buf = lds + (it & 1) * TILE_F;
#pragma unroll
            for (int p = 0; p < BC_PASSES; ++p) {
                const int e = tid + p * kThreads;
                if (BC_UNITS % kThreads == 0 || e < BC_UNITS) {
                    if constexpr (kTok) {
                        const int q = e % NQ, tt = (e / NQ) % kTile, m = e / (NQ * kTile);
                        *reinterpret_cast<float4*>(buf + tt * R + m * N + 4 * q) =
                            make_float4(bc_next[p].get(0), bc_next[p].get(1), bc_next[p].get(2),
                                        bc_next[p].get(3));
                    } else {
                        const int n = e % N, q = (e / N) % (kTile / 4), m = e / (N * (kTile / 4));
                        float* dst = buf + 4 * q * R + m * N + n;
#pragma unroll
                        for (int i = 0; i < 4; ++i) dst[i * R] = bc_next[p].get(i);
                    }
                }
            }
            float xv[2][kH], dv[2][kH], zv[2][kH];
            if constexpr (kTok) {
                // the wave's pieces into its own area as rows, then each lane's kH steps of its
                // channel from there (the area is free: the last sweep's gathers are done)
                char* st = reinterpret_cast<char*>(wa);
#pragma unroll
                for (int j = 0; j < TS::PL; ++j) {
                    const int q = lane + 64 * j;
                    if (TS::PIECES % 64 == 0 || q < TS::PIECES) {
                        const int row = q / TS::PPR, pc = q % TS::PPR;
                        char* dst = st + row * TS::RSB + pc * 16;
                        *reinterpret_cast<uint4*>(dst) = px[j];
                        if (dt_full) *reinterpret_cast<uint4*>(dst + TS::TBYTES) = pd[j];
                        if (kGate && !kAgg) *reinterpret_cast<uint4*>(dst + 2 * TS::TBYTES) = pz[j];
                    }
                }
                wave_sync();
                const char* src = st + c * TS::ELEM;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                    for (int i = 0; i < kH; ++i) {
                        const char* e = src + (kHalf * hh + kH * l + i) * TS::RSB;
                        if constexpr (sizeof(Tin) == 2) {
                            xv[hh][i] = __uint_as_float(uint32_t(*reinterpret_cast<const uint16_t*>(e)) << 16);
                            if (dt_full)
                                dv[hh][i] = __uint_as_float(
                                    uint32_t(*reinterpret_cast<const uint16_t*>(e + TS::TBYTES)) << 16);
                            if (kGate && !kAgg)
                                zv[hh][i] = __uint_as_float(
                                    uint32_t(*reinterpret_cast<const uint16_t*>(e + 2 * TS::TBYTES)) << 16);
                        } else {
                            xv[hh][i] = *reinterpret_cast<const float*>(e);
                            if (dt_full) dv[hh][i] = *reinterpret_cast<const float*>(e + TS::TBYTES);
                            if (kGate && !kAgg) zv[hh][i] = *reinterpret_cast<const float*>(e + 2 * TS::TBYTES);
                        }
                    }
                    if (!dt_full) {
                        const uint32_t* w = reinterpret_cast<const uint32_t*>(pd);
#pragma unroll
                        for (int i = 0; i < kH; ++i) {
                            const int e = hh * kH + i;
                            dv[hh][i] = (sizeof(Tin) == 2)
                                            ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16))
                                            : __uint_as_float(w[e]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    xn[hh].decode(xv[hh]);
                    dn[hh].decode(dv[hh]);
                    if (kGate && !kAgg) zn[hh].decode(zv[hh]);
                }
                // kWiden: widen here, before the next tile's loads reuse the raw registers (left
                // to itself the compiler widens at the first use and keeps a copy of every raw
                // register across the loads: two moves per raw register per tile).  The widened
                // values take more registers until they are used, so only where that leaves the
                // occupancy as it was.
                if constexpr (kWiden) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int i = 0; i < kH; ++i) {
                            asm volatile("" : "+v"(xv[hh][i]), "+v"(dv[hh][i]));
                            if (kGate && !kAgg) asm volatile("" : "+v"(zv[hh][i]));
                        }
                }
            }
            if (it + 1 < n_tiles) issue_loads(t0 + kTile);
            __syncthreads();

#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if (ckr) checkpoint(t0 + kHalf * hh);      // sweeps start on multiples of 16
                // this lane's kH steps of the half: (δ, δ·x) into the channel's row (or kept in
                // registers for the quad broadcast)
                float qdl[kH], qdx[kH], qr[kH];
#pragma unroll
                for (int i = 0; i < kH; ++i) {
                    const float dl = softplus(bias + dv[hh][i]);
                    if (kAgg) dsum += dl;
                    qdl[i] = dl;
                    qdx[i] = dl * xv[hh][i];
                    if constexpr (!kDpp)
                        *reinterpret_cast<float2*>(dd_row + 2 * (kH * l + i)) =
                            make_float2(dl, kZoh ? xv[hh][i] : qdx[i]);
                }
                float qR[kRev ? kH : 1];
                if constexpr (kRev) {
                    // R of this lane's steps: its own later steps, then the later lanes' totals
                    // (quad lanes l+1.., which own the half's later steps)
                    float e = 0.0f;
#pragma unroll
                    for (int i = kH - 1; i >= 0; --i) { qR[i] = e; e += qdl[i]; }
                    const float n1 = qperm<0xF9>(e);                 // quad lane l + 1
                    const float s1 = (l < 3) ? n1 : 0.0f;
                    const float n2 = qperm<0xFE>(e + s1);            // quad lanes l + 2, l + 3
                    const float later = s1 + ((l < 2) ? n2 : 0.0f);
#pragma unroll
                    for (int i = 0; i < kH; ++i) {
                        qR[i] += later;
                        qr[i] = exp2_hw(-qR[i] * kLog2e);   // e^{-R}
                    }
                    // the state entering the half decays by e^{-(n+1)Δ}
                    const float tot = qperm<0x00>(e + later);        // Δ, from quad lane 0
                    float E = exp2_hw(tot * A2[0]);
                    const float eD = exp2_hw(-tot * kLog2e);
#pragma unroll
                    for (int s2 = 0; s2 < S; ++s2) {
                        h[s2] *= E;
                        if (s2 + 1 < S) E *= eD;
                    }
                } else if constexpr (kPow) {
#pragma unroll
                    for (int i = 0; i < kH; ++i) qr[i] = exp2_hw(-qdl[i] * kLog2e);   // e^{-δ}
                }
                if constexpr (!kDpp) wave_sync();

                // recurrence over the half; operands of step t+1 are read during step t
                const float* bh = buf + kHalf * hh * R;
                float part[kHalf];
                {
                    Row<S> bcur, ccur, bnxt, cnxt;
                    float2 dcur, dnxt;
                    bnxt.load(bh + n0);
                    if (!kAgg) cnxt.load(bh + N + n0);
                    if constexpr (!kDpp) dnxt = *reinterpret_cast<const float2*>(dd_row);
#pragma unroll
                    for (int t = 0; t < kHalf; ++t) {
                        bcur = bnxt;
                        if (!kAgg) ccur = cnxt;
                        if constexpr (kDpp) {
                            dcur.x = quad_step(qdl, t);
                            dcur.y = quad_step(qdx, t);
                        } else {
                            dcur = dnxt;
                        }
                        if (t + 1 < kHalf) {
                            bnxt.load(bh + (t + 1) * R + n0);
                            if (!kAgg) cnxt.load(bh + (t + 1) * R + N + n0);
                            if constexpr (!kDpp) dnxt = *reinterpret_cast<const float2*>(dd_row + 2 * (t + 1));
                        }
                        // the next step's LDS reads stay issued here; arithmetic may move across
                        __builtin_amdgcn_sched_barrier(0x7);
                        float acc = 0.0f;
                        if constexpr (kRev) {
                            // δ_t x_t·e^{-(n0+1)R_t}, then one product per next state
                            const float qt = quad_step(qr, t);
                            float p = exp2_hw(quad_step(qR, t) * A2[0]) * dcur.y;
#pragma unroll
                            for (int s = 0; s < S; ++s) {
                                h[s] = fmaf(p, bcur.v[s], h[s]);
                                if (s + 1 < S) p *= qt;
                            }
                        } else if constexpr (kPow) {
                            const float rt = quad_step(qr, t);
                            float abar = exp2_hw(dcur.x * A2[0]);     // r^(n0+1)
#pragma unroll
                            for (int s = 0; s < S; ++s) {
                                h[s] = fmaf(abar, h[s], dcur.y * bcur.v[s]);
                                if (!kAgg) acc = fmaf(ccur.v[s], h[s], acc);
                                if (s + 1 < S) abar *= rt;
                            }
                        } else {
#pragma unroll
                            for (int s = 0; s < S; ++s) {
                                const float t2 = dcur.x * A2[s];
                                const float abar = exp2_hw(t2);
                                // first order: dcur.y = δ·x; exact hold: dcur.y = x, times the gain
                                float bx = dcur.y * bcur.v[s];
                                if (kZoh) bx *= zoh_gain(t2, abar, dcur.x, iA[s]);
                                h[s] = fmaf(abar, h[s], bx);
                                if (!kAgg) acc = fmaf(ccur.v[s], h[s], acc);
                            }
                        }
                        part[t] = acc;
                    }
                }
                // every lane's reads of the rows are done before partials land
                if constexpr (!kDpp) wave_sync();

                if (!kAgg) {
                    // partial readouts through the wave's area: each lane writes its 16, then
                    // gathers the G partials of its own kH steps
#pragma unroll
                    for (int q = 0; q < kHalf; q += 4)
                        *reinterpret_cast<float4*>(mine + q) =
                            make_float4(part[q], part[q + 1], part[q + 2], part[q + 3]);
                    wave_sync();
                    float sum[kH];
                    const int gbase = lane & ~(G - 1);
                    // lane l starts at source l (rotation): lanes served together read
                    // different source rows; the first row starts the sums (no 0 + x)
#pragma unroll
                    for (int r = 0; r < G; ++r) {
                        const int src = (l + r) & (G - 1);
                        Row<kH> pr;
                        pr.load(wa + (gbase + src) * kPS + kH * l);
#pragma unroll
                        for (int i = 0; i < kH; ++i) sum[i] = r ? sum[i] + pr.v[i] : pr.v[i];
                    }
                    float out[kH];
#pragma unroll
                    for (int i = 0; i < kH; ++i) {
                        float sv = fmaf(Dd, xv[hh][i], sum[i]);
                        if (kGate) sv *= silu(zv[hh][i]);
                        out[i] = sv;
                    }
                    if (valid) {
                        const int64_t te = t0 + kHalf * hh + kH * l;
                        if constexpr (kTok) {
                            const uint32_t o = uint32_t(te) * D32 + d32;
#pragma unroll
                            for (int i = 0; i < kH; ++i) yb[o + uint32_t(i) * D32] = out[i];
                        } else {
                            store_k<kH>(yr + te, out);
                        }
                    }
                    wave_sync();  // gathers done before the next half's rows overwrite the area
                }
            }
        }
    };
    if constexpr (kDpp && kMayPow) {
        if (pow_path) run_tiles(std::true_type{});
        else run_tiles(std::false_type{});
    } else {
        run_tiles(std::false_type{});
    }

    // tail: the last (t_end - t_tiles_end) < 32 steps, one step at a time; every lane
    // prepares the step itself and reads its B/C straight from the inputs
    for (int64_t t = t_tiles_end; t < t_end; ++t) {
        if (ckr && t % kCkptSteps == 0) checkpoint(t);
        const float xt = to_f32(xr[t * ts]);
        const float delta = softplus(bias + to_f32(dr[t * dts]));
        const float dxt = delta * xt;
        if (kAgg) dsum += (l == 0) ? delta : 0.0f;
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const float t2 = delta * A2[s];
            const float abar = exp2_hw(t2);
            const int64_t bci = kTok ? t * N + n0 + s : int64_t(n0 + s) * L + t;
            float bx = (kZoh ? xt : dxt) * to_f32(Bb[bci]);
            if (kZoh) bx *= zoh_gain(t2, abar, delta, iA[s]);
            h[s] = fmaf(abar, h[s], bx);
            if (!kAgg) acc = fmaf(to_f32(Cb[bci]), h[s], acc);
        }
        if (!kAgg) {
            acc = group_sum<G>(acc);
            float sv = fmaf(Dd, xt, acc);
            if (kGate) sv *= silu(to_f32(zr[t * ts]));
            if (valid && l == 0) yr[t * ts] = sv;
        }
    }

    if (kAgg) {
        dsum = group_sum<G>(dsum);
        const int64_t aidx = (int64_t(b) * D + d) * K + k;
        if (valid) {
#pragma unroll
            for (int s = 0; s < S; ++s) h_last[aidx * N + n0 + s] = h[s];
            if (l == 0) dsum_out[aidx] = dsum;
        }
    } else if (h_last && k == K - 1 && valid) {
        const int64_t fidx = (int64_t(b) * D + d) * N + n0;
#pragma unroll
        for (int s = 0; s < S; ++s) h_last[fidx + s] = h[s];
    }
}

// grid = (ceil(D / (256/G)), K, B), block = 256.
template <typename Tin, int G, int S, bool kGate, bool kAgg, bool kZoh, bool kTok>
__global__ __launch_bounds__(kThreads) void scang_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const Tin* __restrict__ Bm, const Tin* __restrict__ Cm,
    const float* __restrict__ h_init, float* __restrict__ y, float* __restrict__ h_last,
    float* __restrict__ h_ckpt, float* __restrict__ dsum_out, int64_t L, int64_t D,
    int64_t chunk, int K, DtRows dtr) {
    __shared__ __align__(16) float lds[GroupLds<G, S, Tin, kTok>::FLOATS];
    // early widening (see scang_body) except in the gated bf16 output pass, where it would
    // cost a wave per SIMD
    constexpr bool kWiden = kAgg || !kGate || sizeof(Tin) == 4;
    scang_body<Tin, G, S, kGate, kAgg, kZoh, kTok, true, kWiden>(lds, blockIdx.x, blockIdx.y, blockIdx.z, 0, D, x,
                                                   dt_raw, z, dt_bias, A, Dskip, Bm, Cm, h_init, y,
                                                   h_last, h_ckpt, dsum_out, L, D, chunk, K, dtr);
}

// Single pass over every channel with two layouts in one launch: per batch row, channels
// [0, d4) on four lanes (64 per workgroup) and [d4, D) on eight lanes (32 per workgroup).
// The workgroups are numbered four-lane first, so a round-robin dispatch hands each CU its
// four-lane workgroups and then its eight-lane one: whole rounds of four-lane waves per
// SIMD, the remainder as eight-lane waves that take about half a four-lane wave's time.
// grid = B * (nb4 + nb8), block = 256.
template <typename Tin, int N, bool kGate, bool kZoh, bool kTok>
__global__ __launch_bounds__(kThreads) void scang_mixed_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ dt_raw, const Tin* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const Tin* __restrict__ Bm, const Tin* __restrict__ Cm,
    const float* __restrict__ h_init, float* __restrict__ y, float* __restrict__ h_last,
    float* __restrict__ h_ckpt, int64_t L, int64_t D, int64_t d4, int nb4, int nb8, int B,
    DtRows dtr) {
    constexpr int F4 = GroupLds<4, N / 4, Tin, kTok>::FLOATS, F8 = GroupLds<8, N / 8, Tin, kTok>::FLOATS;
    __shared__ __align__(16) float lds[F4 > F8 ? F4 : F8];
    const int64_t f = blockIdx.x;
    const int64_t n4 = int64_t(B) * nb4;
    // early widening of the raw inputs keeps both layouts' occupancy at N = 16 with the
    // first-order hold (measured resource use; other shapes would lose a wave per SIMD)
    constexpr bool kWiden = N == 16 && !kZoh;
    if (f < n4) {
        scang_body<Tin, 4, N / 4, kGate, false, kZoh, kTok, false, kWiden>(
            lds, f % nb4, 0, int(f / nb4), 0, d4, x, dt_raw, z, dt_bias, A, Dskip, Bm, Cm, h_init,
            y, h_last, h_ckpt, nullptr, L, D, L, 1, dtr);
    } else {
        const int64_t g = f - n4;
        scang_body<Tin, 8, N / 8, kGate, false, kZoh, kTok, true, kWiden>(
            lds, g % nb8, 0, int(g / nb8), d4, D, x, dt_raw, z, dt_bias, A, Dskip, Bm, Cm, h_init,
            y, h_last, h_ckpt, nullptr, L, D, L, 1, dtr);
    }
}

template <typename Tin, int N>
static hipError_t launch_scang_mixed_t(const ScanLaunch& p, hipStream_t s) {
    const int nb8 = int((p.D - p.d4 + 31) / 32);
    dim3 grid(unsigned(p.B * (p.nb4 + nb8)));
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
    const Tin* Bm = static_cast<const Tin*>(p.Bm);
    const Tin* Cm = static_cast<const Tin*>(p.Cm);
    return with_bool(p.z != nullptr, [&](auto gate) {
        return with_bool(p.zoh != 0, [&](auto zoh) {
            return with_bool(p.tok != 0, [&](auto tok) {
                hipLaunchKernelGGL((scang_mixed_kernel<Tin, N, gate.value, zoh.value, tok.value>),
                                   grid, dim3(kThreads), 0, s, x, dr, z, p.dt_bias, p.A, p.Dskip,
                                   Bm, Cm, p.h_init, p.y, p.h_last, p.h_ckpt, p.L, p.D, p.d4, p.nb4,
                                   nb8, int(p.B), p.dtr);
                return hipGetLastError();
            });
        });
    });
}

template <typename Tin, int G, int S>
static hipError_t launch_scang_t(const ScanLaunch& p, hipStream_t s) {
    constexpr int CB = 4 * 64 / G;
    // the last chunk's aggregate has no successor: the carry reads it only into values it
    // never stores (the final state comes from the output pass), so it is not computed
    const unsigned kg = unsigned((p.agg && p.K > 1) ? p.K - 1 : p.K);
    dim3 grid(unsigned((p.D + CB - 1) / CB), kg, unsigned(p.B));
    const Tin* x = static_cast<const Tin*>(p.x);
    const Tin* dr = static_cast<const Tin*>(p.dt_raw);
    const Tin* z = static_cast<const Tin*>(p.z);
    const Tin* Bm = static_cast<const Tin*>(p.Bm);
    const Tin* Cm = static_cast<const Tin*>(p.Cm);
    return with_bool(p.zoh != 0, [&](auto zoh) {
        return with_bool(p.tok != 0, [&](auto tok) {
            auto go = [&](auto gate, auto agg) {
                hipLaunchKernelGGL(
                    (scang_kernel<Tin, G, S, gate.value, agg.value, zoh.value, tok.value>), grid,
                    dim3(kThreads), 0, s, x, dr, z, p.dt_bias, p.A, p.Dskip, Bm, Cm, p.h_init, p.y,
                    p.h_last, p.h_ckpt, p.dsum, p.L, p.D, p.chunk, p.K, p.dtr);
                return hipGetLastError();
            };
            // the aggregate pass has no gate
            if (p.agg) return go(std::false_type{}, std::true_type{});
            if (p.z) return go(std::true_type{}, std::false_type{});
            return go(std::false_type{}, std::false_type{});
        });
    });
}

template <typename Tin>
static hipError_t launch_scang_dt(int N, int G, const ScanLaunch& p, hipStream_t s) {
    if (G == 4) {
        switch (N) {
            case 4: return launch_scang_t<Tin, 4, 1>(p, s);
            case 8: return launch_scang_t<Tin, 4, 2>(p, s);
            case 16: return launch_scang_t<Tin, 4, 4>(p, s);
            case 32: return launch_scang_t<Tin, 4, 8>(p, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (G == 8) {
        switch (N) {
            case 8: return launch_scang_t<Tin, 8, 1>(p, s);
            case 16: return launch_scang_t<Tin, 8, 2>(p, s);
            case 32: return launch_scang_t<Tin, 8, 4>(p, s);
            case 64: return launch_scang_t<Tin, 8, 8>(p, s);
            default: return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scang(int bf16, int N, int G, const ScanLaunch& p, hipStream_t s) {
    return bf16 ? launch_scang_dt<bf16_t>(N, G, p, s) : launch_scang_dt<float>(N, G, p, s);
}

template <typename Tin>
static hipError_t launch_scang_mixed_dt(int N, const ScanLaunch& p, hipStream_t s) {
    switch (N) {
        case 8: return launch_scang_mixed_t<Tin, 8>(p, s);
        case 16: return launch_scang_mixed_t<Tin, 16>(p, s);
        case 32: return launch_scang_mixed_t<Tin, 32>(p, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_scang_mixed(int bf16, int N, const ScanLaunch& p, hipStream_t s) {
    return bf16 ? launch_scang_mixed_dt<bf16_t>(N, p, s) : launch_scang_mixed_dt<float>(N, p, s);
}

}  // namespace ss
