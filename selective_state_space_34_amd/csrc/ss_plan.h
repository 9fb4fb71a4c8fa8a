// Plan choice and workspace layout of the selective-scan library.  Host-only,
// HIP-free: everything here depends on the dims alone, so the same dims always
// give the same plan and the same workspace size.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ss.h"

namespace ss {

struct Plan {
    int64_t B, L, D, N;
    int in_dtype;
    int chunked;     // forward: 0 = single pass, 1 = chunked; backward: always 1
    int64_t chunk;   // steps per chunk (multiple of 8 unless chunk == L)
    int64_t K;       // number of chunks
    int vec;         // L % 8 == 0: 8-step vector loads
    int group;       // forward: lanes per channel of the group kernel (4 or 8), 0 = one lane
    int mixed;       // forward, single pass: four lanes for channels [0, d4), eight for the rest
    int64_t d4;
    int nb4;         // four-lane workgroups per batch row (d4 / 64)
    int zoh;         // exact zero-order-hold input term
    int tok;         // token-major x, z, y, dy, dx, dz [B, L, D] and B, C, dB, dC [B, L, N]
    int dt_shared;   // Δraw one value per token [B, L]
    // workspace carving (byte offsets, 256-aligned)
    //   forward:  off_bc    [B, L, 2N] B|C staging (one-lane kernel)
    //             off_hend  [B, D, K, N] chunk end states, off_dsum [B, D, K] Σδ per chunk,
    //             off_hstart [B, D, K, N] chunk start states (chunked plan)
    //   backward: off_hend  forward pairs -> start states -> dA partials, off_dsum,
    //             off_gend  [B, D, K, N] reverse pairs -> adjoints entering from the right,
    //             off_bcpart [B, NB, L, 2N] dB|dC partials of NB = ceil(D / 64) channel blocks,
    //             off_dtpart [B, D, K, 2] dD, ddt_bias partials,
    //             off_ddt   [B, NB, L] block sums of a shared Δraw's gradient
    size_t off_bc, off_hend, off_dsum, off_hstart, off_gend, off_bcpart, off_dtpart, off_ddt;
    size_t ws_total;
};

// Channels per workgroup of the backward kernels (16 per wave, four waves).
constexpr int64_t kBwdChan = 64;

constexpr int64_t kMaxGridYZ = 65535;

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline bool mul_ok(int64_t a, int64_t b, int64_t lim) { return a > 0 && b > 0 && a <= lim / b; }

// Target number of 64-lane waves for the sequence-parallel plans: sixteen per SIMD of a
// 256-CU, 4-SIMD part, several rounds of resident waves.  Measured against four per SIMD (one
// round): the 2^20-step, 256-channel forward 1654 -> 1596 us with 1024-step instead of 4096-step
// chunks, the 4096-step, 2048-channel forward 230 -> 220 us with 128-step instead of 512-step.
constexpr int64_t kTargetWaves = 16384;
// Single pass when one pass already yields two waves per SIMD (a chunked pass costs a
// second sweep for the chunk aggregates).
constexpr int64_t kSingleWaves = 2048;
// SIMDs of the part (256 CUs x 4): one round of waves
constexpr int64_t kSimds = 1024;

// Channel blocks of the backward (each leaves one row of dB|dC partials per batch row).
inline int64_t bwd_reduce_blocks(const Plan& p) { return (p.D + kBwdChan - 1) / kBwdChan; }

// What the plan is for: the sequence forward, the backward, or the single-token step (which
// uses only the validated sizes and flags, none of the sequence kernels' tiling).
enum PlanFor { kPlanFwd, kPlanBwd, kPlanStep };

inline int make_plan(const ss_dims& d, PlanFor what, Plan* out) {
    const bool backward = what == kPlanBwd;
    Plan p{};
    if (d.in_dtype != SS_F32 && d.in_dtype != SS_BF16) return SS_ERR_DTYPE;
    if (d.plan != SS_PLAN_AUTO && d.plan != SS_PLAN_SINGLE && d.plan != SS_PLAN_CHUNKED)
        return SS_ERR_DTYPE;
    if (d.layout != SS_LAYOUT_AUTO && d.layout != SS_LAYOUT_QUAD && d.layout != SS_LAYOUT_LANE &&
        d.layout != SS_LAYOUT_OCT)
        return SS_ERR_DTYPE;
    if (d.disc != SS_DISC_EULER && d.disc != SS_DISC_ZOH) return SS_ERR_DTYPE;
    if (d.order != SS_ORDER_BDL && d.order != SS_ORDER_BLD) return SS_ERR_DTYPE;
    if (d.dt_layout != SS_DT_FULL && d.dt_layout != SS_DT_SHARED) return SS_ERR_DTYPE;
    if (d.batch <= 0 || d.seqlen <= 0 || d.dim <= 0 || d.dstate <= 0) return SS_ERR_DIMS;
    const int64_t N = d.dstate;
    if (N != 1 && N != 2 && N != 4 && N != 8 && N != 16 && N != 32 && N != 64) return SS_ERR_DIMS;
    // N = 64: the forward on eight lanes of eight states only (one lane per channel or four
    // lanes would hold 64 or 16 states and their B/C operands per lane), no backward (its
    // tile of 16 recomputed states per lane would need 256 registers)
    if (N == 64 && (backward || d.layout == SS_LAYOUT_LANE || d.layout == SS_LAYOUT_QUAD))
        return SS_ERR_UNSUPPORTED;
    if (d.chunk < 0 || (d.chunk % 8) != 0) return SS_ERR_DIMS;
    const int64_t lim = int64_t(1) << 40;  // element count bound of any one array
    if (!mul_ok(d.batch, d.dim, lim) || !mul_ok(d.batch * d.dim, d.seqlen, lim) ||
        !mul_ok(d.batch * d.dstate, d.seqlen, lim) || !mul_ok(d.batch * d.dim, N, lim))
        return SS_ERR_DIMS;
    if (d.batch > kMaxGridYZ) return SS_ERR_DIMS;
    p.B = d.batch; p.L = d.seqlen; p.D = d.dim; p.N = N; p.in_dtype = d.in_dtype;
    p.zoh = d.disc == SS_DISC_ZOH;
    p.tok = d.order == SS_ORDER_BLD;
    p.dt_shared = d.dt_layout == SS_DT_SHARED;
    p.vec = (p.L % 8) == 0;
    // layout: a group of G lanes per channel (G x the waves of one lane per channel).
    // Automatic choice: four lanes wherever they apply.  Measured on MI355X, eight lanes
    // balance the SIMDs better at B*D = 40960 but saturate the LDS (their operand
    // traffic per state-step is higher) and lose on every workload; one lane per channel
    // loses on every workload too.
    // (token-major rows are read element by element, so only channel-major needs L % 8;
    // token-major offsets within a batch row are 32-bit: L·D < 2^31)
    const bool tile_ok = p.tok ? p.L * p.D < (int64_t(1) << 31) : p.vec != 0;
    const int gmax = !tile_ok ? 0 : N >= 8 ? 8 : N >= 4 ? 4 : 0;
    if (d.layout == SS_LAYOUT_LANE) p.group = 0;
    else if (d.layout == SS_LAYOUT_OCT || N == 64) p.group = gmax;
    else p.group = gmax >= 4 ? 4 : 0;
    // N = 64 rows the eight-lane kernel cannot tile (channel-major L % 8 != 0, token-major
    // L·D >= 2^31) would need the one-lane kernel
    if (N == 64 && p.group != 8 && what != kPlanStep) return SS_ERR_UNSUPPORTED;
    const int64_t waves = p.group ? (p.B * p.D * p.group + 63) / 64 : (p.B * p.D + 63) / 64;
    int chunked = backward ? 1 : 0;
    if (!backward) {
        if (d.plan == SS_PLAN_CHUNKED) chunked = 1;
        else if (d.plan == SS_PLAN_SINGLE) chunked = 0;
        else chunked = (waves < kSingleWaves && p.L > 512) ? 1 : 0;
    }
    int64_t chunk = p.L;
    if (backward) {
        // 16-step tiles, at most four per chunk (tile start states live in LDS)
        if (d.chunk > 0 && (d.chunk % 16 != 0 || d.chunk > 64)) return SS_ERR_DIMS;
        chunk = d.chunk > 0 ? d.chunk : 64;
        if (chunk > p.L) chunk = (p.L + 15) / 16 * 16;
    } else if (chunked) {
        if (d.chunk > 0) {
            chunk = d.chunk;
        } else {
            int64_t K = (kTargetWaves + waves - 1) / waves;
            int64_t c = (p.L + K - 1) / K;
            const int64_t cmin = backward ? 64 : 128;
            if (c < cmin) c = cmin;
            // whole 32-step tiles for the group kernel (no per-step tail; checkpoints at its
            // 16-step sweep starts)
            chunk = p.group ? (c + 31) / 32 * 32 : (c + 7) / 8 * 8;
        }
        if (chunk > p.L) chunk = (p.L + 7) / 8 * 8;
    }
    p.chunked = chunked;
    p.chunk = chunk;
    // Mixed layout for a single pass whose four-lane waves leave a last round at most half
    // full: the whole rounds stay on four lanes, the remainder goes to eight lanes (twice the
    // waves, each about half as long), so every SIMD ends up with about the same work.  Used
    // when the whole rounds split evenly over batch rows into 64-channel workgroups.
    p.mixed = 0; p.d4 = 0; p.nb4 = 0;
    if (!backward && !chunked && d.layout == SS_LAYOUT_AUTO && p.group == 4 && N >= 8) {
        const int64_t U = p.B * ((p.D + 15) / 16);       // four-lane waves
        const int64_t full = U / kSimds, rem = U % kSimds;
        if (full >= 1 && rem > 0 && 2 * rem <= kSimds && (full * kSimds) % (4 * p.B) == 0) {
            const int64_t nb4 = full * kSimds / (4 * p.B);
            if (nb4 * 64 < p.D) { p.mixed = 1; p.nb4 = int(nb4); p.d4 = nb4 * 64; }
        }
    }
    p.K = (p.L + chunk - 1) / chunk;
    if (p.K > kMaxGridYZ) return SS_ERR_DIMS;

    size_t off = 0;
    p.off_bc = off;
    // [B, L, 2N] float32 copy of B and C: the one-lane forward kernel only
    if (!backward && !p.group) off = align256(off + size_t(p.B) * size_t(p.L) * size_t(2 * N) * sizeof(float));
    p.off_hend = p.off_dsum = p.off_hstart = p.off_gend = p.off_bcpart = p.off_dtpart = 0;
    if (chunked) {
        const size_t st = size_t(p.B) * size_t(p.K) * size_t(p.D) * size_t(N) * sizeof(float);
        const size_t sm = size_t(p.B) * size_t(p.K) * size_t(p.D) * sizeof(float);
        p.off_hend = off; off = align256(off + st);
        p.off_dsum = off; off = align256(off + sm);
        if (backward) {
            // the carries run in place: no separate start-state buffers
            p.off_gend = off; off = align256(off + st);
            p.off_bcpart = off;
            off = align256(off + size_t(p.B) * size_t(bwd_reduce_blocks(p)) * size_t(p.L) *
                                     size_t(2 * N) * sizeof(float));
            p.off_dtpart = off; off = align256(off + size_t(p.B) * size_t(p.K) * size_t(p.D) * 2 * sizeof(float));
        } else {
            p.off_hstart = off; off = align256(off + st);
        }
    }
    // shared Δraw: the backward's per-64-channel-block sums of its gradient [B, ceil(D/64), L]
    p.off_ddt = 0;
    if (backward && p.dt_shared) {
        p.off_ddt = off;
        off = align256(off + size_t(p.B) * size_t(bwd_reduce_blocks(p)) * size_t(p.L) * sizeof(float));
    }
    p.ws_total = off;
    *out = p;
    return SS_OK;
}

// Selection projection of the block ([Δ | B | C] = x · W_xᵀ): token tiles per wave, splits of
// the K = D sum over workgroups and their length (whole 64-step LDS tiles).
constexpr int64_t kXprojK = 64;
inline int xproj_mt(int N) { return N <= 16 ? 2 : 1; }
inline int64_t xproj_splits(int64_t M, int64_t D, int N) {
    // about 768 workgroups in all (one round at three workgroups per CU, which the kernel's
    // LDS tiles and registers allow for N = 16), each split at least 64 steps of K
    const int64_t tok = 64 * xproj_mt(N);        // tokens per workgroup
    const int64_t mb = (M + tok - 1) / tok;
    int64_t S = (768 + mb - 1) / mb;
    if (S > D / 64) S = D / 64;
    return S < 1 ? 1 : S;
}
inline int64_t xproj_split_len(int64_t D, int64_t S) {
    return ((D + S - 1) / S + kXprojK - 1) / kXprojK * kXprojK;
}

// Workspace carving of ss_block_fwd: every intermediate, the projection partials and the
// scan's own workspace.  Depends on the dims alone.
struct BlockPlan {
    int64_t M, Din, D, N, S;
    ss_dims sd;                 // the scan: float32, token-major, Δraw shared
    size_t off_x, off_z, off_dt, off_B, off_C, off_part, off_scan, scan_ws, total;
};

inline int make_block_plan(const ss_block_dims& bd, BlockPlan* out) {
    BlockPlan bp{};
    if (bd.batch <= 0 || bd.seqlen <= 0 || bd.d_in <= 0 || bd.dim <= 0 || bd.dstate <= 0)
        return SS_ERR_DIMS;
    if (bd.d_in % 8 != 0 || bd.dim % 4 != 0) return SS_ERR_DIMS;
    const int64_t lim = int64_t(1) << 40;
    if (bd.batch > lim / bd.seqlen) return SS_ERR_DIMS;
    bp.M = bd.batch * bd.seqlen; bp.Din = bd.d_in; bp.D = bd.dim; bp.N = bd.dstate;
    if (bp.M > lim / bp.Din || bp.M > lim / (2 * bp.D)) return SS_ERR_DIMS;
    bp.sd = ss_dims{bd.batch, bd.seqlen, bd.dim, bd.dstate, SS_F32, bd.plan, 0, bd.layout,
                    SS_DISC_EULER, SS_ORDER_BLD, SS_DT_SHARED};
    Plan p;
    const int rc = make_plan(bp.sd, kPlanFwd, &p);
    if (rc != SS_OK) return rc;
    bp.S = xproj_splits(bp.M, bp.D, int(bp.N));
    const size_t f = sizeof(float);
    const size_t MD = size_t(bp.M) * size_t(bp.D), MN = size_t(bp.M) * size_t(bp.N);
    size_t off = 0;
    bp.off_x = off; off = align256(off + MD * f);
    bp.off_z = off; off = align256(off + MD * f);
    bp.off_dt = off; off = align256(off + size_t(bp.M) * f);
    bp.off_B = off; off = align256(off + MN * f);
    bp.off_C = off; off = align256(off + MN * f);
    bp.off_part = off;
    off = align256(off + size_t(bp.S) * size_t(bp.M) * size_t(1 + 2 * bp.N) * f);
    bp.off_scan = off; bp.scan_ws = p.ws_total; off = align256(off + p.ws_total);
    bp.total = off;
    *out = bp;
    return SS_OK;
}

}  // namespace ss
