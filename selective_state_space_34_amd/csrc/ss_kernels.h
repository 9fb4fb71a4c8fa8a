// Internal launch interface between the C-ABI layer (ss_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ss {

// Steps between the forward's state checkpoints (the backward's tile length).
constexpr int kCkptSteps = 16;

// Where channel (b, d)'s Δraw values lie: element t at dt_raw[b·sb + d·sd + t·ts].
//   [B, D, L]: (D·L, L, 1);  [B, L, D]: (L·D, 1, D);  one value per token [B, L]: (L, 0, 1).
struct DtRows {
    int64_t sb, sd, ts;
};

// Calls f(std::integral_constant<bool, v>): a runtime flag as a template argument.
template <typename F>
inline hipError_t with_bool(bool v, F&& f) {
    return v ? f(std::true_type{}) : f(std::false_type{});
}

struct ScanLaunch {
    const void* x;
    const void* dt_raw;
    const void* z;          // nullable (no gate); ignored in AGG mode
    const float* dt_bias;
    const float* A;
    const float* Dskip;
    const float* BC;        // [B, L, 2N] float32 staging copy of B and C (one-lane kernel)
    const void* Bm;         // [B, N, L] inputs (group kernel)
    const void* Cm;
    const float* h_init;    // nullable; [B, D, K, N]
    float* y;               // OUT mode
    float* h_last;          // OUT: h_final (nullable); AGG: h_end [B, D, K, N]
    float* h_ckpt;          // OUT: nullable; [B, D, ceil(L / kCkptSteps), N]: state entering
                            // every kCkptSteps-th step
    float* dsum;            // AGG: Σδ per chunk [B, D, K]
    int64_t B, L, D, chunk;
    int K;
    int vec;                // 1: L % 8 == 0, 8-step vector loads
    int agg;                // 1: AGG mode
    int64_t d4;             // mixed layout: channels [0, d4) on four lanes, [d4, D) on eight
    int nb4;                //               four-lane workgroups per batch row (d4 / 64)
    int zoh;                // 1: exact zero-order-hold B̄
    int tok;                // 1: token-major x, z, y [B, L, D] and B, C [B, L, N]
    DtRows dtr;             // Δraw rows
};

// Affine-pair carry across chunks (one workgroup per channel).  Chunk c's pair is
// (exp(A Σδ_c), h_end_c); h_start_c is the state entering chunk c in scan order
// (reverse = 1 scans chunks from last to first, for the adjoint), h_out the state
// after the last one.  h_in, h_out nullable.
struct CarryLaunch {
    const float* h_end;     // [B, D, K, N]
    const float* dsum;      // [B, D, K]
    const float* A;         // [D, N]
    const float* h_in;      // [B, D, N]
    float* h_start;         // [B, D, K, N]
    float* h_out;           // [B, D, N]
    int64_t B, D;
    int K;
    int reverse;
    // optional second set, carried in the same launch when dual = 1
    int dual;
    const float* h_end2;
    const float* h_in2;
    float* h_start2;
    float* h_out2;
    int reverse2;
};

// Backward launches (four lanes per channel).  stage 0: chunk aggregates (h_end, rev_end, dsum);
// stage 1: final pass (h_end holds chunk start states on entry and dA partials on exit,
// rev_end holds the adjoints entering each chunk from the right).
struct BwdLaunch {
    const void* x;
    const void* dt_raw;
    const void* z;
    const float* dy;
    const float* dt_bias;
    const float* A;
    const float* Dskip;
    const void* Bm;    // [B, N, L] inputs
    const void* Cm;
    const float* h_ckpt;  // nullable: the forward's checkpoints; then h_end holds only dA
    float* h_end;      // [B, D, K, N]
    float* rev_end;    // [B, D, K, N]
    float* dsum;       // [B, D, K]
    float* dbc_part;   // [B, ceil(D/64), L, 2N]
    float* ddt_part;   // [B, D, K, 2]
    float* dx;
    float* ddt_raw;
    float* dz;
    float* dA;
    float* dB;
    float* dC;
    float* dD;
    float* ddt_bias;
    int64_t B, L, D, N, chunk;
    int K;
    int vec;
    int stage;
    int tok;           // 1: token-major x, z, dy, dx, dz [B, L, D] and B, C, dB, dC [B, L, N]
    DtRows dtr;        // Δraw rows
    DtRows gdr;        // rows the per-channel Δraw gradient is written to (ddt_raw)
    int zoh;           // 1: gradients of the exact zero-order hold
    float* ddt_shared; // nullable: Δraw shared by the channels; its gradient [B, L]
    float* ddt_blk;    // with ddt_shared: per-64-channel-block sums [B, ceil(D/64), L]
};

// Single-token step: x, dt_raw, z [B, D]; Bm, Cm [B, N]; h_in, h_out [B, D, N] (may be equal).
struct StepLaunch {
    const void* x;
    const void* dt_raw;
    const void* z;          // nullable
    const float* dt_bias;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const float* h_in;
    float* h_out;
    float* y;
    int64_t B, D;
    int N;
    int zoh;                // 1: exact zero-order-hold B̄
    int dt_shared;          // 1: dt_raw [B], one value per token
};

hipError_t launch_bc_stage(int bf16, int N, const void* Bm, const void* Cm, float* BC, int64_t B,
                           int64_t L, int tok, hipStream_t s);
hipError_t launch_scan(int bf16, int N, const ScanLaunch& p, hipStream_t s);
// group-split layout: G = 4 (N in {4, 8, 16, 32}) or G = 8 (N in {8, 16, 32}); L % 8 == 0
// for channel-major inputs
hipError_t launch_scang(int bf16, int N, int G, const ScanLaunch& p, hipStream_t s);
// single pass, N in {8, 16, 32}: four lanes for channels [0, d4), eight for [d4, D)
hipError_t launch_scang_mixed(int bf16, int N, const ScanLaunch& p, hipStream_t s);
hipError_t launch_carry(int N, const CarryLaunch& p, hipStream_t s);
hipError_t launch_step(int bf16, const StepLaunch& p, hipStream_t s);
hipError_t launch_bwd(int bf16, const BwdLaunch& p, hipStream_t s);
hipError_t launch_bwd_reduce(const BwdLaunch& p, hipStream_t s);

// Block projections (ss_block.hip).  C0 | C1 = A [M, K] · W [Nc, K]ᵀ (bf16 in, fp32 out),
// split at column nsplit; K % 8 == 0, 16-byte aligned rows.
hipError_t launch_gemm_bf16_nt(const void* A, const void* W, float* C0, float* C1, int64_t M,
                               int64_t Nc, int64_t K, int64_t nsplit, int64_t ld0, int64_t ld1,
                               hipStream_t s);
// [Δ | B | C] = x [M, D] · Wx [1 + 2N, D]ᵀ (fp32) through split-K partials part
// [S, M, 1 + 2N] (S = xproj_splits, ss_plan.h); D % 4 == 0.
hipError_t launch_xproj(const float* x, const float* Wx, float* part, float* dt, float* Bm,
                        float* Cm, int64_t M, int64_t D, int N, hipStream_t s);

}  // namespace ss
