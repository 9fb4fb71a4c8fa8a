/*
 * ss.h — C ABI of the MI355X (gfx950) selective-scan (S6) library.
 *
 * The operation (sources cited by page title and section):
 *   Page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별"
 *   (booiljung.github.io) — §1.2 selection: Δ_t = softplus(parameter + per-token
 *   input); §2.1 ZOH discretisation Ā_t = exp(Δ_t A) with A diagonal; §2.2 the
 *   recurrence h_t = Ā_t h_{t-1} + B̄_t x_t as an associative scan; §1.1 readout
 *   y_t = C_t h_t; §3.2 kernel fusion (inputs in, only y out; the state never
 *   reaches HBM); §3.3 recomputation of states in the backward pass.
 *   Note "상태공간 모델(SSM)과 Mamba 아키텍처", §3: the SiLU gate branch that
 *   multiplies the scan's output.
 *
 * Per batch row b, channel d and time t (n indexes the N states):
 *   δ      = softplus(dt_bias[d] + dt_raw[b,d,t])
 *   h[n]   = exp(δ·A[d,n])·h[n] + δ·B[b,n,t]·x[b,d,t]      (first-order B̄ = Δ·B)
 *   y[b,d,t] = (Σ_n C[b,n,t]·h[n] + Dskip[d]·x[b,d,t]) · silu(z[b,d,t])   (gate optional)
 * with h = h0[b,d,:] (or 0) before t = 0 and h_final[b,d,:] = h after t = L-1.
 *
 * Layouts (dense, row-major, element strides implied by the dims; shown for the default
 * SS_ORDER_BDL and SS_DT_FULL, see ss_order and ss_dt_layout for the others):
 *   x, dt_raw, z, y, dy, dx, ddt_raw, dz : [B, D, L]
 *   Bm, Cm, dB, dC                        : [B, N, L]
 *   A, dA                                 : [D, N]
 *   dt_bias, Dskip, ddt_bias, dD          : [D]
 *   h0, h_final, dh_final, dh0            : [B, D, N]
 *   h_ckpt                                : [B, D, ceil(L / 16), N]
 * x, dt_raw, z, Bm, Cm have the dtype ss_dims.in_dtype (float32 or bfloat16);
 * every other array, including all outputs and all gradients, is float32.
 *
 * Conventions:
 *   - All pointers are device pointers (hipMalloc'd or equivalent) except the
 *     ss_dims pointer, which is a host pointer read during the call only.
 *   - The caller owns every buffer and the workspace; the library never
 *     allocates, frees or synchronises.  All work is enqueued on `stream`
 *     (0 = the null stream) and the call returns without waiting.  Calls only
 *     launch kernels (no memset, no copy), so they can be captured in a HIP graph
 *     and replayed.
 *   - Outputs are overwritten, never accumulated into (the reduced gradients
 *     dA, dB, dC, dD, ddt_bias included).  Inputs and outputs must not alias.
 *   - The library keeps no state between calls and is re-entrant; concurrent
 *     calls need distinct workspaces.
 *   - Arguments are validated before anything is launched; on an error code
 *     nothing has been enqueued.
 *   - All base pointers must be 16-byte aligned.
 */
#ifndef SS_H_
#define SS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_VERSION_MAJOR 0
#define SS_VERSION_MINOR 7

/* dtype of x, dt_raw, z, Bm, Cm */
typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/* Execution plan.
 *   SS_PLAN_AUTO    — chosen from the dims.
 *   SS_PLAN_SINGLE  — one pass, each channel's whole sequence on one lane.
 *   SS_PLAN_CHUNKED — sequence split into chunks: per-chunk aggregates, a carry
 *                     scan of the affine pairs across chunks (§2.2 operator),
 *                     then the output pass from each chunk's true start state.
 * The backward always runs chunked. */
typedef enum { SS_PLAN_AUTO = 0, SS_PLAN_SINGLE = 1, SS_PLAN_CHUNKED = 2 } ss_plan;

/* Forward lane layout.
 *   SS_LAYOUT_AUTO — chosen from the dims.
 *   SS_LAYOUT_QUAD — the N states of a channel on four lanes (N >= 4; L % 8 == 0 in the
 *                    channel-major order).
 *   SS_LAYOUT_LANE — one lane per channel; when A[d,n] = -(n+1) exactly for every
 *                    channel of a wavefront, exp(δA) is formed as powers of exp(-δ)
 *                    (checked on the device, otherwise the general path runs).
 *   SS_LAYOUT_OCT  — the N states of a channel on eight lanes (N >= 8; L % 8 == 0 in the
 *                    channel-major order).
 * A layout that does not apply to the dims falls back to the widest narrower one that does. */
typedef enum { SS_LAYOUT_AUTO = 0, SS_LAYOUT_QUAD = 1, SS_LAYOUT_LANE = 2, SS_LAYOUT_OCT = 3 } ss_layout;

/* Discretisation of the input term (page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의
 * 압축 및 선별", §2.1; Ā = exp(δA) in both).
 *   SS_DISC_EULER — B̄x = δ·B·x, the first-order form of the hold (the default).
 *   SS_DISC_ZOH   — B̄x = (exp(δA) - 1)/A · B·x, the exact zero-order hold (ss_fwd, ss_bwd
 *                   and ss_step). */
typedef enum { SS_DISC_EULER = 0, SS_DISC_ZOH = 1 } ss_disc;

/* Memory order of the sequence tensors (the pages write x as (B, L, D)).
 *   SS_ORDER_BDL — x, dt_raw, z, y, dy, dx, ddt_raw, dz [B, D, L]; B, C, dB, dC [B, N, L].
 *   SS_ORDER_BLD — token-major: x, dt_raw, z, y, dy, dx, ddt_raw, dz [B, L, D];
 *                  B, C, dB, dC [B, L, N].
 * States (h0, h_final, h_ckpt, dh0, dh_final) are [B, D, N] (h_ckpt [B, D, ceil(L/16), N])
 * in both orders. */
typedef enum { SS_ORDER_BDL = 0, SS_ORDER_BLD = 1 } ss_order;

/* Shape of dt_raw (page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별",
 * §1.2: Δ from a one-output projection of the token, broadcast over the channels).
 *   SS_DT_FULL   — one value per (batch row, channel, step), in the order above.
 *   SS_DT_SHARED — one value per (batch row, step): dt_raw and ddt_raw are [B, L] (ss_step:
 *                  [B]); each channel adds its own dt_bias. */
typedef enum { SS_DT_FULL = 0, SS_DT_SHARED = 1 } ss_dt_layout;

typedef struct ss_dims {
    int64_t batch;    /* B  >= 1 */
    int64_t seqlen;   /* L  >= 1 */
    int64_t dim;      /* D  >= 1 */
    int64_t dstate;   /* N, one of 1, 2, 4, 8, 16, 32, 64.  N = 64: ss_fwd on the eight-lane
                         layout only (layout AUTO or OCT; channel-major rows need L % 8 == 0,
                         token-major L·D < 2^31) and ss_step; ss_bwd, and the layouts and rows
                         the eight-lane kernel cannot take, return SS_ERR_UNSUPPORTED */
    int32_t in_dtype; /* ss_dtype */
    int32_t plan;     /* ss_plan */
    int64_t chunk;    /* chunk length of the chunked plan (multiple of 8; backward: multiple
                         of 16, at most 64); 0 = automatic */
    int32_t layout;   /* ss_layout (forward only) */
    int32_t disc;     /* ss_disc */
    int32_t order;    /* ss_order */
    int32_t dt_layout; /* ss_dt_layout */
} ss_dims;

/* Return codes: 0 on success, negative on error. */
enum {
    SS_OK = 0,
    SS_ERR_NULL = -1,        /* a required pointer is NULL */
    SS_ERR_DIMS = -2,        /* a dim <= 0, N unsupported, sizes overflow, or bad chunk */
    SS_ERR_DTYPE = -3,       /* in_dtype, plan, layout, disc, order or dt_layout not one of the enums */
    SS_ERR_ALIGN = -4,       /* a base pointer is not 16-byte aligned */
    SS_ERR_WORKSPACE = -5,   /* workspace NULL while needed, or workspace_bytes too small */
    SS_ERR_HIP = -6,         /* a HIP call failed; see ss_last_hip_error() */
    SS_ERR_UNSUPPORTED = -7, /* valid arguments this build does not handle */
    SS_ERR_SCRATCH = -8      /* ss_fwd_noalloc: the plan needs more than its static scratch */
};

/* Workspace bytes ss_fwd / ss_bwd need for these dims (written to *bytes).
 * Returns SS_OK, SS_ERR_NULL, SS_ERR_DIMS or SS_ERR_DTYPE. */
int ss_fwd_workspace_size(const ss_dims* dims, size_t* bytes);
int ss_bwd_workspace_size(const ss_dims* dims, size_t* bytes);

/* Forward scan.
 *   x, dt_raw, Bm, Cm, dt_bias, A, Dskip, y : required.
 *   z       : NULL = no gate.
 *   h0      : NULL = zero initial state.
 *   h_final : NULL = final state not written.
 *   h_ckpt  : NULL = not written; else the state entering steps 0, 16, 32, ... (entry i is
 *             the state before step 16·i; entry 0 is h0 or 0): the checkpoints ss_bwd can
 *             take instead of recomputing chunk start states.  A chunked plan of two or
 *             more chunks on the four- or eight-lane layout whose chunk is no multiple of 16
 *             (a user-chosen chunk) returns SS_ERR_UNSUPPORTED.
 *   workspace / workspace_bytes : at least ss_fwd_workspace_size bytes of device memory. */
int ss_fwd(const ss_dims* dims,
           const void* x, const void* dt_raw, const float* dt_bias, const float* A,
           const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
           float* y, float* h_final, float* h_ckpt,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward: gradients of sum(dy·y) + sum(dh_final·h_final) with respect to every
 * input, recomputing the states from the inputs (§3.3) instead of storing them.  With
 * dims->disc = SS_DISC_ZOH they are the gradients of the exact hold (its gain
 * g = (exp(δA) - 1)/A has ∂g/∂δ = exp(δA) and ∂g/∂A = (δ·exp(δA) - g)/A).
 *   Inputs as ss_fwd; dy required; dh_final NULL = zero.
 *   h_ckpt : NULL = the chunk start states are recomputed here; else the checkpoints an
 *            ss_fwd call on these same inputs (and h0) wrote, from which every 16-step
 *            tile's states are recomputed (one forward sweep and one carry fewer).
 *   dx, ddt_raw, ddt_bias, dA, dB, dC, dD : required outputs.
 *   dz  : required iff z is given (else must be NULL).
 *   dh0 : required iff h0 is given (else must be NULL). */
int ss_bwd(const ss_dims* dims,
           const void* x, const void* dt_raw, const float* dt_bias, const float* A,
           const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
           const float* dy, const float* dh_final, const float* h_ckpt,
           float* dx, float* ddt_raw, float* ddt_bias, float* dA, float* dB, float* dC,
           float* dD, float* dz, float* dh0,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Selection projections and gated block around the scan (note "상태공간 모델(SSM)과 Mamba
 * 아키텍처", §3: the input is projected two ways, one branch through the scan and one through
 * the SiLU gate; page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §1.2:
 * B_t, C_t and Δ_t come from linear maps of the token).  Weights are stored (outputs, inputs):
 *   [x | z]     = u · W_inᵀ         u [B, L, d_in] bf16, W_in [2·dim, d_in] bf16, fp32 accumulate
 *   [Δraw|B|C]  = x · W_xᵀ          W_x [1 + 2·dstate, dim] float32
 *   y           = scan of x with Δraw shared by the channels (plus each channel's dt_bias),
 *                 B, C, gate z, A, Dskip, h0 — token-major, float32 throughout
 * and y [B, L, dim] float32 (h_final [B, dim, dstate] optional).  x, z [B, L, dim], dt [B, L],
 * Bm, Cm [B, L, dstate] are float32 outputs when given (else they live in the workspace).
 * d_in % 8 == 0 and dim % 4 == 0 (else SS_ERR_DIMS); plan and layout as for ss_fwd. */
typedef struct ss_block_dims {
    int64_t batch;    /* B >= 1 */
    int64_t seqlen;   /* L >= 1 */
    int64_t d_in;     /* input width, multiple of 8 */
    int64_t dim;      /* D: channels of the scan, multiple of 4 */
    int64_t dstate;   /* N, one of 1, 2, 4, 8, 16, 32, 64 (as ss_dims) */
    int32_t plan;     /* ss_plan of the scan */
    int32_t layout;   /* ss_layout of the scan */
} ss_block_dims;

int ss_block_fwd_workspace_size(const ss_block_dims* dims, size_t* bytes);

/* The block's first stage alone: [x | z] = u · W_inᵀ with u [B, L, d_in], W_in [2·dim, d_in]
 * (bf16) and x, z [B, L, dim] float32 (required).  dstate, plan and layout of dims are not
 * used.  Needs no workspace. */
int ss_in_proj(const ss_block_dims* dims, const void* u, const void* W_in, float* x, float* z,
               hipStream_t stream);

int ss_block_fwd(const ss_block_dims* dims, const void* u, const void* W_in, const float* W_x,
                 const float* dt_bias, const float* A, const float* Dskip, const float* h0,
                 float* y, float* h_final, float* x, float* z, float* dt, float* Bm, float* Cm,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, arguments (minus workspace / workspace_bytes), kernels and results as
 * ss_fwd.  The scratch the chunked and one-lane plans need (ss_fwd_workspace_size bytes) comes
 * from a static device array of SS_NOALLOC_SCRATCH_MIB MiB inside the library, one per GPU,
 * held from the first use on that GPU until the process ends; dims whose workspace size
 * exceeds it return SS_ERR_SCRATCH before anything happens.  The call allocates nothing and
 * calls no allocating routine.  The first call on a GPU that needs scratch looks up the
 * array's device address once (hipGetSymbolAddress, the stream's device made current for it,
 * then restored); a HIP failure there returns SS_ERR_HIP.
 * Every call on one GPU uses the same array: calls that overlap on one GPU (concurrent
 * streams, or several host threads) race on it and give undefined results; calls ordered on
 * one stream are safe.  Nothing in the array needs to start at zero (each call writes every
 * value it reads), so the previous call's contents do no harm. */
#define SS_NOALLOC_SCRATCH_MIB 64
int ss_fwd_noalloc(const ss_dims* dims,
                   const void* x, const void* dt_raw, const float* dt_bias, const float* A,
                   const void* Bm, const void* Cm, const float* Dskip, const void* z,
                   const float* h0, float* y, float* h_final, float* h_ckpt, hipStream_t stream);

/* Single-token (decode) step: the recurrence carried one token further for every (batch
 * row, channel), as in recurrent inference (note "상태공간 모델(SSM)과 Mamba 아키텍처", §2):
 *   δ = softplus(dt_bias + dt_raw);  h ← exp(δ·A)⊙h + δ·B·x;  y = (C·h + Dskip·x)·silu(z)
 *   (with dims->disc = SS_DISC_ZOH the input term is (exp(δA) - 1)/A · B·x)
 *   dims   : batch, dim, dstate, in_dtype, disc, dt_layout as for ss_fwd; seqlen must be 1;
 *            plan, chunk and layout must be 0; order is either (one token: the same memory).
 *   x, z : [B, D] (in_dtype; z NULL = no gate); dt_raw : [B, D], or [B] with SS_DT_SHARED;
 *   Bm, Cm : [B, N] (in_dtype);
 *   A [D, N], dt_bias [D], Dskip [D] : float32.
 *   h_in   : [B, D, N] float32, the state before the token (required).
 *   h_out  : [B, D, N] float32, the state after it; may equal h_in (the state is updated in
 *            place), otherwise it must not overlap h_in.
 *   y      : [B, D] float32.
 * Needs no workspace.  Same conventions and return codes as ss_fwd. */
int ss_step(const ss_dims* dims,
            const void* x, const void* dt_raw, const float* dt_bias, const float* A,
            const void* Bm, const void* Cm, const float* Dskip, const void* z,
            const float* h_in, float* h_out, float* y, hipStream_t stream);

/* Static description of a return code. */
const char* ss_strerror(int code);

/* hipError_t of the last failing HIP call made by this thread inside the library. */
int ss_last_hip_error(void);

/* (SS_VERSION_MAJOR << 16) | SS_VERSION_MINOR */
int ss_version(void);

/* Identity of the sources this library was built from: a NUL-terminated string of 64
 * lowercase hex digits, the SHA-256 over every file of the kernel source directory (name
 * and bytes, in name order), this header and the code-generation flags, fixed at compile
 * time.  A loader compares it with the same digest of the sources it expects, so results
 * are never taken from a library built from other sources.  Static storage; never NULL. */
const char* ss_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_H_ */
