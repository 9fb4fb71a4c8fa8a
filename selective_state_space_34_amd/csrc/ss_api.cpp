// C ABI of the selective-scan library: validation, plan choice, workspace carving
// and kernel launches on the caller's stream.  Declared in include/ss.h.
//
// Every argument check happens before the first HIP call, so an error return
// means nothing was enqueued.  The library allocates nothing: all scratch memory
// comes from the caller's workspace.
#include "ss.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "ss_kernels.h"
#include "ss_plan.h"

// Scratch of ss_fwd_noalloc: a fixed device array instead of a caller's workspace.  Each GPU
// the library runs on holds its own copy (allocated with the code object, kept until the
// process ends).  In host code `scratch` names a host-side stand-in, never the device memory:
// every host use goes through the address hipGetSymbolAddress returns for the device.
constexpr size_t kScratchBytes = size_t(SS_NOALLOC_SCRATCH_MIB) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

#ifndef SS_BUILD_ID
#error "SS_BUILD_ID (the SHA-256 of the sources, 64 hex digits) must be defined by the build"
#endif

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = int(e);
    return SS_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`, looked up once per device with
// that device current (the caller's current device is restored).
int scratch_for_stream(hipStream_t stream, void** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    int dev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return hip_fail(e);
    }
    if (dev < 0 || dev >= kMaxDevices) return SS_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t r = (dev != cur) ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return hip_fail(e);
        if (r != hipSuccess) return hip_fail(r);
        if (!p) return hip_fail(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SS_OK;
}

// Rows of a [B, D, L] (channel-major) or [B, L, D] (token-major) tensor: element (b, d, t) at
// b·sb + d·sd + t·ts.
ss::DtRows seq_rows(const ss::Plan& p) {
    return p.tok ? ss::DtRows{p.L * p.D, 1, p.D} : ss::DtRows{p.D * p.L, p.L, 1};
}

// Rows of dt_raw: as the sequence tensors, or one value per token [B, L] shared by channels.
ss::DtRows dt_rows(const ss::Plan& p) {
    return p.dt_shared ? ss::DtRows{p.L, 0, 1} : seq_rows(p);
}

}  // namespace

extern "C" {

int ss_version(void) { return (SS_VERSION_MAJOR << 16) | SS_VERSION_MINOR; }

const char* ss_build_id(void) { return SS_BUILD_ID; }

int ss_last_hip_error(void) { return g_last_hip_error; }

const char* ss_strerror(int code) {
    switch (code) {
        case SS_OK: return "success";
        case SS_ERR_NULL: return "a required pointer is NULL";
        case SS_ERR_DIMS: return "invalid dimensions (dim <= 0, unsupported dstate, overflow or bad chunk)";
        case SS_ERR_DTYPE: return "invalid dtype or plan";
        case SS_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
        case SS_ERR_WORKSPACE: return "workspace missing or too small";
        case SS_ERR_HIP: return "a HIP runtime call failed";
        case SS_ERR_UNSUPPORTED: return "unsupported by this build";
        case SS_ERR_SCRATCH: return "the call needs more scratch than ss_fwd_noalloc's static buffer holds";
        default: return "unknown error code";
    }
}

int ss_fwd_workspace_size(const ss_dims* dims, size_t* bytes) {
    if (!dims || !bytes) return SS_ERR_NULL;
    ss::Plan p;
    const int rc = ss::make_plan(*dims, ss::kPlanFwd, &p);
    if (rc != SS_OK) return rc;
    *bytes = p.ws_total;
    return SS_OK;
}

int ss_bwd_workspace_size(const ss_dims* dims, size_t* bytes) {
    if (!dims || !bytes) return SS_ERR_NULL;
    ss::Plan p;
    const int rc = ss::make_plan(*dims, ss::kPlanBwd, &p);
    if (rc != SS_OK) return rc;
    *bytes = p.ws_total;
    return SS_OK;
}

}  // extern "C"

namespace {

// Argument checks of the forward, in order; nothing is launched.  Fills the plan.
int fwd_validate(const ss_dims* dims, const void* x, const void* dt_raw, const float* dt_bias,
                 const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                 const float* h0, float* y, float* h_final, float* h_ckpt, ss::Plan* plan) {
    if (!dims) return SS_ERR_NULL;
    ss::Plan& p = *plan;
    int rc = ss::make_plan(*dims, ss::kPlanFwd, &p);
    if (rc != SS_OK) return rc;
    if (!x || !dt_raw || !dt_bias || !A || !Bm || !Cm || !Dskip || !y) return SS_ERR_NULL;
    const void* ptrs[] = {x, dt_raw, dt_bias, A, Bm, Cm, Dskip, y};
    for (const void* q : ptrs)
        if (!aligned16(q)) return SS_ERR_ALIGN;
    if ((z && !aligned16(z)) || (h0 && !aligned16(h0)) || (h_final && !aligned16(h_final)) ||
        (h_ckpt && !aligned16(h_ckpt)))
        return SS_ERR_ALIGN;
    // the group kernel checkpoints at its 16-step sweep starts, which are multiples of 16 when
    // every chunk starts on one: chunk % 16 == 0, or a single chunk (its sweeps start at 0, its
    // per-step tail checkpoints at t % 16 == 0)
    if (h_ckpt && p.group && p.chunked && p.K > 1 && p.chunk % ss::kCkptSteps != 0)
        return SS_ERR_UNSUPPORTED;
    return SS_OK;
}

// The forward's launches on a validated plan; ws holds at least p.ws_total bytes.
int fwd_launch(const ss::Plan& p, const void* x, const void* dt_raw, const float* dt_bias,
               const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
               const float* h0, float* y, float* h_final, float* h_ckpt, char* ws,
               hipStream_t stream) {
    const int bf16 = p.in_dtype == SS_BF16;
    hipError_t e = hipSuccess;
    // the group kernel tiles B/C from the inputs; the one-lane kernel reads a [B, L, 2N] copy
    float* BC = nullptr;
    if (!p.group) {
        BC = reinterpret_cast<float*>(ws + p.off_bc);
        e = ss::launch_bc_stage(bf16, int(p.N), Bm, Cm, BC, p.B, p.L, p.tok, stream);
        if (e != hipSuccess) return hip_fail(e);
    }

    ss::ScanLaunch s{};
    s.x = x; s.dt_raw = dt_raw; s.z = z; s.dt_bias = dt_bias; s.A = A; s.Dskip = Dskip; s.BC = BC;
    s.Bm = Bm; s.Cm = Cm;
    s.B = p.B; s.L = p.L; s.D = p.D; s.vec = p.vec; s.zoh = p.zoh; s.tok = p.tok;
    s.dtr = dt_rows(p);
    if (!p.chunked) {
        s.chunk = p.L; s.K = 1; s.h_init = h0; s.y = y; s.h_last = h_final; s.h_ckpt = h_ckpt; s.agg = 0;
        s.d4 = p.d4; s.nb4 = p.nb4;
        e = p.mixed ? ss::launch_scang_mixed(bf16, int(p.N), s, stream)
            : p.group ? ss::launch_scang(bf16, int(p.N), p.group, s, stream)
                      : ss::launch_scan(bf16, int(p.N), s, stream);
        if (e != hipSuccess) return hip_fail(e);
        return SS_OK;
    }
    float* h_end = reinterpret_cast<float*>(ws + p.off_hend);
    float* dsum = reinterpret_cast<float*>(ws + p.off_dsum);
    float* h_start = reinterpret_cast<float*>(ws + p.off_hstart);
    s.chunk = p.chunk; s.K = int(p.K);
    // 1. per-chunk aggregates
    s.h_init = nullptr; s.y = nullptr; s.h_last = h_end; s.dsum = dsum; s.agg = 1; s.z = nullptr;
    e = p.group ? ss::launch_scang(bf16, int(p.N), p.group, s, stream) : ss::launch_scan(bf16, int(p.N), s, stream);
    if (e != hipSuccess) return hip_fail(e);
    // 2. carry across chunks
    ss::CarryLaunch c{};
    c.h_end = h_end; c.dsum = dsum; c.A = A; c.h_in = h0; c.h_start = h_start; c.h_out = nullptr;
    c.B = p.B; c.D = p.D; c.K = int(p.K); c.reverse = 0;
    e = ss::launch_carry(int(p.N), c, stream);
    if (e != hipSuccess) return hip_fail(e);
    // 3. output pass from each chunk's true start state
    s.z = z; s.h_init = h_start; s.y = y; s.h_last = h_final; s.h_ckpt = h_ckpt; s.dsum = nullptr;
    s.agg = 0;
    e = p.group ? ss::launch_scang(bf16, int(p.N), p.group, s, stream) : ss::launch_scan(bf16, int(p.N), s, stream);
    if (e != hipSuccess) return hip_fail(e);
    return SS_OK;
}

}  // namespace

extern "C" {

int ss_fwd(const ss_dims* dims, const void* x, const void* dt_raw, const float* dt_bias,
           const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
           const float* h0, float* y, float* h_final, float* h_ckpt, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
    ss::Plan p;
    const int rc = fwd_validate(dims, x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, y, h_final,
                                h_ckpt, &p);
    if (rc != SS_OK) return rc;
    if (p.ws_total > 0 && (!workspace || workspace_bytes < p.ws_total)) return SS_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return SS_ERR_ALIGN;
    return fwd_launch(p, x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, y, h_final, h_ckpt,
                      static_cast<char*>(workspace), stream);
}

int ss_fwd_noalloc(const ss_dims* dims, const void* x, const void* dt_raw, const float* dt_bias,
                   const float* A, const void* Bm, const void* Cm, const float* Dskip,
                   const void* z, const float* h0, float* y, float* h_final, float* h_ckpt,
                   hipStream_t stream) {
    ss::Plan p;
    int rc = fwd_validate(dims, x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, y, h_final, h_ckpt,
                          &p);
    if (rc != SS_OK) return rc;
    if (p.ws_total > kScratchBytes) return SS_ERR_SCRATCH;
    // nothing needs to start at zero: every scratch value the kernels read was written earlier
    // in the same call (the aggregates, then the carry's start states)
    void* ws = nullptr;
    if (p.ws_total > 0) {
        rc = scratch_for_stream(stream, &ws);
        if (rc != SS_OK) return rc;
    }
    return fwd_launch(p, x, dt_raw, dt_bias, A, Bm, Cm, Dskip, z, h0, y, h_final, h_ckpt,
                      static_cast<char*>(ws), stream);
}

int ss_step(const ss_dims* dims, const void* x, const void* dt_raw, const float* dt_bias,
            const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
            const float* h_in, float* h_out, float* y, hipStream_t stream) {
    if (!dims) return SS_ERR_NULL;
    if (dims->plan != SS_PLAN_AUTO || dims->layout != SS_LAYOUT_AUTO) return SS_ERR_DTYPE;
    if (dims->seqlen != 1 || dims->chunk != 0) return SS_ERR_DIMS;
    ss::Plan p;
    const int rc = ss::make_plan(*dims, ss::kPlanStep, &p);
    if (rc != SS_OK) return rc;
    if (!x || !dt_raw || !dt_bias || !A || !Bm || !Cm || !Dskip || !h_in || !h_out || !y)
        return SS_ERR_NULL;
    const void* ptrs[] = {x, dt_raw, dt_bias, A, Bm, Cm, Dskip, h_in, h_out, y};
    for (const void* q : ptrs)
        if (!aligned16(q)) return SS_ERR_ALIGN;
    if (z && !aligned16(z)) return SS_ERR_ALIGN;
    ss::StepLaunch s{};
    s.x = x; s.dt_raw = dt_raw; s.z = z; s.dt_bias = dt_bias; s.A = A; s.Bm = Bm; s.Cm = Cm;
    s.Dskip = Dskip; s.h_in = h_in; s.h_out = h_out; s.y = y; s.B = p.B; s.D = p.D; s.N = int(p.N);
    s.zoh = p.zoh;
    s.dt_shared = p.dt_shared;
    const hipError_t e = ss::launch_step(p.in_dtype == SS_BF16, s, stream);
    if (e != hipSuccess) return hip_fail(e);
    return SS_OK;
}

int ss_bwd(const ss_dims* dims, const void* x, const void* dt_raw, const float* dt_bias,
           const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
           const float* h0, const float* dy, const float* dh_final, const float* h_ckpt, float* dx,
           float* ddt_raw,
           float* ddt_bias, float* dA, float* dB, float* dC, float* dD, float* dz, float* dh0,
           void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!dims) return SS_ERR_NULL;
    ss::Plan p;
    const int rc = ss::make_plan(*dims, ss::kPlanBwd, &p);
    if (rc != SS_OK) return rc;
    if (!x || !dt_raw || !dt_bias || !A || !Bm || !Cm || !Dskip || !dy) return SS_ERR_NULL;
    if (!dx || !ddt_raw || !ddt_bias || !dA || !dB || !dC || !dD) return SS_ERR_NULL;
    if ((z != nullptr) != (dz != nullptr)) return SS_ERR_NULL;
    if ((h0 != nullptr) != (dh0 != nullptr)) return SS_ERR_NULL;
    const void* req[] = {x, dt_raw, dt_bias, A, Bm, Cm, Dskip, dy, dx, ddt_raw, ddt_bias, dA, dB, dC, dD};
    for (const void* q : req)
        if (!aligned16(q)) return SS_ERR_ALIGN;
    const void* opt[] = {z, h0, dh_final, dz, dh0, h_ckpt};
    for (const void* q : opt)
        if (q && !aligned16(q)) return SS_ERR_ALIGN;
    if (!workspace || workspace_bytes < p.ws_total) return SS_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SS_ERR_ALIGN;

    char* ws = static_cast<char*>(workspace);
    const int bf16 = p.in_dtype == SS_BF16;
    hipError_t e = hipSuccess;

    ss::BwdLaunch bl{};
    bl.x = x; bl.dt_raw = dt_raw; bl.z = z; bl.dy = dy; bl.dt_bias = dt_bias; bl.A = A;
    bl.Dskip = Dskip; bl.Bm = Bm; bl.Cm = Cm; bl.h_ckpt = h_ckpt;
    bl.h_end = reinterpret_cast<float*>(ws + p.off_hend);
    bl.rev_end = reinterpret_cast<float*>(ws + p.off_gend);
    bl.dsum = reinterpret_cast<float*>(ws + p.off_dsum);
    bl.dbc_part = reinterpret_cast<float*>(ws + p.off_bcpart);
    bl.ddt_part = reinterpret_cast<float*>(ws + p.off_dtpart);
    bl.dx = dx; bl.ddt_raw = ddt_raw; bl.dz = dz; bl.dA = dA; bl.dB = dB; bl.dC = dC; bl.dD = dD;
    bl.ddt_bias = ddt_bias;
    bl.B = p.B; bl.L = p.L; bl.D = p.D; bl.N = p.N; bl.chunk = p.chunk; bl.K = int(p.K);
    bl.vec = p.vec;
    bl.tok = p.tok;
    bl.zoh = p.zoh;
    bl.dtr = dt_rows(p);
    bl.gdr = seq_rows(p);
    bl.ddt_shared = nullptr;
    bl.ddt_blk = nullptr;
    if (p.dt_shared) {
        // the final pass sums each 64-channel block; the reduction sums the blocks
        bl.ddt_raw = nullptr;
        bl.ddt_shared = ddt_raw;
        bl.ddt_blk = reinterpret_cast<float*>(ws + p.off_ddt);
    }
    // 1. chunk aggregates (forward and reverse pairs)
    bl.stage = 0;
    e = ss::launch_bwd(bf16, bl, stream);
    if (e != hipSuccess) return hip_fail(e);
    // 2. carries, in place: adjoints entering each chunk from the right, from dh_final,
    //    whose final value is dh0; without checkpoints also the chunk start states from h0
    ss::CarryLaunch c{};
    c.dsum = bl.dsum; c.A = A; c.B = p.B; c.D = p.D; c.K = int(p.K);
    c.h_end = bl.rev_end; c.h_start = bl.rev_end; c.h_in = dh_final; c.h_out = dh0; c.reverse = 1;
    if (!h_ckpt) {
        c.dual = 1;
        c.h_end2 = bl.h_end; c.h_start2 = bl.h_end; c.h_in2 = h0; c.h_out2 = nullptr; c.reverse2 = 0;
    }
    e = ss::launch_carry(int(p.N), c, stream);
    if (e != hipSuccess) return hip_fail(e);
    // 3. final pass: recomputed states, adjoint sweep, per-element gradients, partials
    bl.stage = 1;
    e = ss::launch_bwd(bf16, bl, stream);
    if (e != hipSuccess) return hip_fail(e);
    // 4. reductions into dB, dC, dA, dD, ddt_bias
    e = ss::launch_bwd_reduce(bl, stream);
    if (e != hipSuccess) return hip_fail(e);
    return SS_OK;
}

int ss_in_proj(const ss_block_dims* dims, const void* u, const void* W_in, float* x, float* z,
               hipStream_t stream) {
    if (!dims) return SS_ERR_NULL;
    ss::BlockPlan bp;
    const int rc = ss::make_block_plan(*dims, &bp);
    if (rc != SS_OK) return rc;
    if (!u || !W_in || !x || !z) return SS_ERR_NULL;
    if (!aligned16(u) || !aligned16(W_in) || !aligned16(x) || !aligned16(z)) return SS_ERR_ALIGN;
    const hipError_t e = ss::launch_gemm_bf16_nt(u, W_in, x, z, bp.M, 2 * bp.D, bp.Din, bp.D,
                                                 bp.D, bp.D, stream);
    if (e != hipSuccess) return hip_fail(e);
    return SS_OK;
}

int ss_block_fwd_workspace_size(const ss_block_dims* dims, size_t* bytes) {
    if (!dims || !bytes) return SS_ERR_NULL;
    ss::BlockPlan bp;
    const int rc = ss::make_block_plan(*dims, &bp);
    if (rc != SS_OK) return rc;
    *bytes = bp.total;
    return SS_OK;
}

int ss_block_fwd(const ss_block_dims* dims, const void* u, const void* W_in, const float* W_x,
                 const float* dt_bias, const float* A, const float* Dskip, const float* h0,
                 float* y, float* h_final, float* x, float* z, float* dt, float* Bm, float* Cm,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!dims) return SS_ERR_NULL;
    ss::BlockPlan bp;
    const int rc = ss::make_block_plan(*dims, &bp);
    if (rc != SS_OK) return rc;
    if (!u || !W_in || !W_x || !dt_bias || !A || !Dskip || !y) return SS_ERR_NULL;
    const void* req[] = {u, W_in, W_x, dt_bias, A, Dskip, y};
    for (const void* q : req)
        if (!aligned16(q)) return SS_ERR_ALIGN;
    const void* opt[] = {h0, h_final, x, z, dt, Bm, Cm};
    for (const void* q : opt)
        if (q && !aligned16(q)) return SS_ERR_ALIGN;
    if (!workspace || workspace_bytes < bp.total) return SS_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SS_ERR_ALIGN;

    char* ws = static_cast<char*>(workspace);
    float* xb = x ? x : reinterpret_cast<float*>(ws + bp.off_x);
    float* zb = z ? z : reinterpret_cast<float*>(ws + bp.off_z);
    float* dtb = dt ? dt : reinterpret_cast<float*>(ws + bp.off_dt);
    float* Bb = Bm ? Bm : reinterpret_cast<float*>(ws + bp.off_B);
    float* Cb = Cm ? Cm : reinterpret_cast<float*>(ws + bp.off_C);
    float* part = reinterpret_cast<float*>(ws + bp.off_part);
    // 1. [x | z] = u · W_inᵀ on the matrix cores
    hipError_t e = ss::launch_gemm_bf16_nt(u, W_in, xb, zb, bp.M, 2 * bp.D, bp.Din, bp.D, bp.D,
                                           bp.D, stream);
    if (e != hipSuccess) return hip_fail(e);
    // 2. [Δraw | B | C] = x · W_xᵀ
    e = ss::launch_xproj(xb, W_x, part, dtb, Bb, Cb, bp.M, bp.D, int(bp.N), stream);
    if (e != hipSuccess) return hip_fail(e);
    // 3. the gated scan, token-major with the shared Δraw
    return ss_fwd(&bp.sd, xb, dtb, dt_bias, A, Bb, Cb, Dskip, zb, h0, y, h_final, nullptr,
                  ws + bp.off_scan, bp.scan_ws, stream);
}

}  // extern "C"
