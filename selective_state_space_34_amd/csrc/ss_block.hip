// The projections around the scan in a Mamba block, for gfx950.
//
// Note "상태공간 모델(SSM)과 Mamba 아키텍처", §3: the block projects its input two ways, one
// branch through the selective scan and one through the SiLU gate; page "3.2 선택적 스캔
// (Selective Scan) 알고리즘과 정보의 압축 및 선별", §1.2: B_t, C_t and Δ_t are linear maps
// of the token.  With weights stored (outputs, inputs):
//   [x | z]    = u · W_inᵀ        u [M, K] bf16, W_in [2D, K] bf16: a dense contraction,
//                                  run on the matrix cores (gemm_bf16_nt_kernel)
//   [Δ | B | C] = x · W_xᵀ        x [M, D] fp32, W_x [1 + 2N, D] fp32: 1 + 2N outputs per
//                                  token, a skinny product kept in fp32 on the vector ALUs
//                                  (xproj_partial_kernel, xproj_reduce_kernel)
// M = B·L tokens.  x and z stay float32, so the scan that follows sees the projections
// at float32 accuracy.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- bf16 GEMM, both operands K-contiguous ("NT") ------------------------------------------
// Block tile 256 (rows of A) x 128 (rows of W) x 64 (K); four waves in a 2 x 2 arrangement,
// each owning a 128 x 64 piece as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.  Operand layouts
// of that instruction (lane l, element e of 8): A row l % 32, k = 8·(l / 32) + e; B column
// l % 32, same k; accumulator element r: row 8·(r / 4) + 4·(l / 32) + r % 4, column l % 32.
// One LDS stage with the next K tile prefetched into registers: load(k+1) -> MFMAs on the
// LDS copy of k -> barrier -> registers to LDS -> barrier.  Inside a K tile each 16-deep
// step's fragments are read while the previous step's MFMAs run (two fragment sets; the
// accumulators then sit in arch VGPRs, 254 in all, still two waves per SIMD).  LDS rows are padded by 8
// elements (144 bytes), which keeps the 16-byte fragment reads of 16 lanes on disjoint banks.
constexpr int kGM = 256, kGN = 128, kGK = 64;
constexpr int kGPad = kGK + 8;                   // LDS row stride (elements)
constexpr int kGThreads = 256;
constexpr int kAChunks = kGM * kGK / 8 / kGThreads;   // 16-byte pieces per thread: 8
constexpr int kBChunks = kGN * kGK / 8 / kGThreads;   // 4

__device__ __forceinline__ uint4 load16_or_zero(const bf16_t* base, int64_t row, int64_t nrows,
                                                int64_t ld, int64_t k, int64_t K) {
    if (row < nrows && k < K) return *reinterpret_cast<const uint4*>(base + row * ld + k);
    return make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

// C0 / C1 [M, ·] = (A [M, K] · W [Nc, K]ᵀ) split at column nsplit: columns [0, nsplit) go to
// C0 (row stride ld0), [nsplit, Nc) to C1 at column - nsplit (row stride ld1).  K % 8 == 0.
// grid = ceil(M / 256) · ceil(Nc / 128) (one dimension, remapped below), block = 256.
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_bf16_nt_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, float* __restrict__ C0,
    float* __restrict__ C1, int64_t M, int64_t Nc, int64_t K, int64_t nsplit, int64_t ld0,
    int64_t ld1, int tiles_m, int tiles_n) {
    __shared__ __align__(16) bf16_t As[kGM * kGPad];
    __shared__ __align__(16) bf16_t Ws[kGN * kGPad];

    // Tile order: the dispatcher deals workgroups to the 8 XCDs in turn, so workgroup g
    // runs on XCD g % 8.  Give each XCD a contiguous range of tiles, walked in column
    // strips 8 row tiles tall, so the tiles an XCD runs together share A and W rows in its
    // own L2.
    const int ntiles = tiles_m * tiles_n;
    const int g = blockIdx.x;
    const int t = (ntiles % 8 == 0) ? (g % 8) * (ntiles / 8) + g / 8 : g;
    constexpr int kGroupM = 8;
    const int group = t / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = (tiles_m - first_m < kGroupM) ? tiles_m - first_m : kGroupM;
    const int tm = first_m + (t % (kGroupM * tiles_n)) % gm;
    const int tn = (t % (kGroupM * tiles_n)) / gm;
    const int64_t m0 = int64_t(tm) * kGM, n0 = int64_t(tn) * kGN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;      // wave's 128 x 64 piece
    const int lr = lane & 31, lk = (lane >> 5) * 8;

    // global -> register staging: thread covers 16-byte piece (tid % 8) of rows tid / 8 + 32 i
    const int prow = tid >> 3, pcol = (tid & 7) * 8;
    uint4 ra[kAChunks], rw[kBChunks];
    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i)
            ra[i] = load16_or_zero(A, m0 + prow + 32 * i, M, K, k0 + pcol, K);
#pragma unroll
        for (int i = 0; i < kBChunks; ++i)
            rw[i] = load16_or_zero(W, n0 + prow + 32 * i, Nc, K, k0 + pcol, K);
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i)
            *reinterpret_cast<uint4*>(As + (prow + 32 * i) * kGPad + pcol) = ra[i];
#pragma unroll
        for (int i = 0; i < kBChunks; ++i)
            *reinterpret_cast<uint4*>(Ws + (prow + 32 * i) * kGPad + pcol) = rw[i];
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (K + kGK - 1) / kGK;
    load_tile(0);
    store_tile();
    __syncthreads();
    // fragments of K step ks + 16 are read while the MFMAs of step ks run
    auto read_frag = [&](int ks, bf16x8 (&af)[4], bf16x8 (&bfr)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + 32 * i + lr) * kGPad + ks + lk);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8*>(Ws + (wn * 64 + 32 * j + lr) * kGPad + ks + lk);
    };
    for (int64_t kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_tile((kt + 1) * kGK);
        bf16x8 fa[2][4], fb[2][2];
        read_frag(0, fa[0], fb[0]);
#pragma unroll
        for (int q = 0; q < kGK / 16; ++q) {
            if (q + 1 < kGK / 16) read_frag(16 * (q + 1), fa[(q + 1) & 1], fb[(q + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q & 1][i], fb[q & 1][j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            __syncthreads();
            store_tile();
            __syncthreads();
        }
    }

    // epilogue: for a fixed r, the 32 lanes of a half-wave hold 32 consecutive columns
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + 32 * j + lr;
            if (col >= Nc) continue;
            float* out = col < nsplit ? C0 + col : C1 + (col - nsplit);
            const int64_t ld = col < nsplit ? ld0 : ld1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 128 + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
                if (row < M) out[row * ld] = acc[i][j][r];
            }
        }
    }
}

// ---- selection projections -----------------------------------------------------------------
// part[s, m, o] = Σ_{k in split s} x[m, k] · Wx[o, k], o < P = 1 + 2N: a product with few
// columns, register-tiled on the vector ALUs.  Thread (token group tg, output group og) owns
// 4 tokens x 4 outputs (16 accumulators); per K step it reads 4 x values and 4 weights as two
// 16-byte LDS reads for 16 FMAs.  A workgroup covers TM = 4·TG tokens and all outputs, and
// one split of K, staged 32 steps at a time: x rows are read coalesced (8 threads per 128-byte
// row piece) and stored transposed, [k][token], so a thread's 4 tokens are adjacent.
// grid = (ceil(M / TM), S), block = TG·OG threads.  D % 4 == 0.
template <int P>
struct XprojShape {
    static constexpr int OG = (P + 3) / 4;           // output groups of 4
    static constexpr int TG = 256 / OG;              // token groups of 4
    static constexpr int TM = 4 * TG;                // tokens per workgroup
    static constexpr int THREADS = TG * OG;
    static constexpr int KT = 32;                    // K steps per LDS stage
    static constexpr int XS = TM + 4;                // row stride of the transposed x tile
    static constexpr int WS = 4 * OG;                // row stride of the weight tile
};

template <int P>
__global__ __launch_bounds__(256) void xproj_partial_kernel(
    const float* __restrict__ x, const float* __restrict__ Wx, float* __restrict__ part,
    int64_t M, int64_t D, int64_t kc) {
    using Sh = XprojShape<P>;
    __shared__ __align__(16) float xs[Sh::KT * Sh::XS];
    __shared__ __align__(16) float wsh[Sh::KT * Sh::WS];
    const int tid = threadIdx.x;
    const int tg = tid % Sh::TG, og = tid / Sh::TG;
    const int s = blockIdx.y;
    const int64_t m0 = int64_t(blockIdx.x) * Sh::TM;
    const int64_t k0 = int64_t(s) * kc;
    const int64_t k1 = (k0 + kc < D) ? k0 + kc : D;

    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = 0.0f;

    for (int64_t kb = k0; kb < k1; kb += Sh::KT) {
        const int nk = int((k1 - kb < Sh::KT) ? k1 - kb : Sh::KT);   // a multiple of 4
        __syncthreads();                                               // previous stage read
        for (int e = tid; e < Sh::TM * (Sh::KT / 4); e += Sh::THREADS) {
            const int tok = e / (Sh::KT / 4), q = e % (Sh::KT / 4);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m0 + tok < M && 4 * q < nk) v = *reinterpret_cast<const float4*>(x + (m0 + tok) * D + kb + 4 * q);
            xs[(4 * q + 0) * Sh::XS + tok] = v.x;
            xs[(4 * q + 1) * Sh::XS + tok] = v.y;
            xs[(4 * q + 2) * Sh::XS + tok] = v.z;
            xs[(4 * q + 3) * Sh::XS + tok] = v.w;
        }
        for (int e = tid; e < Sh::WS * (Sh::KT / 4); e += Sh::THREADS) {
            const int o = e / (Sh::KT / 4), q = e % (Sh::KT / 4);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (o < P && 4 * q < nk) v = *reinterpret_cast<const float4*>(Wx + int64_t(o) * D + kb + 4 * q);
            wsh[(4 * q + 0) * Sh::WS + o] = v.x;
            wsh[(4 * q + 1) * Sh::WS + o] = v.y;
            wsh[(4 * q + 2) * Sh::WS + o] = v.z;
            wsh[(4 * q + 3) * Sh::WS + o] = v.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < Sh::KT; ++k) {
            const float4 xv = *reinterpret_cast<const float4*>(xs + k * Sh::XS + 4 * tg);
            const float4 wv = *reinterpret_cast<const float4*>(wsh + k * Sh::WS + 4 * og);
            const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
            const float wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(xa[a], wa[c], acc[a][c]);
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t m = m0 + 4 * tg + a;
        if (m >= M) continue;
        float* pr = part + (int64_t(s) * M + m) * P;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (4 * og + c < P) pr[4 * og + c] = acc[a][c];
    }
}

// Σ over the S splits -> Δraw [M], B [M, N], C [M, N].  One thread per (m, o).
__global__ __launch_bounds__(256) void xproj_reduce_kernel(const float* __restrict__ part,
                                                           float* __restrict__ dt,
                                                           float* __restrict__ Bm,
                                                           float* __restrict__ Cm, int64_t M,
                                                           int N, int S) {
    const int P = 1 + 2 * N;
    const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (e >= M * P) return;
    float v = 0.0f;
    for (int s = 0; s < S; ++s) v += part[int64_t(s) * M * P + e];
    const int64_t m = e / P;
    const int o = int(e % P);
    if (o == 0) dt[m] = v;
    else if (o <= N) Bm[m * N + o - 1] = v;
    else Cm[m * N + o - 1 - N] = v;
}

hipError_t launch_gemm_bf16_nt(const void* A, const void* W, float* C0, float* C1, int64_t M,
                               int64_t Nc, int64_t K, int64_t nsplit, int64_t ld0, int64_t ld1,
                               hipStream_t s) {
    const int64_t tm = (M + kGM - 1) / kGM, tn = (Nc + kGN - 1) / kGN;
    hipLaunchKernelGGL(gemm_bf16_nt_kernel, dim3(unsigned(tm * tn)), dim3(kGThreads), 0, s,
                       static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(W), C0, C1, M,
                       Nc, K, nsplit, ld0, ld1, int(tm), int(tn));
    return hipGetLastError();
}

static int xproj_tile_tokens(int N) {
    switch (N) {
        case 1: return XprojShape<3>::TM;
        case 2: return XprojShape<5>::TM;
        case 4: return XprojShape<9>::TM;
        case 8: return XprojShape<17>::TM;
        case 16: return XprojShape<33>::TM;
        case 32: return XprojShape<65>::TM;
        default: return XprojShape<129>::TM;
    }
}

int64_t xproj_splits(int64_t M, int64_t D, int N) {
    // about 1024 workgroups in all, each split at least 64 steps of K
    const int64_t mb = (M + xproj_tile_tokens(N) - 1) / xproj_tile_tokens(N);
    int64_t S = (1024 + mb - 1) / mb;
    if (S > D / 64) S = D / 64;
    return S < 1 ? 1 : S;
}

int64_t xproj_split_len(int64_t D, int64_t S) { return ((D + S - 1) / S + 3) / 4 * 4; }

template <int P>
static hipError_t launch_xproj_p(const float* x, const float* Wx, float* part, int64_t M,
                                 int64_t D, int64_t S, int64_t kc, hipStream_t s) {
    using Sh = XprojShape<P>;
    hipLaunchKernelGGL((xproj_partial_kernel<P>),
                       dim3(unsigned((M + Sh::TM - 1) / Sh::TM), unsigned(S)), dim3(Sh::THREADS),
                       0, s, x, Wx, part, M, D, kc);
    return hipGetLastError();
}

hipError_t launch_xproj(const float* x, const float* Wx, float* part, float* dt, float* Bm,
                        float* Cm, int64_t M, int64_t D, int N, hipStream_t s) {
    const int64_t S = xproj_splits(M, D, N);
    const int64_t kc = xproj_split_len(D, S);
    hipError_t e;
    switch (N) {
        case 1: e = launch_xproj_p<3>(x, Wx, part, M, D, S, kc, s); break;
        case 2: e = launch_xproj_p<5>(x, Wx, part, M, D, S, kc, s); break;
        case 4: e = launch_xproj_p<9>(x, Wx, part, M, D, S, kc, s); break;
        case 8: e = launch_xproj_p<17>(x, Wx, part, M, D, S, kc, s); break;
        case 16: e = launch_xproj_p<33>(x, Wx, part, M, D, S, kc, s); break;
        case 32: e = launch_xproj_p<65>(x, Wx, part, M, D, S, kc, s); break;
        case 64: e = launch_xproj_p<129>(x, Wx, part, M, D, S, kc, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t tot = M * (1 + 2 * N);
    hipLaunchKernelGGL(xproj_reduce_kernel, dim3(unsigned((tot + 255) / 256)), dim3(256), 0, s,
                       part, dt, Bm, Cm, M, N, int(S));
    return hipGetLastError();
}

}  // namespace ss
