// The projections around the scan in a Mamba block, for gfx950.
//
// Note "상태공간 모델(SSM)과 Mamba 아키텍처", §3: the block projects its input two ways, one
// branch through the selective scan and one through the SiLU gate; page "3.2 선택적 스캔
// (Selective Scan) 알고리즘과 정보의 압축 및 선별", §1.2: B_t, C_t and Δ_t are linear maps
// of the token.  With weights stored (outputs, inputs):
//   [x | z]    = u · W_inᵀ        u [M, K] bf16, W_in [2D, K] bf16: a dense contraction,
//                                  run on the matrix cores (gemm_bf16_nt_kernel)
//   [Δ | B | C] = x · W_xᵀ        x [M, D] fp32, W_x [1 + 2N, D] fp32: 1 + 2N outputs per
//                                  token, a skinny contraction kept in fp32: B and C on the
//                                  fp32 matrix cores, Δ as a vector dot product beside them
//                                  (xproj_mfma_kernel, xproj_reduce_kernel)
// M = B·L tokens.  x and z stay float32, so the scan that follows sees the projections
// at float32 accuracy.
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_plan.h"

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
// part[s, m, o] = Σ_{k in split s} x[m, k] · Wx[o, k], o < P = 1 + 2N: a dense contraction over
// K = D with few columns, run on the fp32 matrix cores (v_mfma_f32_16x16x4f32: 16 x 16 output,
// K = 4; operand a of lane l is A[l % 16][l / 16], operand b is B[l / 16][l % 16], and the
// accumulator's element v is C[4·(l / 16) + v][l % 16]).  P = 1 + 2N: the 2N outputs of B and
// C fill whole 16-wide tiles for N >= 8, and output 0 (Δraw) is a dot product per lane on the
// vector ALUs instead of a third, mostly empty tile.  A wave owns MT tiles of 16 tokens and the
// NT output tiles over one K split.  The workgroup stages 64-step tiles of its tokens' x rows
// and of the weight rows in LDS, each global load covering 256-byte runs of a row (reading x
// straight into the MFMA operands instead scattered 64-byte pieces over 16 rows per load and
// ran at a third of the DRAM rate), the next tile prefetched into registers.  Per 16-deep
// chunk lane (r, g) = (l % 16, l / 16) reads one 16-byte run of each of its tokens' x rows,
// x[m + r][kc + 4g .. kc + 4g + 3], and the same run of each output tile's weight row and of
// row 0; MFMA j of the chunk takes element j of both runs, so it sums the products at
// k = kc + 4g + j over g: the four MFMAs cover the chunk's 16 steps (the order of k inside a
// chunk is permuted the same way for both operands), and output 0's four-term partials are
// summed over the four lanes g of a token at the end.  Workgroup = 4 waves = 64·MT tokens.
// grid = (ceil(M / (64·MT)), S), block = 256.  D % 4 == 0; split lengths are multiples of 64.
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-token tiles per wave (MT): each weight run loaded feeds MT MFMAs.  Two tiles measured
// 1.7 % faster on the block step than one at N = 16, four no faster than two at half the
// occupancy; above three output tiles (N > 16) one token tile keeps the registers in reach.

// K steps per LDS tile and the tiles' row stride (floats; 4 of padding)
constexpr int kXK = 64;
constexpr int kXRS = kXK + 4;

template <int NT, int MT>
__global__ __launch_bounds__(256) void xproj_mfma_kernel(
    const float* __restrict__ x, const float* __restrict__ Wx, float* __restrict__ part,
    int64_t M, int64_t D, int P, int64_t kc) {
    constexpr int XT = 64 * MT;                  // tokens per workgroup
    constexpr int XQ = XT * (kXK / 4) / 256;     // x float4 pieces per thread per tile
    constexpr int PR = 1 + 16 * NT;              // weight rows staged (P <= PR)
    constexpr int WQ = (PR * (kXK / 4) + 255) / 256;
    __shared__ __align__(16) float xs[XT * kXRS];
    __shared__ __align__(16) float ws[PR * kXRS];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int s = blockIdx.y;
    const int64_t m0 = int64_t(blockIdx.x) * XT;
    const int64_t k0 = int64_t(s) * kc;
    const int64_t k1 = (k0 + kc < D) ? k0 + kc : D;
    const int64_t nt = (k1 > k0) ? (k1 - k0 + kXK - 1) / kXK : 0;

    // staging: 16 consecutive threads cover one row's 64 steps (256 bytes); steps at or past
    // k1 and rows past M or P load nothing and stage zeros
    float4 px[XQ], pw[WQ];
    auto load_tile = [&](int64_t kt) {
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int e = tid + 256 * q, row = e >> 4, c4 = e & 15;
            const int64_t k = kt + 4 * c4, m = m0 + row;
            px[q] = (m < M && k < k1) ? *reinterpret_cast<const float4*>(x + m * D + k)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int q = 0; q < WQ; ++q) {
            const int e = tid + 256 * q, row = e >> 4, c4 = e & 15;
            const int64_t k = kt + 4 * c4;
            pw[q] = (row < P && k < k1) ? *reinterpret_cast<const float4*>(Wx + int64_t(row) * D + k)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int e = tid + 256 * q;
            *reinterpret_cast<float4*>(xs + (e >> 4) * kXRS + 4 * (e & 15)) = px[q];
        }
#pragma unroll
        for (int q = 0; q < WQ; ++q) {
            const int e = tid + 256 * q;
            if (e < PR * (kXK / 4)) *reinterpret_cast<float4*>(ws + (e >> 4) * kXRS + 4 * (e & 15)) = pw[q];
        }
    };

    f32x4 acc[MT][NT];
    float dacc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        dacc[i] = 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (nt > 0) {
        load_tile(k0);
        store_tile();
        __syncthreads();
    }
    for (int64_t it = 0; it < nt; ++it) {
        if (it + 1 < nt) load_tile(k0 + (it + 1) * kXK);
#pragma unroll
        for (int cc = 0; cc < kXK / 16; ++cc) {
            // chunk cc: lane (r, g) takes the runs at steps 16cc + 4g .. 16cc + 4g + 3
            const int kl = 16 * cc + 4 * g;
            float4 xa[MT], wb[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                xa[i] = *reinterpret_cast<const float4*>(xs + (wave * 16 * MT + 16 * i + r) * kXRS + kl);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                wb[t] = *reinterpret_cast<const float4*>(ws + (1 + 16 * t + r) * kXRS + kl);
            const float4 w0 = *reinterpret_cast<const float4*>(ws + kl);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float bv = j == 0 ? wb[t].x : j == 1 ? wb[t].y : j == 2 ? wb[t].z : wb[t].w;
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        const float av = j == 0 ? xa[i].x : j == 1 ? xa[i].y : j == 2 ? xa[i].z : xa[i].w;
                        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[i][t], 0, 0, 0);
                    }
                }
#pragma unroll
            for (int i = 0; i < MT; ++i)
                dacc[i] += fmaf(xa[i].w, w0.w, fmaf(xa[i].z, w0.z, fmaf(xa[i].y, w0.y, xa[i].x * w0.x)));
        }
        if (it + 1 < nt) {
            __syncthreads();
            store_tile();
            __syncthreads();
        }
    }
    // element v of tile (i, t): token m0 + 16(MT·wave + i) + 4g + v, output 1 + 16t + r
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + 16 * (MT * wave + i) + 4 * g + v;
            if (m >= M) continue;
            float* pr = part + (int64_t(s) * M + m) * P;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (1 + 16 * t + r < P) pr[1 + 16 * t + r] = acc[i][t][v];
        }
    // output 0: the four lanes g of token m0 + 16(MT·wave + i) + r hold partial dot products
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        float d = dacc[i];
        d += __shfl_xor(d, 16, 64);
        d += __shfl_xor(d, 32, 64);
        const int64_t m = m0 + 16 * (MT * wave + i) + r;
        if (g == 0 && m < M) part[(int64_t(s) * M + m) * P] = d;
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

template <int NT, int MT>
static hipError_t launch_xproj_t(const float* x, const float* Wx, float* part, int64_t M,
                                 int64_t D, int P, int64_t S, int64_t kc, hipStream_t s) {
    const int64_t tok = 64 * MT;
    hipLaunchKernelGGL((xproj_mfma_kernel<NT, MT>), dim3(unsigned((M + tok - 1) / tok), unsigned(S)),
                       dim3(256), 0, s, x, Wx, part, M, D, P, kc);
    return hipGetLastError();
}

hipError_t launch_xproj(const float* x, const float* Wx, float* part, float* dt, float* Bm,
                        float* Cm, int64_t M, int64_t D, int N, hipStream_t s) {
    const int64_t S = xproj_splits(M, D, N);
    const int64_t kc = xproj_split_len(D, S);
    const int P = 1 + 2 * N;
    hipError_t e;
    switch (N) {   // ceil(2N / 16) output tiles; token tiles per wave as xproj_mt(N)
        case 1: case 2: case 4: case 8: e = launch_xproj_t<1, 2>(x, Wx, part, M, D, P, S, kc, s); break;
        case 16: e = launch_xproj_t<2, 2>(x, Wx, part, M, D, P, S, kc, s); break;
        case 32: e = launch_xproj_t<4, 1>(x, Wx, part, M, D, P, S, kc, s); break;
        case 64: e = launch_xproj_t<8, 1>(x, Wx, part, M, D, P, S, kc, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t tot = M * (1 + 2 * N);
    hipLaunchKernelGGL(xproj_reduce_kernel, dim3(unsigned((tot + 255) / 256)), dim3(256), 0, s,
                       part, dt, Bm, Cm, M, N, int(S));
    return hipGetLastError();
}

}  // namespace ss
