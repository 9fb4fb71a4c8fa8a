// Inter-chunk carry of the sequence-parallel scan, for gfx950.
//
// Page "3.2 선택적 스캔(Selective Scan) 알고리즘과 정보의 압축 및 선별", §2.2: the
// step h -> Ā h + B̄x is an affine map, and composing two of them,
//   (a_j, b_j) • (a_i, b_i) = (a_j a_i, a_j b_i + b_j)   (i earlier, j later),
// is associative, so prefixes over chunks can be taken in any bracketing.  A
// chunk's pair is (Π_t Ā_t, local state from zero) = (exp(A Σδ), h_end).
//
// The page's tree (up-sweep / down-sweep) is replaced by the wavefront's own
// cross-lane network: one workgroup per channel, lane = run of consecutive chunks,
//   1. each lane composes its run sequentially (all N states at once),
//   2. an inclusive Kogge–Stone scan across the 64 lanes with DPP row_shr:1/2/4/8
//      inside rows of 16, then row_bcast:15 and row_bcast:31 across rows,
//   3. the (up to 16) wave totals meet in LDS and each wave folds the totals of
//      the waves before it onto the initial state,
//   4. wave_shr:1 turns the inclusive prefix into each lane's entering state, and
//      the lane walks its run again writing every chunk's start state.
// With few chunks and many channels a plain sequential walk per (channel, state) is
// faster (carry_seq_kernel): the scan's depth is then small and its lanes mostly idle.  At
// N = 64 the walk is always used: the per-channel scan would hold 4 x 64 values per lane.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ss {

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xf, false));
}

// Inclusive scan of affine pairs across the 64 lanes of a wavefront: on return lane i
// holds (P, H) = e_i • e_{i-1} • ... • e_0.  Lanes that receive nothing compose with
// the identity (1, 0).
__device__ __forceinline__ void wave_scan_affine(float& P, float& H) {
#define SS_STEP(CTRL, MASK)                         \
    {                                               \
        const float pp = dpp<CTRL, MASK>(1.0f, P);  \
        const float hp = dpp<CTRL, MASK>(0.0f, H);  \
        H = fmaf(P, hp, H);                         \
        P = P * pp;                                 \
    }
    SS_STEP(0x111, 0xf)  // row_shr:1
    SS_STEP(0x112, 0xf)  // row_shr:2
    SS_STEP(0x114, 0xf)  // row_shr:4
    SS_STEP(0x118, 0xf)  // row_shr:8
    SS_STEP(0x142, 0xa)  // row_bcast:15 -> rows 1, 3
    SS_STEP(0x143, 0xc)  // row_bcast:31 -> rows 2, 3
#undef SS_STEP
}

// One launch may carry two independent sets (blockIdx.z selects): the backward runs
// its forward-state carry and its reverse-adjoint carry together.
struct CarrySet {
    const float* h_end;
    const float* h_in;
    float* h_start;
    float* h_out;
    int reverse;
};

template <int N>
__global__ __launch_bounds__(1024) void carry_kernel(CarrySet s0, CarrySet s1,
                                                     const float* __restrict__ dsum,
                                                     const float* __restrict__ A, int64_t D, int K,
                                                     int m) {
    const CarrySet& cs = blockIdx.z ? s1 : s0;
    const float* h_end = cs.h_end;
    const float* h_in = cs.h_in;
    float* h_start = cs.h_start;
    float* h_out = cs.h_out;
    const int reverse = cs.reverse;
    __shared__ float wP[16][N];
    __shared__ float wH[16][N];
    const int64_t d = blockIdx.x;
    const int b = blockIdx.y;
    const int g = threadIdx.x;
    const int lane = g & 63, wave = g >> 6;
    float A2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = A[d * N + n] * kLog2e;

    const int j0 = g * m;
    const int j1 = (j0 + m < K) ? j0 + m : K;
    auto chunk_of = [&](int j) { return reverse ? K - 1 - j : j; };

    float P[N], H[N];
#pragma unroll
    for (int n = 0; n < N; ++n) { P[n] = 1.0f; H[n] = 0.0f; }
    for (int j = j0; j < j1; ++j) {
        const int64_t base = (int64_t(b) * D + d) * K + chunk_of(j);
        const float s = dsum[base];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float pc = exp2_hw(A2[n] * s);
            H[n] = fmaf(pc, H[n], h_end[base * N + n]);
            P[n] *= pc;
        }
    }
#pragma unroll
    for (int n = 0; n < N; ++n) wave_scan_affine(P[n], H[n]);
    if (lane == 63) {
#pragma unroll
        for (int n = 0; n < N; ++n) { wP[wave][n] = P[n]; wH[wave][n] = H[n]; }
    }
    __syncthreads();
    float st[N];
    const int64_t ci = (int64_t(b) * D + d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) st[n] = h_in ? h_in[ci + n] : 0.0f;
    for (int w = 0; w < wave; ++w) {
#pragma unroll
        for (int n = 0; n < N; ++n) st[n] = fmaf(wP[w][n], st[n], wH[w][n]);
    }
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float pe = dpp<0x138, 0xf>(1.0f, P[n]);  // wave_shr:1: lane i gets lane i-1
        const float he = dpp<0x138, 0xf>(0.0f, H[n]);
        st[n] = fmaf(pe, st[n], he);
    }
    for (int j = j0; j < j1; ++j) {
        const int64_t base = (int64_t(b) * D + d) * K + chunk_of(j);
        const float s = dsum[base];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            // read before write: h_start may alias h_end (each lane owns its chunks)
            const float he = h_end[base * N + n];
            h_start[base * N + n] = st[n];
            st[n] = fmaf(exp2_hw(A2[n] * s), st[n], he);
        }
    }
    if (h_out && j0 < K && j1 == K) {
#pragma unroll
        for (int n = 0; n < N; ++n) h_out[ci + n] = st[n];
    }
}

// Few chunks (K <= kSeqMaxK) and many channels: one thread per (batch row, channel, state)
// walks its K chunks in order.  The chunk pairs are loaded kSeqBatch at a time ahead of
// the dependent chain of FMAs.  Threads run along n, then d: each chunk's N states of a
// channel are contiguous, so a group of N threads reads one contiguous run.
constexpr int kSeqMaxK = 128;
constexpr int kSeqBatch = 16;

__global__ __launch_bounds__(256) void carry_seq_kernel(CarrySet s0, CarrySet s1,
                                                        const float* __restrict__ dsum,
                                                        const float* __restrict__ A, int64_t BDN,
                                                        int64_t D, int N, int K) {
    const CarrySet& cs = blockIdx.y ? s1 : s0;
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= BDN) return;
    const int n = int(i % N);
    const int64_t bd = i / N;                  // b * D + d
    const int64_t d = bd % D;
    const float a2 = A[d * N + n] * kLog2e;
    float st = cs.h_in ? cs.h_in[bd * N + n] : 0.0f;
    for (int j0 = 0; j0 < K; j0 += kSeqBatch) {
        float he[kSeqBatch], sm[kSeqBatch];
#pragma unroll
        for (int u = 0; u < kSeqBatch; ++u) {
            const int j = j0 + u;
            const int c = cs.reverse ? K - 1 - j : j;
            const int64_t base = bd * K + c;
            he[u] = (j < K) ? cs.h_end[base * N + n] : 0.0f;
            sm[u] = (j < K) ? dsum[base] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kSeqBatch; ++u) {
            const int j = j0 + u;
            if (j < K) {
                const int c = cs.reverse ? K - 1 - j : j;
                // read before write: h_start may alias h_end (the loads above came first)
                cs.h_start[(bd * K + c) * N + n] = st;
                st = fmaf(exp2_hw(a2 * sm[u]), st, he[u]);
            }
        }
    }
    if (cs.h_out) cs.h_out[bd * N + n] = st;
}

template <int N>
static hipError_t launch_carry_t(const CarryLaunch& p, hipStream_t s) {
    const int m = (p.K + 1023) / 1024;
    const int lanes = (p.K + m - 1) / m;
    const int threads = (lanes + 63) / 64 * 64;
    const CarrySet s0{p.h_end, p.h_in, p.h_start, p.h_out, p.reverse};
    const CarrySet s1{p.h_end2, p.h_in2, p.h_start2, p.h_out2, p.reverse2};
    dim3 grid(unsigned(p.D), unsigned(p.B), p.dual ? 2u : 1u);
    hipLaunchKernelGGL(carry_kernel<N>, grid, dim3(threads), 0, s, s0, s1, p.dsum, p.A, p.D, p.K, m);
    return hipGetLastError();
}

hipError_t launch_carry(int N, const CarryLaunch& p, hipStream_t s) {
    const int64_t BDN = p.B * p.D * N;
    // one thread per (channel, state) walking the chunks; also every N = 64 carry, whose
    // per-channel kernel would hold 4 x 64 values per thread
    if ((p.K <= kSeqMaxK && BDN >= 16384) || N == 64) {
        const CarrySet s0{p.h_end, p.h_in, p.h_start, p.h_out, p.reverse};
        const CarrySet s1{p.h_end2, p.h_in2, p.h_start2, p.h_out2, p.reverse2};
        dim3 grid(unsigned((BDN + 255) / 256), p.dual ? 2u : 1u);
        hipLaunchKernelGGL(carry_seq_kernel, grid, dim3(256), 0, s, s0, s1, p.dsum, p.A, BDN, p.D, N,
                           p.K);
        return hipGetLastError();
    }
    switch (N) {
        case 1: return launch_carry_t<1>(p, s);
        case 2: return launch_carry_t<2>(p, s);
        case 4: return launch_carry_t<4>(p, s);
        case 8: return launch_carry_t<8>(p, s);
        case 16: return launch_carry_t<16>(p, s);
        case 32: return launch_carry_t<32>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ss
