// Split-bf16 router GEMM for gfx950: fp32 router weights kept as two bf16
// parts, scores = X W_high^T + (X W_low^T) / 256 in fp32.
//
// Method: SGLang post, section "Router GEMM: balancing routing precision and
// throughput".  The router's fp32 weights W are split once into W_high (the
// bf16 truncation of W) and W_low (the bf16 of the scaled residual
// (W - W_high) * 256), so W ~ W_high + W_low / 256 keeps the low mantissa bits
// a plain bf16 cast would drop; the product runs as two bf16 matrix products
// that share the activation operand, accumulate in fp32 and meet in an
// epilogue that applies the 1/256 and writes fp32 scores.
//
// gfx950 mapping.  The shapes are thin (K = 4096, N = 192 experts, M tokens
// from 1 to thousands), so the kernel is built for streaming the weights and
// the activations once:
//   * MFMA 16x16x32 bf16 with X as the A operand and W^T as the B operand,
//     both loaded straight from global memory into registers (16 B per lane:
//     a row's 8 consecutive k of the 32 of a step); the high and low weight
//     products share every X operand and keep separate fp32 accumulators.
//   * A workgroup (4 waves) covers 64 experts (16 per wave) and 16 * MT
//     tokens over one K range; the loads of 4 k-steps are issued before their
//     MFMAs (a second register buffer, to overlap the next chunk's loads
//     with these MFMAs, measured slower: one wave per SIMD).
//   * Up to 16 tokens, one launch: a workgroup of 16 waves per 16 experts,
//     each wave one sixteenth of K, the partial tiles added in LDS in wave
//     order.  Beyond that, a workgroup of 4 waves covers 64 experts; when the
//     grid is still small, K is split over workgroups, each split writes its
//     epilogue-combined partial, and a second kernel adds the splits in a
//     fixed order.  Both forms are deterministic.
#include "lbsa_device.h"

namespace lbsa {
namespace {

using namespace dev;

constexpr int kRouterThreads = 256;
constexpr int kRouterCols = 16 * 4;           // experts per workgroup (16 per wave)
constexpr int kRouterUnroll = 4;              // k-steps of 32 whose loads are issued together
constexpr int kRouterKChunk = 32 * kRouterUnroll;

struct RouterArgs {
    const uint16_t* x;        // bf16 [M][K]
    const uint16_t* w_hi;     // bf16 [N][K]
    const uint16_t* w_lo;
    float* dst;               // S == 1: scores [M][N]; else partials [S][M][N]
    int32_t M, N, K, S;
};

// fp32 weights -> (truncated bf16, bf16 of the residual x 256), 8 per thread.
__global__ __launch_bounds__(256) void split_weights_kernel(const float* __restrict__ w, uint16_t* __restrict__ hi,
                                                            uint16_t* __restrict__ lo, long long n8) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const float4 a = reinterpret_cast<const float4*>(w)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(w)[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t u0 = __float_as_uint(v[2 * j]), u1 = __float_as_uint(v[2 * j + 1]);
        const uint32_t t0 = u0 & 0xFFFF0000u, t1 = u1 & 0xFFFF0000u;      // truncation
        h[j] = (u0 >> 16) | (u1 & 0xFFFF0000u);
        // the residual keeps the dropped 16 mantissa bits exactly; times 256 is exact
        l[j] = bf16x2_pack((v[2 * j] - __uint_as_float(t0)) * 256.f, (v[2 * j + 1] - __uint_as_float(t1)) * 256.f);
    }
    reinterpret_cast<uint4*>(hi)[i] = make_uint4(h[0], h[1], h[2], h[3]);
    reinterpret_cast<uint4*>(lo)[i] = make_uint4(l[0], l[1], l[2], l[3]);
}

// The operands of one 128-k chunk for one lane: 4 k-steps of the high and
// low weight rows (B) and of MT token rows (A).
template <int MT>
struct Chunk {
    uint4 bh[kRouterUnroll], bl[kRouterUnroll], ax[kRouterUnroll][MT];
    __device__ void load(const uint4* wh, const uint4* wl, const uint4* const (&xr)[MT], int c) {
#pragma unroll
        for (int u = 0; u < kRouterUnroll; ++u) {
            bh[u] = wh[c + 4 * u];
            bl[u] = wl[c + 4 * u];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) ax[u][mt] = xr[mt][c + 4 * u];
        }
    }
    __device__ void mma(f32x4 (&hi)[MT], f32x4 (&lo)[MT]) const {
#pragma unroll
        for (int u = 0; u < kRouterUnroll; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                hi[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax[u][mt]), as_bf16x8(bh[u]), hi[mt], 0, 0, 0);
                lo[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax[u][mt]), as_bf16x8(bl[u]), lo[mt], 0, 0, 0);
            }
    }
};

template <int MT>
__global__ __launch_bounds__(kRouterThreads) void router_gemm_kernel(RouterArgs a) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * kRouterCols + 16 * w;           // this wave's 16 experts
    if (n0 >= a.N) return;                                      // uniform: past the last expert
    const int m0 = blockIdx.y * 16 * MT;
    const int kper = a.K / a.S, kb = blockIdx.z * kper;

    // B operands: expert n0 + r, k = kb + 32 step + 8 g ..; A operands: token
    // m0 + 16 mt + r (rows past M read the last row and are never stored)
    const uint4* wh = reinterpret_cast<const uint4*>(a.w_hi + (size_t)(n0 + r) * a.K + kb) + g;
    const uint4* wl = reinterpret_cast<const uint4*>(a.w_lo + (size_t)(n0 + r) * a.K + kb) + g;
    const uint4* xr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        xr[mt] = reinterpret_cast<const uint4*>(a.x + (size_t)min(m0 + 16 * mt + r, a.M - 1) * a.K + kb) + g;

    f32x4 acc_hi[MT], acc_lo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        acc_hi[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_lo[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int c = 0; c < kper / 8; c += kRouterKChunk / 8) {
        Chunk<MT> ch;
        ch.load(wh, wl, xr, c);
        ch.mma(acc_hi, acc_lo);
    }

    // epilogue: lane (g, r) holds tokens 4 g + i of each tile, expert n0 + r
    float* dst = a.dst + (size_t)blockIdx.z * a.M * a.N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 16 * mt + 4 * g + i;
            if (m < a.M) dst[(size_t)m * a.N + n0 + r] = acc_hi[mt][i] + acc_lo[mt][i] * (1.f / 256.f);
        }
}

// Few tokens (up to 16): one workgroup of 16 waves per 16 experts, wave w
// taking the w-th sixteenth of K; the 16 partial tiles meet in LDS and are
// added in wave order.  One launch, no workspace.
constexpr int kWideWaves = 16;
__global__ __launch_bounds__(64 * kWideWaves) void router_gemm_wide_kernel(RouterArgs a) {
    __shared__ f32x4 red[kWideWaves][64];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int kper = a.K / kWideWaves, kb = w * kper;
    const uint4* wh = reinterpret_cast<const uint4*>(a.w_hi + (size_t)(n0 + r) * a.K + kb) + g;
    const uint4* wl = reinterpret_cast<const uint4*>(a.w_lo + (size_t)(n0 + r) * a.K + kb) + g;
    const uint4* const xr[1] = {reinterpret_cast<const uint4*>(a.x + (size_t)min(r, a.M - 1) * a.K + kb) + g};
    f32x4 acc_hi[1] = {f32x4{0.f, 0.f, 0.f, 0.f}}, acc_lo[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int c = 0; c < kper / 8; c += kRouterKChunk / 8) {
        Chunk<1> ch;
        ch.load(wh, wl, xr, c);
        ch.mma(acc_hi, acc_lo);
    }
    red[w][lane] = acc_hi[0] + acc_lo[0] * (1.f / 256.f);
    __syncthreads();
    if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        f32x4 sum = red[0][l];
#pragma unroll
        for (int ww = 1; ww < kWideWaves; ++ww) sum += red[ww][l];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l >> 4) + i;
            if (m < a.M) a.dst[(size_t)m * a.N + n0 + (l & 15)] = sum[i];
        }
    }
}

// scores = sum over the S splits' partials, in split order; 4 scores per thread.
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                            long long n4, int S) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int j = 1; j < S; ++j) {
        const float4 v = reinterpret_cast<const float4*>(part)[(long long)j * n4 + i];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = s;
}

}  // namespace

RouterPlan router_plan(int M, int N, int K) {
    RouterPlan p;
    p.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.wide = M <= 16 && K % (kWideWaves * kRouterKChunk) == 0;
    if (p.wide) {
        p.S = 1;
        p.workspace = 0;
        return p;
    }
    const long long tiles = (long long)((N + kRouterCols - 1) / kRouterCols) * ((M + 16 * p.MT - 1) / (16 * p.MT));
    // split K (halving while the halves stay whole chunks of 128 k) until the
    // grid holds 512 workgroups
    p.S = 1;
    while (tiles * p.S < 512 && K % (2 * p.S * kRouterKChunk) == 0) p.S *= 2;
    p.workspace = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
    return p;
}

hipError_t launch_router_split(const float* w, void* hi, void* lo, long long count, hipStream_t stream) {
    const long long n8 = count / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(split_weights_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, w,
                       static_cast<uint16_t*>(hi), static_cast<uint16_t*>(lo), n8);
    return hipGetLastError();
}

hipError_t launch_router_gemm(const void* x, const void* w_hi, const void* w_lo, int M, int N, int K, float* out,
                              void* workspace, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const RouterPlan p = router_plan(M, N, K);
    RouterArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.w_hi = static_cast<const uint16_t*>(w_hi);
    a.w_lo = static_cast<const uint16_t*>(w_lo);
    a.dst = p.S > 1 ? static_cast<float*>(workspace) : out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.S = p.S;
    if (p.wide) {
        hipLaunchKernelGGL(router_gemm_wide_kernel, dim3(N / 16), dim3(64 * kWideWaves), 0, stream, a);
        return hipGetLastError();
    }
    const dim3 grid((N + kRouterCols - 1) / kRouterCols, (M + 16 * p.MT - 1) / (16 * p.MT), p.S);
    if (p.MT == 1) hipLaunchKernelGGL((router_gemm_kernel<1>), grid, dim3(kRouterThreads), 0, stream, a);
    else if (p.MT == 2) hipLaunchKernelGGL((router_gemm_kernel<2>), grid, dim3(kRouterThreads), 0, stream, a);
    else hipLaunchKernelGGL((router_gemm_kernel<4>), grid, dim3(kRouterThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.S == 1) return e;
    const long long n4 = (long long)M * N / 4;
    hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(workspace), out, n4, p.S);
    return hipGetLastError();
}

}  // namespace lbsa
