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
// from 1 to thousands): the weights (3 MiB as two bf16 parts) are the whole
// traffic for few tokens, the activations for many.
//   * MFMA 16x16x32 bf16, X the A operand and W^T the B operand.  A lane
//     (g, r) = (lane / 16, lane % 16) takes 16 consecutive k (16 g .. of a
//     64-k step) of its row r and feeds them to two MFMAs of 32 k each (b =
//     0, 1: the first and the second 8); A and B take the same k order, so
//     each MFMA still sums 32 exact bf16 products.  The high and low weight
//     products share every X operand and keep separate fp32 accumulators;
//     the epilogue adds hi + lo / 256.
//   * The split weights are stored blocked for these loads: per 16 experts
//     and 64 k, a 2 KiB block of [b][lane][8 k] (one per part), so each
//     wave's W load is one contiguous 1 KiB read.  Row-major W would spread
//     it over 16 rows, half of each 128-byte line per load.
//   * Thin form (few tokens): a workgroup of 4 waves covers 16 experts and
//     16 MT tokens over 256 k (64 per wave, all loads issued at once); the 4
//     wave partials meet in LDS in wave order.  K is split over workgroups,
//     so the 3 MiB of weights are read by some 200 workgroups at once.
//   * Tile form (many tokens): a workgroup of 4 waves (one per SIMD, so each
//     has the whole register file: 96 accumulator registers and the W operands
//     of two steps) covers 64 tokens x 192 experts over K / S <= 1024 k.  Its
//     whole X tile is loaded into LDS at the start (asynchronous global->LDS
//     loads, shared by the 4 waves); W goes straight to registers, one step
//     ahead, since no other wave of the workgroup reads a wave's experts.
//     Workgroups are ordered so that each of the 8 XCDs (L2 domains; the
//     dispatcher deals workgroups to them in turn) works on one part of K and
//     keeps only that slice of W in its L2.
//   * A split of K over S workgroups writes S partial planes; a second kernel
//     adds them in split order (deterministic), spread over the whole GPU.
#include "lbsa_device.h"

namespace lbsa {
namespace {

using namespace dev;

constexpr int kStep = 64;                         // k per wave step: 16 per lane group, two MFMAs
constexpr int kThinWaves = 4;
constexpr int kThinK = kThinWaves * kStep;        // k per thin workgroup
constexpr int kTileMT = 4;                        // 16-token tiles per tile workgroup
constexpr int kTileNB = 3;                        // 16-expert tiles per wave
constexpr int kTileEW = 4;                        // expert waves
constexpr int kTileWaves = kTileEW;
constexpr int kTileRows = 16 * kTileMT;
constexpr int kTileCols = 16 * kTileNB * kTileEW; // experts per tile workgroup
constexpr int kChunk = 128;                       // k per X chunk in LDS
constexpr int kStageBytes = kTileRows * kChunk * 2;
constexpr int kTileXBytes = kTileRows * kRouterTileMaxK * 2;  // the whole X tile of a workgroup
constexpr int kXLoads = kStageBytes / (16 * 64 * kTileEW);   // 16-byte LDS loads per lane per chunk
constexpr int kWLoads = 4 * kTileNB;              // 16-byte W loads per lane per step (hi, lo; 32 bytes each)
static_assert(kXLoads == 4, "one chunk = 4 loads per lane");
static_assert(kTileXBytes <= 160 * 1024 - 64, "X tile fits in LDS");
static_assert(kTileMT == 4, "the A reads of a step are one 4-read block");
static_assert(kThinK == kRouterKAlign && 2 * kChunk == kRouterKAlign, "K granularity of both forms");

struct RouterArgs {
    const uint16_t* x;        // bf16 [M][K]
    const uint16_t* w_hi;     // bf16, blocked (see router_w_index)
    const uint16_t* w_lo;
    float* dst;               // S == 1: scores [M][N]; else partials [S][M][N]
    int32_t M, N, K, S;
    int32_t tiles_n, tiles;   // output tiles along N, in all
};

// Element (n, k) of a blocked weight part: block (n / 16, k / 64) of 1024
// elements, inside it [b][lane][e] with lane = 16 g + n % 16 for k % 64 =
// 16 g + 8 b + e.
__host__ __device__ inline size_t router_w_index(int n, int k, int K) {
    const int kk = k & 63;
    return ((size_t)(n >> 4) * (K >> 6) + (k >> 6)) * 1024 + ((kk >> 3) & 1) * 512 + ((kk >> 4) * 16 + (n & 15)) * 8 +
           (kk & 7);
}

// fp32 weights [N][K] -> (truncated bf16, bf16 of the residual x 256), both
// blocked; 8 consecutive k of one row per thread (contiguous in the block).
__global__ __launch_bounds__(256) void split_weights_kernel(const float* __restrict__ w, uint16_t* __restrict__ hi,
                                                            uint16_t* __restrict__ lo, long long n8, int K) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const int n = (int)(i / (K / 8)), k = (int)(i % (K / 8)) * 8;
    const size_t o = router_w_index(n, k, K) / 8;
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
    reinterpret_cast<uint4*>(hi)[o] = make_uint4(h[0], h[1], h[2], h[3]);
    reinterpret_cast<uint4*>(lo)[o] = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ inline f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ inline void load32(uint4 (&v)[2], const uint16_t* p) {
    v[0] = reinterpret_cast<const uint4*>(p)[0];
    v[1] = reinterpret_cast<const uint4*>(p)[1];
}

// The lane's two 16-byte W operands (b = 0, 1) of expert tile et, step s.
__device__ inline void load_wb(uint4 (&v)[2], const uint16_t* part, int et, int s, int K, int lane) {
    const uint4* p = reinterpret_cast<const uint4*>(part + ((size_t)et * (K >> 6) + s) * 1024) + lane;
    v[0] = p[0];
    v[1] = p[64];
}

// scores = the S partial planes added in split order; 4 scores per thread,
// a thread's loads issued 8 planes at a time.
__global__ __launch_bounds__(256) void router_reduce_kernel(const f32x4* __restrict__ part, f32x4* __restrict__ out,
                                                            long long n4, int S) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    f32x4 s = part[i];
    for (int j0 = 1; j0 < S; j0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(long long)min(j0 + u, S - 1) * n4 + i];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < S) s += v[u];
    }
    out[i] = s;
}

// Thin form: workgroup (expert tile, token tile, split z); wave w takes the
// 64 k at 256 z + 64 w, lane (g, r) the 16 k at 16 g of that step for expert
// row r and token rows r of each 16-token tile.
template <int MT>
__global__ __launch_bounds__(64 * kThinWaves) void router_thin_kernel(RouterArgs a) {
    __shared__ f32x4 red[kThinWaves - 1][MT][64];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int et = blockIdx.x, n0 = 16 * et;
    const int m0 = blockIdx.y * 16 * MT;
    const int z = blockIdx.z;
    const int k = z * kThinK + w * kStep + 16 * g;

    f32x4 hi[MT], lo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) hi[mt] = lo[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        uint4 bh[2], bl[2], ax[MT][2];
        load_wb(bh, a.w_hi, et, k >> 6, a.K, lane);
        load_wb(bl, a.w_lo, et, k >> 6, a.K, lane);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) load32(ax[mt], a.x + (size_t)min(m0 + 16 * mt + r, a.M - 1) * a.K + k);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                hi[mt] = mfma(ax[mt][b], bh[b], hi[mt]);
                lo[mt] = mfma(ax[mt][b], bl[b], lo[mt]);
            }
    }
    f32x4 v[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) v[mt] = hi[mt] + lo[mt] * (1.f / 256.f);
    if (w > 0)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[w - 1][mt][lane] = v[mt];
    __syncthreads();
    if (w == 0) {
        float* dst = a.dst + (size_t)z * a.M * a.N;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int ww = 0; ww < kThinWaves - 1; ++ww) v[mt] += red[ww][mt][lane];     // wave order
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * mt + 4 * g + i;
                if (m < a.M) dst[(size_t)m * a.N + n0 + r] = v[mt][i];
            }
        }
    }
}

// Tile form.  One workgroup per (expert block of 192, token tile of 64,
// split z), laid out over the XCDs as described at the top.  Wave ew takes
// expert tiles 3 ew .. 3 ew + 2 of the block.  The workgroup's whole X tile
// (64 rows x K / S <= 1024 k) is loaded into LDS at the start; the loop then
// only streams W, one 64-k step ahead, and needs no barrier.  Workgroups
// start at different steps of their k range (rotated order), so the
// workgroups of an XCD that share a slice of W touch different parts of it
// at a time and most of their W loads hit the XCD's L2.
__global__ __launch_bounds__(64 * kTileWaves) void router_tile_kernel(RouterArgs a) {
    __shared__ __attribute__((aligned(16))) char xs[kTileXBytes];
    const int ew = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;

    const int L = blockIdx.x;
    int z, q, row;
    if (8 % a.S == 0) {                         // S in {1, 2, 4, 8}: XCD x works on part x % S
        const int xcd = L & 7, xp = 8 / a.S;
        row = L >> 3;
        z = xcd % a.S;
        q = row * xp + xcd / a.S;
    } else if (a.S % 8 == 0) {                  // S = 8 zp: XCD x on parts x zp .. x zp + zp - 1
        const int xcd = L & 7, zp = a.S >> 3;
        row = L >> 3;
        z = xcd * zp + row % zp;
        q = row / zp;
    } else {
        row = L / a.S;
        z = L % a.S;
        q = row;
    }
    if (q >= a.tiles) return;                   // whole workgroup: grid padding
    const int nb = q % a.tiles_n, m0 = (q / a.tiles_n) * kTileRows;
    const int kper = a.K / a.S, kz = z * kper;
    const int nch = kper / kChunk, nst = 2 * nch;
    const int ntile = a.N / 16;
    const int rot = row % nst;

    // X: lane's 4 pieces of 16 bytes per 128-k chunk; LDS position p of chunk
    // c holds row p / 16, piece (p % 16) ^ (row % 16) of its 128 k
    {
        uint32_t xoff[kXLoads];
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int p = 256 * i + 64 * ew + lane, prow = p >> 4, pc = (p & 15) ^ (prow & 15);
            xoff[i] = (uint32_t)min(m0 + prow, a.M - 1) * (uint32_t)a.K + (uint32_t)(kz + 8 * pc);
        }
        lds_char* xl = (lds_char*)xs;
        for (int c = 0; c < nch; ++c)
#pragma unroll
            for (int i = 0; i < kXLoads; ++i)
                dma16(a.x + xoff[i] + c * kChunk, xl + c * kStageBytes + 4096 * i + 1024 * ew);
    }
    // W: blocks of this wave's expert tiles (past the last tile: the last
    // one, computed and not stored) from step kz / 64 on, the lane's 16 bytes
    uint32_t woff[kTileNB];
#pragma unroll
    for (int j = 0; j < kTileNB; ++j) {
        const int et = min(nb * kTileNB * kTileEW + ew * kTileNB + j, ntile - 1);
        woff[j] = ((uint32_t)et * (uint32_t)(a.K >> 6) + (uint32_t)(kz >> 6)) * 1024u + 8u * lane;
    }
    const uint32_t xs_a = lds_addr((lds_char*)xs);

    f32x4 hi[kTileMT][kTileNB], lo[kTileMT][kTileNB];
#pragma unroll
    for (int mt = 0; mt < kTileMT; ++mt)
#pragma unroll
        for (int j = 0; j < kTileNB; ++j) hi[mt][j] = lo[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto step_of = [&](int t) { const int u = t + rot; return u < nst ? u : u - nst; };
    // w[j][0] = W_high, w[j][1] = W_low, halves b = 0, 1, of step s (64 k)
    auto load_w = [&](uint4 (&w)[kTileNB][2][2], int s) {
        const uint32_t o = s * 1024u;
#pragma unroll
        for (int j = 0; j < kTileNB; ++j) {
            const uint4* ph = reinterpret_cast<const uint4*>(a.w_hi + woff[j] + o);
            const uint4* pl = reinterpret_cast<const uint4*>(a.w_lo + woff[j] + o);
            w[j][0][0] = ph[0];
            w[j][0][1] = ph[64];
            w[j][1][0] = pl[0];
            w[j][1][1] = pl[64];
        }
    };
    // A operand of token tile mt, half b of the lane's 16 k in step s: row
    // 16 mt + r of chunk s / 2, logical piece 8 (s % 2) + 2 g + b
    auto step = [&](const uint4 (&w)[kTileNB][2][2], int s) {
        const uint32_t base = xs_a + (s >> 1) * kStageBytes + r * (kChunk * 2);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t pos = 16 * ((8 * (s & 1) + 2 * g + b) ^ r);
            uint4 ax[kTileMT];
            const uint32_t ad[4] = {base + pos, base + 16 * (kChunk * 2) + pos, base + 32 * (kChunk * 2) + pos,
                                    base + 48 * (kChunk * 2) + pos};
            lds_read4x16(ax, ad);
#pragma unroll
            for (int mt = 0; mt < kTileMT; ++mt)
#pragma unroll
                for (int j = 0; j < kTileNB; ++j) {
                    hi[mt][j] = mfma(ax[mt], w[j][0][b], hi[mt][j]);
                    lo[mt][j] = mfma(ax[mt], w[j][1][b], lo[mt][j]);
                }
        }
    };

    // Issue order: X (all), W(t0), W(t1), then W(t + 2) after step t.  Every
    // wait leaves exactly the one newest W step in flight.
    uint4 wa[kTileNB][2][2], wb[kTileNB][2][2];
    load_w(wa, step_of(0));
    load_w(wb, step_of(1));
    wait_vmcnt<kWLoads>();                      // X and W(t0) landed
    lds_barrier();                              // every wave's part of X
    // (the last pair of steps is peeled: a uniform loop body keeps the
    // compiler's own wait counts exact instead of waiting for every load)
    for (int t = 0; t + 2 < nst; t += 2) {
        step(wa, step_of(t));
        load_w(wa, step_of(t + 2));
        wait_vmcnt<kWLoads>();                  // W(t + 1) landed
        step(wb, step_of(t + 1));
        load_w(wb, step_of(t + 3));
        wait_vmcnt<kWLoads>();                  // W(t + 2) landed
    }
    step(wa, step_of(nst - 2));
    wait_vmcnt<0>();
    step(wb, step_of(nst - 1));

    // epilogue: hi + lo / 256
    float* dst = a.dst + (size_t)z * a.M * a.N;
#pragma unroll
    for (int mt = 0; mt < kTileMT; ++mt)
#pragma unroll
        for (int j = 0; j < kTileNB; ++j) {
            const f32x4 sc = hi[mt][j] + lo[mt][j] * (1.f / 256.f);
            const int et = nb * kTileNB * kTileEW + ew * kTileNB + j;
            if (et >= ntile) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * mt + 4 * g + i;
                if (m < a.M) dst[(size_t)m * a.N + 16 * et + r] = sc[i];
            }
        }
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

RouterPlan router_plan(int M, int N, int K) {
    RouterPlan p{};
    p.tile = M > kRouterThinMaxM;
    if (!p.tile) {
        p.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        p.tiles_n = N / 16;
        p.S = K / kThinK;
    } else {
        p.MT = kTileMT;
        p.tiles_n = ceil_div(N, kTileCols);
        const long long tiles = (long long)p.tiles_n * ceil_div(M, kTileRows);
        // parts of K: whole 256-k multiples of at most kRouterTileMaxK each (the
        // X tile lives in LDS); then more parts while the grid stays within
        // one workgroup per CU, up to kRouterTileMaxS
        const int units = K / kRouterKAlign;
        p.S = 1;
        while (K / p.S > kRouterTileMaxK || units % p.S != 0) ++p.S;
        while (2 * p.S <= kRouterTileMaxS && units % (2 * p.S) == 0 && tiles * p.S * 2 <= kRouterTileTarget) p.S *= 2;
    }
    p.workspace = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
    return p;
}

hipError_t launch_router_split(const float* w, void* hi, void* lo, int N, int K, hipStream_t stream) {
    const long long n8 = (long long)N * K / 8;
    if (n8 == 0) return hipSuccess;
    return launch(split_weights_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, w,
                  static_cast<uint16_t*>(hi), static_cast<uint16_t*>(lo), n8, K);
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
    a.tiles_n = p.tiles_n;
    hipError_t e;
    if (p.tile) {
        a.tiles = p.tiles_n * ceil_div(M, kTileRows);
        const long long grid = 8 % p.S == 0 ? 8LL * ceil_div(a.tiles, 8 / p.S) : (long long)a.tiles * p.S;
        e = launch(router_tile_kernel, dim3((unsigned)grid), dim3(64 * kTileWaves), 0, stream, a);
    } else {
        a.tiles = p.tiles_n * ceil_div(M, 16 * p.MT);
        const dim3 grid(p.tiles_n, a.tiles / p.tiles_n, p.S);
        if (p.MT == 1) e = launch(router_thin_kernel<1>, grid, dim3(64 * kThinWaves), 0, stream, a);
        else if (p.MT == 2) e = launch(router_thin_kernel<2>, grid, dim3(64 * kThinWaves), 0, stream, a);
        else e = launch(router_thin_kernel<4>, grid, dim3(64 * kThinWaves), 0, stream, a);
    }
    if (e != hipSuccess || p.S == 1) return e;
    const long long n4 = (long long)M * N / 4;
    return launch(router_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                  static_cast<const f32x4*>(workspace), reinterpret_cast<f32x4*>(out), n4, p.S);
}

}  // namespace lbsa
