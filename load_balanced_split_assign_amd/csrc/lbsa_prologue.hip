// Fused attention prologue for gfx950: QK-Norm, then RoPE, then Q out (bf16,
// or fp8 codes with one scale per token and head), and K / V written into the
// paged cache (bf16, or fp8 codes with per-token-per-head scales).
//
// Method: vLLM post, section "A fused attention prologue" (SGLang post: the
// attention prologue section): one kernel starts from the fused QKV
// projection, normalises Q and K before rotating them (the Hy3 order), writes
// K and V straight into the paged cache and, in fp8, emits the query as fp8
// with its per-token, per-head scale, so that the attention kernel never
// re-quantises.
//
// Readings (the pages give the order, not the formulas):
//   * QK-Norm: RMSNorm over head_dim with one weight vector for the query heads
//     and one for the KV heads;
//   * RoPE: the pairs (d, d + 64) rotate by pos * theta^(-2d/128), d < 64;
//   * fp8: scale = max|x| / 448 per token and head (1 for an all-zero head),
//     codes rounded to nearest even; V is neither normalised nor rotated.
//
// gfx950 mapping.  A 32-lane half-wave owns one head vector (128 values): lane
// j holds d = 4j .. 4j + 3 for j < 16 and d = 64 + 4(j - 16) .. for j >= 16, so
// a RoPE pair sits in lanes j and j ^ 16 and the norm and the fp8 maximum are
// 32-lane reductions.  Every load and store of a head is one coalesced 256 B
// (bf16) or 128 B (fp8) access.  A workgroup (8 half-waves) takes 8 head
// vectors of one token; it first computes the token's 64 (cos, sin) pairs in
// fp64 (exact angle, then rounded to fp32) into LDS.
#include "lbsa_internal.h"

namespace lbsa {
namespace {

constexpr int kPrologueThreads = 256;
constexpr int kHeadsPerBlock = kPrologueThreads / 32;

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// 32-lane reductions inside a half-wave (xor partners stay in the half).
__device__ inline float half_sum(float v) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ inline float half_max(float v) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// 4 values -> 4 e4m3fn codes (one dword, value 0 in the low byte), rounded to
// nearest even by the hardware convert; inputs are clamped to +-448 first.
__device__ inline uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    c = fminf(fmaxf(c, -448.f), 448.f);
    d = fminf(fmaxf(d, -448.f), 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0, 1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);        // bytes 2, 3
    return (uint32_t)w;
}

struct PrologueArgs {
    const uint16_t* qkv;
    const int32_t* positions;
    const int64_t* slots;
    const float* qw;
    const float* kw;
    uint8_t* q_out;        // bf16 [T][Hq][128] or e4m3 [T][Hq][128]
    float* q_scale;        // fp8: [T][Hq]
    uint8_t* k_cache;
    uint8_t* v_cache;
    float* k_scale;        // fp8: [pages][Hkv][64]
    float* v_scale;
    int64_t num_pages;
    double theta;
    float eps;
    int32_t T, Hq, Hkv, fp8;
};

__global__ __launch_bounds__(kPrologueThreads) void prologue_kernel(PrologueArgs a) {
    __shared__ float cs[64], sn[64];
    const int NV = a.Hq + 2 * a.Hkv;
    const int blocks_per_token = (NV + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const int t = blockIdx.x / blocks_per_token;
    const int hv = (blockIdx.x - t * blocks_per_token) * kHeadsPerBlock + (threadIdx.x >> 5);
    const int j = threadIdx.x & 31;
    const int pos = a.positions[t];

    // the token's rotation: angle pos * theta^(-i/64) in fp64, then fp32 cos / sin
    if (threadIdx.x < 64) {
        const int i = threadIdx.x;
        const double ang = (double)pos * exp2(-(double)i / 64.0 * log2(a.theta));
        double s, c;
        sincos(ang, &s, &c);
        cs[i] = (float)c;
        sn[i] = (float)s;
    }
    __syncthreads();
    if (hv >= NV) return;

    const int d0 = j < 16 ? 4 * j : 64 + 4 * (j - 16);     // first of this lane's 4 dims
    const int i0 = d0 & 63;                                  // its rotation index
    const uint2 raw = *reinterpret_cast<const uint2*>(a.qkv + ((size_t)t * NV + hv) * kHeadDim + d0);
    float x[4] = {bf16_to_f32((uint16_t)raw.x), bf16_to_f32((uint16_t)(raw.x >> 16)),
                  bf16_to_f32((uint16_t)raw.y), bf16_to_f32((uint16_t)(raw.y >> 16))};

    const bool is_q = hv < a.Hq, is_k = !is_q && hv < a.Hq + a.Hkv;
    if (is_q || is_k) {
        // QK-Norm
        const float4 w = *reinterpret_cast<const float4*>((is_q ? a.qw : a.kw) + d0);
        const float ss = half_sum(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
        const float r = 1.f / sqrtf(ss * (1.f / kHeadDim) + a.eps);
        x[0] *= w.x * r;
        x[1] *= w.y * r;
        x[2] *= w.z * r;
        x[3] *= w.w * r;
        // RoPE: this lane's partner holds the other half of each pair
        float y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float other = __shfl_xor(x[k], 16, 64);
            const float c = cs[i0 + k], s = sn[i0 + k];
            y[k] = j < 16 ? x[k] * c - other * s : x[k] * c + other * s;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = y[k];
    }

    // fp8: per-head scale from the 32-lane maximum
    float scale = 1.f, inv = 1.f;
    if (a.fp8) {
        const float amax = half_max(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
        if (amax > 0.f) {
            scale = amax / 448.f;
            inv = 448.f / amax;
        }
    }

    if (is_q) {
        const size_t row = (size_t)t * a.Hq + hv;
        if (a.fp8) {
            *reinterpret_cast<uint32_t*>(a.q_out + row * kHeadDim + d0) =
                f32x4_to_e4m3(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
            if (j == 0) a.q_scale[row] = scale;
        } else {
            uint2 o;
            o.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
            o.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
            *reinterpret_cast<uint2*>(a.q_out + row * kHeadDim * 2 + d0 * 2) = o;
        }
        return;
    }

    // K or V into the paged cache: slot = page * 64 + row in the page
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= a.num_pages * kTile) return;          // padding token / out of range
    const int h = is_k ? hv - a.Hq : hv - a.Hq - a.Hkv;
    const int64_t page = slot / kTile, row = slot - page * kTile;
    uint8_t* cache = is_k ? a.k_cache : a.v_cache;
    const size_t elem = ((size_t)slot * a.Hkv + h) * kHeadDim + d0;   // token-major [page][row][h][d]
    if (a.fp8) {
        *reinterpret_cast<uint32_t*>(cache + elem) = f32x4_to_e4m3(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
        if (j == 0) (is_k ? a.k_scale : a.v_scale)[((size_t)page * a.Hkv + h) * kTile + row] = scale;
    } else {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
        *reinterpret_cast<uint2*>(cache + elem * 2) = o;
    }
}

}  // namespace

hipError_t launch_prologue(const uint16_t* qkv, const int32_t* positions, const int64_t* slots,
                           const float* qw, const float* kw, double theta, float eps, int T, int Hq,
                           int Hkv, bool fp8, void* q_out, float* q_scale, void* k_cache, void* v_cache,
                           float* k_scale, float* v_scale, int64_t num_pages, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    PrologueArgs a;
    a.qkv = qkv;
    a.positions = positions;
    a.slots = slots;
    a.qw = qw;
    a.kw = kw;
    a.q_out = static_cast<uint8_t*>(q_out);
    a.q_scale = q_scale;
    a.k_cache = static_cast<uint8_t*>(k_cache);
    a.v_cache = static_cast<uint8_t*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.num_pages = num_pages;
    a.theta = theta;
    a.eps = eps;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.fp8 = fp8 ? 1 : 0;
    const int NV = Hq + 2 * Hkv;
    const long long grid = (long long)T * ((NV + kHeadsPerBlock - 1) / kHeadsPerBlock);
    hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)grid), dim3(kPrologueThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lbsa
