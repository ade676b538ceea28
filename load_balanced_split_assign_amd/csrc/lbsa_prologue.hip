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
// gfx950 mapping.  The kernel streams bytes: per head vector 256 B in, 256 B
// (bf16) or 128 B + a scale (fp8) out, and about a hundred VALU instructions
// per 4 heads, so it is bound by HBM once enough loads are in flight.
//   * A 16-lane DPP row owns one head vector: lane j holds d = 8j .. 8j + 7
//     (one 16 B load, one 16 B or 8 B store), so a RoPE pair (d, d + 64) sits
//     in lanes j and j ^ 8, one row_ror:8 apart, and the norm and the fp8
//     maximum are 4-step DPP reductions inside the row: no LDS round trip.
//   * A wave takes 4 consecutive head vectors (a "group"); the types (Q, K, V)
//     may differ between its rows, so each lane selects its own weights,
//     output and destination, and nothing branches on the type.
//   * A workgroup (4 waves) takes K groups per wave of one token, issues all
//     its loads before anything else, then puts the token's 64 (cos, sin) into
//     LDS (angle and its reduction to [-pi, pi] in fp64, fp32 sin / cos).  The
//     host picks K (1 .. 8) so that the grid still holds enough workgroups:
//     decode batches split a token over several workgroups, prefill gives one
//     workgroup a whole token.
//   * bf16 results leave through gfx950's v_cvt_pk_bf16_f32 (round to nearest
//     even), fp8 codes through v_cvt_pk_fp8_f32 after a clamp to +-448.
#include <cmath>

#include "lbsa_internal.h"

namespace lbsa {
namespace {

constexpr int kPrologueThreads = 256;       // 4 waves
constexpr int kGroupHeads = 4;              // head vectors per wave (16 lanes each)
constexpr int kWaves = kPrologueThreads / 64;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// DPP controls: rotate a 16-lane row by 8 / 4, swap within a quad by 2 / 1.
constexpr int kRor8 = 0x128, kRor4 = 0x124, kQuadXor2 = 0x4E, kQuadXor1 = 0xB1;

template <int CTRL>
__device__ inline float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum / maximum over the 16 lanes of a DPP row, in every lane of the row:
// after ror 8 and ror 4 lane j holds its residue class mod 4, the two quad
// swaps join the classes.
__device__ inline float row_sum(float v) {
    v += dpp<kRor8>(v);
    v += dpp<kRor4>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kQuadXor1>(v);
    return v;
}
__device__ inline float row_max(float v) {
    v = fmaxf(v, dpp<kRor8>(v));
    v = fmaxf(v, dpp<kRor4>(v));
    v = fmaxf(v, dpp<kQuadXor2>(v));
    v = fmaxf(v, dpp<kQuadXor1>(v));
    return v;
}

__device__ inline uint32_t bf16x2_bits(float lo, float hi) {
    const bf16x2v h = __builtin_convertvector((f32x2){lo, hi}, bf16x2v);   // round to nearest even
    return __builtin_bit_cast(uint32_t, h);
}

// 4 values -> 4 e4m3fn codes (one dword, first value in the low byte), rounded
// to nearest even by the hardware convert; inputs are clamped to +-448 first.
__device__ inline uint32_t e4m3x4_bits(float a, float b, float c, float d) {
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
    uint8_t* k_cache;      // [pages][64][Hkv][128]
    uint8_t* v_cache;
    float* k_scale;        // fp8: [pages][Hkv][64]
    float* v_scale;
    int64_t num_slots;     // pages * 64
    double log2_theta;
    float eps;
    int32_t Hq, Hkv, slices;
};

enum HeadType : int { kQ = 0, kK = 1, kV = 2 };

// What every group of a workgroup shares: the token, its rotation and the
// lane's weights.
struct TokenCtx {
    int t;
    int64_t slot;
    float cosv[8], sinv[8];     // sinv carries the sign of the lane's half
    float wq[8], wk[8];
};

// One group (4 head vectors of one type, one per DPP row) in registers:
// QK-Norm + RoPE for Q and K, the fp8 scale, the store.  `live` is false for
// the rows past the type's last head (they hold a copy of it).
template <int TYPE, bool FP8>
__device__ inline void finish_group(const PrologueArgs& a, const TokenCtx& c, uint4 raw, int h, bool live,
                                    int j) {
    const int d0 = 8 * j;
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        y[2 * e] = __uint_as_float(rw[e] << 16);
        y[2 * e + 1] = __uint_as_float(rw[e] & 0xFFFF0000u);
    }
    if (TYPE != kV) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
        const float r = __builtin_amdgcn_rsqf(row_sum(ss) * (1.f / kHeadDim) + a.eps);
        float xn[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xn[e] = y[e] * ((TYPE == kQ ? c.wq[e] : c.wk[e]) * r);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = xn[e] * c.cosv[e] + dpp<kRor8>(xn[e]) * c.sinv[e];
    }
    if (!live) return;

    uint8_t* dst;
    float* sdst;
    if (TYPE == kQ) {
        const size_t row = (size_t)c.t * a.Hq + h;
        dst = a.q_out + (row * kHeadDim + d0) * (FP8 ? 1 : 2);
        sdst = a.q_scale + row;
    } else {
        dst = (TYPE == kK ? a.k_cache : a.v_cache) + (((size_t)c.slot * a.Hkv + h) * kHeadDim + d0) * (FP8 ? 1 : 2);
        sdst = (TYPE == kK ? a.k_scale : a.v_scale) + ((size_t)(c.slot >> 6) * a.Hkv + h) * kTile + (c.slot & 63);
    }
    if (FP8) {
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
        amax = row_max(amax);
        float scale = 1.f, inv = 1.f;
        if (amax > 0.f) {
            scale = amax * (1.f / 448.f);
            inv = 448.f * __builtin_amdgcn_rcpf(amax);
        }
        uint2 o;
        o.x = e4m3x4_bits(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
        o.y = e4m3x4_bits(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
        *reinterpret_cast<uint2*>(dst) = o;
        if (j == 0) *sdst = scale;
    } else {
        uint4 o = raw;                                           // V is copied bit for bit
        if (TYPE != kV) {
            o.x = bf16x2_bits(y[0], y[1]);
            o.y = bf16x2_bits(y[2], y[3]);
            o.z = bf16x2_bits(y[4], y[5]);
            o.w = bf16x2_bits(y[6], y[7]);
        }
        *reinterpret_cast<uint4*>(dst) = o;
    }
}

template <int K, bool FP8>
__global__ __launch_bounds__(kPrologueThreads) void prologue_kernel(PrologueArgs a) {
    __shared__ float cs[64], sn[64];
    // groups of the token: the query heads, then the key heads, then the value
    // heads, 4 to a group (a type's last group may be partly idle)
    const int GQ = (a.Hq + kGroupHeads - 1) / kGroupHeads, GKV = (a.Hkv + kGroupHeads - 1) / kGroupHeads;
    const int G = GQ + 2 * GKV, NV = a.Hq + 2 * a.Hkv;
    const int t = blockIdx.x / a.slices;
    const int g0 = (blockIdx.x - t * a.slices) * (kWaves * K);   // first group of this workgroup
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int j = lane & 15, sub = lane >> 4;
    const int d0 = 8 * j;

    // 1. every load of this workgroup's head vectors, before anything waits
    //    (idle rows load their type's last head again: no lane branches)
    TokenCtx c;
    c.t = t;
    {
        const float4 q0 = *reinterpret_cast<const float4*>(a.qw + d0), q1 = *reinterpret_cast<const float4*>(a.qw + d0 + 4);
        const float4 k0 = *reinterpret_cast<const float4*>(a.kw + d0), k1 = *reinterpret_cast<const float4*>(a.kw + d0 + 4);
        const float wq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        const float wk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            c.wq[e] = wq[e];
            c.wk[e] = wk[e];
        }
    }
    uint4 raw[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int g = g0 + wave + kWaves * k;
        if (g < G) {
            int hv;
            if (g < GQ) hv = min(kGroupHeads * g + sub, a.Hq - 1);
            else if (g < GQ + GKV) hv = a.Hq + min(kGroupHeads * (g - GQ) + sub, a.Hkv - 1);
            else hv = a.Hq + a.Hkv + min(kGroupHeads * (g - GQ - GKV) + sub, a.Hkv - 1);
            raw[k] = *reinterpret_cast<const uint4*>(a.qkv + ((size_t)t * NV + hv) * kHeadDim + d0);
        }
    }
    c.slot = a.slots[t];
    const bool slot_ok = c.slot >= 0 && c.slot < a.num_slots;

    // 2. the token's rotation, one (cos, sin) per lane of wave 0: the angle
    //    pos * theta^(-i/64) in fp64, reduced to [-pi, pi] in fp64, then fp32
    if (threadIdx.x < 64) {
        const int i = threadIdx.x;
        const double ang = (double)a.positions[t] * exp2(-(double)i * (1.0 / 64.0) * a.log2_theta);
        const double two_pi = 6.283185307179586476925286766559;
        const float red = (float)(ang - two_pi * rint(ang * (1.0 / two_pi)));
        float s, co;
        sincosf(red, &s, &co);
        cs[i] = co;
        sn[i] = s;
    }
    __syncthreads();
    // lane j rotates its dims with index (d0 & 63) .. + 7; the lower half of a
    // pair subtracts the partner's sine term, the upper half adds it
    {
        const int i0 = d0 & 63;
        const float sg = j < 8 ? -1.f : 1.f;
        const float4 c0 = *reinterpret_cast<const float4*>(cs + i0), c1 = *reinterpret_cast<const float4*>(cs + i0 + 4);
        const float4 s0 = *reinterpret_cast<const float4*>(sn + i0), s1 = *reinterpret_cast<const float4*>(sn + i0 + 4);
        const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            c.cosv[e] = cv[e];
            c.sinv[e] = sg * sv[e];
        }
    }
    // one wait for all loads (vmcnt(0)); the stores below then never make a
    // later group wait for an earlier group's store
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));

    // 3. per group: norm, rotate, quantise, store
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int g = g0 + wave + kWaves * k;
        if (g >= G) break;
        if (g < GQ) {
            const int h = kGroupHeads * g + sub;
            finish_group<kQ, FP8>(a, c, raw[k], h, h < a.Hq, j);
        } else if (slot_ok) {                                    // padding tokens write no cache row
            const bool is_k = g < GQ + GKV;
            const int h = kGroupHeads * (is_k ? g - GQ : g - GQ - GKV) + sub;
            if (is_k) finish_group<kK, FP8>(a, c, raw[k], h, h < a.Hkv, j);
            else finish_group<kV, FP8>(a, c, raw[k], h, h < a.Hkv, j);
        }
    }
}

template <int K>
hipError_t launch_k(const PrologueArgs& a, bool fp8, unsigned grid, hipStream_t stream) {
    return fp8 ? launch(prologue_kernel<K, true>, dim3(grid), dim3(kPrologueThreads), 0, stream, a)
               : launch(prologue_kernel<K, false>, dim3(grid), dim3(kPrologueThreads), 0, stream, a);
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
    a.num_slots = num_pages * kTile;
    a.log2_theta = std::log2(theta);
    a.eps = eps;
    a.Hq = Hq;
    a.Hkv = Hkv;
    // K groups per wave: the largest of 8, 4, 2, 1 that still leaves at least
    // kMinPrologueBlocks workgroups (a whole token per workgroup for prefill,
    // a token spread over several for small decode batches)
    const int G = (Hq + kGroupHeads - 1) / kGroupHeads + 2 * ((Hkv + kGroupHeads - 1) / kGroupHeads);
    constexpr long long kMinPrologueBlocks = 2048;
    int K = 8;
    while (K > 1 && (long long)T * ((G + kWaves * K - 1) / (kWaves * K)) < kMinPrologueBlocks) K /= 2;
    a.slices = (G + kWaves * K - 1) / (kWaves * K);
    const unsigned grid = (unsigned)((long long)T * a.slices);
    switch (K) {
        case 8: return launch_k<8>(a, fp8, grid, stream);
        case 4: return launch_k<4>(a, fp8, grid, stream);
        case 2: return launch_k<2>(a, fp8, grid, stream);
        default: return launch_k<1>(a, fp8, grid, stream);
    }
}

}  // namespace lbsa
