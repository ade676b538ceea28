// Split (persistent), static split-KV and combine kernels for gfx950.
//
// Method: HPC-Ops vLLM post, section "The solution: a per-step, load-balanced
// decode scheduler", bullet "Compute and combine" (SGLang post: "Scheduling
// around live KV work"): each persistent workgroup loops over the descriptors
// of its bin, computes attention over the descriptor's consecutive 64-token
// tiles, writes a partial output with its log-sum-exp to a split buffer and
// moves on until its bin is drained; a combine kernel then reads the chunk
// count of each (head, request) and merges the partials under the global
// softmax normalisation into bf16.
//
// gfx950 mapping (one split workgroup = 4 wave64; all 8 query heads of one KV
// head are served together):
//   * wave w owns tokens [16w, 16w + 16) of every tile; its lane (r, g),
//     r = lane % 16, g = lane / 16, loads token row r of that slice with
//     128-bit global loads straight into MFMA operand registers (16 rows x 64
//     contiguous bytes per load instruction);
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows = 16 tokens, columns =
//     16 query heads of which 8 are real), fp32 accumulation;
//   * online softmax per wave in the exp2 domain; the row max needs two
//     cross-lane exchanges per tile, the row sum is reduced once per chunk;
//   * V is staged in LDS (wave-private, rows padded to 288 B) and read back
//     transposed with ds_read_b64_tr_b16 as the A operand of
//     O^T += V^T P^T (v_mfma_f32_16x16x16_bf16); P comes straight from the
//     S^T accumulator registers (its layout is already the B operand);
//   * fp8 (OCP e4m3fn) K/V are widened to bf16 in registers with
//     v_cvt_f32_fp8 + v_perm_b32 (exact), the per-token K scale multiplies the score
//     column and the per-token V scale is folded into p before PV;
//   * at the end of a chunk the 4 waves merge their (max, sum, O) through LDS
//     and one partial (fp32 O normalised, natural-log LSE) is written.
#include "lbsa_internal.h"

namespace lbsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// 16-byte store into LDS (HIP's uint4 has no address-space-3 assignment).
__device__ inline void lds_store16(lds_char* p, uint4 v) {
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

constexpr int kWaves = kSplitThreads / 64;
constexpr int kVPitch = 288;                 // bytes per staged V row (256 + 32 pad)
constexpr int kWaveLds = 16 * kVPitch;       // 4608 B per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline uint32_t bf16x2_bits(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;          // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// 4 e4m3fn codes (one dword) -> 4 bf16 (two dwords); exact, since every e4m3
// value has at most 4 significant bits.  Each byte is widened on its own
// (v_cvt_f32_fp8 with a byte select) and the upper halves of two fp32 results
// are packed with v_perm_b32.  (Taking the second element of the packed
// two-byte convert and masking it was miscompiled by this toolchain: the
// packing read element 0 twice.)
__device__ inline uint2 fp8x4_to_bf16x4(uint32_t w) {
    const uint32_t f0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(w, 0));
    const uint32_t f1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(w, 1));
    const uint32_t f2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(w, 2));
    const uint32_t f3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_f32_fp8(w, 3));
    uint2 r;
    r.x = __builtin_amdgcn_perm(f1, f0, 0x07060302u);   // {f0.hi16, f1.hi16}
    r.y = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    return r;
}

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// 8 e4m3 codes (two dwords) -> one bf16x8 operand.
__device__ inline uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    uint2 a = fp8x4_to_bf16x4(w0), b = fp8x4_to_bf16x4(w1);
    return make_uint4(a.x, a.y, b.x, b.y);
}

// Per-wave registers of one tile (the wave's 16-token slice).
template <bool FP8> struct Tile;
template <> struct Tile<false> {
    uint4 k[4], v[4];          // lane (r, g): token r, 16-byte chunks g + 4s
};
template <> struct Tile<true> {
    uint4 k[2], v[2];          // lane (r, g): token r, 16-byte chunks g + 4s
    f32x4 ks, vs;              // scales of score rows 4g .. 4g+3
};

// d offset (elements) of k-step s (8 elements) for lane group g; Q and K use
// the same map, so the QK^T contraction covers every d exactly once.
template <bool FP8> __device__ inline int kstep_d0(int g, int s) {
    return FP8 ? 16 * (g + 4 * (s >> 1)) + 8 * (s & 1) : 8 * (g + 4 * s);
}

// Uniform (scalar-cache) view of read-only metadata: page table, task map,
// lengths.  Loads through it with a wave-uniform address become s_load.
template <typename T>
__device__ inline const __attribute__((address_space(4))) T* uniform_ptr(const void* p) {
    return (const __attribute__((address_space(4))) T*)(p);
}

// Issue the loads of one tile (this wave's 16-token slice of page `page`).
// Branch-free: every row of the page is read, rows past the live length are
// zeroed later, so the compiler can keep NB tiles of loads in flight.
template <bool FP8>
__device__ inline void load_tile(Tile<FP8>& t, const AttnArgs& a, int64_t page, int h,
                                 uint32_t lane_off, uint32_t scale_off) {
    constexpr size_t kRowBytes = FP8 ? kHeadDim : 2 * kHeadDim;
    const size_t page_bytes = (size_t)kTile * (size_t)a.Hkv * kRowBytes;
    const char* kb = static_cast<const char*>(a.k_cache) + (size_t)page * page_bytes + lane_off;
    const char* vb = static_cast<const char*>(a.v_cache) + (size_t)page * page_bytes + lane_off;
    constexpr int kChunks = FP8 ? 2 : 4;
#pragma unroll
    for (int s = 0; s < kChunks; ++s) t.k[s] = *reinterpret_cast<const uint4*>(kb + 64 * s);
#pragma unroll
    for (int s = 0; s < kChunks; ++s) t.v[s] = *reinterpret_cast<const uint4*>(vb + 64 * s);
    if constexpr (FP8) {
        const size_t sc = ((size_t)page * a.Hkv + h) * kTile + scale_off;
        t.ks = *reinterpret_cast<const f32x4*>(a.k_scale + sc);
        t.vs = *reinterpret_cast<const f32x4*>(a.v_scale + sc);
    }
}

// Running state of one wave over one chunk.
struct WaveState {
    f32x4 acc[8];     // O^T[d = 16 db + 4 g + i][head r]
    float m;          // running max (log2 domain) of head r, uniform over g
    float l;          // this lane's share of the running sum of head r
};

// QK^T, staging of V into LDS, online softmax and PV for one tile.
template <bool FP8>
__device__ inline void tile_step(const Tile<FP8>& t, const bf16x8 (&q)[4], float sl2, int tok0,
                                 int L, int w, int r, int g, lds_char* vl, WaveState& st) {
    // row r of this slice is token tok0 + 16 w + r; rows past L hold whatever the
    // page tail holds (even NaN) and are zeroed before V reaches the MFMA.
    const bool row_live = tok0 + 16 * w + r < L;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    // ---- S^T = K Q^T: rows = this wave's 16 tokens, cols = 16 heads --------
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!FP8) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[ks]), q[ks], s, 0, 0, 0);
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 c = t.k[ks >> 1];
            const uint4 kb = (ks & 1) ? fp8x8_to_bf16x8(c.z, c.w) : fp8x8_to_bf16x8(c.x, c.y);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb), q[ks], s, 0, 0, 0);
        }
    }

    // ---- stage V (bf16) in this wave's LDS rows ----------------------------
    lds_char* row = vl + r * kVPitch;
    if constexpr (!FP8) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            lds_store16(row + 16 * (g + 4 * c), row_live ? t.v[c] : z4);
    } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint4 raw = row_live ? t.v[c] : z4;
            const int e0 = 16 * (g + 4 * c);              // first element of this 16-code chunk
            lds_store16(row + 2 * e0, fp8x8_to_bf16x8(raw.x, raw.y));
            lds_store16(row + 2 * e0 + 16, fp8x8_to_bf16x8(raw.z, raw.w));
        }
    }

    // ---- online softmax over the 4 score rows of this lane ------------------
    const int pos0 = tok0 + 16 * w + 4 * g;       // token of score row i is pos0 + i
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = s[i] * sl2;
        if constexpr (FP8) x *= t.ks[i];
        sc[i] = (pos0 + i < L) ? x : kNegInf;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(st.m, mt);
    const bool none = (m_new == kNegInf);        // no live token seen yet
    const float alpha = none ? 1.f : exp2_fast(st.m - m_new);
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = none ? 0.f : exp2_fast(sc[i] - m_new);
        psum += p[i];
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
    if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] *= (pos0 + i < L) ? t.vs[i] : 0.f;
    }
    s16x4 pb;
    {
        const uint32_t lo = bf16x2_bits(p[0], p[1]), hi = bf16x2_bits(p[2], p[3]);
        pb = __builtin_bit_cast(s16x4, make_uint2(lo, hi));
    }

    // ---- O^T += V^T P^T ------------------------------------------------------
    // ds_read_b64_tr_b16: in each 16-lane group, lane k supplies the address of
    // 4 consecutive d of token row 4g + k/4; lane i = 4a + c then receives
    // V[4g + j][16 db + i] for j = 0..3 -- the A operand (d x tokens).
    lds_char* tr = vl + (4 * g + (r >> 2)) * kVPitch + 8 * (r & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) s16x4*>(tr + 32 * db));
        st.acc[db] = st.acc[db] * alpha;
        st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, st.acc[db], 0, 0, 0);
    }
}

// Attention of the 8 query heads of KV head h of request b over tiles
// [t0, t1) (tokens < L), written as partial `slot`.  `NB` tiles are in flight
// per wave ahead of the one being computed.
template <bool FP8, int NB>
__device__ void process_chunk(const AttnArgs& a, int h, int b, int t0, int t1, int L, int64_t slot,
                              lds_char* lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    lds_char* vl = lds + w * kWaveLds;

    // ---- query operand (B of S^T = K Q^T): head r of the group, zero r >= 8 -
    bf16x8 q[4];
    float sl2 = a.scale_log2;
    {
        const int hq = h * kGroup + (r & 7);
        const size_t qrow = (size_t)b * a.Hq + hq;
        if constexpr (!FP8) {
            const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qrow * kHeadDim);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint4 v = qp[kstep_d0<false>(g, s) / 8];
                if (r >= kGroup) v = make_uint4(0, 0, 0, 0);
                q[s] = as_bf16x8(v);
            }
        } else {
            const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qrow * kHeadDim;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint2 v = *reinterpret_cast<const uint2*>(qp + kstep_d0<true>(g, s));
                uint4 c = fp8x8_to_bf16x8(v.x, v.y);
                if (r >= kGroup) c = make_uint4(0, 0, 0, 0);
                q[s] = as_bf16x8(c);
            }
            sl2 *= a.q_scale[qrow];
        }
    }

    WaveState st;
#pragma unroll
    for (int db = 0; db < 8; ++db) st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = kNegInf;
    st.l = 0.f;

    // ---- tile pipeline: NB tiles in flight ahead of the one being computed --
    // Page ids come through the scalar cache one tile before their loads are
    // issued; tiles past the chunk end re-read its last page (never used), so
    // the loop body has no data-dependent branch around a load.
    const int n = t1 - t0;
    const auto* pt = uniform_ptr<int32_t>(a.page_table) + (size_t)b * a.max_pages + t0;
    constexpr uint32_t kRowBytes = FP8 ? kHeadDim : 2 * kHeadDim;
    const uint32_t lane_off = ((uint32_t)(16 * w + r) * (uint32_t)a.Hkv + (uint32_t)h) * kRowBytes + 16u * g;
    const uint32_t scale_off = 16u * w + 4u * g;
    bool bad = false;
    auto page_at = [&](int k) -> int64_t { return (int64_t)pt[min(k, n - 1)]; };
    auto fetch = [&](Tile<FP8>& t, int64_t page) {
        const bool ok = page >= 0 && page < a.num_pages;
        bad |= !ok;
        load_tile<FP8>(t, a, ok ? page : 0, h, lane_off, scale_off);
    };

    Tile<FP8> buf[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) fetch(buf[u], page_at(u));
    int64_t next_page = page_at(NB);
    for (int k = 0; k < n; k += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int kk = k + u;
            const Tile<FP8> t = buf[u];                  // tile kk has landed
            const int64_t pg = next_page;
            next_page = page_at(kk + NB + 1);
            fetch(buf[u], pg);                           // tile kk + NB
            if (kk < n) tile_step<FP8>(t, q, sl2, 64 * (t0 + kk), L, w, r, g, vl, st);
        }
    }

    // ---- merge the 4 waves through LDS and write the partial ----------------
    float lsum = st.l;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    __attribute__((address_space(3))) float* o_w = reinterpret_cast<__attribute__((address_space(3))) float*>(vl);
    if (r < kGroup) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
            *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(o_w + r * kHeadDim + 16 * db + 4 * g) = st.acc[db];
        if (g == 0) {
            o_w[kGroup * kHeadDim + r] = st.m;
            o_w[kGroup * kHeadDim + kGroup + r] = lsum;
        }
    }
    if (lane == 0) o_w[kGroup * kHeadDim + 2 * kGroup] = bad ? 1.f : 0.f;
    __syncthreads();
    {
        const int tid = threadIdx.x;
        const int hh = tid >> 5, d4 = (tid & 31) * 4;
        float M = kNegInf;
        bool any_bad = false;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const __attribute__((address_space(3))) float* ow =
                reinterpret_cast<const __attribute__((address_space(3))) float*>(lds + ww * kWaveLds);
            M = fmaxf(M, ow[kGroup * kHeadDim + hh]);
            any_bad |= ow[kGroup * kHeadDim + 2 * kGroup] != 0.f;
        }
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        float lt = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const __attribute__((address_space(3))) float* ow =
                reinterpret_cast<const __attribute__((address_space(3))) float*>(lds + ww * kWaveLds);
            const float mw = ow[kGroup * kHeadDim + hh];
            const float sw = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
            lt += sw * ow[kGroup * kHeadDim + kGroup + hh];
            o += sw * *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(ow + hh * kHeadDim + d4);
        }
        float lse;
        if (any_bad || M == kNegInf) {
            const float nan = __builtin_nanf("");
            o = f32x4{nan, nan, nan, nan};
            lse = nan;
        } else {
            o *= 1.f / lt;
            lse = (M + __builtin_log2f(lt)) * kLn2;
        }
        *reinterpret_cast<f32x4*>(a.part_o + ((size_t)slot * kGroup + hh) * kHeadDim + d4) = o;
        if ((tid & 31) == 0) a.part_lse[(size_t)slot * kGroup + hh] = lse;
    }
    __syncthreads();   // LDS is reused by the next chunk
}

constexpr int kPipe = 2;   // tiles in flight per wave ahead of the computed one

template <bool FP8>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds_raw[kWaves * kWaveLds];
    lds_char* lds = (lds_char*)(lds_raw);   // address-space cast to LDS
    const MapLayout ML = map_layout(a.B, a.Hkv, a.P);
    const auto* hdr = uniform_ptr<int32_t>(a.map + ML.header);
    if (hdr[LBSA_HDR_ERROR] != 0 || hdr[LBSA_HDR_P] != a.P || hdr[LBSA_HDR_B] != a.B ||
        hdr[LBSA_HDR_HKV] != a.Hkv)
        return;
    const auto* bdb = uniform_ptr<int32_t>(a.map + ML.bin_desc_begin);
    const auto* desc = uniform_ptr<int32_t>(a.map + ML.desc);
    const auto* seqlens = uniform_ptr<int32_t>(a.map + ML.seqlens);
    const int cap = a.Hkv * a.B + a.P;
    for (int j = blockIdx.x; j < a.P; j += gridDim.x) {
        const int d0 = max(0, min(bdb[j], cap));
        const int d1 = max(d0, min(bdb[j + 1], cap));
        for (int d = d0; d < d1; ++d) {
            const int h = desc[4 * d], b = desc[4 * d + 1], t0 = desc[4 * d + 2], t1 = desc[4 * d + 3];
            if (h < 0 || h >= a.Hkv || b < 0 || b >= a.B || t0 < 0 || t1 <= t0 || t1 > a.max_pages)
                continue;
            const int L = min(seqlens[b], a.max_pages * kTile);
            process_chunk<FP8, kPipe>(a, h, b, t0, t1, L, d, lds);
        }
    }
}

template <bool FP8>
__global__ __launch_bounds__(kSplitThreads) void static_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds_raw[kWaves * kWaveLds];
    lds_char* lds = (lds_char*)(lds_raw);   // address-space cast to LDS
    const int S = a.P;
    const int split = blockIdx.x % S;
    const int rest = blockIdx.x / S;
    const int b = rest % a.B, h = rest / a.B;
    const int64_t slot = ((int64_t)h * a.B + b) * S + split;
    int L = uniform_ptr<int32_t>(a.seqlens)[b];
    const bool len_ok = L >= 0 && L <= a.max_pages * kTile;
    if (!len_ok) L = 0;
    const int n = (L + kTile - 1) / kTile;
    const int t0 = (int)((int64_t)split * n / S);
    const int t1 = (int)((int64_t)(split + 1) * n / S);
    if (t1 <= t0) {   // empty split: weight 0 in the combine
        const int tid = threadIdx.x;
        const int hh = tid >> 5, d4 = (tid & 31) * 4;
        *reinterpret_cast<f32x4*>(a.part_o + ((size_t)slot * kGroup + hh) * kHeadDim + d4) = f32x4{0.f, 0.f, 0.f, 0.f};
        if ((tid & 31) == 0) a.part_lse[(size_t)slot * kGroup + hh] = len_ok ? kNegInf : __builtin_nanf("");
        return;
    }
    process_chunk<FP8, kPipe>(a, h, b, t0, t1, L, slot, lds);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One workgroup per (request, query head): 8 slices of 32 threads stride over
// the chunks, each thread owns 4 consecutive d.
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(AttnArgs a, int static_mode) {
    __shared__ float red_m[8];
    __shared__ float red_w[8];
    __shared__ __attribute__((aligned(16))) float red_o[8][kHeadDim];
    const int row = blockIdx.x;
    const int b = row / a.Hq, hq = row - b * a.Hq;
    const int h = hq / kGroup, gq = hq - h * kGroup;
    const int64_t seg = (int64_t)h * a.B + b;
    const int tid = threadIdx.x, cs = tid >> 5, d4 = (tid & 31) * 4;
    uint16_t* out = static_cast<uint16_t*>(a.out) + ((size_t)b * a.Hq + hq) * kHeadDim + d4;

    int64_t d0 = 0;
    int n = 0;
    bool poison = false;
    if (static_mode) {
        d0 = seg * a.P;
        n = a.P;
    } else {
        const MapLayout ML = map_layout(a.B, a.Hkv, a.P);
        const int32_t* hdr = reinterpret_cast<const int32_t*>(a.map + ML.header);
        if (hdr[LBSA_HDR_P] != a.P || hdr[LBSA_HDR_B] != a.B || hdr[LBSA_HDR_HKV] != a.Hkv) {
            poison = true;
        } else if (hdr[LBSA_HDR_ERROR] == 0) {
            const int cap = a.Hkv * a.B + a.P;
            d0 = reinterpret_cast<const int32_t*>(a.map + ML.seg_first_desc)[seg];
            n = reinterpret_cast<const int32_t*>(a.map + ML.seg_num_chunks)[seg];
            if (d0 < 0 || n < 0 || d0 + n > cap) { poison = true; n = 0; }
        }
    }

    // pass 1: global max of the chunk LSEs
    float m = kNegInf;
    for (int c = cs; c < n; c += 8) m = fmaxf(m, a.part_lse[(d0 + c) * kGroup + gq]);
    if ((tid & 31) == 0) red_m[cs] = m;
    __syncthreads();
    float M = red_m[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) M = fmaxf(M, red_m[i]);

    // pass 2: weighted sum of the partial outputs
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float ws = 0.f;
    if (M != kNegInf) {
#pragma unroll 4
        for (int c = cs; c < n; c += 8) {
            const float l = a.part_lse[(d0 + c) * kGroup + gq];
            const float wgt = exp2_fast((l - M) * kLog2e);
            ws += wgt;
            o += wgt * *reinterpret_cast<const f32x4*>(a.part_o + ((d0 + c) * kGroup + gq) * kHeadDim + d4);
        }
    }
    if ((tid & 31) == 0) red_w[cs] = ws;
    *reinterpret_cast<f32x4*>(&red_o[cs][d4]) = o;
    __syncthreads();
    if (cs == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float wt = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc += *reinterpret_cast<const f32x4*>(&red_o[i][d4]);
            wt += red_w[i];
        }
        if (M == kNegInf || n == 0) acc = f32x4{0.f, 0.f, 0.f, 0.f};
        else acc *= 1.f / wt;
        if (poison || M != M) {
            const float nan = __builtin_nanf("");
            acc = f32x4{nan, nan, nan, nan};
        }
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(out) = packed;
    }
}

}  // namespace

hipError_t launch_split(const AttnArgs& a, bool fp8, hipStream_t stream) {
    if (fp8) hipLaunchKernelGGL(split_kernel<true>, dim3(a.P), dim3(kSplitThreads), 0, stream, a);
    else hipLaunchKernelGGL(split_kernel<false>, dim3(a.P), dim3(kSplitThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_static(const AttnArgs& a, bool fp8, hipStream_t stream) {
    const long long grid = (long long)a.P * a.B * a.Hkv;
    if (fp8) hipLaunchKernelGGL(static_kernel<true>, dim3((unsigned)grid), dim3(kSplitThreads), 0, stream, a);
    else hipLaunchKernelGGL(static_kernel<false>, dim3((unsigned)grid), dim3(kSplitThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, bool static_mode, hipStream_t stream) {
    const long long grid = (long long)a.B * a.Hq;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(kCombineThreads), 0, stream, a,
                       static_mode ? 1 : 0);
    return hipGetLastError();
}

hipError_t split_occupancy(bool fp8, int* blocks_per_cu) {
    if (fp8)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, split_kernel<true>, kSplitThreads, 0);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, split_kernel<false>, kSplitThreads, 0);
}

}  // namespace lbsa
