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
// gfx950 mapping.  One split workgroup = 4 wave64 serving all 8 query heads of
// one KV head; wave w owns tokens [16w, 16w + 16) of every 64-token tile.
//   * Tile stream: a workgroup's bin is one stream of tiles across all of its
//     descriptors.  Each wave keeps a private ring of kStages LDS stages and
//     fills it with asynchronous global->LDS loads (global_load_lds_dwordx4):
//     while tile k is computed, tiles k+1 .. k+kStages-1 are in flight, also
//     across descriptor boundaries, so the memory pipe never drains inside a
//     bin.  The compiler does not track these LDS writes; the kernel waits
//     for each stage itself with s_waitcnt vmcnt(N), N = loads issued after
//     that stage (vector memory operations complete in order).
//   * Loads are coalesced: each 64-lane load moves whole 256-byte K/V rows
//     (4 rows per instruction for bf16, 8 rows of 128 B for fp8).  Inside a
//     row the 16-byte chunks are XOR-swizzled by the row index, so the MFMA
//     operand reads (16 rows, same column) hit 16 different LDS bank groups.
//   * Rows past the live length are fetched from the tile's first row (always
//     live) instead, so no tail garbage or NaN ever reaches LDS; their scores
//     are masked to -inf, so they contribute nothing.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows = 16 tokens, columns =
//     16 query heads of which 8 are real), fp32 accumulation; online softmax
//     per wave in the exp2 domain.
//   * O^T += V^T P^T with v_mfma_f32_16x16x16_bf16: V^T comes from LDS through
//     ds_read_b64_tr_b16, P straight from the S^T accumulator registers (its
//     layout is already the B operand).
//   * fp8 (OCP e4m3fn) K is widened to bf16 in registers (v_cvt_f32_fp8 +
//     v_perm_b32, exact), fp8 V is widened into a bf16 LDS area before the
//     transposed reads; the per-token K scale multiplies the score column and
//     the per-token V scale is folded into p before PV.
//   * At the end of a descriptor the 4 waves merge (max, sum, O) through LDS
//     and one partial (fp32 O normalised, natural-log LSE) is written.
#include "lbsa_internal.h"

namespace lbsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = kSplitThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline uint4 lds_load16(const lds_char* p) {
    return __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p));
}
__device__ inline uint2 lds_load8(const lds_char* p) {
    return __builtin_bit_cast(uint2, *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(p));
}
__device__ inline void lds_store16(lds_char* p, uint4 v) {
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

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

// 8 e4m3 codes (two dwords) -> 8 bf16 (one 16-byte operand).
__device__ inline uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    uint2 a = fp8x4_to_bf16x4(w0), b = fp8x4_to_bf16x4(w1);
    return make_uint4(a.x, a.y, b.x, b.y);
}

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Uniform (scalar-cache) view of read-only metadata: page table, task map,
// lengths.  Loads through it with a wave-uniform address become s_load.
template <typename T>
__device__ inline const __attribute__((address_space(4))) T* uniform_ptr(const void* p) {
    return (const __attribute__((address_space(4))) T*)(p);
}

// s_waitcnt vmcnt(n) with the LDS and export counters left unconstrained,
// followed by a compiler barrier so no LDS access moves above it.
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __asm__ volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Per-wave LDS ring stage.  bf16: K 16 x 256 B, V 16 x 256 B; fp8: K 16 x 128 B,
// V 16 x 128 B, scales (k[16], v[16], q[8]).  The group's Q rows (8 x 256 B or
// 8 x 128 B) of each stage live in a separate array.
// ---------------------------------------------------------------------------
template <bool FP8> struct Stage {
    static constexpr int kRow = FP8 ? 128 : 256;        // bytes of one K/V/Q row
    static constexpr int K = 0;
    static constexpr int V = 16 * kRow;
    static constexpr int SC = 32 * kRow;                // fp8 only
    static constexpr int BYTES = SC + (FP8 ? 256 : 0);   // 8192 (bf16) / 4352 (fp8)
    static constexpr int Q_BYTES = 8 * kRow;              // Q rows of the group, own array per stage
    static constexpr int LOADS = FP8 ? 6 : 10;          // Q, K, V (and scale) loads issued per tile
    static constexpr int STAGES = FP8 ? 4 : 3;          // ring depth
    static constexpr int VB = FP8 ? 16 * 256 : 0;       // fp8: bf16 copy of the V slice
};

// 16-byte chunk swizzle inside a row: LDS chunk c' holds row chunk c' ^ f(row).
template <bool FP8> __device__ inline int swz(int row) { return FP8 ? ((row >> 1) & 7) : (row & 15); }
__device__ inline int swz_bf16(int row) { return row & 15; }

// LDS of one split / static workgroup.  Every ring stage is its own
// __shared__ object: the compiler's wait-count insertion can then tell which
// asynchronous load an LDS read depends on (distinct underlying objects) and
// does not fall back to waiting for all of them.
constexpr int kMergeWave = (kGroup * kHeadDim + 2 * kGroup + 4) * 4;   // O, m, l, flag per wave
constexpr int kMergeBytes = kWaves * kMergeWave;
template <bool FP8> struct Smem {
    lds_char* stage[4];   // [kWaves][Stage::BYTES] each; the first STAGES are used
    lds_char* qst[4];     // [kWaves][Stage::Q_BYTES] each
    lds_char* vb;         // fp8: [kWaves][4096] bf16 copy of the V slice
    lds_char* merge;      // [kMergeBytes]
};
template <bool FP8> constexpr int stage_array_bytes(int u) {
    return u < Stage<FP8>::STAGES ? kWaves * Stage<FP8>::BYTES : 16;
}
template <bool FP8> constexpr int q_array_bytes(int u) {
    return u < Stage<FP8>::STAGES ? kWaves * Stage<FP8>::Q_BYTES : 16;
}
constexpr int kVbBytes = kWaves * 16 * 256;

// One descriptor of the tile stream (all fields wave-uniform).
struct Desc {
    int h, b, t0, t1, L;
    int64_t slot;
};

// Asynchronous global -> LDS loads: lane i's 16 (or 4) bytes land at
// lds + 16 i (or 4 i).  Non-template wrappers keep the target builtin out of
// dependent (template) contexts.
__device__ inline void dma16(const void* g, lds_char* l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ inline void dma4(const void* g, lds_char* l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}

// Issue the asynchronous loads of one tile into `st` (this wave's 16-token
// slice of page `page`): K and V rows (whole rows, chunk-swizzled), the fp8
// scales, and -- for the first tile of a descriptor -- the group's Q rows.
template <bool FP8>
__device__ inline void issue_tile(const AttnArgs& a, lds_char* __restrict__ st, lds_char* __restrict__ qs,
                                  int64_t page, const Desc& d, int tile, int w, int lane) {
    using SL = Stage<FP8>;
    constexpr size_t kRow = SL::kRow;
    const int tok0 = 64 * tile;
    const char* kc = static_cast<const char*>(a.k_cache);
    const char* vc = static_cast<const char*>(a.v_cache);
    {   // the group's Q rows, every tile (uniform load count; only a descriptor's first tile reads them)
        const char* q = static_cast<const char*>(a.q) + ((size_t)d.b * a.Hq + (size_t)d.h * kGroup) * kRow;
        if constexpr (!FP8) {
#pragma unroll
            for (int s = 0; s < 2; ++s)      // 4 heads x 256 B per load
                dma16(q + 1024 * s + 16 * lane, qs + 1024 * s);
        } else {                             // 8 heads x 128 B
            dma16(q + 16 * lane, qs);
        }
    }
    constexpr int kRowsPerLoad = 1024 / kRow;          // 4 (bf16) or 8 (fp8)
    constexpr int kChunks = kRow / 16;
#pragma unroll
    for (int s = 0; s < 16 / kRowsPerLoad; ++s) {
        const int row = kRowsPerLoad * s + lane / kChunks;        // row of this wave's slice
        const int cl = lane % kChunks;                            // LDS chunk
        const int trow = (tok0 + 16 * w + row < d.L) ? 16 * w + row : 0;   // dead rows read row 0
        const size_t goff = (((size_t)page * kTile + trow) * a.Hkv + d.h) * kRow + 16 * (cl ^ swz<FP8>(row));
        dma16(kc + goff, st + SL::K + 1024 * s);
        dma16(vc + goff, st + SL::V + 1024 * s);
    }
    if constexpr (FP8) {
        // lanes 0-15: k scale of rows 0-15, 16-31: v scale, 32-39: q scale of the group
        const int row = lane & 15;
        const int trow = (tok0 + 16 * w + row < d.L) ? 16 * w + row : 0;
        const size_t sidx = ((size_t)page * a.Hkv + d.h) * kTile + trow;
        const float* src = lane < 16 ? a.k_scale + sidx
                         : lane < 32 ? a.v_scale + sidx
                                     : a.q_scale + (size_t)d.b * a.Hq + (size_t)d.h * kGroup + (lane & 7);
        dma4(src, st + SL::SC);
    }
}

// The 8 transposed V reads of one tile (one per 16-wide d block), issued
// together and completed (lgkmcnt(0)) before returning.  Written as one asm
// block: the compiler models the transposed-read intrinsic without the LDS
// alias information it uses for ordinary LDS loads, and would otherwise wait
// for every asynchronous load in flight before each of them.  The LDS data
// they read is ordered by the caller's explicit vmcnt wait (memory clobber).
__device__ inline void vt_read8(s16x4 (&va)[8], const uint32_t (&addr)[8]) {
    typedef short s16x4_v __attribute__((ext_vector_type(4)));
    s16x4_v o0, o1, o2, o3, o4, o5, o6, o7;
    __asm__ volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(o4), "=&v"(o5), "=&v"(o6), "=&v"(o7)
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7])
        : "memory");
    va[0] = __builtin_bit_cast(s16x4, o0);
    va[1] = __builtin_bit_cast(s16x4, o1);
    va[2] = __builtin_bit_cast(s16x4, o2);
    va[3] = __builtin_bit_cast(s16x4, o3);
    va[4] = __builtin_bit_cast(s16x4, o4);
    va[5] = __builtin_bit_cast(s16x4, o5);
    va[6] = __builtin_bit_cast(s16x4, o6);
    va[7] = __builtin_bit_cast(s16x4, o7);
}

// Two 16-byte LDS reads completed before returning (asm for the same reason
// as vt_read8: the fp8 V rows come from asynchronous loads ordered by the
// caller's explicit vmcnt wait).
__device__ inline void lds_read2x16(uint4& x, uint4& y, uint32_t ax, uint32_t ay) {
    u32x4 ox, oy;
    __asm__ volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(ox), "=&v"(oy)
        : "v"(ax), "v"(ay)
        : "memory");
    x = __builtin_bit_cast(uint4, ox);
    y = __builtin_bit_cast(uint4, oy);
}

// Running state of one wave over one descriptor.
struct WaveState {
    f32x4 acc[8];     // O^T[d = 16 db + 4 g + i][head r]
    float m;          // running max (log2 domain) of head r, uniform over g
    float l;          // this lane's share of the running sum of head r
};

// Q operand of a descriptor (B of S^T = K Q^T) from the stage of its first
// tile: head r of the group, zero for r >= 8.  Also returns the score scale.
template <bool FP8>
__device__ inline void read_q(const lds_char* __restrict__ qs, const lds_char* __restrict__ st, int r, int g,
                              float scale_log2, bf16x8 (&q)[4], float& sl2) {
    using SL = Stage<FP8>;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const int hr = r & 7;
    sl2 = scale_log2;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint4 v;
        if constexpr (!FP8) {
            v = lds_load16(qs + hr * 256 + 16 * (g + 4 * ks));
        } else {
            const uint2 c = lds_load8(qs + hr * 128 + 16 * (g + 4 * (ks >> 1)) + 8 * (ks & 1));
            v = fp8x8_to_bf16x8(c.x, c.y);
        }
        q[ks] = as_bf16x8(r < kGroup ? v : z);
    }
    if constexpr (FP8) sl2 *= *reinterpret_cast<const __attribute__((address_space(3))) float*>(st + SL::SC + 4 * (32 + hr));
}

// QK^T, online softmax and PV of one tile held in stage `st`.
template <bool FP8>
__device__ inline void tile_compute(const lds_char* __restrict__ st, lds_char* __restrict__ vb, const bf16x8 (&q)[4], float sl2, int tok0,
                                    int L, int w, int r, int g, WaveState& ws) {
    using SL = Stage<FP8>;
    // ---- S^T = K Q^T: rows = this wave's 16 tokens, cols = 16 heads --------
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!FP8) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 k = lds_load16(st + SL::K + r * 256 + 16 * ((g + 4 * ks) ^ swz<false>(r)));
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k), q[ks], s, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint4 c = lds_load16(st + SL::K + r * 128 + 16 * ((g + 4 * p) ^ swz<true>(r)));
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fp8x8_to_bf16x8(c.x, c.y)), q[2 * p], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fp8x8_to_bf16x8(c.z, c.w)), q[2 * p + 1], s, 0, 0, 0);
        }
        // widen this lane's two V chunks of row r into the bf16 copy (same swizzle as bf16 V)
        uint4 raw[2];
        lds_read2x16(raw[0], raw[1], (uint32_t)(size_t)(st + SL::V + r * 128 + 16 * (g ^ swz<true>(r))),
                     (uint32_t)(size_t)(st + SL::V + r * 128 + 16 * ((g + 4) ^ swz<true>(r))));
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = g + 4 * p;
            lds_store16(vb + r * 256 + 16 * ((2 * c) ^ swz_bf16(r)), fp8x8_to_bf16x8(raw[p].x, raw[p].y));
            lds_store16(vb + r * 256 + 16 * ((2 * c + 1) ^ swz_bf16(r)), fp8x8_to_bf16x8(raw[p].z, raw[p].w));
        }
    }

    // ---- online softmax over the 4 score rows of this lane ------------------
    const int pos0 = tok0 + 16 * w + 4 * g;       // token of score row i is pos0 + i
    f32x4 ks4, vs4;
    if constexpr (FP8) {
        ks4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(st + SL::SC + 16 * g);
        vs4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(st + SL::SC + 64 + 16 * g);
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = s[i] * sl2;
        if constexpr (FP8) x *= ks4[i];
        sc[i] = (pos0 + i < L) ? x : kNegInf;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(ws.m, mt);
    const bool none = (m_new == kNegInf);        // no live token seen yet
    const float alpha = none ? 1.f : exp2_fast(ws.m - m_new);
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = none ? 0.f : exp2_fast(sc[i] - m_new);
        psum += p[i];
    }
    ws.l = ws.l * alpha + psum;
    ws.m = m_new;
    if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] *= vs4[i];
    }
    const s16x4 pb = __builtin_bit_cast(s16x4, make_uint2(bf16x2_bits(p[0], p[1]), bf16x2_bits(p[2], p[3])));

    // ---- O^T += V^T P^T ------------------------------------------------------
    // ds_read_b64_tr_b16: in each 16-lane group, lane k supplies the address of
    // 4 consecutive d of token row 4g + k/4; lane i = 4a + c then receives
    // V[4g + j][16 db + i] for j = 0..3 -- the A operand (d x tokens).
    const lds_char* vbase = FP8 ? (const lds_char*)vb : st + SL::V;
    const int vrow = 4 * g + (r >> 2);
    const uint32_t vr = (uint32_t)(size_t)(vbase + vrow * 256 + 8 * (r & 1));   // LDS byte address
    uint32_t addr[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) addr[db] = vr + 16u * (uint32_t)((2 * db + ((r >> 1) & 1)) ^ swz_bf16(vrow));
    s16x4 va[8];
    vt_read8(va, addr);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        ws.acc[db] = ws.acc[db] * alpha;
        ws.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[db], pb, ws.acc[db], 0, 0, 0);
    }
}

// Workgroup barrier for LDS exchange only.  __syncthreads() also fences
// global memory, which would wait for every asynchronous load in flight; the
// merge only needs this wave's LDS writes done (lgkmcnt(0)) before s_barrier.
__device__ inline void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0), vmcnt(63)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// End of a descriptor: merge the 4 waves' (max, sum, O) through LDS and write
// the partial (normalised O, natural-log LSE) of slot d.slot.
__device__ inline void finish_desc(const AttnArgs& a, lds_char* merge, const WaveState& ws, bool bad,
                                   int64_t slot, int w, int lane, int r, int g) {
    float lsum = ws.l;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    __attribute__((address_space(3))) float* o_w =
        reinterpret_cast<__attribute__((address_space(3))) float*>(merge + w * kMergeWave);
    if (r < kGroup) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
            *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(o_w + r * kHeadDim + 16 * db + 4 * g) = ws.acc[db];
        if (g == 0) {
            o_w[kGroup * kHeadDim + r] = ws.m;
            o_w[kGroup * kHeadDim + kGroup + r] = lsum;
        }
    }
    if (lane == 0) o_w[kGroup * kHeadDim + 2 * kGroup] = bad ? 1.f : 0.f;
    lds_barrier();
    {
        const int tid = threadIdx.x;
        const int hh = tid >> 5, d4 = (tid & 31) * 4;
        float M = kNegInf;
        bool any_bad = false;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const __attribute__((address_space(3))) float* ow =
                reinterpret_cast<const __attribute__((address_space(3))) float*>(merge + ww * kMergeWave);
            M = fmaxf(M, ow[kGroup * kHeadDim + hh]);
            any_bad |= ow[kGroup * kHeadDim + 2 * kGroup] != 0.f;
        }
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        float lt = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const __attribute__((address_space(3))) float* ow =
                reinterpret_cast<const __attribute__((address_space(3))) float*>(merge + ww * kMergeWave);
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
    lds_barrier();   // the merge area is reused by the next descriptor
}

// Descriptor sources of the tile stream.
struct MapDescs {           // descriptors [d0, d1) of a task-map bin
    const __attribute__((address_space(4))) int32_t* desc;
    const __attribute__((address_space(4))) int32_t* seqlens;
    int d0, d1, Hkv, B, max_pages;
    __device__ int count() const { return d1 - d0; }
    // descriptor i (0-based in the bin); an invalid one (corrupt map) has no tiles
    __device__ Desc get(int i) const {
        const int d = d0 + i;
        Desc x;
        x.h = desc[4 * d];
        x.b = desc[4 * d + 1];
        x.t0 = desc[4 * d + 2];
        x.t1 = desc[4 * d + 3];
        x.slot = d;
        if (x.h < 0 || x.h >= Hkv || x.b < 0 || x.b >= B || x.t0 < 0 || x.t1 <= x.t0 || x.t1 > max_pages) {
            x.h = 0; x.b = 0; x.t0 = 0; x.t1 = 0; x.L = 0;
        } else {
            x.L = min(seqlens[x.b], max_pages * kTile);
        }
        return x;
    }
};

struct OneDesc {            // the static kernel's single chunk
    Desc d;
    __device__ int count() const { return 1; }
    __device__ Desc get(int) const { return d; }
};

// Cursor over the tiles of a descriptor source (wave-uniform).
template <class Src>
struct Cursor {
    const Src* src;
    int i;          // descriptor ordinal
    int t;          // tile of that descriptor
    Desc d;
    __device__ void seek_valid() {      // skip descriptors without tiles
        while (i < src->count()) {
            d = src->get(i);
            if (d.t1 > d.t0) { t = d.t0; return; }
            ++i;
        }
    }
    __device__ void begin(const Src* s) { src = s; i = 0; seek_valid(); }
    __device__ void next() {
        if (++t >= d.t1) { ++i; seek_valid(); }
    }
};

// Issue the next tile of the load cursor into ring stage `slot`.
template <bool FP8, class Src>
__device__ inline void issue_step(const AttnArgs& a, Cursor<Src>& lc, int& issued, int ntiles, uint32_t& bad_bits,
                                  lds_char* st, lds_char* qs, int slot, int w, int lane) {
    const int64_t pg = (int64_t)uniform_ptr<int32_t>(a.page_table)[(size_t)lc.d.b * a.max_pages + lc.t];
    const bool ok = pg >= 0 && pg < a.num_pages;
    bad_bits = (bad_bits & ~(1u << slot)) | ((uint32_t)(!ok) << slot);
    issue_tile<FP8>(a, st, qs, ok ? pg : 0, lc.d, lc.t, w, lane);
    if (++issued < ntiles) lc.next();
}

// Stream every tile of `src` through this workgroup (see the header comment).
template <bool FP8, class Src>
__device__ void run_stream(const AttnArgs& a, const Src& src, int ntiles, const Smem<FP8>& sm) {
    using SL = Stage<FP8>;
    constexpr int S = SL::STAGES;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    auto stage = [&](int u) -> lds_char* { return sm.stage[u] + w * SL::BYTES; };
    auto qstage = [&](int u) -> lds_char* { return sm.qst[u] + w * SL::Q_BYTES; };
    lds_char* vb = sm.vb + w * (16 * 256);
    lds_char* merge = sm.merge;

    // load cursor: runs S-1 tiles ahead; past the last tile it re-issues the
    // last tile (into a free stage, never read) so every step issues the same
    // number of loads and the vmcnt bound below stays exact.
    Cursor<Src> lc;
    lc.begin(&src);
    int issued = 0;
    uint32_t bad_bits = 0;          // bit u: the tile in stage u has an out-of-range page id
#pragma unroll
    for (int u = 0; u < S - 1; ++u) issue_step<FP8>(a, lc, issued, ntiles, bad_bits, stage(u), qstage(u), u, w, lane);

    Cursor<Src> cc;
    cc.begin(&src);
    WaveState ws;
    bf16x8 q[4];
    float sl2 = 0.f;
    bool bad = false;
    for (int k = 0; k < ntiles; k += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int kk = k + u;
            issue_step<FP8>(a, lc, issued, ntiles, bad_bits, stage((u + S - 1) % S), qstage((u + S - 1) % S),
                            (u + S - 1) % S, w, lane);                  // tile kk + S - 1
            wait_vmcnt<(S - 1) * SL::LOADS>();                // tile kk has landed
            if (kk < ntiles) {
                const lds_char* st = stage(u);
                if (cc.t == cc.d.t0) {                            // first tile of a descriptor
                    read_q<FP8>(qstage(u), st, r, g, a.scale_log2, q, sl2);
#pragma unroll
                    for (int db = 0; db < 8; ++db) ws.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
                    ws.m = kNegInf;
                    ws.l = 0.f;
                    bad = false;
                }
                bad |= (bad_bits >> u) & 1u;
                tile_compute<FP8>(st, vb, q, sl2, 64 * cc.t, cc.d.L, w, r, g, ws);
                if (cc.t + 1 == cc.d.t1) finish_desc(a, merge, ws, bad, cc.d.slot, w, lane, r, g);
                cc.next();
            }
        }
    }
    wait_vmcnt<0>();   // no load may still target LDS when the workgroup retires
}

template <bool FP8>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char s0[stage_array_bytes<FP8>(0)];
    __shared__ __attribute__((aligned(16))) char s1[stage_array_bytes<FP8>(1)];
    __shared__ __attribute__((aligned(16))) char s2[stage_array_bytes<FP8>(2)];
    __shared__ __attribute__((aligned(16))) char s3[stage_array_bytes<FP8>(3)];
    __shared__ __attribute__((aligned(16))) char q0[q_array_bytes<FP8>(0)];
    __shared__ __attribute__((aligned(16))) char q1[q_array_bytes<FP8>(1)];
    __shared__ __attribute__((aligned(16))) char q2[q_array_bytes<FP8>(2)];
    __shared__ __attribute__((aligned(16))) char q3[q_array_bytes<FP8>(3)];
    __shared__ __attribute__((aligned(16))) char svb[FP8 ? kVbBytes : 16];
    __shared__ __attribute__((aligned(16))) char smerge[kMergeBytes];
    Smem<FP8> sm;   // address-space casts to LDS
    sm.stage[0] = (lds_char*)s0;
    sm.stage[1] = (lds_char*)s1;
    sm.stage[2] = (lds_char*)s2;
    sm.stage[3] = (lds_char*)s3;
    sm.qst[0] = (lds_char*)q0;
    sm.qst[1] = (lds_char*)q1;
    sm.qst[2] = (lds_char*)q2;
    sm.qst[3] = (lds_char*)q3;
    sm.vb = (lds_char*)svb;
    sm.merge = (lds_char*)smerge;
    const MapLayout ML = map_layout(a.B, a.Hkv, a.P);
    const auto* hdr = uniform_ptr<int32_t>(a.map + ML.header);
    if (hdr[LBSA_HDR_ERROR] != 0 || hdr[LBSA_HDR_P] != a.P || hdr[LBSA_HDR_B] != a.B ||
        hdr[LBSA_HDR_HKV] != a.Hkv)
        return;
    const auto* bdb = uniform_ptr<int32_t>(a.map + ML.bin_desc_begin);
    const int cap = a.Hkv * a.B + a.P;
    for (int j = blockIdx.x; j < a.P; j += gridDim.x) {
        MapDescs src;
        src.desc = uniform_ptr<int32_t>(a.map + ML.desc);
        src.seqlens = uniform_ptr<int32_t>(a.map + ML.seqlens);
        src.d0 = max(0, min(bdb[j], cap));
        src.d1 = max(src.d0, min(bdb[j + 1], cap));
        src.Hkv = a.Hkv;
        src.B = a.B;
        src.max_pages = a.max_pages;
        int ntiles = 0;
        for (int i = 0; i < src.count(); ++i) {
            const Desc d = src.get(i);
            ntiles += d.t1 - d.t0;
        }
        if (ntiles > 0) run_stream<FP8>(a, src, ntiles, sm);
    }
}

template <bool FP8>
__global__ __launch_bounds__(kSplitThreads) void static_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char s0[stage_array_bytes<FP8>(0)];
    __shared__ __attribute__((aligned(16))) char s1[stage_array_bytes<FP8>(1)];
    __shared__ __attribute__((aligned(16))) char s2[stage_array_bytes<FP8>(2)];
    __shared__ __attribute__((aligned(16))) char s3[stage_array_bytes<FP8>(3)];
    __shared__ __attribute__((aligned(16))) char q0[q_array_bytes<FP8>(0)];
    __shared__ __attribute__((aligned(16))) char q1[q_array_bytes<FP8>(1)];
    __shared__ __attribute__((aligned(16))) char q2[q_array_bytes<FP8>(2)];
    __shared__ __attribute__((aligned(16))) char q3[q_array_bytes<FP8>(3)];
    __shared__ __attribute__((aligned(16))) char svb[FP8 ? kVbBytes : 16];
    __shared__ __attribute__((aligned(16))) char smerge[kMergeBytes];
    Smem<FP8> sm;   // address-space casts to LDS
    sm.stage[0] = (lds_char*)s0;
    sm.stage[1] = (lds_char*)s1;
    sm.stage[2] = (lds_char*)s2;
    sm.stage[3] = (lds_char*)s3;
    sm.qst[0] = (lds_char*)q0;
    sm.qst[1] = (lds_char*)q1;
    sm.qst[2] = (lds_char*)q2;
    sm.qst[3] = (lds_char*)q3;
    sm.vb = (lds_char*)svb;
    sm.merge = (lds_char*)smerge;
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
    if (t1 <= t0) {   // empty split: weight 0 in the combine (NaN if the length was invalid)
        const int tid = threadIdx.x;
        const int hh = tid >> 5, d4 = (tid & 31) * 4;
        *reinterpret_cast<f32x4*>(a.part_o + ((size_t)slot * kGroup + hh) * kHeadDim + d4) = f32x4{0.f, 0.f, 0.f, 0.f};
        if ((tid & 31) == 0) a.part_lse[(size_t)slot * kGroup + hh] = len_ok ? kNegInf : __builtin_nanf("");
        return;
    }
    OneDesc src;
    src.d.h = h;
    src.d.b = b;
    src.d.t0 = t0;
    src.d.t1 = t1;
    src.d.L = L;
    src.d.slot = slot;
    run_stream<FP8>(a, src, t1 - t0, sm);
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
