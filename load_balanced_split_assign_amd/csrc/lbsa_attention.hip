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
//     descriptors.  Each wave keeps a private ring of LDS stages and fills it
//     with asynchronous global->LDS loads (global_load_lds): while tile k is
//     computed, the next stages' tiles are in flight, also across descriptor
//     boundaries, so the memory pipe never drains inside a bin.  The kernel
//     waits for each stage itself with s_waitcnt vmcnt(N), N = loads issued
//     after that stage (vector memory operations complete in order).
//   * Loads are coalesced: each 64-lane load moves whole K/V rows (4 rows of
//     256 B for bf16, 8 rows of 128 B for fp8) from a uniform page base plus a
//     per-lane offset fixed for the whole stream.  Inside a row the 16-byte
//     chunks are XOR-swizzled by the row index, so the MFMA operand reads (16
//     rows, same column) hit 16 different LDS bank groups.
//   * Rows past the live length are fetched from the page's first row (always
//     live) instead, so no tail garbage or NaN ever reaches LDS; their scores
//     are masked to -inf, so they contribute nothing.
//   * S^T = K Q^T with MFMA 16x16x32 (rows = 16 tokens, columns = 16 query
//     rows: the 8 heads of the group for one query token per request, of
//     which 8 columns are real, or 8 heads x 2 query tokens for multi-token
//     decode, all 16 real), fp32 accumulation in two independent chains:
//     bf16 operands for bf16 KV, the fp8 MFMA on the raw e4m3 codes of K and
//     Q for fp8 KV (the per-token K scale and per-head Q scale multiply the
//     score).  With 2 query tokens the later one sees one token more (causal
//     among the new tokens): a per-column length limit in the score mask.
//   * Online softmax in the exp2 domain with a lazy running max: a tile whose
//     scores stay within kSlack of the running max is exponentiated against
//     it directly; only when a wave-wide ballot finds a larger score does the
//     wave reduce the max across lanes and rescale its accumulators.
//   * O^T += V^T P^T with MFMA 16x16x16 bf16: V^T comes from LDS through
//     transposed reads, P straight from the S^T accumulator registers (its
//     layout is already the B operand).  bf16 V: ds_read_b64_tr_b16.  fp8 V:
//     ds_read_b64_tr_b8 straight from the ring stage, each read giving a lane
//     the 4 tokens of two d blocks, widened exactly to bf16 in registers; the
//     per-token V scale is folded into p.
//   * At the end of a descriptor the 4 waves merge (max, sum, O) through LDS
//     and one partial (fp32 O normalised, natural-log LSE) is written.
#include "lbsa_device.h"

namespace lbsa {
namespace {

using namespace dev;

constexpr float kSlack = 8.0f;   // log2 headroom of the lazy running max (p <= 256)

// ---------------------------------------------------------------------------
// Per-wave LDS ring stage.  bf16: K 16 x 256 B, V 16 x 256 B.  fp8: K 16 x 128
// B, V 16 x 128 B, k scales (256 B: rows 0-15, then copies), v scales (256 B),
// the q scales of the tile's descriptor (256 B: heads 0-7, then copies) and,
// on a descriptor's first tile, its Q codes (8 heads x 128 B).  Q and its
// scales travel through the ring so that reading them needs no wait on a
// register load (which the compiler turns into a wait for the whole ring).
// ---------------------------------------------------------------------------
// QL = query tokens per request (1, or 2 for multi-token decode): the Q codes
// of a descriptor are QL x 8 heads x 128 B.  fp8 runs a 2-stage ring, so a
// workgroup needs under 80 KiB of LDS and two share a CU: an fp8 tile carries
// half the bytes of a bf16 one for the same work, and the second workgroup
// computes while the first waits on its LDS round trips and loads (16% faster
// than one workgroup per CU with a 5-stage ring).  With QL = 2 its merge slot
// holds half of O at a time (two passes of 64 dims) to fit.  bf16 keeps one
// workgroup per CU and 3 stages (two per CU, with half-size bins and twice
// the descriptors, was slower on the small batches and no faster on the
// large ones).
template <bool FP8, int QL = 1> struct Stage {
    static constexpr int kRow = FP8 ? 128 : 256;        // bytes of one K/V row
    static constexpr int K = 0;
    static constexpr int V = 16 * kRow;
    static constexpr int KS = 32 * kRow;                // fp8 only: k scales
    static constexpr int VS = KS + 256;                 // fp8 only: v scales
    static constexpr int QS = VS + 256;                 // fp8 only: the 8 QL q scales of the descriptor
    static constexpr int QD = QS + 256;                 // fp8 only: Q codes, QL x 8 heads x 128 B (first tiles)
    static constexpr int BYTES = FP8 ? QD + 1024 * QL : 32 * kRow;   // 5888 / 6912 (fp8), 8192 (bf16)
    static constexpr int KV_LOADS = 16 * kRow / 1024;   // loads per K (or V) slice: 4 (bf16) / 2 (fp8)
    // ring loads issued for every tile (fp8 adds one more, the Q codes, on a
    // descriptor's first tile; the waits count only the fixed ones, which can
    // only make them wait for a little more than the stage)
    static constexpr int LOADS = 2 * KV_LOADS + (FP8 ? 3 : 0);
    // ring depth: STAGES - 1 tiles in flight per wave (a 3-stage fp8 ring, which
    // fits once the merge slot lives in the ring, measured 3% slower)
    static constexpr int STAGES = FP8 ? 2 : 3;
};
static_assert((Stage<false>::STAGES - 1) * Stage<false>::LOADS < 64, "vmcnt range");
static_assert((Stage<true>::STAGES - 1) * Stage<true>::LOADS < 64, "vmcnt range");

// 16-byte chunk swizzle inside a row: LDS chunk c' holds row chunk c' ^ f(row).
// K rows use swz; V rows, which are read transposed, use swz_v (bf16) or
// swz_v8 (fp8), chosen so that a transposed pass has no bank conflict.
template <bool FP8> __device__ inline int swz(int row) { return FP8 ? ((row >> 1) & 7) : (row & 15); }
// fp8 V: one 16-lane pass of ds_read_b64_tr_b8 reads chunks 2c and 2c + 1 of the
// 4 rows 4g .. 4g + 3 (8 B per lane, 128 B).  A 128-byte row spans half of the
// 32 four-byte banks, so the bank group of a chunk is its swizzled index alone;
// 2 (row & 3) sends the four rows' chunk pairs to four different pairs of bank
// groups.
__device__ inline int swz_v8(int row) { return 2 * (row & 3); }
template <bool FP8> __device__ inline int swz_vrow(int row) { return FP8 ? swz_v8(row) : swz_v(row); }

// LDS of one split / static workgroup.  Every ring stage is its own
// __shared__ object: the compiler's wait-count insertion can then tell which
// asynchronous load an LDS read depends on (distinct underlying objects) and
// does not fall back to waiting for all of them.
//
// At the end of a descriptor each wave puts its (O, m, l, flag) in a merge slot.
// bf16: one slot per wave (Slot::kWave bytes) of its own.  fp8: the wave's slice
// of the ring stage it has just computed -- that stage is consumed, and no
// load targets it again before the merge's closing barrier (the next load into
// it is issued in the following step) -- so the fp8 ring gets one more stage
// in the same LDS (two workgroups per CU).  fp8 with QL = 2 merges O in two
// passes of 64 dims (a slot holds half of O).
template <bool FP8, int QL> struct Slot {
    static constexpr int kRows = kGroup * QL;                          // query rows of a descriptor
    static constexpr int kPasses = (FP8 && QL == 2) ? 2 : 1;           // passes over the 128 dims
    static constexpr int kDims = kHeadDim / kPasses;                   // dims of O per pass
    static constexpr int kMerge = (kRows * kDims + 2 * kRows + 4) * 4;   // O (one pass), m, l, flag per wave
    static constexpr bool kInStage = FP8;                              // merge in the consumed ring stage
    static constexpr int kWave = kInStage ? Stage<FP8, QL>::BYTES : (kMerge + 255) / 256 * 256;   // slot stride
    static constexpr int kBytes = kInStage ? 16 : kWaves * kWave;      // the separate slot array
};
static_assert(Slot<true, 1>::kMerge <= Stage<true, 1>::BYTES && Slot<true, 2>::kMerge <= Stage<true, 2>::BYTES,
              "an fp8 merge slot fits the wave's stage slice");
constexpr int kMaxStages = 6;
template <bool FP8> struct Smem {
    lds_char* stage[kMaxStages];   // [kWaves][Stage::BYTES] each; the first STAGES are used
    lds_char* merge;               // [kWaves][Slot::kWave]
};
template <bool FP8, int QL> constexpr int stage_array_bytes(int u) {
    return u < Stage<FP8, QL>::STAGES ? kWaves * Stage<FP8, QL>::BYTES : 16;
}
template <bool FP8, int QL> constexpr int smem_bytes() {
    return kWaves * Stage<FP8, QL>::BYTES * Stage<FP8, QL>::STAGES + Slot<FP8, QL>::kBytes;
}
static_assert(smem_bytes<false, 1>() <= 160 * 1024 && smem_bytes<true, 1>() <= 80 * 1024, "LDS (fp8: 2 per CU)");
static_assert(smem_bytes<false, 2>() <= 160 * 1024 && smem_bytes<true, 2>() <= 80 * 1024, "LDS (fp8: 2 per CU)");

// One descriptor of the tile stream (all fields wave-uniform).
struct Desc {
    int h, b, t0, t1, L;
    int slot;        // partial slot (< Hkv * B + P, or the static grid size: both below 2^31)
};

// Per-lane constants of the asynchronous loads (fixed for a wave's stream).
template <bool FP8> struct LaneLoads {
    uint32_t kv_live[Stage<FP8>::KV_LOADS];   // byte offset in a page of this lane's 16 B of K (h = 0)
    uint32_t v_live[Stage<FP8>::KV_LOADS];    // the same for V (its own swizzle)
    uint32_t kv_dead[Stage<FP8>::KV_LOADS];   // a chunk of the page's row 0
    int row[Stage<FP8>::KV_LOADS];            // slice row loaded by this lane
    int scale_row;                            // fp8: slice row of this lane's scale (lane % 16)
    __device__ void init(int Hkv, int w, int lane) {
        using SL = Stage<FP8>;
        constexpr int kRowsPerLoad = 1024 / SL::kRow;
        constexpr int kChunks = SL::kRow / 16;
#pragma unroll
        for (int s = 0; s < SL::KV_LOADS; ++s) {
            row[s] = kRowsPerLoad * s + lane / kChunks;
            const uint32_t chunk = 16u * (uint32_t)((lane % kChunks) ^ swz<FP8>(row[s]));
            const uint32_t chunk_v = 16u * (uint32_t)((lane % kChunks) ^ swz_vrow<FP8>(row[s]));
            const uint32_t row_off = (uint32_t)(16 * w + row[s]) * (uint32_t)Hkv * SL::kRow;
            kv_live[s] = row_off + chunk;
            v_live[s] = row_off + chunk_v;
            kv_dead[s] = chunk;
        }
        scale_row = lane & 15;
    }
};

// Issue the asynchronous loads of one tile into stage `st`: this wave's 16 K
// and V rows of page `page` and, for fp8, their k/v scales, all non-temporal
// (a step reads each page once).
template <bool FP8, int QL>
__device__ inline void issue_tile(const AttnArgs& a, const LaneLoads<FP8>& ll, lds_char* __restrict__ st,
                                  int64_t page, const Desc& d, int tile, int w) {
    using SL = Stage<FP8, QL>;
    const size_t pbase = ((size_t)page * kTile * a.Hkv + d.h) * SL::kRow;
    const char* kb = static_cast<const char*>(a.k_cache) + pbase;
    const char* vb = static_cast<const char*>(a.v_cache) + pbase;
    const int tok0 = 64 * tile + 16 * w;
    const bool full = tok0 + 16 <= d.L;                 // every row of this slice is live
#pragma unroll
    for (int s = 0; s < SL::KV_LOADS; ++s) {
        const bool live = full || tok0 + ll.row[s] < d.L;
        dma16_nt(kb + (live ? ll.kv_live[s] : ll.kv_dead[s]), st + SL::K + 1024 * s);
        dma16_nt(vb + (live ? ll.v_live[s] : ll.kv_dead[s]), st + SL::V + 1024 * s);
    }
    if constexpr (FP8) {
        const size_t sbase = ((size_t)page * a.Hkv + d.h) * kTile;
        const int srow = (full || tok0 + ll.scale_row < d.L) ? 16 * w + ll.scale_row : 0;
        dma4_nt(a.k_scale + sbase + srow, st + SL::KS);
        dma4_nt(a.v_scale + sbase + srow, st + SL::VS);
        // lane i brings the scale of query (i / 8) % QL, head i % 8 (q_scale [B][QL][Hq])
        const int qi = QL == 1 ? 0 : (threadIdx.x >> 3) & (QL - 1);
        dma4(a.q_scale + ((size_t)(d.b * QL + qi) * a.Hq + (size_t)d.h * kGroup) + (threadIdx.x & 7), st + SL::QS);
    }
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Four fp32 -> four bf16 in one 8-byte store.
__device__ inline void store_bf16x4(uint16_t* p, f32x4 v) {
    uint2 packed;
    packed.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
    packed.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = packed;
}

// Running state of one wave over one descriptor.
struct WaveState {
    f32x4 acc[8];     // O^T[d = 16 db + 4 g + i][head r]
    float m;          // running reference max (log2 domain) of head r, uniform over g
    float l;          // this lane's share of the running sum of head r
};

// Q operand of a descriptor (B of S^T = K Q^T): head r of the group (zero for
// r >= 8), as bf16 (bf16 KV: register loads) or raw e4m3 codes (fp8 KV: read
// from the ring stage of the descriptor's first tile).
template <bool FP8> struct QOp;
template <> struct QOp<false> { uint4 v[4]; };
template <> struct QOp<true> { uint4 v[2]; };

// bf16: plain loads into registers, issued when the load cursor enters a
// descriptor (its first tile), several tiles before the compute cursor needs
// them; column r holds query r / 8, head r % 8 (q [B][QL][Hq][128]).  fp8:
// the QL x 8 x 128 B of Q codes go into the stage with that first tile (lane
// i moves bytes [16 i, 16 i + 16) of each query's row-major block).
template <bool FP8, int QL>
__device__ inline void load_q(const AttnArgs& a, const Desc& d, int r, int g, QOp<FP8>& q, lds_char* st) {
    if constexpr (!FP8) {
        const int qi = QL == 1 ? 0 : (r >> 3) & (QL - 1);
        const size_t row = (size_t)(d.b * QL + qi) * a.Hq + (size_t)d.h * kGroup + (r & 7);
        const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + row * 256);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) q.v[ks] = qp[g + 4 * ks];
    } else {
#pragma unroll
        for (int qi = 0; qi < QL; ++qi) {
            const size_t row0 = (size_t)(d.b * QL + qi) * a.Hq + (size_t)d.h * kGroup;
            dma16(static_cast<const char*>(a.q) + row0 * 128 + 16 * (threadIdx.x & 63),
                  st + Stage<true, QL>::QD + 1024 * qi);
        }
    }
}

// QK^T, online softmax and PV of one tile held in stage `st`.  `lim` is the
// token limit of this lane's column (its query sees tokens < lim).
template <bool FP8, int QL>
__device__ inline void tile_compute(const lds_char* __restrict__ st, const QOp<FP8>& q, float sl2, int tok0,
                                    int lim, int w, int r, int g, WaveState& ws) {
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    const bool qlive = r < kGroup * QL;
    using SL = Stage<FP8, QL>;
    // ---- operands from LDS, then S^T = K Q^T (rows = 16 tokens, cols = 16 heads)
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    const int vrow = 4 * g + (r >> 2);            // transposed-read row of this lane
    s16x4 va[8];
    f32x4 ks4, vs4;
    if constexpr (!FP8) {
        uint32_t ka[4], vaddr[8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[ks] = lds_addr(st + SL::K + r * 256 + 16 * ((g + 4 * ks) ^ swz<false>(r)));
        const uint32_t vr = lds_addr(st + SL::V + vrow * 256 + 8 * (r & 1));
#pragma unroll
        for (int db = 0; db < 8; ++db) vaddr[db] = vr + 16u * (uint32_t)((2 * db + ((r >> 1) & 1)) ^ swz_v(vrow));
        uint4 k[4];
        lds_read_tile_bf16(k, va, ka, vaddr);
        bf16x8 qv[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qv[ks] = as_bf16x8(qlive ? q.v[ks] : z4);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[0]), qv[0], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[1]), qv[1], sb, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[2]), qv[2], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[3]), qv[3], sb, 0, 0, 0);
    } else {
        uint32_t addr[4], vaddr[4];
        addr[0] = lds_addr(st + SL::K + r * 128 + 16 * (g ^ swz<true>(r)));         // K k-steps 0, 1
        addr[1] = lds_addr(st + SL::K + r * 128 + 16 * ((g + 4) ^ swz<true>(r)));   // K k-steps 2, 3
        addr[2] = lds_addr(st + SL::KS + 16 * g);                                   // k scales, rows 4g..
        addr[3] = lds_addr(st + SL::VS + 16 * g);                                   // v scales, rows 4g..
        // V^T by transposed byte reads: in the 16-lane group g, lanes 2j and 2j + 1
        // name the two halves of "row" j = (token 4g + j % 4, chunk 2 db + j / 4);
        // lane i then receives byte i of each of the 8 rows: the 4 tokens of dim
        // 32 db + i (bytes 0-3) and of dim 32 db + 16 + i (bytes 4-7).
        const int vt = 4 * g + ((r >> 1) & 3);
        const uint32_t vrow = lds_addr(st + SL::V + vt * 128 + 8 * (r & 1));
#pragma unroll
        for (int db = 0; db < 4; ++db) vaddr[db] = vrow + 16u * (uint32_t)((2 * db + (r >> 3)) ^ swz_v8(vt));
        uint4 o[4];
        uint2 vv[4];
        lds_read_tile_fp8_tr(o, vv, addr, vaddr);
        const uint4 c0 = o[0], c1 = o[1];
        ks4 = __builtin_bit_cast(f32x4, o[2]);
        vs4 = __builtin_bit_cast(f32x4, o[3]);
        const uint4 q0 = qlive ? q.v[0] : z4, q1 = qlive ? q.v[1] : z4;
        auto lo = [](uint4 x) { return (long)(((uint64_t)x.y << 32) | x.x); };
        auto hi = [](uint4 x) { return (long)(((uint64_t)x.w << 32) | x.z); };
        sa = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(lo(c0), lo(q0), sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(hi(c0), hi(q0), sb, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(lo(c1), lo(q1), sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(hi(c1), hi(q1), sb, 0, 0, 0);
        // the 4 tokens of each d block as bf16, in token order (exact widening)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            va[2 * db] = __builtin_bit_cast(s16x4, fp8x4_to_bf16x4(vv[db].x));
            va[2 * db + 1] = __builtin_bit_cast(s16x4, fp8x4_to_bf16x4(vv[db].y));
        }
    }
    const f32x4 s = sa + sb;

    // ---- online softmax over the 4 score rows of this lane ------------------
    const int pos0 = tok0 + 16 * w + 4 * g;       // token of score row i is pos0 + i
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = s[i] * sl2;
        if constexpr (FP8) x *= ks4[i];
        sc[i] = (pos0 + i < lim) ? x : kNegInf;
    }
    const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__builtin_amdgcn_ballot_w64(lmax > ws.m + kSlack) != 0) {
        // a score above the reference: new reference = max over the 16 tokens
        float mt = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(ws.m, mt);
        // 0 when nothing was accumulated yet (also when this column is still
        // fully masked, m_new = -inf: a wave-wide rescale may come from another
        // column, and -inf - -inf would give NaN)
        const float alpha = ws.m == kNegInf ? 0.f : exp2_fast(ws.m - m_new);
        ws.l *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) ws.acc[db] *= alpha;
        ws.m = m_new;
    }
    const float mref = (ws.m == kNegInf) ? 0.f : ws.m;   // all scores -inf so far: p = 0
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = exp2_fast(sc[i] - mref);
        ws.l += p[i];
    }
    if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] *= vs4[i];
    }
    const s16x4 pb = __builtin_bit_cast(s16x4, make_uint2(bf16x2_bits(p[0], p[1]), bf16x2_bits(p[2], p[3])));

    // ---- O^T += V^T P^T ------------------------------------------------------
    // ds_read_b64_tr_b16: in each 16-lane group, lane k supplies the address of
    // 4 consecutive d of token row 4g + k/4; lane i = 4a + c then receives
    // V[4g + j][16 db + i] for j = 0..3 -- the A operand (d x tokens).
#pragma unroll
    for (int db = 0; db < 8; ++db)
        ws.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[db], pb, ws.acc[db], 0, 0, 0);
}

// End of a descriptor: merge the 4 waves' (max, sum, O) through LDS and write
// the partial (normalised O, natural-log LSE) of its slot: QL x 8 rows, row
// r = 8 query + head.  Every descriptor holds a token the last query sees, so
// a row of that query with nothing accumulated means bad data (NaN); an
// earlier query may legitimately see none of the descriptor's tokens, which
// gives an empty partial (O = 0, LSE = -inf) that the combine skips.
// With a.direct_out set, a descriptor that covers its whole (kv_head, request)
// segment -- the segment's only chunk -- is already the final result: its
// normalised O goes straight to the bf16 output rows (the merge of a single
// chunk is the identity) and the combine leaves those rows alone.
template <bool FP8, int QL>
__device__ inline void finish_desc(const AttnArgs& a, lds_char* merge, const WaveState& ws, bool bad,
                                   const Desc& dd, int w, int lane, int r, int g) {
    const size_t slot = (size_t)dd.slot;
    const bool whole = a.direct_out != 0 && dd.t0 == 0 && dd.t1 == (dd.L + kTile - 1) / kTile;
    using SM = Slot<FP8, QL>;
    constexpr int R = SM::kRows, DW = SM::kDims, DBP = DW / 16;   // rows, dims and d blocks per pass
    float lsum = ws.l;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    lds_float* o_w = reinterpret_cast<lds_float*>(merge + w * SM::kWave);
#pragma unroll
    for (int dp = 0; dp < SM::kPasses; ++dp) {
        if (r < R) {
#pragma unroll
            for (int e = 0; e < DBP; ++e)
                *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(o_w + r * DW + 16 * e + 4 * g) =
                    ws.acc[DBP * dp + e];
            if (dp == 0 && g == 0) {
                o_w[R * DW + r] = ws.m;
                o_w[R * DW + R + r] = lsum;
            }
        }
        if (dp == 0 && lane == 0) o_w[R * DW + 2 * R] = bad ? 1.f : 0.f;
        lds_barrier();
#pragma unroll
        for (int pass = 0; pass < QL; ++pass) {
            const int tid = threadIdx.x;
            const int hh = kGroup * pass + (tid >> 5), d4 = (tid & 31) * 4;
            if (d4 < DW) {
                float M = kNegInf;
                bool any_bad = false;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    const lds_float* ow = reinterpret_cast<const lds_float*>(merge + ww * SM::kWave);
                    M = fmaxf(M, ow[R * DW + hh]);
                    any_bad |= ow[R * DW + 2 * R] != 0.f;
                }
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
                float lt = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    const lds_float* ow = reinterpret_cast<const lds_float*>(merge + ww * SM::kWave);
                    const float mw = ow[R * DW + hh];
                    const float sw = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
                    lt += sw * ow[R * DW + R + hh];
                    o += sw * *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(ow + hh * DW + d4);
                }
                float lse;
                if (!any_bad && M == kNegInf && pass < QL - 1) {
                    o = f32x4{0.f, 0.f, 0.f, 0.f};                 // an earlier query that sees none of it
                    lse = kNegInf;
                } else if (any_bad || M == kNegInf || !(lt > 0.f)) {
                    const float nan = __builtin_nanf("");
                    o = f32x4{nan, nan, nan, nan};
                    lse = nan;
                } else {
                    o *= 1.f / lt;
                    lse = (M + __builtin_log2f(lt)) * kLn2;
                }
                if (whole) {
                    // row (request, query pass, head h * 8 + tid / 32) of out [B][QL][Hq][128]
                    const size_t orow = ((size_t)dd.b * QL + pass) * a.Hq + (size_t)dd.h * kGroup + (tid >> 5);
                    store_bf16x4(static_cast<uint16_t*>(a.out) + orow * kHeadDim + DW * dp + d4, o);
                } else {
                    *reinterpret_cast<f32x4*>(a.part_o + ((size_t)slot * R + hh) * kHeadDim + DW * dp + d4) = o;
                    if (dp == 0 && (tid & 31) == 0) a.part_lse[(size_t)slot * R + hh] = lse;
                }
            }
        }
        lds_barrier();   // the merge area is reused by the next pass / descriptor
    }
}

// Descriptor sources of the tile stream.
// A descriptor as loaded from the map, before validation.
struct RawDesc {
    int h, b, t0, t1, L;
};

struct MapDescs {           // descriptors [d0, d0 + n) of a task-map bin
    const __attribute__((address_space(4))) int32_t* desc;
    const __attribute__((address_space(4))) int32_t* dlen;
    RawDesc head;           // descriptor d0, from the bin's head record
    int d0, n, Hkv, B, max_pages;
    __device__ int count() const { return n; }
    // the bin's first descriptor (from the head record; no load)
    __device__ Desc first() const { return check(0, head); }
    // descriptor i >= 1 of the bin (loaded from the map).  The cursors read the
    // head record only in first(), so it is dead inside the stream loop.
    __device__ Desc get(int i) const { return check(i, raw(i)); }
    // the raw record of descriptor i >= 1 (loads; validated by check)
    __device__ RawDesc raw(int i) const {
        const int d = d0 + i;
        return RawDesc{desc[4 * d], desc[4 * d + 1], desc[4 * d + 2], desc[4 * d + 3], dlen[d]};
    }
    // an invalid descriptor (corrupt map) has no tiles
    __device__ Desc check(int i, RawDesc x) const {
        const int d = d0 + i;
        Desc y;
        y.slot = d;
        if (x.h < 0 || x.h >= Hkv || x.b < 0 || x.b >= B || x.t0 < 0 || x.t1 <= x.t0 || x.t1 > max_pages ||
            x.L < 0) {
            y.h = 0; y.b = 0; y.t0 = 0; y.t1 = 0; y.L = 0;
        } else {
            y.h = x.h; y.b = x.b; y.t0 = x.t0; y.t1 = x.t1;
            y.L = min(x.L, max_pages * kTile);
        }
        return y;
    }
};

struct OneDesc {            // the static kernel's single chunk
    Desc d;
    __device__ int count() const { return 1; }
    __device__ Desc first() const { return d; }
    __device__ Desc get(int) const { return d; }
    __device__ RawDesc raw(int) const { return RawDesc{d.h, d.b, d.t0, d.t1, d.L}; }
    __device__ Desc check(int, RawDesc) const { return d; }
};

// Cursor over the tiles of a descriptor source (wave-uniform).  Past the last
// tile it parks on that tile (or on tile 0 of an empty descriptor), so every
// page-table index it yields stays in bounds whatever the map holds.
template <class Src>
struct Cursor {
    const Src* src;
    int i;          // descriptor ordinal
    int t;          // tile of that descriptor
    Desc d;
    __device__ void seek_valid() {      // skip descriptors without tiles, from descriptor i >= 1
        while (i < src->count()) {
            const Desc x = src->get(i);
            if (x.t1 > x.t0) { d = x; t = x.t0; return; }
            ++i;
        }
        t = max(d.t0, d.t1 - 1);
    }
    __device__ void begin(const Src* s) {
        src = s;
        i = 0;
        d = s->first();
        t = d.t0;
        if (d.t1 <= d.t0) {
            ++i;
            seek_valid();
        }
    }
    __device__ void next() {
        if (++t >= d.t1) { ++i; seek_valid(); }
    }
    // The load cursor: the record of descriptor i + 1 is loaded when descriptor
    // i is entered, so it has arrived -- behind the ring wait of the steps in
    // between -- by the time the cursor switches to it, and a switch waits for
    // no map load.
    RawDesc nx;
    __device__ void begin_prefetching(const Src* s) {
        begin(s);
        if (i + 1 < src->count()) nx = src->raw(i + 1);
    }
    __device__ void next_prefetched() {
        if (++t < d.t1) return;
        ++i;
        while (i < src->count()) {
            const Desc x = src->check(i, nx);
            if (i + 1 < src->count()) nx = src->raw(i + 1);
            if (x.t1 > x.t0) { d = x; t = x.t0; return; }
            ++i;
        }
        t = max(d.t0, d.t1 - 1);
    }
};

// Issue the next tile of the load cursor into ring stage `slot` (and, when it
// is the first tile of a descriptor, that descriptor's Q into qslot).  Past
// the last tile it issues the same number of loads, of row 0 of the last page
// only (one cache line per row chunk), into a stage that is never read, so
// every step issues the same number of ring loads.  `page` is the page id of
// the cursor's tile, loaded one step ahead; the next one is fetched here.
template <bool FP8, int QL, class Src>
__device__ inline void issue_step(const AttnArgs& a, const LaneLoads<FP8>& ll, Cursor<Src>& lc, int& issued,
                                  int ntiles, int& page, uint32_t& bad_bits, lds_char* st, QOp<FP8>& qslot,
                                  int slot, int w, int r, int g) {
    const bool ok = page >= 0 && page < a.num_pages;
    bad_bits = (bad_bits & ~(1u << slot)) | ((uint32_t)(!ok) << slot);
    const bool real = issued < ntiles;
    if (real && lc.t == lc.d.t0) load_q<FP8, QL>(a, lc.d, r, g, qslot, st);
    Desc d = lc.d;
    if (!real) d.L = 0;     // past the end: every row counts as dead, so only row 0 of the page is read
    issue_tile<FP8, QL>(a, ll, st, ok ? page : 0, d, lc.t, w);
    if (++issued < ntiles) {
        lc.next_prefetched();
        page = uniform_ptr<int32_t>(a.page_table)[(size_t)lc.d.b * a.max_pages + lc.t];
    }
}

// Stream the tiles of `src` through this workgroup (see the header comment).
// `ntiles` is the number of tiles the source holds (at least 1); with a
// corrupt map that holds fewer, the cursors repeat their last tile.
template <bool FP8, int QL, class Src>
__device__ void run_stream(const AttnArgs& a, const Src& src, int ntiles, const Smem<FP8>& sm) {
    using SL = Stage<FP8, QL>;
    constexpr int S = SL::STAGES;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    // column r's query sees the request's tokens below L - (QL - 1 - query)
    const int lim_off = (QL == 1 ? 0 : min(r >> 3, QL - 1)) - (QL - 1);
    auto stage = [&](int u) -> lds_char* { return sm.stage[u] + w * SL::BYTES; };
    LaneLoads<FP8> ll;
    ll.init(a.Hkv, w, lane);

    // load cursor: runs S-1 tiles ahead of the compute cursor
    Cursor<Src> lc;
    lc.begin_prefetching(&src);
    int issued = 0;
    int page = uniform_ptr<int32_t>(a.page_table)[(size_t)lc.d.b * a.max_pages + lc.t];
    uint32_t bad_bits = 0;          // bit u: the tile in stage u has an out-of-range page id
    QOp<FP8> qring[S];              // Q of the descriptor whose first tile sits in stage u
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
        issue_step<FP8, QL>(a, ll, lc, issued, ntiles, page, bad_bits, stage(u), qring[u], u, w, r, g);

    Cursor<Src> cc;
    cc.begin(&src);
    WaveState ws;
    QOp<FP8> q;
    float sl2 = 0.f;
    bool bad = false;
    for (int k = 0; k < ntiles; k += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int kk = k + u;
            issue_step<FP8, QL>(a, ll, lc, issued, ntiles, page, bad_bits, stage((u + S - 1) % S),
                                qring[(u + S - 1) % S], (u + S - 1) % S, w, r, g);   // tile kk + S - 1
            wait_vmcnt<(S - 1) * SL::LOADS>();                             // tile kk has landed
            if (kk < ntiles) {
                if (cc.t == cc.d.t0) {                                     // first tile of a descriptor
                    // column r: row r of the QL x 8 Q block, scale r of the 8 QL scales
                    constexpr int kColMask = kGroup * QL - 1;
                    if constexpr (FP8)
                        lds_read2x16(q.v[0], q.v[1], lds_addr(stage(u) + SL::QD) + 128 * (r & kColMask) + 16 * g,
                                     lds_addr(stage(u) + SL::QD) + 128 * (r & kColMask) + 16 * g + 64);
                    else
                        q = qring[u];
                    sl2 = a.scale_log2;
                    if constexpr (FP8) sl2 *= lds_read_f32(lds_addr(stage(u) + SL::QS) + 4 * (r & kColMask));
#pragma unroll
                    for (int db = 0; db < 8; ++db) ws.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
                    ws.m = kNegInf;
                    ws.l = 0.f;
                    bad = false;
                }
                bad |= (bad_bits >> u) & 1u;
                tile_compute<FP8, QL>(stage(u), q, sl2, 64 * cc.t, cc.d.L + lim_off, w, r, g, ws);
                if (cc.t + 1 == cc.d.t1)
                    finish_desc<FP8, QL>(a, Slot<FP8, QL>::kInStage ? sm.stage[u] : sm.merge, ws, bad, cc.d, w, lane,
                                         r, g);
                cc.next();
            }
        }
    }
    wait_vmcnt<0>();   // no load may still target LDS when the workgroup moves on
}

#define LBSA_DECLARE_SMEM(FP8, QL)                                                  \
    __shared__ __attribute__((aligned(16))) char s0[stage_array_bytes<FP8, QL>(0)]; \
    __shared__ __attribute__((aligned(16))) char s1[stage_array_bytes<FP8, QL>(1)]; \
    __shared__ __attribute__((aligned(16))) char s2[stage_array_bytes<FP8, QL>(2)]; \
    __shared__ __attribute__((aligned(16))) char s3[stage_array_bytes<FP8, QL>(3)]; \
    __shared__ __attribute__((aligned(16))) char s4[stage_array_bytes<FP8, QL>(4)]; \
    __shared__ __attribute__((aligned(16))) char s5[stage_array_bytes<FP8, QL>(5)]; \
    __shared__ __attribute__((aligned(16))) char sslot[Slot<FP8, QL>::kBytes];      \
    Smem<FP8> sm; /* address-space casts to LDS */                             \
    sm.stage[0] = (lds_char*)s0;                                               \
    sm.stage[1] = (lds_char*)s1;                                               \
    sm.stage[2] = (lds_char*)s2;                                               \
    sm.stage[3] = (lds_char*)s3;                                               \
    sm.stage[4] = (lds_char*)s4;                                               \
    sm.stage[5] = (lds_char*)s5;                                               \
    sm.merge = (lds_char*)sslot

// One workgroup per bin (grid = P).  The header words and the bin's head
// record are independent loads, so the first page-table and K/V loads follow
// after a single round trip to the map.
// Keeps a loaded value (and so its load) alive up to this point without using
// it: a compiler-only barrier, no instruction.  Used to make loads that the
// compiler would otherwise sink into later branches go out together.
__device__ inline void keep(int x) { __asm__ volatile("" ::"s"(x)); }
__device__ inline void keep(const void* p) { __asm__ volatile("" ::"s"(p)); }
__device__ inline void keep(float x) { __asm__ volatile("" ::"s"(x)); }

// The kernel arguments the tile stream reads, fetched in the kernel's first
// round trip rather than after the map checks.
template <bool FP8>
__device__ inline void keep_stream_args(const AttnArgs& a) {
    keep(a.q);
    keep(a.k_cache);
    keep(a.v_cache);
    keep(a.page_table);
    keep(a.scale_log2);
    if constexpr (FP8) {
        keep(a.q_scale);
        keep(a.k_scale);
        keep(a.v_scale);
    }
}

// One workgroup per bin (grid = P).  Every map word the start needs -- the
// header words and the bin's head record -- is loaded up front and checked in a
// single branch, so the loads go out together and the first page-table and
// K/V loads follow after one round trip to the map (checked one by one, the
// compiler sinks each load into the branch that tests it, and the start takes
// a round trip per check).
template <bool FP8, int QL>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(const uint8_t* map, int B, int Hkv, int P, int max_pages, AttnArgs a) {
    LBSA_DECLARE_SMEM(FP8, QL);
    const MapLayout ML = map_layout(B, Hkv, P);
    const int j = blockIdx.x;
    const auto* hdr = uniform_ptr<int32_t>(map + ML.header);
    const auto* rec = uniform_ptr<int32_t>(map + ML.bin_head) + (size_t)kBinHeadWords * j;
    // The combine kernel starts by reading each segment's chunk range: the
    // workgroups load one word of each 64-byte line of those two arrays (8 bytes
    // per segment, contiguous; the index is clamped into them) in the same round
    // trip as their own map words, so that the combine finds them in the
    // caches.  The load is asm, issued before the map loads (its memory clobber
    // keeps them after it), so the wait for the map words covers it too; its
    // register stays live (keep, below) until after that wait, since the load
    // writes it whenever it returns.
    const int seg_words = 2 * Hkv * B;
    const int32_t* seg_line = reinterpret_cast<const int32_t*>(map + ML.seg_first_desc) + min(16 * j, seg_words - 1);
    int touched;
    __asm__ volatile("s_load_dword %0, %1, 0x0" : "=s"(touched) : "s"(seg_line) : "memory");
    const int h_err = hdr[LBSA_HDR_ERROR], h_p = hdr[LBSA_HDR_P], h_b = hdr[LBSA_HDR_B], h_hkv = hdr[LBSA_HDR_HKV];
    const int h_k = hdr[LBSA_HDR_K], h_q = hdr[LBSA_HDR_Q], h_r = hdr[LBSA_HDR_R];
    const int r_h = rec[BH_H], r_b = rec[BH_B], r_t0 = rec[BH_T0], r_t1 = rec[BH_T1];
    const int r_first = rec[BH_FIRST], r_count = rec[BH_COUNT], r_len = rec[BH_L];
    const int cap = Hkv * B + P;
    // tiles of bin j from the header's bin sizes (the descriptors' tiles sum to it)
    const int ntiles = min(h_q + (j < h_r ? 1 : 0), B * max_pages) * (j < h_k ? 1 : 0);
    const bool run = (h_err == 0) & (h_p == P) & (h_b == B) & (h_hkv == Hkv) & (r_count > 0) &
                     (r_first >= 0) & (r_count <= cap - r_first) & (ntiles > 0);
    keep(h_q);
    keep(h_r);
    keep(r_h);
    keep(r_b);
    keep(r_t0);
    keep(r_t1);
    keep(r_len);
    keep_stream_args<FP8>(a);
    keep(touched);   // waited for with the map words: from here its register is the compiler's again
    if (!run) return;
    MapDescs src;
    src.desc = uniform_ptr<int32_t>(map + ML.desc);
    src.dlen = uniform_ptr<int32_t>(map + ML.desc_len);
    src.d0 = r_first;
    src.n = r_count;
    src.Hkv = Hkv;
    src.B = B;
    src.max_pages = a.max_pages;
    src.head = RawDesc{r_h, r_b, r_t0, r_t1, r_len};
    run_stream<FP8, QL>(a, src, ntiles, sm);
}

template <bool FP8, int QL>
__global__ __launch_bounds__(kSplitThreads) void static_kernel(AttnArgs a) {
    LBSA_DECLARE_SMEM(FP8, QL);
    const int S = a.P;
    const int split = blockIdx.x % S;
    const int rest = blockIdx.x / S;
    const int b = rest % a.B, h = rest / a.B;
    const int slot = (h * a.B + b) * S + split;
    // every kernel argument in one round trip, before the length is loaded
    __asm__ volatile("" ::"s"(a.q), "s"(a.k_cache), "s"(a.v_cache), "s"(a.page_table), "s"(a.seqlens),
                     "s"(a.part_lse), "s"(a.part_o), "s"(a.scale_log2), "s"(a.num_pages), "s"(a.max_pages));
    if constexpr (FP8) __asm__ volatile("" ::"s"(a.q_scale), "s"(a.k_scale), "s"(a.v_scale));
    int L = uniform_ptr<int32_t>(a.seqlens)[b];
    const bool len_ok = L >= 0 && L <= a.max_pages * kTile;
    if (!len_ok) L = 0;
    const int n = (L + kTile - 1) / kTile;
    const int t0 = (int)((int64_t)split * n / S);
    const int t1 = (int)((int64_t)(split + 1) * n / S);
    if (t1 <= t0) {   // empty split: weight 0 in the combine (NaN if the length was invalid)
        constexpr int R = Slot<FP8, QL>::kRows;
        const int tid = threadIdx.x;
#pragma unroll
        for (int pass = 0; pass < QL; ++pass) {
            const int hh = kGroup * pass + (tid >> 5), d4 = (tid & 31) * 4;
            *reinterpret_cast<f32x4*>(a.part_o + ((size_t)slot * R + hh) * kHeadDim + d4) = f32x4{0.f, 0.f, 0.f, 0.f};
            if ((tid & 31) == 0) a.part_lse[(size_t)slot * R + hh] = len_ok ? kNegInf : __builtin_nanf("");
        }
        return;
    }
    OneDesc src;
    src.d.h = h;
    src.d.b = b;
    src.d.t0 = t0;
    src.d.t1 = t1;
    src.d.L = L;
    src.d.slot = slot;
    run_stream<FP8, QL>(a, src, t1 - t0, sm);
}

// Online LSE merge of one chunk into a running (max, weight sum, weighted O).
__device__ inline void merge_chunk(float l, f32x4 x, float& m, float& wsum, f32x4& o, bool& nan_seen) {
    if (l != l) { nan_seen = true; return; }
    if (l == kNegInf) return;                           // empty chunk (static split) or padding
    if (l > m) {
        const float sc = exp2_fast((m - l) * kLog2e);   // 0 when m = -inf
        wsum *= sc;
        o *= sc;
        m = l;
    }
    const float wgt = exp2_fast((l - m) * kLog2e);
    wsum += wgt;
    o += wgt * x;
}

// Merge of chunks [d0, d0 + n) of partial row rr (R rows per slot) into the
// bf16 output row dst by one workgroup of 256 threads.  They form 8 slices of
// 32 (4 consecutive dims per thread); slice z merges chunks z, z + 8, ... with
// a running (max LSE, weight sum, weighted O).  The loads of up to UNROLL
// chunks per slice (8 UNROLL per row) are all issued before the first of them
// is used, so a row of up to 8 UNROLL chunks costs one round trip to the
// partials.  The 8 slice states are then merged through LDS under the global
// maximum.  A poisoned row is written as NaN.  The static combine, one
// workgroup per output row of every request, takes UNROLL = 8 (16 needed more
// registers, and the lower occupancy cost more than the round trips it
// saved); the long segments of the task-map combine, a few workgroups with
// up to hundreds of chunks each, take 16.
constexpr int kCombineUnroll = 8;
struct RowMergeLds {
    float m[8];
    float w[8];
    int nan;
    __attribute__((aligned(16))) float o[8][kHeadDim];
};
template <int UNROLL = kCombineUnroll>
__device__ inline void merge_row(const AttnArgs& a, int64_t d0, int n, int R, int rr, uint16_t* dst, bool poison,
                                 RowMergeLds& red) {
    constexpr int kSlices = 8;
    const int tid = threadIdx.x, slice = tid >> 5, d4 = (tid & 31) * 4;
    if (tid == 0) red.nan = 0;
    float m = kNegInf, wsum = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    bool nan_seen = false;
    auto pr = [&](int c) { return (d0 + c) * R + rr; };
    for (int c0 = slice; c0 < n; c0 += UNROLL * kSlices) {
        float l[UNROLL];
        f32x4 x[UNROLL];
        // every load first (a slice past the row's last chunk loads nothing), then
        // the merges
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int c = c0 + u * kSlices;
            if (c < n) {
                l[u] = a.part_lse[pr(c)];
                x[u] = *reinterpret_cast<const f32x4*>(a.part_o + pr(c) * kHeadDim + d4);
            } else {
                l[u] = kNegInf;
                x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) merge_chunk(l[u], x[u], m, wsum, o, nan_seen);
    }
    __syncthreads();                                    // red.nan initialised
    if (nan_seen) red.nan = 1;
    if ((tid & 31) == 0) {
        red.m[slice] = m;
        red.w[slice] = wsum;
    }
    *reinterpret_cast<f32x4*>(&red.o[slice][d4]) = o;
    __syncthreads();
    if (slice == 0) {
        float M = kNegInf;
#pragma unroll
        for (int i = 0; i < kSlices; ++i) M = fmaxf(M, red.m[i]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float W = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int i = 0; i < kSlices; ++i) {
                const float sc = exp2_fast((red.m[i] - M) * kLog2e);   // 0 for empty slices
                W += sc * red.w[i];
                acc += sc * *reinterpret_cast<const f32x4*>(&red.o[i][d4]);
            }
            acc *= 1.f / W;
        }
        if (poison || red.nan) {
            const float nan = __builtin_nanf("");
            acc = f32x4{nan, nan, nan, nan};
        }
        store_bf16x4(dst + d4, acc);
    }
}

// The combine of the static split: one workgroup per output row (request,
// query token, query head), merging the row's P chunks (slots seg * P + s).
__global__ __launch_bounds__(kCombineThreads) void combine_static_kernel(int B, int P, int Hq, int QL, AttnArgs a) {
    __shared__ RowMergeLds red;
    const int row = blockIdx.x;                         // (b * QL + query) * Hq + hq
    const int bq = row / Hq, hq = row - bq * Hq;
    const int b = bq / QL, qi = bq - b * QL;
    const int h = hq / kGroup, gq = hq - h * kGroup;
    const int64_t seg = (int64_t)h * B + b;
    merge_row(a, seg * P, P, kGroup * QL, kGroup * qi + gq, static_cast<uint16_t*>(a.out) + (size_t)row * kHeadDim,
              false, red);
}

// The combine of the task-map path, over the map's segments (KV head h,
// request b) and their 8 * QL rows rr = 8 * query token + head of the group.
//  - Workgroups [0, E), E = 8 QL max_long_segments(Hkv*B + P): workgroup e
//    takes row e mod 8 QL of the (e / 8 QL)-th long segment of the map's list
//    (more than kCombineSegChunks chunks) and merges it with merge_row; past
//    the list's end it returns.  They come first so that the largest merges
//    start first.
//  - Workgroups [E, E + Hkv*B): one per segment; thread t holds 4 dims of row
//    t / 32 (and of row t / 32 + 8 when QL = 2) and merges the segment's up to
//    kCombineSegChunks chunks from registers, all loaded in one round trip.  A
//    segment with one chunk was written by the split kernel when direct_out is
//    set: its workgroup returns after the map words; a long one is left to the
//    first range.
// A map built for another shape, or one whose lengths were invalid (the split
// kernel computed nothing), poisons the call: every output row is NaN (written
// by the segment workgroups).  Against one workgroup per output row (most of
// which would only read a chunk count), a batch of 64 requests with 64 query
// heads launches 2-3x fewer workgroups, and each row of a long segment still
// has a workgroup of its own.
template <int QL>
__global__ __launch_bounds__(kCombineThreads) void combine_map_kernel(const uint8_t* map, int B, int Hkv, int P, int Hq,
                                                                       AttnArgs a) {
    __shared__ RowMergeLds red;
    constexpr int R = kGroup * QL;                      // partial rows per slot
    const MapLayout ML = map_layout(B, Hkv, P);
    const int S = Hkv * B, cap = S + P;
    const int E = R * max_long_segments(cap);
    const int tid = threadIdx.x, d4 = (tid & 31) * 4;
    const auto* hdr = uniform_ptr<int32_t>(map + ML.header);
    auto out_row = [&](int h, int b, int rr) {
        const int qi = rr >> 3, gq = rr & 7;
        return static_cast<uint16_t*>(a.out) + ((size_t)(b * QL + qi) * Hq + (size_t)h * kGroup + gq) * kHeadDim;
    };
    if ((int)blockIdx.x < E) {
        const int k = (int)blockIdx.x / R, rr = (int)blockIdx.x - k * R;
        // the record and the header words in one round trip, with the kernel
        // arguments still to come (k < max_long_segments(cap): in bounds)
        const auto* ent = uniform_ptr<int32_t>(map + ML.long_seg) + 4 * k;
        const int seg = ent[0], d0 = ent[1], n = ent[2];
        const int h_p = hdr[LBSA_HDR_P], h_b = hdr[LBSA_HDR_B], h_hkv = hdr[LBSA_HDR_HKV];
        const int h_err = hdr[LBSA_HDR_ERROR], h_nlong = hdr[LBSA_HDR_NLONG];
        __asm__ volatile("" ::"s"(a.part_lse), "s"(a.part_o), "s"(a.out));
        keep(seg);
        keep(d0);
        keep(n);
        keep(h_nlong);
        // a poisoned map is written as NaN by the segment workgroups; a record
        // that does not describe a long segment of this map is not merged
        const bool bad_map = (h_p != P) | (h_b != B) | (h_hkv != Hkv) | (h_err != 0);
        if (bad_map || k >= h_nlong || seg < 0 || seg >= S || d0 < 0 || n <= kCombineSegChunks || n > cap - d0)
            return;
        const int h = seg / B, b = seg - h * B;
        merge_row<2 * kCombineUnroll>(a, d0, n, R, rr, out_row(h, b, rr), false, red);
        return;
    }
    const int seg = (int)blockIdx.x - E, h = seg / B, b = seg - h * B;
    const int d0 = uniform_ptr<int32_t>(map + ML.seg_first_desc)[seg];
    const int n = uniform_ptr<int32_t>(map + ML.seg_num_chunks)[seg];
    const int h_p = hdr[LBSA_HDR_P], h_b = hdr[LBSA_HDR_B], h_hkv = hdr[LBSA_HDR_HKV];
    const int h_err = hdr[LBSA_HDR_ERROR];
    __asm__ volatile("" ::"s"(a.part_lse), "s"(a.part_o), "s"(a.out), "s"(a.direct_out));
    keep(d0);
    keep(n);
    keep(h_err);
    const int r0 = tid >> 5;
    const bool bad_map = (h_p != P) | (h_b != B) | (h_hkv != Hkv) | (h_err != 0);
    if (bad_map | (d0 < 0) | (n < 0) | (n > cap - d0)) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int i = 0; i < QL; ++i) store_bf16x4(out_row(h, b, r0 + kGroup * i) + d4, f32x4{nan, nan, nan, nan});
        return;
    }
    if ((a.direct_out && n == 1) || n > kCombineSegChunks) return;
    if (n == 0) {                                       // an empty request: O = 0
#pragma unroll
        for (int i = 0; i < QL; ++i) store_bf16x4(out_row(h, b, r0 + kGroup * i) + d4, f32x4{0.f, 0.f, 0.f, 0.f});
        return;
    }
    // every load first, branch-free: a chunk past the segment's last re-reads
    // the last one (same cache lines) and is dropped by its -inf LSE
    float l[QL][kCombineSegChunks];
    f32x4 x[QL][kCombineSegChunks];
#pragma unroll
    for (int i = 0; i < QL; ++i) {
#pragma unroll
        for (int c = 0; c < kCombineSegChunks; ++c) {
            const size_t pr = (size_t)(d0 + min(c, n - 1)) * R + r0 + kGroup * i;
            const float lv = a.part_lse[pr];
            l[i][c] = c < n ? lv : kNegInf;
            x[i][c] = *reinterpret_cast<const f32x4*>(a.part_o + pr * kHeadDim + d4);
        }
    }
#pragma unroll
    for (int i = 0; i < QL; ++i) {
        float m = kNegInf, wsum = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        bool nan_seen = false;
#pragma unroll
        for (int c = 0; c < kCombineSegChunks; ++c) merge_chunk(l[i][c], x[i][c], m, wsum, o, nan_seen);
        if (m != kNegInf) o *= 1.f / wsum;
        if (nan_seen) {
            const float nan = __builtin_nanf("");
            o = f32x4{nan, nan, nan, nan};
        }
        store_bf16x4(out_row(h, b, r0 + kGroup * i) + d4, o);
    }
}

}  // namespace

hipError_t launch_split(const AttnArgs& a, bool fp8, hipStream_t stream) {
    const dim3 grid(a.P), block(kSplitThreads);
    if (a.QL == 2)
        return fp8 ? launch(split_kernel<true, 2>, grid, block, 0, stream, a.map, a.B, a.Hkv, a.P, a.max_pages, a)
                   : launch(split_kernel<false, 2>, grid, block, 0, stream, a.map, a.B, a.Hkv, a.P, a.max_pages, a);
    return fp8 ? launch(split_kernel<true, 1>, grid, block, 0, stream, a.map, a.B, a.Hkv, a.P, a.max_pages, a)
               : launch(split_kernel<false, 1>, grid, block, 0, stream, a.map, a.B, a.Hkv, a.P, a.max_pages, a);
}

hipError_t launch_static(const AttnArgs& a, bool fp8, hipStream_t stream) {
    const dim3 grid((unsigned)((long long)a.P * a.B * a.Hkv)), block(kSplitThreads);
    if (a.QL == 2)
        return fp8 ? launch(static_kernel<true, 2>, grid, block, 0, stream, a)
                   : launch(static_kernel<false, 2>, grid, block, 0, stream, a);
    return fp8 ? launch(static_kernel<true, 1>, grid, block, 0, stream, a)
               : launch(static_kernel<false, 1>, grid, block, 0, stream, a);
}

hipError_t launch_combine(const AttnArgs& a, bool static_mode, hipStream_t stream) {
    if (static_mode)
        return launch(combine_static_kernel, dim3((unsigned)((long long)a.B * a.QL * a.Hq)), dim3(kCombineThreads), 0,
                      stream, a.B, a.P, a.Hq, a.QL, a);
    const long long S = (long long)a.B * a.Hkv;
    const long long grid = (long long)kGroup * a.QL * max_long_segments(S + a.P) + S;
    if (a.QL == 2)
        return launch(combine_map_kernel<2>, dim3((unsigned)grid), dim3(kCombineThreads), 0, stream, a.map, a.B, a.Hkv,
                      a.P, a.Hq, a);
    return launch(combine_map_kernel<1>, dim3((unsigned)grid), dim3(kCombineThreads), 0, stream, a.map, a.B, a.Hkv,
                  a.P, a.Hq, a);
}

hipError_t split_occupancy(bool fp8, int q_len, int* blocks_per_cu) {
    if (q_len == 2) {
        if (fp8)
            return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, split_kernel<true, 2>, kSplitThreads, 0);
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, split_kernel<false, 2>, kSplitThreads, 0);
    }
    if (fp8)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, split_kernel<true, 1>, kSplitThreads, 0);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, split_kernel<false, 1>, kSplitThreads, 0);
}

}  // namespace lbsa
