// Internal declarations shared by the HIP translation units of liblbsa.so.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lbsa.h"

namespace lbsa {

constexpr int kTile = 64;       // tokens per tile = tokens per page
constexpr int kHeadDim = 128;
constexpr int kGroup = 8;       // query heads per KV head
constexpr int kSplitThreads = 256;   // 4 wave64 per split workgroup
constexpr int kAssignThreads = 256;
constexpr int kCombineThreads = 256;
constexpr int kMaxAssignLdsWords = 16384;  // (B + 1) + (Hkv*B + 1) + B int32 in 64 KiB
constexpr int kAutoTilesPerWorkgroup = 32;  // lbsa_auto_workgroups: tiles per resident workgroup for two waves

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Events armed by lbsa_time_next_kernel for the next launch on this host
// thread; taking them disarms the hook.
struct KernelEvents {
    hipEvent_t start, stop;
};
KernelEvents take_kernel_events();

// Every kernel of the library is launched here: through hipExtLaunchKernelGGL,
// which stamps the armed events at the kernel's own start and end, when the
// timing hook is armed, else as a plain launch.
template <class F, class... Args>
inline hipError_t launch(F kernel, dim3 grid, dim3 block, uint32_t lds_bytes, hipStream_t stream, Args... args) {
    const KernelEvents ev = take_kernel_events();
    if (ev.start != nullptr || ev.stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, ev.start, ev.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
    return hipGetLastError();
}

// Byte offsets of the task-map arrays for (B, Hkv, P).
struct MapLayout {
    size_t header, bin_desc_begin, desc, seg_first_desc, seg_num_chunks, seqlens, bin_head, desc_len, long_seg,
        total;
};

// A segment of more than kCombineSegChunks chunks is "long": the assign lists
// it as (segment, first descriptor, chunks, 0), and the combine merges each of
// its rows in a workgroup of its own; shorter segments are merged whole by one
// workgroup.  With at most Hkv*B + P descriptors there are at most
// max_long_segments of them.
constexpr int kCombineSegChunks = 8;
__host__ __device__ inline int max_long_segments(int64_t cap) { return (int)(cap / (kCombineSegChunks + 1)); }

// Words of one bin_head record: the bin's first descriptor, its slot, the
// bin's descriptor count and the request's length (everything a split
// workgroup needs to start streaming).
constexpr int kBinHeadWords = 8;
enum { BH_H = 0, BH_B = 1, BH_T0 = 2, BH_T1 = 3, BH_FIRST = 4, BH_COUNT = 5, BH_L = 6 };

__host__ __device__ inline MapLayout map_layout(int B, int Hkv, int P) {
    MapLayout m;
    const size_t S = (size_t)Hkv * (size_t)B;
    const size_t cap = S + (size_t)P;
    m.header = 0;
    m.bin_desc_begin = 64;
    m.desc = align_up(m.bin_desc_begin + 4 * ((size_t)P + 1), 16);
    m.seg_first_desc = m.desc + 16 * cap;
    m.seg_num_chunks = m.seg_first_desc + 4 * S;
    m.seqlens = m.seg_num_chunks + 4 * S;
    m.bin_head = align_up(m.seqlens + 4 * (size_t)B, 32);
    m.desc_len = m.bin_head + 4 * kBinHeadWords * (size_t)P;
    m.long_seg = align_up(m.desc_len + 4 * cap, 16);
    m.total = align_up(m.long_seg + 16 * (size_t)max_long_segments((int64_t)cap), 256);
    return m;
}

// ---------------------------------------------------------------------------
// Prefill / extend on the task map.  Request b brings q_b new tokens (the last
// q_b of its L_b cached ones); its queries form blocks of kQBlock positions,
// and a segment is (KV head, request, query block) spanning the tiles that the
// block's last query sees.  Segments are walked head-major, batch-minor, query
// block innermost, with the decode budget, fill and spill.  Q and out are
// packed [sum q_b][Hq][128].
// ---------------------------------------------------------------------------
constexpr int kQBlock = 24;                 // query positions per block (one split workgroup's columns:
                                            // 4 waves x 3 MFMA column blocks of 2 positions x 8 heads)
static_assert(kQBlock == LBSA_QBLOCK, "the public block size");
constexpr int kVarlenDescWords = 8;         // h, b, k, t0, t1, L, q, qstart: one 32-byte record
enum { VD_H = 0, VD_B = 1, VD_K = 2, VD_T0 = 3, VD_T1 = 4, VD_L = 5, VD_Q = 6, VD_QS = 7 };
constexpr int kVarlenRows = kQBlock * kGroup;   // partial rows per slot: position p, head g -> p * 8 + g

// Query blocks a map must hold: sum_b ceil(q_b / 24) <= B + total_q / 24.
__host__ __device__ inline int64_t varlen_max_blocks(int B, int64_t total_q) { return B + total_q / kQBlock; }

// Byte offsets of a prefill / extend task map for B requests, Hkv KV heads, P
// bins and at most NQ query blocks per KV head.  desc_slot[d] is the partial
// slot of descriptor d: 2 j for the first descriptor of bin j, 2 j + 1 for
// the others (only a bin's first and last descriptors can be cut).
// claim_order lists the descriptors of each group of bins (kVarlenGroups
// groups of consecutive bins, group x = bins [x P / 8, (x + 1) P / 8)) in the
// order the split kernel's workgroups claim them: by decreasing length class
// (the tile count below 8, then four classes per power of two), equal classes
// by decreasing index.
struct VarlenMapLayout {
    size_t header, bin_desc_begin, desc, desc_slot, claim_order, seg_first_desc, seg_num_chunks, seg_slot0,
        blk_req, blk_k, qbase, qstart, seqlens, qlens, total;
};

__host__ __device__ inline VarlenMapLayout varlen_map_layout(int B, int Hkv, int P, int64_t NQ) {
    VarlenMapLayout m;
    const size_t S = (size_t)Hkv * (size_t)NQ;
    const size_t cap = S + (size_t)P;
    m.header = 0;
    m.bin_desc_begin = 64;
    m.desc = align_up(m.bin_desc_begin + 4 * ((size_t)P + 1), 32);
    m.desc_slot = m.desc + 4 * kVarlenDescWords * cap;
    m.claim_order = m.desc_slot + 4 * cap;
    m.seg_first_desc = m.claim_order + 4 * cap;
    m.seg_num_chunks = m.seg_first_desc + 4 * S;
    m.seg_slot0 = m.seg_num_chunks + 4 * S;
    m.blk_req = m.seg_slot0 + 4 * S;
    m.blk_k = m.blk_req + 4 * (size_t)NQ;
    m.qbase = m.blk_k + 4 * (size_t)NQ;
    m.qstart = m.qbase + 4 * ((size_t)B + 1);
    m.seqlens = m.qstart + 4 * ((size_t)B + 1);
    m.qlens = m.seqlens + 4 * (size_t)B;
    m.total = align_up(m.qlens + 4 * (size_t)B, 256);
    return m;
}

// The varlen workspace starts with the counters of the split kernel, cleared
// before every launch: one claim counter per group of bins (a group per XCD),
// then an arrival counter per bin (for the cut segment whose first chunk the
// bin holds); the partial slots follow.
constexpr int kVarlenGroups = 8;
__host__ __device__ inline size_t varlen_counter_bytes(int P) { return align_up(4 * ((size_t)kVarlenGroups + P), 256); }

// LDS words the varlen assign kernel needs: lengths, q lengths, their two
// prefixes, the tile prefix over query blocks, the chunk prefix over
// segments, the claim-order histogram and each query block's request.
constexpr int kVarlenClaimHistWords = 2048;
// The varlen assign runs in one workgroup with every prefix in LDS: up to
// 144 KiB of prefixes plus the histogram (gfx950 gives a workgroup 160 KiB).
constexpr int kMaxVarlenAssignLdsWords = 36864 + kVarlenClaimHistWords;
__host__ __device__ inline size_t varlen_assign_lds_words(int B, int Hkv, int64_t NQ) {
    return 4 * (size_t)B + 2 + ((size_t)NQ + 1) + ((size_t)Hkv * NQ + 1) + kVarlenClaimHistWords + (size_t)NQ;
}

// Byte offsets of the partial buffers for `slots` partials of (q_len x G) x D
// (one row per query token and head of the group).
struct WsLayout {
    size_t part_lse, part_o, total;
};

__host__ __device__ inline WsLayout ws_layout(size_t slots, int q_len) {
    const size_t rows = slots * (size_t)kGroup * (size_t)q_len;
    WsLayout w;
    w.part_lse = 0;
    w.part_o = align_up(4 * rows, 256);
    w.total = align_up(w.part_o + 4 * rows * kHeadDim, 256);
    return w;
}

constexpr int kMaxQLen = 2;     // query tokens per request the decode kernels take

// Arguments of the attention kernels (passed by value).
struct AttnArgs {
    const void* q;
    const float* q_scale;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* page_table;
    const int32_t* seqlens;      // static path only (the split path reads the map copy)
    const uint8_t* map;          // task map base (split / combine)
    float* part_lse;
    float* part_o;
    void* out;
    int32_t num_pages;           // pages in each cache (capped at INT32_MAX: page ids are int32)
    int32_t B, Hq, Hkv, max_pages;
    int32_t P;                   // split: bins; static: number of splits
    int32_t QL;                  // query tokens per request (1 .. kMaxQLen)
    int32_t direct_out;          // split: a segment's only chunk goes straight to out (bf16); combine:
                                 // skip the rows of single-chunk segments (map path only)
    float scale_log2;            // softmax_scale * log2(e)
};

// Host launchers (defined in the .hip files).
hipError_t launch_assign(const int32_t* seqlens, int B, int Hq, int Hkv, int P, int F,
                         int max_pages, void* map, hipStream_t stream);
hipError_t launch_assign_varlen(const int32_t* seqlens, const int32_t* qlens, int B, int Hq, int Hkv, int P, int F,
                                int max_pages, int64_t total_q, int64_t nq_max, void* map, hipStream_t stream);
hipError_t launch_split(const AttnArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_static(const AttnArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_combine(const AttnArgs& a, bool static_mode, hipStream_t stream);
hipError_t split_occupancy(bool fp8, int q_len, int* blocks_per_cu);
hipError_t launch_varlen(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                         const void* map, int B, int Hq, int Hkv, int P, int64_t nq_max, int max_pages,
                         int64_t num_pages, int64_t total_q, float scale_log2, int32_t* counters, float* part_lse,
                         float* part_o, void* out, int workgroups, hipStream_t stream);
hipError_t varlen_occupancy(int* blocks_per_cu);
hipError_t launch_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                          const int32_t* seqlens, int B, int QL, int Hq, int Hkv, int max_pages,
                          int64_t num_pages, float scale_log2, void* out, int cb, hipStream_t stream);
// Router GEMM launch plan.  Thin form (few tokens): MT 16-token tiles per
// workgroup of 16 experts, K split in S = K / 256 parts.  Tile form: 64 tokens
// x 192 experts per workgroup, S parts of K of at most kRouterTileMaxK each.
// S > 1: the parts' fp32 partial planes [S][M][N] go to the workspace and a
// second kernel adds them.
constexpr int kRouterKAlign = 256;          // K granularity of both forms
constexpr int kRouterThinMaxM = 256;        // thin form up to this many tokens
constexpr int kRouterTileMaxK = 1024;       // k per tile workgroup (its X tile in LDS)
constexpr int kRouterTileMaxS = 16;         // parts of K a tile-form split aims at, at most
constexpr int kRouterTileTarget = 256;      // tile-form workgroups aimed at (one per CU)
struct RouterPlan {
    bool tile;
    int MT, S, tiles_n;
    size_t workspace;
};
RouterPlan router_plan(int M, int N, int K);
hipError_t launch_router_split(const float* w, void* hi, void* lo, int N, int K, hipStream_t stream);
hipError_t launch_router_gemm(const void* x, const void* w_hi, const void* w_lo, int M, int N, int K, float* out,
                              void* workspace, hipStream_t stream);
hipError_t launch_prologue(const uint16_t* qkv, const int32_t* positions, const int64_t* slots,
                           const float* qw, const float* kw, double theta, float eps, int T, int Hq,
                           int Hkv, bool fp8, void* q_out, float* q_scale, void* k_cache, void* v_cache,
                           float* k_scale, float* v_scale, int64_t num_pages, hipStream_t stream);

}  // namespace lbsa
