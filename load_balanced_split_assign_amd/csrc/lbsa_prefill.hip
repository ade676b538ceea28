// Prefill / extend attention over the paged KV cache for gfx950 (bf16).
//
// Method: the vLLM post's Table 4 ("Attention latency vs FlashAttention,
// Triton and FlashInfer") measures the same attention backend on prefill and
// extend shapes; the SGLang post's "Attention" section frames decode and
// prefill as one backend over the paged store.  Prefill and extend are causal
// attention of a request's q_len new tokens (the last q_len of its L cached
// tokens, written into the cache beforehand) over the cache: query i sees
// tokens [0, L - q_len + i].
//
// gfx950 mapping.  The work is a dense contraction, so it is built around the
// MFMA tiles the decode kernel already uses, with K/V reuse across many query
// columns:
//   * A workgroup (4 wave64) owns one KV head of one request and a block of
//     query positions; every query column is a (position, head of the group)
//     pair, 16 columns per MFMA block, CB blocks per wave (CB = 1 or 2, i.e.
//     2 or 4 positions per wave).  Q stays in registers for the whole run.
//   * The 64-token K/V tiles (one page of the KV head) stream through a
//     2-stage LDS ring (64 KiB) shared by the 4 waves: each wave issues the
//     async global->LDS loads of 16 of the 64 rows, waits for them with its
//     own vmcnt, and one workgroup barrier per tile publishes the tile and
//     frees the stage written next.  At 64 KiB of LDS and under 256 VGPRs two
//     workgroups share a compute unit, so one's softmax (VALU) overlaps the
//     other's MFMAs; that overlap outweighs the larger K/V reuse of 4 blocks
//     per wave or a deeper ring, which both leave one wave per SIMD.
//   * Per 32-token half-tile: S^T = K Q^T (MFMA 16x16x32 bf16, one chain of 4
//     per 16 tokens and block; K is read from LDS once per wave for all CB
//     blocks), an online softmax per column in the exp2 domain with a lazy
//     running max, then O^T += V^T P^T with MFMA 16x16x32 bf16 over the 32
//     tokens (V^T through ds_read_b64_tr_b16, P straight from the S^T
//     accumulators).  Half-tiles that reach a column's limit set the scores
//     above it to -inf; the softmax scale folds into one fma before each
//     exp2; the denominator is one more MFMA with an all-ones A operand over
//     the same bf16 P as the numerator.
//   * The tile loop is unrolled over the 2 ring stages and the 2 halves, so
//     each LDS read is a per-lane base address plus an immediate offset.
//   * Built with the MFMA accumulators in VGPRs (-amdgpu-mfma-vgpr-form): the
//     rescale of the online softmax multiplies them with VALU instructions,
//     which cannot address AGPRs, and the AGPR form copied every accumulator
//     on every step.
//   * Causality: column limits mask the diagonal tiles; a wave skips the tiles
//     past its own last position; the grid starts with the query blocks that
//     see the most tiles (longest first), and the blocks of one (request, KV
//     head) share an XCD whenever batch * Hkv is a multiple of 8, so their K/V
//     reuse stays in one L2.
#include <type_traits>

#include "lbsa_device.h"

namespace lbsa {
namespace {

using namespace dev;

constexpr int kPfStages = 2;
constexpr int kPfRow = 256;                         // bytes of one bf16 K/V row
constexpr int kPfSlice = 16 * kPfRow;               // one wave's 16 rows of a tile
constexpr int kPfHalf = 64 * kPfRow;                // K (or V) of one 64-token tile
constexpr int kPfStageBytes = 2 * kPfHalf;          // 32 KiB: K then V
constexpr int kPfLoads = 8;                         // ring loads per lane per tile (4 K + 4 V)
constexpr float kPfSlack = 8.0f;                    // log2 headroom of the lazy running max
static_assert(kPfStages * kPfStageBytes <= 80 * 1024, "two workgroups per compute unit");
static_assert((kPfStages - 2) * kPfLoads < 64, "vmcnt range");

struct PrefillArgs {
    const uint16_t* q;           // [B][QL][Hq][128]
    const uint16_t* k_cache;     // [pages][64][Hkv][128]
    const uint16_t* v_cache;
    const int32_t* page_table;   // [B][max_pages]
    const int32_t* seqlens;      // [B]
    uint16_t* out;               // [B][QL][Hq][128]
    int64_t num_pages;
    int32_t B, QL, Hq, Hkv, max_pages;
    int32_t qblocks;             // query blocks per (request, KV head)
    float scale_log2;            // softmax_scale * log2(e)
};

__device__ inline int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }



template <int CB>
__global__ __launch_bounds__(kSplitThreads) void prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) char ring_mem[kPfStages * kPfStageBytes];
    lds_char* const ring = (lds_char*)ring_mem;         // stage u at u * kPfStageBytes
    constexpr int kPosWave = 2 * CB, kPosBlock = kWaves * kPosWave;

    // heaviest query blocks first; consecutive workgroups take different
    // (request, KV head) pairs of the same query block
    const int nbh = a.B * a.Hkv;
    const int qb = a.qblocks - 1 - (int)(blockIdx.x / (unsigned)nbh);
    const int bh = (int)(blockIdx.x % (unsigned)nbh);
    const int b = bh / a.Hkv, h = bh - b * a.Hkv;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;

    int L = uniform_ptr<int32_t>(a.seqlens)[b];
    const bool len_ok = L >= 0 && L <= a.max_pages * kTile;
    if (!len_ok) L = 0;
    const int off = L - a.QL;                             // query i sees tokens < off + i + 1

    // columns of this lane: position p0 + 2 cb + r / 8, head r % 8
    const int p0 = qb * kPosBlock + w * kPosWave;
    int pos[CB], lim[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        pos[cb] = p0 + 2 * cb + (r >> 3);
        lim[cb] = pos[cb] < a.QL ? clampi(off + pos[cb] + 1, 0, L) : 0;
    }
    // smallest limit over this wave's live columns (its first position): tokens
    // below it are visible to every live column
    const int lim_lo = p0 < a.QL ? clampi(off + p0 + 1, 0, L) : 0;
    const int pw_last = min(p0 + kPosWave, a.QL) - 1;     // this wave's last live position
    const int lim_wave = pw_last >= p0 ? clampi(off + pw_last + 1, 0, L) : 0;
    const int pb_last = min(qb * kPosBlock + kPosBlock, a.QL) - 1;
    const int lim_blk = pb_last >= qb * kPosBlock ? clampi(off + pb_last + 1, 0, L) : 0;
    const int ntiles = (lim_blk + kTile - 1) / kTile;

    f32x4 acc[CB][8];
    float m[CB];
    f32x4 l[CB];        // column sums of P, from an MFMA with an all-ones A: every element holds it
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[cb] = kNegInf;
        l[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bool bad = !len_ok;

    if (ntiles > 0) {
        // Q of every column of this lane (B operand: 8 dims per k-step), then
        // wait for it once before the ring starts
        uint4 q[CB][4];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const bool live = pos[cb] < a.QL;
            const int p = live ? pos[cb] : 0;
            const uint4* qp = reinterpret_cast<const uint4*>(
                a.q + ((size_t)(b * a.QL + p) * a.Hq + (size_t)h * kGroup + (r & 7)) * kHeadDim);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) q[cb][ks] = live ? qp[g + 4 * ks] : make_uint4(0, 0, 0, 0);
        }
        wait_vmcnt<0>();

        // this lane's 4 K and 4 V chunks of every tile: rows 16 w + 4 s + lane / 16,
        // chunk lane % 16, XOR-swizzled by the row inside the wave's 16
        uint32_t live_off[4], live_off_v[4], dead_off[4];
        int lrow[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            lrow[s] = 4 * s + (lane >> 4);
            const uint32_t chunk = 16u * (uint32_t)((lane & 15) ^ lrow[s]);
            const uint32_t chunk_v = 16u * (uint32_t)((lane & 15) ^ swz_v(lrow[s]));
            const uint32_t row_off = (uint32_t)(16 * w + lrow[s]) * (uint32_t)a.Hkv * kPfRow;
            live_off[s] = row_off + chunk;
            live_off_v[s] = row_off + chunk_v;
            dead_off[s] = 16u * (uint32_t)(lane & 15);    // row 0 of the page: always live
        }
        const auto* pt = uniform_ptr<int32_t>(a.page_table) + (size_t)b * a.max_pages;
        auto issue = [&](int t, lds_char* st) {
            int64_t page = pt[t];
            if (page < 0 || page >= a.num_pages) {
                bad = true;
                page = 0;
            }
            const size_t pbase = ((size_t)page * kTile * a.Hkv + h) * kPfRow;
            const char* kb = reinterpret_cast<const char*>(a.k_cache) + pbase;
            const char* vb = reinterpret_cast<const char*>(a.v_cache) + pbase;
            const int tok0 = kTile * t + 16 * w;
            const bool full = tok0 + 16 <= L;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bool live = full || tok0 + lrow[s] < L;
                dma16(kb + (live ? live_off[s] : dead_off[s]), st + w * kPfSlice + 1024 * s);
                dma16(vb + (live ? live_off_v[s] : dead_off[s]), st + kPfHalf + w * kPfSlice + 1024 * s);
            }
        };
        for (int u = 0; u < kPfStages - 1; ++u) issue(min(u, ntiles - 1), ring + u * kPfStageBytes);

        // lane parts of the ring read addresses (stage 0, first 16 rows); the
        // stage and the 16-row sub-tile are the reads' immediate offsets
        uint32_t ka[4], vaddr[8];
        {
            const uint32_t rb = lds_addr(ring);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ka[ks] = rb + r * kPfRow + 16 * ((g + 4 * ks) ^ r);
            const int vrow = 4 * g + (r >> 2);
            const uint32_t vr = rb + kPfHalf + vrow * kPfRow + 8 * (r & 1);
#pragma unroll
            for (int db = 0; db < 8; ++db)
                vaddr[db] = vr + 16u * (uint32_t)((2 * db + ((r >> 1) & 1)) ^ swz_v(vrow));
        }

        const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
        // 32 tokens [t32, t32 + 32) of the tile whose rows start at ring byte OFF
        auto half_step = [&](auto off_c, int t32) {
            constexpr int OFF = decltype(off_c)::value;
            // ---- K (A operand of S^T) and V^T reads of 32 tokens, two 16-token
            // sub-tiles, shared by all CB blocks
            uint4 kk[2][4];
            s16x4 va[2][8];
            lds_read_tile_bf16_at<OFF>(kk[0], va[0], ka, vaddr);
            lds_read_tile_bf16_at<OFF + 16 * kPfRow>(kk[1], va[1], ka, vaddr);

            // ---- S^T = K Q^T: s[cb][sub][i] is token t32 + 16 sub + 4 g + i
            f32x4 s[CB][2];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    f32x4 sa = {0.f, 0.f, 0.f, 0.f};
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[sub][0]), as_bf16x8(q[cb][0]), sa, 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[sub][1]), as_bf16x8(q[cb][1]), sa, 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[sub][2]), as_bf16x8(q[cb][2]), sa, 0, 0, 0);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[sub][3]), as_bf16x8(q[cb][3]), sa, 0, 0, 0);
                    s[cb][sub] = sa;
                }
            }

            // ---- online softmax over the 8 scores of this lane per block.  Half-
            // tiles that reach a live column's limit get -inf above it (raw score
            // domain); then one path for all: the scale folds into the fma before
            // each exp2 (exp2(-inf) = 0), and the block maximum is the scale times
            // the raw maximum (the scale is positive).  The maximum propagates NaN
            // (v_maximum3), which needs no canonicalising of the MFMA results.
            const int tok = t32 + 4 * g;
            if (t32 + 31 >= lim_lo) {                                     // uniform
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (tok + 16 * sub + i >= lim[cb]) s[cb][sub][i] = kNegInf;
            }
            float lmax[CB];
            bool need = false;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const f32x4 x0 = s[cb][0], x1 = s[cb][1];
                float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x0[0], x0[1]), x0[2]);
                mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, x0[3]), x1[0]);
                mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, x1[1]), x1[2]);
                mx = __builtin_elementwise_maximum(mx, x1[3]);
                lmax[cb] = mx * a.scale_log2;
                need |= lmax[cb] > m[cb] + kPfSlack;
            }
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                // a score above a column's reference: new reference = max over
                // the column's 32 tokens (0 rescale for a column still fully masked)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    float mt = fmaxf(lmax[cb], __shfl_xor(lmax[cb], 16, 64));
                    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
                    const float m_new = fmaxf(m[cb], mt);
                    const float alpha = m[cb] == kNegInf ? 0.f : exp2_fast(m[cb] - m_new);
                    l[cb] *= alpha;
#pragma unroll
                    for (int db = 0; db < 8; ++db) acc[cb][db] *= alpha;
                    m[cb] = m_new;
                }
            }

            // ---- P and O^T += V^T P^T with MFMA 16x16x32: k = the 32 tokens,
            // lane group g holding tokens 4g .. 4g + 3 of both sub-tiles, in the
            // same order in the V^T operand (two transposed reads) and in P
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const float mref = m[cb] == kNegInf ? 0.f : m[cb];
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = exp2_fast(fmaf(s[cb][j >> 2][j & 3], a.scale_log2, -mref));
                const bf16x8 pb = __builtin_bit_cast(
                    bf16x8, make_uint4(bf16x2_pack(p[0], p[1]), bf16x2_pack(p[2], p[3]),
                                       bf16x2_pack(p[4], p[5]), bf16x2_pack(p[6], p[7])));
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const bf16x8 vt = __builtin_bit_cast(
                        bf16x8, make_uint4(__builtin_bit_cast(uint2, va[0][db]).x,
                                           __builtin_bit_cast(uint2, va[0][db]).y,
                                           __builtin_bit_cast(uint2, va[1][db]).x,
                                           __builtin_bit_cast(uint2, va[1][db]).y));
                    acc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb, acc[cb][db], 0, 0, 0);
                }
                // the softmax denominator over the same bf16 P as the numerator
                l[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, l[cb], 0, 0, 0);
            }
        };

        // tile k sits in ring stage U = k % 2.  Every tile issues the same number
        // of loads (past the end the last tile is loaded again into a stage
        // nobody reads), so one wait count fits all
        auto tile_step = [&](auto u_c, int k) {
            constexpr int U = decltype(u_c)::value;
            wait_vmcnt<(kPfStages - 2) * kPfLoads>();                 // this wave's rows of tile k
            lds_barrier();                                          // everyone's rows; stage of k-1 free
            issue(min(k + kPfStages - 1, ntiles - 1), ring + (1 - U) * kPfStageBytes);
            if (kTile * k >= lim_wave) return;                      // nothing of it is visible here
            half_step(std::integral_constant<int, U * kPfStageBytes>{}, kTile * k);
            if (kTile * k + 32 < lim_wave)
                half_step(std::integral_constant<int, U * kPfStageBytes + 32 * kPfRow>{}, kTile * k + 32);
        };
        static_assert(kPfStages == 2, "tile_step alternates two stages");
        for (int k = 0; k < ntiles; k += 2) {
            tile_step(std::integral_constant<int, 0>{}, k);
            if (k + 1 < ntiles) tile_step(std::integral_constant<int, 1>{}, k + 1);
        }
        wait_vmcnt<0>();   // no load may still target LDS when the workgroup ends
    }

    // ---- normalise and store: lane (g, r) holds dims 16 db + 4 g .. + 3 of column r
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const float lt = l[cb][0];
        if (pos[cb] >= a.QL) continue;
        float inv = lt > 0.f ? 1.f / lt : 0.f;            // a query that sees nothing: zeros
        if (bad) inv = __builtin_nanf("");
        uint16_t* o = a.out + ((size_t)(b * a.QL + pos[cb]) * a.Hq + (size_t)h * kGroup + (r & 7)) * kHeadDim + 4 * g;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const f32x4 v = acc[cb][db] * inv;
            *reinterpret_cast<uint2*>(o + 16 * db) = make_uint2(bf16x2_pack(v[0], v[1]), bf16x2_pack(v[2], v[3]));
        }
    }
}

template <int CB>
hipError_t launch_cb(PrefillArgs a, hipStream_t stream) {
    constexpr int kPosBlock = kWaves * 2 * CB;
    a.qblocks = (a.QL + kPosBlock - 1) / kPosBlock;
    const long long grid = (long long)a.qblocks * a.B * a.Hkv;
    return launch(prefill_kernel<CB>, dim3((unsigned)grid), dim3(kSplitThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                          const int32_t* seqlens, int B, int QL, int Hq, int Hkv, int max_pages,
                          int64_t num_pages, float scale_log2, void* out, int cb, hipStream_t stream) {
    PrefillArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint16_t*>(k_cache);
    a.v_cache = static_cast<const uint16_t*>(v_cache);
    a.page_table = page_table;
    a.seqlens = seqlens;
    a.out = static_cast<uint16_t*>(out);
    a.num_pages = num_pages;
    a.B = B;
    a.QL = QL;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.max_pages = max_pages;
    a.qblocks = 0;
    a.scale_log2 = scale_log2;
    if (cb <= 0) {
        // two query blocks per wave (K/V reuse) while that still leaves two
        // workgroups per compute unit in the grid, else one
        const long long bh = (long long)B * Hkv;
        cb = bh * ((QL + kWaves * 4 - 1) / (kWaves * 4)) >= 512 ? 2 : 1;
    }
    return cb == 2 ? launch_cb<2>(a, stream) : launch_cb<1>(a, stream);
}

}  // namespace lbsa
