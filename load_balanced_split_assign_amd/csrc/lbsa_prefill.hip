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
//     pair, 16 columns per MFMA block, CB blocks per wave (CB = 1, 2 or 3,
//     i.e. 2, 4 or 6 positions per wave).  Q stays in registers for the whole
//     run.  Every wave reads each K/V element from LDS once for all its
//     columns, so the LDS bytes per MFMA fall as 1 / CB: at CB = 2 the LDS
//     reads take about as long as the MFMAs.
//   * The 64-token K/V tiles (one page of the KV head) stream through a
//     2-stage LDS ring (64 KiB) shared by the 4 waves: each wave issues the
//     async global->LDS loads of 16 of the 64 rows, waits for them with its
//     own vmcnt, and one workgroup barrier per tile publishes the tile and
//     frees the stage written next.  At 64 KiB of LDS and up to 256 VGPRs two
//     workgroups share a compute unit, so one's softmax (VALU) overlaps the
//     other's MFMAs; that overlap outweighs the larger K/V reuse of 4 blocks
//     per wave or a deeper ring, which both leave one wave per SIMD.
//   * Per 32-token half-tile: S^T = K Q^T (MFMA 16x16x32 bf16, one chain of 4
//     per 16 tokens and block; K is read from LDS once per wave for all CB
//     blocks), an online softmax per column in the exp2 domain with a lazy
//     running max, then O^T += V^T P^T with MFMA 16x16x32 bf16 over the 32
//     tokens (V^T through ds_read_b64_tr_b16, P straight from the S^T
//     accumulators; P of every block first, then the MFMAs, each V^T operand
//     shared by the blocks).  At CB = 3 the operands of a half-tile pass
//     through the same registers one after another (K of one 16-token
//     sub-tile, then the other, then V^T, read while the S MFMAs run), which
//     keeps the kernel at 256 VGPRs and two waves per SIMD.  Half-tiles that reach a column's limit set the scores
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

// x, through an empty asm that the compiler must assume changes it: values
// derived from the result are computed where it is taken, not hoisted out of an
// enclosing loop (where they would occupy registers across the whole loop).
__device__ inline int opaque(int x) {
    __asm__ volatile("" : "+v"(x));
    return x;
}

// The K rows of one 16-token sub-tile at ring byte OFF (A operands of S^T),
// complete on return.
template <int OFF>
__device__ inline void lds_read_k16_at(uint4 (&k)[4], const uint32_t (&ka)[4]) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
    u32x4 k0, k1, k2, k3;
    __asm__ volatile(
        "ds_read_b128 %0, %4 offset:%8\n\t"
        "ds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\t"
        "ds_read_b128 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3)
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "i"(OFF)
        : "memory");
    k[0] = __builtin_bit_cast(uint4, k0);
    k[1] = __builtin_bit_cast(uint4, k1);
    k[2] = __builtin_bit_cast(uint4, k2);
    k[3] = __builtin_bit_cast(uint4, k3);
}

// The transposed V reads of the same half-tile (V^T operands of PV), complete
// on return.
template <int OFF>
__device__ inline void lds_read_vt32_at(s16x4 (&va)[2][8], const uint32_t (&vaddr)[8]) {
    static_assert(OFF >= 0 && OFF + 16 * kPfRow < 65536, "DS offset field");
    typedef short s16x4_v __attribute__((ext_vector_type(4)));
    s16x4_v o[16];
    __asm__ volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %2, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%25\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
        "ds_read_b64_tr_b16 %12, %20 offset:%25\n\t"
        "ds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
          "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]),
          "=&v"(o[15])
        : "v"(vaddr[0]), "v"(vaddr[1]), "v"(vaddr[2]), "v"(vaddr[3]), "v"(vaddr[4]), "v"(vaddr[5]), "v"(vaddr[6]),
          "v"(vaddr[7]), "i"(OFF), "i"(OFF + 16 * kPfRow)
        : "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        va[0][i] = __builtin_bit_cast(s16x4, o[i]);
        va[1][i] = __builtin_bit_cast(s16x4, o[8 + i]);
    }
}



// One query block of one (request, KV head) over the KV tiles [t0, t1) of the
// request: what a prefill workgroup computes for its block, and what a
// persistent workgroup computes for one descriptor of a prefill / extend map.
struct QBlock {
    const uint16_t* q0;          // row of the block's first position, head 0 (row p at q0 + p * Hq * 128)
    const uint16_t* k_cache;     // [pages][64][Hkv][128]
    const uint16_t* v_cache;
    const int32_t* pt;           // the request's page-table row
    int64_t num_pages;
    int Hq, Hkv, h;
    int L;                       // the request's cached tokens (0 if invalid)
    int live;                    // positions of the block that are real queries
    int off;                     // block position p sees tokens [0, off + p]
    float scale_log2;
};

// Column state of one wave after a block: acc[cb][db] = O^T (unnormalised),
// m[cb] the log2-domain reference maximum, l[cb] the column sums of P (every
// element holds the sum).  Position of block column (cb, r): kPosWave w + 2 cb + r / 8.
template <int CB>
struct QBlockState {
    f32x4 acc[CB][8];
    float m[CB];
    f32x4 l[CB];
    bool bad;
};

// LEAN: form the 8 DMA offsets of a tile at each tile from three lane registers
// instead of holding them (the task-map kernel, whose claim loop needs the
// registers); the grid kernel holds them and saves the VALU work.
template <int CB, bool LEAN = false>
__device__ __attribute__((always_inline)) inline void attend_qblock(const QBlock& a, lds_char* ring, int t0, int t1,
                                                                    QBlockState<CB>& st, int tid, int first_page = -1) {
    constexpr int kPosWave = 2 * CB;
    // three blocks per wave fit two waves per SIMD only with the K and V^T
    // operands of a half-tile in registers one after the other
    constexpr bool kLateV = CB >= 3;
    // tid: the thread index (the task-map kernel passes it through opaque(), so
    // that the lane values below are formed per descriptor, not held across its
    // claim loop)
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int L = a.L;

    // columns of this lane: block position p0 + 2 cb + r / 8, head r % 8
    const int p0 = w * kPosWave;
    int pos[CB], lim[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        pos[cb] = p0 + 2 * cb + (r >> 3);
        lim[cb] = pos[cb] < a.live ? clampi(a.off + pos[cb] + 1, 0, L) : 0;
    }
    // smallest limit over this wave's live columns (its first position): tokens
    // below it are visible to every live column
    const int lim_lo = p0 < a.live ? clampi(a.off + p0 + 1, 0, L) : 0;
    const int pw_last = min(p0 + kPosWave, a.live) - 1;   // this wave's last live position
    const int lim_wave = pw_last >= p0 ? clampi(a.off + pw_last + 1, 0, L) : 0;

#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) st.acc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m[cb] = kNegInf;
        st.l[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (t1 <= t0) return;

    // Q of every column of this lane (B operand: 8 dims per k-step), then wait
    // for it once before the ring starts
    uint4 q[CB][4];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const bool live = pos[cb] < a.live;
        const int p = live ? pos[cb] : 0;
        const uint4* qp =
            reinterpret_cast<const uint4*>(a.q0 + ((size_t)p * a.Hq + (size_t)a.h * kGroup + (r & 7)) * kHeadDim);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) q[cb][ks] = live ? qp[g + 4 * ks] : make_uint4(0, 0, 0, 0);
    }
    wait_vmcnt<0>();

    // this lane's 4 K and 4 V chunks of every tile: rows 16 w + 4 s + lane / 16,
    // chunk lane % 16, XOR-swizzled by the row inside the wave's 16.  With row =
    // 4 s + lane / 16 each swizzle is a lane part XOR an s part (K: chunk ^ row;
    // V: swz_v(4 s + g4) = swz_v(g4) ^ swz_v(4 s)); LEAN launders the three lane
    // registers at each tile, so that the compiler forms the 8 offsets there
    // rather than hoisting them out of the tile loop
    const int g4 = lane >> 4;
    const uint32_t ck0 = (uint32_t)((lane & 15) ^ g4);
    const uint32_t cv0 = (uint32_t)((lane & 15) ^ swz_v(g4));
    const uint32_t lrow0 = (uint32_t)(16 * w + g4) * (uint32_t)a.Hkv * kPfRow;
    const auto* pt = uniform_ptr<int32_t>(a.pt);
    auto issue_page = [&](int64_t page, int t, lds_char* stg) {
        if (page < 0 || page >= a.num_pages) {
            st.bad = true;
            page = 0;
        }
        const size_t pbase = ((size_t)page * kTile * a.Hkv + a.h) * kPfRow;
        const char* kb = reinterpret_cast<const char*>(a.k_cache) + pbase;
        const char* vb = reinterpret_cast<const char*>(a.v_cache) + pbase;
        const int tok0 = kTile * t + 16 * w;
        const bool full = tok0 + 16 <= L;
        uint32_t ck = ck0, cv = cv0, lr = lrow0;
        if constexpr (LEAN) __asm__ volatile("" : "+v"(ck), "+v"(cv), "+v"(lr));
        const uint32_t dead = 16u * (uint32_t)(lane & 15);   // row 0 of the page: always live
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bool live = full || tok0 + 4 * s + g4 < L;
            const uint32_t row_off = lr + (uint32_t)(4 * s) * (uint32_t)a.Hkv * kPfRow;
            const uint32_t ko = row_off + 16u * (ck ^ (uint32_t)(4 * s));
            const uint32_t vo = row_off + 16u * (cv ^ (uint32_t)swz_v(4 * s));
            dma16(kb + (live ? ko : dead), stg + w * kPfSlice + 1024 * s);
            dma16(vb + (live ? vo : dead), stg + kPfHalf + w * kPfSlice + 1024 * s);
        }
    };
    auto issue = [&](int t, lds_char* stg) { issue_page(pt[t], t, stg); };
    static_assert(kPfStages == 2, "one tile issued ahead");
    // the first tile, with its page id from the caller when it has one
    issue_page(first_page >= 0 ? (int64_t)first_page : (int64_t)pt[t0], t0, ring);

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
        if constexpr (!kLateV) {
            lds_read_tile_bf16_at<OFF>(kk[0], va[0], ka, vaddr);
            lds_read_tile_bf16_at<OFF + 16 * kPfRow>(kk[1], va[1], ka, vaddr);
        }

        // ---- S^T = K Q^T: s[cb][sub][i] is token t32 + 16 sub + 4 g + i
        f32x4 s[CB][2];
        auto s_mfmas = [&](int sub, const uint4 (&k)[4]) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                f32x4 sa = {0.f, 0.f, 0.f, 0.f};
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[0]), as_bf16x8(q[cb][0]), sa, 0, 0, 0);
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[1]), as_bf16x8(q[cb][1]), sa, 0, 0, 0);
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[2]), as_bf16x8(q[cb][2]), sa, 0, 0, 0);
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[3]), as_bf16x8(q[cb][3]), sa, 0, 0, 0);
                s[cb][sub] = sa;
            }
        };
        if constexpr (kLateV) {
            // one 16-token sub-tile of K in registers at a time
            lds_read_k16_at<OFF>(kk[0], ka);
            s_mfmas(0, kk[0]);
            __builtin_amdgcn_sched_barrier(0);
            lds_read_k16_at<OFF + 16 * kPfRow>(kk[0], ka);
            s_mfmas(1, kk[0]);
        } else {
            s_mfmas(0, kk[0]);
            s_mfmas(1, kk[1]);
        }
        // the V^T reads go out while the S MFMAs run, into the registers the
        // K operands have just left
        if constexpr (kLateV) {
            __builtin_amdgcn_sched_barrier(0);   // the S MFMAs stay above: kk is dead before va
            lds_read_vt32_at<OFF>(va, vaddr);
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
            need |= lmax[cb] > st.m[cb] + kPfSlack;
        }
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            // a score above a column's reference: new reference = max over
            // the column's 32 tokens (0 rescale for a column still fully masked)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                float mt = fmaxf(lmax[cb], __shfl_xor(lmax[cb], 16, 64));
                mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
                const float m_new = fmaxf(st.m[cb], mt);
                const float alpha = st.m[cb] == kNegInf ? 0.f : exp2_fast(st.m[cb] - m_new);
                st.l[cb] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db) st.acc[cb][db] *= alpha;
                st.m[cb] = m_new;
            }
        }

        // ---- P and O^T += V^T P^T with MFMA 16x16x32: k = the 32 tokens,
        // lane group g holding tokens 4g .. 4g + 3 of both sub-tiles, in the
        // same order in the V^T operand (two transposed reads) and in P.  P of
        // every block first (the scores die there), then the MFMAs, each V^T
        // operand shared by the blocks
        bf16x8 pb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const float mref = st.m[cb] == kNegInf ? 0.f : st.m[cb];
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = exp2_fast(fmaf(s[cb][j >> 2][j & 3], a.scale_log2, -mref));
            pb[cb] = __builtin_bit_cast(
                bf16x8, make_uint4(bf16x2_pack(p[0], p[1]), bf16x2_pack(p[2], p[3]),
                                   bf16x2_pack(p[4], p[5]), bf16x2_pack(p[6], p[7])));
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const bf16x8 vt = __builtin_bit_cast(
                bf16x8, make_uint4(__builtin_bit_cast(uint2, va[0][db]).x, __builtin_bit_cast(uint2, va[0][db]).y,
                                   __builtin_bit_cast(uint2, va[1][db]).x, __builtin_bit_cast(uint2, va[1][db]).y));
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                st.acc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb[cb], st.acc[cb][db], 0, 0, 0);
        }
        // the softmax denominator over the same bf16 P as the numerator
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            st.l[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[cb], st.l[cb], 0, 0, 0);
    };

    // tile k sits in ring stage U = (k - t0) % 2.  Every tile issues the same
    // number of loads (past the end the last tile is loaded again into a stage
    // nobody reads), so one wait count fits all
    auto tile_step = [&](auto u_c, int k) {
        constexpr int U = decltype(u_c)::value;
        wait_vmcnt<(kPfStages - 2) * kPfLoads>();                 // this wave's rows of tile k
        lds_barrier();                                          // everyone's rows; stage of k-1 free
        issue(min(k + kPfStages - 1, t1 - 1), ring + (1 - U) * kPfStageBytes);
        if (kTile * k >= lim_wave) return;                      // nothing of it is visible here
        half_step(std::integral_constant<int, U * kPfStageBytes>{}, kTile * k);
        if (kTile * k + 32 < lim_wave)
            half_step(std::integral_constant<int, U * kPfStageBytes + 32 * kPfRow>{}, kTile * k + 32);
    };
    static_assert(kPfStages == 2, "tile_step alternates two stages");
    for (int k = t0; k < t1; k += 2) {
        tile_step(std::integral_constant<int, 0>{}, k);
        if (k + 1 < t1) tile_step(std::integral_constant<int, 1>{}, k + 1);
    }
    wait_vmcnt<0>();   // no load may still target LDS when the block ends
}

template <int CB>
__global__ __launch_bounds__(kSplitThreads, 2) void prefill_kernel(PrefillArgs a) {
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
    const int pos0 = qb * kPosBlock;
    QBlock blk;
    blk.q0 = a.q + (size_t)(b * a.QL + pos0) * a.Hq * kHeadDim;
    blk.k_cache = a.k_cache;
    blk.v_cache = a.v_cache;
    blk.pt = a.page_table + (size_t)b * a.max_pages;
    blk.num_pages = a.num_pages;
    blk.Hq = a.Hq;
    blk.Hkv = a.Hkv;
    blk.h = h;
    blk.L = L;
    blk.live = max(0, min(kPosBlock, a.QL - pos0));
    blk.off = L - a.QL + pos0;                            // block position p sees tokens < off + p + 1
    blk.scale_log2 = a.scale_log2;
    const int pb_last = blk.live - 1;
    const int lim_blk = pb_last >= 0 ? clampi(blk.off + pb_last + 1, 0, L) : 0;
    const int ntiles = (lim_blk + kTile - 1) / kTile;

    QBlockState<CB> st;
    st.bad = !len_ok;
    attend_qblock<CB>(blk, ring, 0, ntiles, st, (int)threadIdx.x);

    // ---- normalise and store: lane (g, r) holds dims 16 db + 4 g .. + 3 of column r
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int p = w * kPosWave + 2 * cb + (r >> 3);
        const float lt = st.l[cb][0];
        if (p >= blk.live) continue;
        float inv = lt > 0.f ? 1.f / lt : 0.f;            // a query that sees nothing: zeros
        if (st.bad) inv = __builtin_nanf("");
        uint16_t* o = a.out + ((size_t)(b * a.QL + pos0 + p) * a.Hq + (size_t)h * kGroup + (r & 7)) * kHeadDim + 4 * g;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const f32x4 v = st.acc[cb][db] * inv;
            *reinterpret_cast<uint2*>(o + 16 * db) = make_uint2(bf16x2_pack(v[0], v[1]), bf16x2_pack(v[2], v[3]));
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill / extend on the task map.  A map built with query blocks
// (lbsa_plan_varlen) holds descriptors: one query block of one (request, KV
// head) over a range of its KV tiles, each computed by the same block loop as
// the grid kernel above.  A descriptor that covers its whole segment writes the
// bf16 output rows of its block; a cut one -- only a bin's first or last
// descriptor can be cut -- writes its partial (normalised O, natural-log LSE)
// to the slot the map gives it (2 j first, 2 j + 1 last, for bin j), and the
// workgroup that writes the last of a cut segment's chunks merges them all
// into the output rows (an arrival counter per cut segment, indexed by the bin
// of its first chunk: a bin starts at most one cut segment).
//
// Execution order on gfx950.  The bins fix where segments are cut; the
// persistent workgroups then claim the descriptors one at a time.  A
// workgroup per bin would leave the last-dispatched of the two workgroups of a
// compute unit behind (the older one wins issue arbitration), and its bin
// would end last, alone on the unit.  The P bins form 8 groups of consecutive
// bins, group x for the workgroups of XCD x (workgroups are dispatched to the
// 8 XCDs in turn), so the K/V of a group's query blocks stays in one L2; a
// workgroup claims its group's descriptors in the map's claim order (each
// request's query blocks with the most tiles first, as the grid kernel orders
// them: workgroups that claim together stream the same tiles together, and
// the last claims are short), then helps the other groups.
// ---------------------------------------------------------------------------
struct VarlenArgs {
    const uint16_t* q;           // packed [total_q][Hq][128]
    const uint16_t* k_cache;
    const uint16_t* v_cache;
    const int32_t* page_table;   // [B][max_pages]
    int32_t* counters;           // kVarlenGroups claim counters, then P arrival counters; zero at launch
    float* part_lse;             // [2 P][128]: row p * 8 + g of a slot
    float* part_o;               // [2 P][128][128]
    uint16_t* out;               // packed like q
    int64_t num_pages;
    int32_t Hq, max_pages, total_q;
    float scale_log2;
};

// Four fp32 -> four bf16 (round to nearest even) in one 8-byte store.
__device__ inline void store_bf16x4(uint16_t* p, f32x4 v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(bf16x2_pack(v[0], v[1]), bf16x2_pack(v[2], v[3]));
}

__device__ inline int varlen_extent(int L, int q, int k) {   // tiles the block's last query sees
    return (L - q + min(q, kQBlock * (k + 1)) + kTile - 1) / kTile;
}

// The claim and arrival counters of one launch start at zero (a fill kernel,
// not a memset, so the launches can be captured in a graph).
__global__ void varlen_reset_kernel(int32_t* counters, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) counters[i] = 0;
}

// Merge of the n >= 2 chunks of one cut segment into its bf16 output rows, by
// the whole workgroup: 8 rows at a time (row p * 8 + g of the block), 32
// threads x 4 dims per row, the loads of up to 8 chunks issued before the
// merge.  Chunk c sits in slot slot0 (c = 0) or 2 (bin0 + c): a cut
// segment's chunks lie in consecutive bins, each after the first starting its
// bin.  A NaN LSE (an invalid page) makes the row NaN.
constexpr int kVarlenMergeUnroll = 8;

__device__ inline void merge_cut_segment(const VarlenArgs& a, int slot0, int n, uint16_t* out_rows, int live) {
    const int tid = opaque((int)threadIdx.x), d4 = (tid & 31) * 4;
    const int bin0 = slot0 >> 1;
    for (int row = tid >> 5; row < kVarlenRows; row += kSplitThreads / 32) {
        const int p = row >> 3, gg = row & 7;
        if (p >= live) break;                           // rows are position-major: the rest are dead too
        float m = kNegInf, wsum = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        bool nan_seen = false;
        for (int c0 = 0; c0 < n; c0 += kVarlenMergeUnroll) {
            float l[kVarlenMergeUnroll];
            f32x4 x[kVarlenMergeUnroll];
#pragma unroll
            for (int i = 0; i < kVarlenMergeUnroll; ++i) {
                const int c = c0 + i;
                if (c < n) {
                    const size_t pr = (size_t)(c == 0 ? slot0 : 2 * (bin0 + c)) * kVarlenRows + row;
                    l[i] = a.part_lse[pr];
                    x[i] = *reinterpret_cast<const f32x4*>(a.part_o + pr * kHeadDim + d4);
                } else {
                    l[i] = kNegInf;
                    x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int i = 0; i < kVarlenMergeUnroll; ++i) {
                if (l[i] != l[i]) { nan_seen = true; continue; }
                if (l[i] == kNegInf) continue;
                if (l[i] > m) {
                    const float sc = exp2_fast((m - l[i]) * kLog2e);   // 0 when m = -inf
                    wsum *= sc;
                    o *= sc;
                    m = l[i];
                }
                const float wgt = exp2_fast((l[i] - m) * kLog2e);
                wsum += wgt;
                o += wgt * x[i];
            }
        }
        o *= wsum > 0.f ? 1.f / wsum : 0.f;
        if (nan_seen) {
            const float nan = __builtin_nanf("");
            o = f32x4{nan, nan, nan, nan};
        }
        store_bf16x4(out_rows + ((size_t)p * a.Hq + gg) * kHeadDim + d4, o);
    }
}

__global__ __launch_bounds__(kSplitThreads, 2) void varlen_split_kernel(const uint8_t* map, int B, int Hkv, int P,
                                                                     int nq_max, VarlenArgs a) {
    __shared__ __attribute__((aligned(16))) char ring_mem[kPfStages * kPfStageBytes];
    __shared__ int claim_lds, arrive_lds;
    lds_char* const ring = (lds_char*)ring_mem;
    constexpr int CB = 3, kPosWave = 2 * CB;
    static_assert(kWaves * kPosWave == kQBlock, "one workgroup holds one query block");
    const VarlenMapLayout ML = varlen_map_layout(B, Hkv, P, nq_max);
    const auto* hdr = uniform_ptr<int32_t>(map + ML.header);
    const auto* bdb = uniform_ptr<int32_t>(map + ML.bin_desc_begin);
    const int h_err = hdr[LBSA_HDR_ERROR], h_p = hdr[LBSA_HDR_P], h_b = hdr[LBSA_HDR_B], h_hkv = hdr[LBSA_HDR_HKV];
    const int ndesc = hdr[LBSA_HDR_NDESC], NQ = hdr[14];
    const int cap = Hkv * nq_max + P;
    if (h_err != 0 || h_p != P || h_b != B || h_hkv != Hkv || ndesc < 0 || ndesc > cap || NQ < 0 || NQ > nq_max) {
        // a map built for another shape or from invalid lengths: every output
        // row is NaN (packed rows of all heads, spread over the workgroups)
        const float nan = __builtin_nanf("");
        const size_t n4 = (size_t)a.total_q * a.Hq * (kHeadDim / 4);
        const size_t stride = (size_t)gridDim.x * kSplitThreads;
        for (size_t i = (size_t)blockIdx.x * kSplitThreads + threadIdx.x; i < n4; i += stride)
            store_bf16x4(a.out + 4 * i, f32x4{nan, nan, nan, nan});
        return;
    }
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const auto* descs = uniform_ptr<int32_t>(map + ML.desc);
    const auto* dslot = uniform_ptr<int32_t>(map + ML.desc_slot);
    const auto* order = uniform_ptr<int32_t>(map + ML.claim_order);
    const auto* qbase = uniform_ptr<int32_t>(map + ML.qbase);
    const auto* snc = uniform_ptr<int32_t>(map + ML.seg_num_chunks);
    const auto* sslot0 = uniform_ptr<int32_t>(map + ML.seg_slot0);
    int32_t* const arrive = a.counters + kVarlenGroups;
    const auto* ptab = uniform_ptr<int32_t>(a.page_table);

    // ---- claims: group gx's descriptors are [lo, hi), claim i takes order[lo + i]
    int gx = (int)(blockIdx.x % kVarlenGroups), tried = 0, lo = 0, hi = 0;
    auto group_bounds = [&]() {
        const int l = bdb[(int)((int64_t)gx * P / kVarlenGroups)];
        const int e = bdb[(int)((int64_t)(gx + 1) * P / kVarlenGroups)];
        const bool ok = 0 <= l && l <= e && e <= ndesc;              // a corrupt map: the group is skipped
        lo = ok ? l : 0;
        hi = ok ? e : 0;
    };
    // thread 0 adds to the counter; the value reaches the other waves through LDS
    auto claim_issue = [&]() { return threadIdx.x == 0 ? atomicAdd(a.counters + gx, 1) : 0; };
    // the descriptor of claim v (thread 0's), or of the next claims once this
    // group is drained; -1 when every group is
    auto claim_take = [&](int v) {
        while (true) {
            if (threadIdx.x == 0) claim_lds = v;
            lds_barrier();
            const int i = __builtin_amdgcn_readfirstlane(claim_lds);
            lds_barrier();                                              // read before thread 0 writes again
            if (i < hi - lo) {
                const int d = order[lo + i];
                return d >= lo && d < hi ? d : hi - 1 - i;    // a corrupt order: the index itself
            }
            if (++tried == kVarlenGroups) return -1;
            gx = gx + 1 == kVarlenGroups ? 0 : gx + 1;
            group_bounds();
            v = claim_issue();
        }
    };
    group_bounds();
    int d = claim_take(claim_issue());
    while (d >= 0) {
        // the next claim is in flight while this descriptor computes
        const int v_next = claim_issue();
        int x[kVarlenDescWords];
#pragma unroll
        for (int i = 0; i < kVarlenDescWords; ++i) x[i] = descs[(size_t)kVarlenDescWords * d + i];
        const int slot = dslot[d];
        const int h = x[VD_H], b = x[VD_B], k = x[VD_K], t0 = x[VD_T0], t1 = x[VD_T1];
        const int L = x[VD_L], q = x[VD_Q], qs = x[VD_QS];
        // a record this map cannot hold (corrupt map): skipped, nothing read out of bounds
        const bool rec_ok = h >= 0 && h < Hkv && b >= 0 && b < B && L >= 0 && L <= a.max_pages * kTile && q >= 1 &&
                            q <= L && k >= 0 && kQBlock * k < q && qs >= 0 && qs <= a.total_q - q && t0 >= 0 &&
                            t1 > t0 && t1 <= varlen_extent(L, q, k);
        const bool whole = rec_ok && t0 == 0 && t1 == varlen_extent(L, q, k);
        if (rec_ok && (whole || (slot >= 0 && slot < 2 * P))) {
            QBlock blk;
            blk.q0 = a.q + (size_t)(qs + kQBlock * k) * a.Hq * kHeadDim;
            blk.k_cache = a.k_cache;
            blk.v_cache = a.v_cache;
            blk.pt = a.page_table + (size_t)b * a.max_pages;
            blk.num_pages = a.num_pages;
            blk.Hq = a.Hq;
            blk.Hkv = Hkv;
            blk.h = h;
            blk.L = L;
            blk.live = min(kQBlock, q - kQBlock * k);
            blk.off = L - q + kQBlock * k;
            blk.scale_log2 = a.scale_log2;
            QBlockState<CB> st;
            st.bad = false;
            attend_qblock<CB, true>(blk, ring, t0, t1, st, opaque((int)threadIdx.x), ptab[(size_t)b * a.max_pages + t0]);
            const int el = opaque((int)threadIdx.x) & 63, er = el & 15, eg = el >> 4;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int p = w * kPosWave + 2 * cb + (er >> 3), gg = er & 7;
                if (p >= blk.live) continue;
                const float lt = st.l[cb][0];
                float inv = lt > 0.f ? 1.f / lt : 0.f;        // a query that sees none of these tokens: O = 0
                if (st.bad) inv = __builtin_nanf("");
                if (whole) {
                    uint16_t* o =
                        a.out + ((size_t)(qs + kQBlock * k + p) * a.Hq + (size_t)h * kGroup + gg) * kHeadDim + 4 * eg;
#pragma unroll
                    for (int db = 0; db < 8; ++db) store_bf16x4(o + 16 * db, st.acc[cb][db] * inv);
                } else {
                    const size_t row = (size_t)slot * kVarlenRows + p * kGroup + gg;
                    float* o = a.part_o + row * kHeadDim + 4 * eg;
#pragma unroll
                    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(o + 16 * db) = st.acc[cb][db] * inv;
                    if (eg == 0) {
                        float lse = lt > 0.f ? (st.m[cb] + __builtin_log2f(lt)) * kLn2 : kNegInf;
                        if (st.bad) lse = __builtin_nanf("");
                        a.part_lse[row] = lse;
                    }
                }
            }
            if (!whole) {
                // the segment's chunk count and first slot (s = h * NQ + its block)
                const int u = qbase[b] + k;
                const int sg = h * NQ + (u >= 0 && u < NQ ? u : 0);
                const int n = snc[sg], slot0 = sslot0[sg];
                const bool seg_ok = u >= 0 && u < NQ && n >= 2 && slot0 >= 0 && (slot0 >> 1) + n <= P;
                // every wave's partial stores are done before thread 0 counts the
                // chunk in; the acquire-release add publishes them at device scope
                // and, for the last arrival, makes the other chunks visible
                __syncthreads();
                if (threadIdx.x == 0)
                    arrive_lds = seg_ok ? __hip_atomic_fetch_add(arrive + (slot0 >> 1), 1, __ATOMIC_ACQ_REL,
                                                                 __HIP_MEMORY_SCOPE_AGENT)
                                        : -1;
                __syncthreads();
                if (seg_ok && __builtin_amdgcn_readfirstlane(arrive_lds) == n - 1) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    uint16_t* rows = a.out + ((size_t)(qs + kQBlock * k) * a.Hq + (size_t)h * kGroup) * kHeadDim;
                    merge_cut_segment(a, slot0, n, rows, blk.live);
                }
            }
        }
        d = claim_take(v_next);   // its barriers also keep the ring until every wave is done with it
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

hipError_t launch_varlen(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                         const void* map, int B, int Hq, int Hkv, int P, int64_t nq_max, int max_pages,
                         int64_t num_pages, int64_t total_q, float scale_log2, int32_t* counters, float* part_lse,
                         float* part_o, void* out, int workgroups, hipStream_t stream) {
    VarlenArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint16_t*>(k_cache);
    a.v_cache = static_cast<const uint16_t*>(v_cache);
    a.page_table = page_table;
    a.counters = counters;
    a.part_lse = part_lse;
    a.part_o = part_o;
    a.out = static_cast<uint16_t*>(out);
    a.num_pages = num_pages;
    a.Hq = Hq;
    a.max_pages = max_pages;
    a.total_q = (int32_t)total_q;
    a.scale_log2 = scale_log2;
    const uint8_t* m = static_cast<const uint8_t*>(map);
    // the counter reset stays outside the kernel timing hook, which stamps
    // the split kernel
    const int words = kVarlenGroups + P;
    const int blocks = min((words + 255) / 256, 64);
    hipLaunchKernelGGL(varlen_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, counters, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch(varlen_split_kernel, dim3((unsigned)workgroups), dim3(kSplitThreads), 0, stream, m, B, Hkv, P,
                  (int)nq_max, a);
}

hipError_t varlen_occupancy(int* blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, varlen_split_kernel, kSplitThreads, 0);
}

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
        // the widest block (most K/V reuse per LDS read) whose grid still
        // fills the device: 3 blocks per wave from two full rounds of two
        // workgroups per compute unit (with fewer, a grid of equal blocks
        // leaves the last round partly idle and 2 blocks per wave are as
        // fast), 2 from one round
        const long long bh = (long long)B * Hkv;
        cb = bh * ((QL + kWaves * 6 - 1) / (kWaves * 6)) >= 1024  ? 3
             : bh * ((QL + kWaves * 4 - 1) / (kWaves * 4)) >= 512 ? 2
                                                                  : 1;
    }
    if (cb == 3) return launch_cb<3>(a, stream);
    return cb == 2 ? launch_cb<2>(a, stream) : launch_cb<1>(a, stream);
}

}  // namespace lbsa
