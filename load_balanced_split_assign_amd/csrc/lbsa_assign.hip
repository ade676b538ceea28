// Assign kernel: builds the per-step task map on the device.
//
// Method: HPC-Ops vLLM post, section "The solution: a per-step, load-balanced
// decode scheduler", bullet "Assign" (and the SGLang post's "Scheduling around
// live KV work"): every live KV sequence is cut into 64-token tiles, tiles are
// walked head-major / batch-minor, a per-workgroup budget comes from total
// tiles / workgroups with a minimum-work floor, and bins are filled to the
// budget and then spill into the next bin.  The map is built from device-side
// lengths once per decode step and reused by every layer.
//
// Budget reading: K = min(P, max(1, floor(T/F))) active bins, the first T mod K
// bins hold ceil(T/K) tiles and the rest floor(T/K) -- fill-then-spill with
// bin sizes that differ by at most one tile.
//
// GPU formulation (one workgroup, integer only, no atomics, so the map is
// bit-reproducible).  The sequential fill-and-spill walk is equivalent to
// cutting the global tile range [0, T) at two sets of points: segment starts
// and bin starts bin_start(j) = j*q + min(j, r).  Hence
//   chunks(s) = bin_of(last tile of s) - bin_of(first tile of s) + 1,
// descriptor slots are the exclusive prefix of chunks(s) in (h, b) order, and
// each bin's descriptors are emitted by one thread walking the bin's tile range
// from its first slot.  Every step is a scan, a search or a short walk, so the
// 256 threads share the work.
#include <mutex>

#include "lbsa_internal.h"

namespace lbsa {
namespace {

// Inclusive scan of one int per lane over the 64-lane wave with DPP moves:
// shifts by 1, 2, 4 and 8 inside each 16-lane row (lanes without a source
// add 0), then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into
// rows 2 and 3.
__device__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Block-wide exclusive scan of one int per thread; returns the prefix and
// writes the block total to *total (all threads).  `red` holds one int per
// wave and must not be reused by the next scan (one barrier per scan).
__device__ int block_exclusive_scan(int v, int* red, int* total) {
    constexpr int kWaves = kAssignThreads / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int x = wave_inclusive_scan(v);
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int t = red[i];
        before += i < wave ? t : 0;
        all += t;
    }
    *total = all;
    return before + x - v;
}

// Group of bin j: the largest x with floor(x P / 8) <= j.
__device__ inline int group_of_bin(int j, int P) {
    int x = 0;
    while (x + 1 < kVarlenGroups && (int)((int64_t)(x + 1) * P / kVarlenGroups) <= j) ++x;
    return x;
}

// Claim-order sort key of a descriptor of `len` tiles in group x: groups in
// order, lengths decreasing by class (exact below 8 tiles, then four classes
// per power of two).
constexpr int kLenClasses = 64;
constexpr int kClaimKeys = kVarlenGroups * kLenClasses;
constexpr int kWaveQuarters = kAssignThreads / 64;
static_assert(kClaimKeys * kWaveQuarters == kVarlenClaimHistWords, "LDS words reserved for the claim order");
__device__ inline int claim_key(int x, int len) {
    int c = len;
    if (len >= 8) {
        const int e = 31 - __builtin_clz((unsigned)len);            // floor(log2 len) >= 3
        c = 8 + 4 * (e - 3) + ((len >> (e - 2)) & 3);              // the two bits below the leading one
    }
    c = min(max(c, 0), kLenClasses - 1);
    return x * kLenClasses + (kLenClasses - 1 - c);
}

struct Bins {
    int K, q, r;
    __device__ int start(int j) const { return j * q + min(j, r); }
    // bin holding global tile x (0 <= x < T)
    __device__ int of(int x) const {
        const int big = r * (q + 1);
        return x < big ? x / (q + 1) : r + (x - big) / q;
    }
};

// first index i in [0, n] with a[i] > x (a non-decreasing, length n + 1)
__device__ int upper_bound(const int* a, int n, int x) {
    int lo = 0, hi = n + 1;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (a[mid] > x) hi = mid; else lo = mid + 1;
    }
    return lo;
}

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(
    const int32_t* __restrict__ seqlens, int B, int Hq, int Hkv, int P, int F, int max_pages,
    uint8_t* __restrict__ map) {
    extern __shared__ int smem[];
    __shared__ int red[3][kAssignThreads / 64];
    // every kernel argument in one round trip, before anything uses one (else the
    // compiler fetches them in several dependent rounds)
    __asm__ volatile("" ::"s"(seqlens), "s"(map), "s"(B), "s"(Hq), "s"(Hkv), "s"(P), "s"(F), "s"(max_pages));
    const MapLayout L = map_layout(B, Hkv, P);
    int32_t* hdr = reinterpret_cast<int32_t*>(map + L.header);
    int32_t* bdb = reinterpret_cast<int32_t*>(map + L.bin_desc_begin);
    int4* desc = reinterpret_cast<int4*>(map + L.desc);
    int32_t* sfd_g = reinterpret_cast<int32_t*>(map + L.seg_first_desc);
    int32_t* snc_g = reinterpret_cast<int32_t*>(map + L.seg_num_chunks);
    int32_t* sl_g = reinterpret_cast<int32_t*>(map + L.seqlens);
    int4* head = reinterpret_cast<int4*>(map + L.bin_head);
    int32_t* dlen = reinterpret_cast<int32_t*>(map + L.desc_len);
    int4* long_seg = reinterpret_cast<int4*>(map + L.long_seg);

    const int S = Hkv * B;
    int* prefix = smem;            // [B + 1]  exclusive prefix of n_b
    int* sfd = smem + B + 1;       // [S + 1]  exclusive prefix of chunks(s)
    int* lens = sfd + S + 1;       // [B]      the lengths (read once from global)
    const int tid = threadIdx.x;

    // ---- tile census: n_b = ceil(L_b / 64) (one pass over the lengths, n_b
    // stashed in LDS), validation, exclusive prefix over b -------------------
    const int per = (B + kAssignThreads - 1) / kAssignThreads;
    const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
    int bad = 0, local = 0;
    for (int b = b0; b < b1; ++b) {
        const int len = seqlens[b];
        sl_g[b] = len;
        lens[b] = len;
        const bool ok = len >= 0 && (long long)len <= (long long)max_pages * kTile;
        bad |= !ok;
        const int nb = ok ? (len + kTile - 1) / kTile : 0;
        prefix[b] = nb;
        local += nb;
    }
    const int error = __syncthreads_or(bad);   // a bad length empties the map
    if (error) local = 0;
    int N;
    int run = block_exclusive_scan(local, red[0], &N);
    for (int b = b0; b < b1; ++b) {
        const int nb = error ? 0 : prefix[b];
        prefix[b] = run;
        run += nb;
    }
    if (tid == 0) prefix[B] = N;
    __syncthreads();

    // ---- budget ------------------------------------------------------------
    const int T = Hkv * N;
    Bins bins;
    bins.K = 0; bins.q = 0; bins.r = 0;
    if (T > 0) {
        bins.K = min(P, max(1, T / F));
        bins.q = T / bins.K;
        bins.r = T % bins.K;
    }

    // ---- chunks per segment s = h*B + b and their exclusive prefix ---------
    // (chunk counts are parked in sfd[] until the scan turns them into offsets)
    const int sper = (S + kAssignThreads - 1) / kAssignThreads;
    const int s0 = min(S, tid * sper), s1 = min(S, s0 + sper);
    local = 0;
    int nlong_local = 0;
    for (int s = s0; s < s1; ++s) {
        const int h = s / B, b = s - h * B;
        const int a = h * N + prefix[b];
        const int n = prefix[b + 1] - prefix[b];
        const int c = n ? bins.of(a + n - 1) - bins.of(a) + 1 : 0;
        sfd[s] = c;
        local += c;
        nlong_local += c > kCombineSegChunks;
    }
    int ndesc, nlong;
    run = block_exclusive_scan(local, red[1], &ndesc);
    // the long segments (more than kCombineSegChunks chunks) in segment order,
    // for the combine; at most max_long_segments(S + P) of them
    int lrun = block_exclusive_scan(nlong_local, red[2], &nlong);
    for (int s = s0; s < s1; ++s) {
        const int c = sfd[s];
        sfd[s] = run;
        sfd_g[s] = run;
        snc_g[s] = c;
        if (c > kCombineSegChunks) long_seg[lrun++] = make_int4(s, run, c, 0);
        run += c;
    }
    if (tid == 0) sfd[S] = ndesc;
    __syncthreads();

    // ---- bins: thread j walks bin j's tile range [bin_start(j), bin_start(j+1))
    // segment by segment and emits its descriptors, which take consecutive
    // slots from the bin's first one (the first slot of bin j counts every
    // chunk of earlier segments plus the chunks of its first segment that lie
    // in earlier bins) -------------------------------------------------------
    for (int j = tid; j <= P; j += kAssignThreads) {
        int v = ndesc;
        int4 rec0 = make_int4(0, 0, 0, 0);
        int len0 = 0, count = 0;
        if (j < bins.K) {
            int x = bins.start(j);
            const int xe = bins.start(j + 1);
            int h = x / N;
            int b = upper_bound(prefix, B, x - h * N) - 1;
            int a = h * N + prefix[b];
            v = sfd[h * B + b] + (j - bins.of(a));
            const int cap = S + P;                             // descriptor slots in the map
            for (int d = v; d < cap; ++d) {
                const int e = h * N + prefix[b + 1];          // end of segment (h, b)
                const int t1 = min(e, xe);
                const int4 dd = make_int4(h, b, x - a, t1 - a);
                desc[d] = dd;
                dlen[d] = lens[b];
                if (d == v) { rec0 = dd; len0 = lens[b]; }
                ++count;
                if (t1 >= xe) break;
                // next non-empty segment: step over a few empty requests, else search
                x = t1;
                int k = 0;
                do {
                    if (++b == B) { b = 0; ++h; }
                } while (prefix[b + 1] == prefix[b] && ++k < 4);
                if (prefix[b + 1] == prefix[b]) {
                    h = x / N;
                    b = upper_bound(prefix, B, x - h * N) - 1;
                }
                a = h * N + prefix[b];
            }
        }
        bdb[j] = v;
        if (j < P) {
            head[2 * j] = rec0;
            head[2 * j + 1] = make_int4(v, count, len0, 0);
        }
    }

    if (tid == 0) {
        hdr[0] = T;
        hdr[1] = bins.K;
        hdr[2] = bins.q;
        hdr[3] = bins.r;
        hdr[4] = ndesc;
        hdr[5] = P;
        hdr[6] = F;
        hdr[7] = B;
        hdr[8] = Hq;
        hdr[9] = Hkv;
        hdr[10] = error;
        hdr[11] = N;
        hdr[12] = max_pages;
        hdr[13] = kTile;
        hdr[14] = nlong;
        hdr[15] = 0;
    }
}

// ---------------------------------------------------------------------------
// Assign with query blocks (prefill / extend and decode rows on one map).  The
// same cut of [0, T) at segment starts and bin starts, over segments
// (h, request, query block): block u of one KV head belongs to request
// blk_req[u] and spans ntile(u) = ceil(min(L, L - q + 16 (k + 1)) / 64) tiles;
// segment s = h * NQ + u.  Besides the decode map's arrays it records, per
// segment, the partial slot of its first chunk (2 * bin, + 1 when the chunk is
// not its bin's first descriptor: only a bin's first and last descriptors can
// cut a segment, so partial slots are numbered by bin), and per query block
// its request and index, for the combine.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAssignThreads) void assign_varlen_kernel(
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ qlens, int B, int Hq, int Hkv, int P, int F,
    int max_pages, int total_q, int nq_max, uint8_t* __restrict__ map) {
    extern __shared__ int smem[];
    __shared__ int red[4][kAssignThreads / 64];
    const VarlenMapLayout L = varlen_map_layout(B, Hkv, P, nq_max);
    int32_t* hdr = reinterpret_cast<int32_t*>(map + L.header);
    int32_t* bdb = reinterpret_cast<int32_t*>(map + L.bin_desc_begin);
    int32_t* desc = reinterpret_cast<int32_t*>(map + L.desc);
    int32_t* dslot = reinterpret_cast<int32_t*>(map + L.desc_slot);
    int32_t* order = reinterpret_cast<int32_t*>(map + L.claim_order);
    int32_t* sfd_g = reinterpret_cast<int32_t*>(map + L.seg_first_desc);
    int32_t* snc_g = reinterpret_cast<int32_t*>(map + L.seg_num_chunks);
    int32_t* slot0_g = reinterpret_cast<int32_t*>(map + L.seg_slot0);
    int32_t* breq_g = reinterpret_cast<int32_t*>(map + L.blk_req);
    int32_t* bk_g = reinterpret_cast<int32_t*>(map + L.blk_k);
    int32_t* qbase_g = reinterpret_cast<int32_t*>(map + L.qbase);
    int32_t* qstart_g = reinterpret_cast<int32_t*>(map + L.qstart);
    int32_t* sl_g = reinterpret_cast<int32_t*>(map + L.seqlens);
    int32_t* ql_g = reinterpret_cast<int32_t*>(map + L.qlens);

    int* lens = smem;                  // [B]
    int* qls = lens + B;               // [B]
    int* qbase = qls + B;              // [B + 1] exclusive prefix of the query blocks per request
    int* qstart = qbase + B + 1;       // [B + 1] exclusive prefix of q_b (packed query rows)
    int* tpre = qstart + B + 1;        // [nq_max + 1] exclusive prefix of the blocks' tiles
    int* sfd = tpre + nq_max + 1;      // [Hkv * nq_max + 1] exclusive prefix of chunks(s)
    int* hist = sfd + (size_t)Hkv * nq_max + 1;        // [kClaimKeys][kWaveQuarters] claim-order histogram
    int* blkreq = hist + kClaimKeys * kWaveQuarters;   // [nq_max] request of each query block
    const int tid = threadIdx.x;

    // ---- lengths, validation, query blocks and packed rows per request -----
    const int per = (B + kAssignThreads - 1) / kAssignThreads;
    const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
    int bad = 0, nq_local = 0, q_local = 0;
    for (int b = b0; b < b1; ++b) {
        const int len = seqlens[b], q = qlens[b];
        sl_g[b] = len;
        ql_g[b] = q;
        lens[b] = len;
        qls[b] = q;
        bad |= !(len >= 0 && (long long)len <= (long long)max_pages * kTile && q >= 1 && q <= len);
        nq_local += q >= 1 ? (q + kQBlock - 1) / kQBlock : 0;
        q_local += q >= 1 ? q : 0;
    }
    int NQ, QT;
    int runb = block_exclusive_scan(nq_local, red[0], &NQ);
    int runq = block_exclusive_scan(q_local, red[1], &QT);
    // bad lengths, or query counts that disagree with the packed Q the caller sized
    const int error = __syncthreads_or(bad) || QT != total_q || NQ > nq_max;
    if (error) NQ = 0;
    for (int b = b0; b < b1; ++b) {
        const int q = qls[b];
        qbase[b] = error ? 0 : runb;
        qstart[b] = error ? 0 : runq;
        runb += q >= 1 ? (q + kQBlock - 1) / kQBlock : 0;
        runq += q >= 1 ? q : 0;
    }
    if (tid == 0) {
        qbase[B] = NQ;
        qstart[B] = error ? 0 : QT;
    }
    __syncthreads();
    for (int b = tid; b <= B; b += kAssignThreads) {
        qbase_g[b] = qbase[b];
        qstart_g[b] = qstart[b];
    }

    // ---- tiles of every query block: request by search over qbase ----------
    const int uper = (NQ + kAssignThreads - 1) / kAssignThreads;
    const int u0 = min(NQ, tid * uper), u1 = min(NQ, u0 + uper);
    int t_local = 0;
    for (int u = u0; u < u1; ++u) {
        const int b = upper_bound(qbase, B, u) - 1;
        const int k = u - qbase[b];
        breq_g[u] = b;
        blkreq[u] = b;
        bk_g[u] = k;
        const int seen = lens[b] - qls[b] + min(qls[b], kQBlock * (k + 1));
        const int nt = (seen + kTile - 1) / kTile;
        tpre[u] = nt;
        t_local += nt;
    }
    int N;
    int run = block_exclusive_scan(t_local, red[2], &N);
    for (int u = u0; u < u1; ++u) {
        const int nt = tpre[u];
        tpre[u] = run;
        run += nt;
    }
    if (tid == 0) tpre[NQ] = N;
    __syncthreads();

    // ---- budget -------------------------------------------------------------
    const int T = Hkv * N;
    Bins bins;
    bins.K = 0; bins.q = 0; bins.r = 0;
    if (T > 0) {
        bins.K = min(P, max(1, T / F));
        bins.q = T / bins.K;
        bins.r = T % bins.K;
    }

    // ---- chunks per segment s = h * NQ + u and their prefix ------------------
    // (counts in LDS with interleaved segments, then a scan over contiguous
    // ranges of them)
    const int S = Hkv * NQ;
    for (int s = tid; s < S; s += kAssignThreads) {
        const int h = s / NQ, u = s - h * NQ;
        const int a = h * N + tpre[u], n = tpre[u + 1] - tpre[u];
        sfd[s] = n ? bins.of(a + n - 1) - bins.of(a) + 1 : 0;
    }
    __syncthreads();
    const int sper = (S + kAssignThreads - 1) / kAssignThreads;
    const int s0 = min(S, tid * sper), s1 = min(S, s0 + sper);
    int c_local = 0;
    for (int s = s0; s < s1; ++s) c_local += sfd[s];
    int ndesc;
    run = block_exclusive_scan(c_local, red[3], &ndesc);
    for (int s = s0; s < s1; ++s) {
        const int c = sfd[s];
        sfd[s] = run;
        run += c;
    }
    if (tid == 0) sfd[S] = ndesc;
    // claim-order histogram: per sort key and per wave's quarter of the
    // descriptors (the quarters in decreasing index order: wave 0 the highest)
    for (int i = tid; i < kClaimKeys * kWaveQuarters; i += kAssignThreads) hist[i] = 0;
    const int quarter = (ndesc + kWaveQuarters - 1) / kWaveQuarters;
    __syncthreads();

    // ---- descriptors, segment by segment: chunk c of segment s is descriptor
    // sfd[s] + c, its part of bin bins.of(a) + c (the same numbering as a walk
    // of every bin in order).  Neighbouring threads take neighbouring
    // segments, so the records of one-chunk segments are written together.
    // The chunk that starts at its bin's first tile is the bin's first
    // descriptor: exactly one per bin below K. ----------------------------------
    for (int s = tid; s < S; s += kAssignThreads) {
        const int h = s / NQ, u = s - h * NQ;
        const int a = h * N + tpre[u], n = tpre[u + 1] - tpre[u];
        const int d0 = sfd[s], nc = sfd[s + 1] - d0;
        const int j0 = n ? bins.of(a) : 0;
        sfd_g[s] = d0;
        snc_g[s] = nc;
        slot0_g[s] = 2 * j0 + (n && a != bins.start(j0) ? 1 : 0);
        const int b = blkreq[u];
        const int k = u - qbase[b], L = lens[b], q = qls[b], qs = qstart[b];
        for (int c = 0; c < nc; ++c) {
            const int j = j0 + c, d = d0 + c;
            const int bs = bins.start(j);
            const int ts = max(a, bs), te = min(a + n, bins.start(j + 1));
            int32_t* rec = desc + (size_t)kVarlenDescWords * d;
            *reinterpret_cast<int4*>(rec) = make_int4(h, b, k, ts - a);
            *reinterpret_cast<int4*>(rec + 4) = make_int4(te - a, L, q, qs);
            dslot[d] = 2 * j + (ts != bs ? 1 : 0);
            if (ts == bs) bdb[j] = d;
            atomicAdd(&hist[claim_key(group_of_bin(j, P), te - ts) * kWaveQuarters + (ndesc - 1 - d) / quarter], 1);
        }
    }
    for (int j = bins.K + tid; j <= P; j += kAssignThreads) bdb[j] = ndesc;
    __syncthreads();   // records and bin starts written by this workgroup

    // ---- claim order: in each group of bins, the descriptors by decreasing
    // length class (claim_key), equal classes by decreasing index.  The walk
    // counted them per (key, quarter); the exclusive scan in (key, quarter)
    // order gives each wave the first position of every key in its quarter (the
    // groups are consecutive descriptor ranges from 0, so positions are claim
    // positions); then wave w places its quarter, highest index first, 64 at a
    // time, ranking equal keys by lane.
    {
        constexpr int per_t = kClaimKeys * kWaveQuarters / kAssignThreads;
        static_assert((kClaimKeys * kWaveQuarters) % kAssignThreads == 0, "entries split evenly over the threads");
        int sum = 0;
        for (int i = 0; i < per_t; ++i) sum += hist[tid * per_t + i];
        int total;
        int pre = block_exclusive_scan(sum, red[0], &total);
        for (int i = 0; i < per_t; ++i) {
            const int c = hist[tid * per_t + i];
            hist[tid * per_t + i] = pre;
            pre += c;
        }
    }
    __syncthreads();
    {
        const int lane = tid & 63, wv = tid >> 6;
        const uint64_t lt_mask = (1ull << lane) - 1;
        const int top = ndesc - 1 - wv * quarter, bottom = max(ndesc - (wv + 1) * quarter, 0);
        // the next 64 descriptors' tile range and slot are loaded while these are placed
        int n_t0 = 0, n_t1 = 0, n_slot = 0;
        auto fetch = [&](int c) {
            const int dd = c - lane;
            if (dd >= bottom) {
                const int32_t* rec = desc + (size_t)kVarlenDescWords * dd;
                n_t0 = rec[VD_T0];
                n_t1 = rec[VD_T1];
                n_slot = dslot[dd];
            }
        };
        fetch(top);
        for (int c0 = top; c0 >= bottom; c0 -= 64) {
            const int t0v = n_t0, t1v = n_t1, slv = n_slot;
            fetch(c0 - 64);
            const int d = c0 - lane;
            const bool valid = d >= bottom;
            const int key = valid ? claim_key(group_of_bin(slv >> 1, P), t1v - t0v) : -1;
            int rank = 0, count = 0;
            uint64_t pending = __builtin_amdgcn_ballot_w64(valid);
            while (pending) {
                const int leader = __builtin_ctzll(pending);
                const int lk = __builtin_amdgcn_readlane(key, leader);
                const uint64_t m = __builtin_amdgcn_ballot_w64(valid && key == lk);
                if (valid && key == lk) {
                    rank = __builtin_popcountll(m & lt_mask);
                    count = __builtin_popcountll(m);
                }
                pending &= ~m;
            }
            if (valid) {
                int* slot = &hist[key * kWaveQuarters + wv];
                const int base = *slot;
                order[base + rank] = d;
                if (rank == count - 1) *slot = base + count;   // the key's last lane moves it on
            }
        }
    }

    if (tid == 0) {
        hdr[0] = T;
        hdr[1] = bins.K;
        hdr[2] = bins.q;
        hdr[3] = bins.r;
        hdr[4] = ndesc;
        hdr[5] = P;
        hdr[6] = F;
        hdr[7] = B;
        hdr[8] = Hq;
        hdr[9] = Hkv;
        hdr[10] = error;
        hdr[11] = N;
        hdr[12] = max_pages;
        hdr[13] = kTile;
        hdr[14] = NQ;
        hdr[15] = kQBlock;
    }
}

}  // namespace

hipError_t launch_assign_varlen(const int32_t* seqlens, const int32_t* qlens, int B, int Hq, int Hkv, int P, int F,
                                int max_pages, int64_t total_q, int64_t nq_max, void* map, hipStream_t stream) {
    const size_t lds = sizeof(int) * varlen_assign_lds_words(B, Hkv, nq_max);
    // the prefixes and the histogram take up to 152 KiB: allow the kernel
    // gfx950's larger LDS once per process
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&assign_varlen_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)(sizeof(int) * (size_t)kMaxVarlenAssignLdsWords));
    });
    if (attr != hipSuccess) return attr;
    return launch(assign_varlen_kernel, dim3(1), dim3(kAssignThreads), (uint32_t)lds, stream, seqlens, qlens, B, Hq,
                  Hkv, P, F, max_pages, (int)total_q, (int)nq_max, static_cast<uint8_t*>(map));
}

hipError_t launch_assign(const int32_t* seqlens, int B, int Hq, int Hkv, int P, int F,
                         int max_pages, void* map, hipStream_t stream) {
    const size_t lds = sizeof(int) * (2 * (size_t)B + 1 + (size_t)Hkv * B + 1);
    return launch(assign_kernel, dim3(1), dim3(kAssignThreads), (uint32_t)lds, stream, seqlens, B, Hq, Hkv, P, F,
                  max_pages, static_cast<uint8_t*>(map));
}

}  // namespace lbsa
