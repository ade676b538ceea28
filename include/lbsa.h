/*
 * lbsa.h -- C ABI of the MI355X (gfx950) load-balanced paged decode attention
 * library (liblbsa.so).
 *
 * The method (HPC-Ops attention backend, described in the HPC-Ops vLLM
 * integration post, section "The solution: a per-step, load-balanced decode
 * scheduler", and in the SGLang post, section "Scheduling around live KV
 * work"):
 *   1. an assign kernel slices every live KV sequence into 64-token tiles,
 *      walks them head-major / batch-minor, and fills persistent-workgroup
 *      bins up to a budget (total tiles / workgroups, with a minimum-work
 *      floor), spilling into the next bin -- the task map, built once per
 *      decode step from device-side lengths and reused by every layer;
 *   2. a persistent split kernel: each workgroup drains its bin, computing
 *      attention over each descriptor's consecutive tiles and writing a
 *      partial output with its log-sum-exp;
 *   3. a combine kernel reads the chunk count of each (request, head) and
 *      merges the partials under the global softmax normalisation into bf16.
 * A static split-KV kernel (fixed split count per request; the posts' "static
 * split-KV" comparison point, section "The challenge: mixed-length decode in
 * every batch") is exported as the scheduling baseline.
 *
 * Conventions for every entry point:
 *   - all pointers named *_d are DEVICE pointers allocated by the caller; the
 *     library never allocates, frees or synchronises; work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream) and returns at once;
 *   - argument errors are detected on the host BEFORE anything is enqueued and
 *     reported as a negative status; nothing is written in that case;
 *   - data errors only visible on the device (a length outside
 *     [0, max_pages_per_seq * 64]) are reported in the task-map header word
 *     LBSA_HDR_ERROR and give an empty map, and a decode with that map writes
 *     NaN in every output row; a page-table entry outside [0, num_pages)
 *     poisons the affected rows with NaN instead of reading out of bounds;
 *   - supported shapes: head_dim 128, page_size 64, query-group size
 *     num_heads / num_kv_heads = 8, q_len 1 or 2 query tokens per request.
 *
 * Multi-token decode (q_len = 2: verifying the draft token of Hy3's MTP
 * speculative layer, vLLM post, the Hy3 model paragraph): the q_len new
 * tokens of a request are the last q_len of its L cached tokens, and query i
 * (0-based) attends to tokens [0, L - q_len + i] -- causal among the new
 * tokens; a query that sees no token (L < q_len) gives a zero row.  The task
 * map does not depend on q_len (tiles count KV tokens).
 *
 * Tensor layouts (row-major, contiguous):
 *   q           [batch][q_len][num_heads][128]   bf16, or e4m3fn with q_scale
 *   q_scale     [batch][q_len][num_heads]        fp32 (fp8 only)
 *   k/v cache   [num_pages][64][num_kv_heads][128] bf16 or e4m3fn (token-major)
 *   k/v scale   [num_pages][num_kv_heads][64]    fp32 (fp8 only)
 *   page_table  [batch][max_pages_per_seq]       int32 physical page ids
 *   seqlens     [batch]                          int32 live KV lengths
 *   out         [batch][q_len][num_heads][128]   bf16
 * Query head hq reads KV head hq / (num_heads / num_kv_heads).
 */
#ifndef LBSA_H
#define LBSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define LBSA_OK 0
#define LBSA_ERR_INVALID_ARGUMENT (-1) /* null pointer, size <= 0, buffer too small, Hq % Hkv != 0 */
#define LBSA_ERR_UNSUPPORTED (-2)      /* head_dim != 128, page_size != 64, group != 8, q_len > 2, too large */
#define LBSA_ERR_HIP (-3)              /* a HIP runtime call or launch failed */

/* ---- constants ---------------------------------------------------------- */
#define LBSA_KV_BF16 0
#define LBSA_KV_FP8_E4M3 1       /* OCP E4M3FN codes with fp32 per-token-per-head scales */
#define LBSA_PAGE_SIZE 64        /* tokens per page = tokens per tile */
#define LBSA_HEAD_DIM 128
#define LBSA_GROUP 8             /* query heads per KV head */
#define LBSA_DEFAULT_MIN_TILES 2 /* default minimum-work floor, tiles per active bin */
#define LBSA_MAX_Q_LEN 2         /* query tokens per request the decode entry points take */

/* Task-map header words (int32), see lbsa_plan. */
#define LBSA_HDR_T 0        /* total tiles over all (kv_head, request) segments */
#define LBSA_HDR_K 1        /* active bins = min(P, max(1, floor(T / F))), 0 if T = 0 */
#define LBSA_HDR_Q 2        /* floor(T / K) */
#define LBSA_HDR_R 3        /* T mod K: bins [0, R) hold Q + 1 tiles, the rest Q */
#define LBSA_HDR_NDESC 4    /* descriptors in the map */
#define LBSA_HDR_P 5        /* bins = persistent workgroups of the split kernel */
#define LBSA_HDR_F 6        /* minimum-work floor (tiles) */
#define LBSA_HDR_B 7
#define LBSA_HDR_HQ 8
#define LBSA_HDR_HKV 9
#define LBSA_HDR_ERROR 10   /* 0 ok; 1 = a length outside [0, max_pages * 64] (map empty) */
#define LBSA_HDR_N 11       /* tiles per KV head = sum_b ceil(L_b / 64) */
#define LBSA_HDR_MAX_PAGES 12
#define LBSA_HDR_PAGE_SIZE 13
#define LBSA_HDR_NLONG 14   /* segments of more than 8 chunks, listed in long_seg */
#define LBSA_HDR_WORDS 16

/* Byte offsets of the arrays inside a task map (all from the map base). */
typedef struct {
    size_t header;          /* int32[16] */
    size_t bin_desc_begin;  /* int32[P + 1]: bin j owns descriptors [begin[j], begin[j+1]) */
    size_t desc;            /* int32x4[Hkv*B + P]: (kv_head, request, tile_begin, tile_end),
                               request-local tile indices; descriptor d writes partial slot d */
    size_t seg_first_desc;  /* int32[Hkv*B], index h*B + b: first descriptor of the segment */
    size_t seg_num_chunks;  /* int32[Hkv*B]: descriptors (chunks) of the segment */
    size_t seqlens;         /* int32[B]: copy of the lengths the map was built from */
    size_t bin_head;        /* int32[P][8], 32-byte records: (kv_head, request, tile_begin,
                               tile_end) of bin j's first descriptor, that descriptor's index,
                               the bin's descriptor count, the request's length, 0; all zero
                               but the index (= Ndesc) for a bin without descriptors */
    size_t desc_len;        /* int32[Hkv*B + P]: length of descriptor d's request */
    size_t long_seg;        /* int32x4[(Hkv*B + P) / 9]: (h*B + b, first descriptor, chunks, 0)
                               of each segment with more than 8 chunks, in segment order;
                               the first header[LBSA_HDR_NLONG] records are valid.  The
                               combine merges such a segment one output row per workgroup,
                               a shorter one whole in one workgroup. */
    size_t total;           /* bytes */
} lbsa_task_map_layout;

/* Byte offsets inside the decode workspace (row 8 * query + head of the group). */
typedef struct {
    size_t part_lse;        /* fp32 [Hkv*B + P][q_len * 8]: natural-log LSE of each partial */
    size_t part_o;          /* fp32 [Hkv*B + P][q_len * 8][128]: normalised partial outputs */
    size_t total;
} lbsa_workspace_layout;

/* Human-readable name of a status code (static storage). */
const char* lbsa_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int lbsa_version(void);

/* Kernel timing hook.  Arms caller-owned HIP events (hipEvent_t, created with
 * timing enabled) for the next kernels that this host thread launches through
 * the library: such a launch goes through hipExtLaunchKernel, which records its
 * start event when the kernel begins and its stop event when it ends, so
 * hipEventElapsedTime(start, stop) is the kernel's own duration, without the
 * dispatch gap that a marker recorded between launches adds.
 *   lbsa_time_next_kernels: the next n launches (0 <= n <= 8) stamp
 *     (start_events[i], stop_events[i]) in launch order; an entry point that
 *     launches several kernels (lbsa_decode: split, then combine) uses one pair
 *     per kernel.  n = 0 disarms.  Either event of a pair may be NULL.
 *   lbsa_time_next_kernel: the same for one launch; NULL, NULL disarms.
 * Arming replaces whatever was armed before.  Pairs left over stay armed for
 * the following launches, except that an entry point which returns without
 * launching anything (an argument it rejected, nothing to do) disarms the hook,
 * so no event is ever stamped by an unrelated later launch.  The library never
 * creates, waits on or destroys the events.  Thread-local; returns LBSA_OK, or
 * LBSA_ERR_INVALID_ARGUMENT for n outside [0, 8] or NULL arrays with n > 0. */
int lbsa_time_next_kernels(int32_t n, void* const* start_events, void* const* stop_events);
int lbsa_time_next_kernel(void* start_event, void* stop_event);

/* Default number of persistent workgroups on `device` for `kv_dtype` and
 * q_len (1 or 2): compute units x resident workgroups per CU of that split
 * kernel (occupancy query), so every bin is resident at once.  On MI355X the
 * fp8 kernels hold two workgroups per CU (P = 512), the bf16 ones one
 * (P = 256); a task map planned for one P serves either q_len, and a larger
 * P than resident runs in waves of workgroups.  Writes *out_P. */
int lbsa_default_workgroups(int device, int32_t kv_dtype, int32_t q_len, int32_t* out_P);

/* Number of bins (P) for a batch of total_tiles = sum over KV heads and
 * requests of ceil(L / 64), known to a serving engine on the host: twice the
 * resident workgroups when num_kv_heads > 1 and there are at least 32 tiles
 * per resident workgroup, else lbsa_default_workgroups.  The second wave of
 * bins goes to the workgroups that finish first.  On MI355X equal bins do not
 * finish together when several KV heads share the batch: a bin's speed
 * depends on which KV head it streams (measured: 179-241 us across the 8
 * heads of a 64-request fp8 batch, 92-111 us on the skewed bf16 batch), and
 * with two waves those batches ran 4-6% faster; with one KV head, or a few
 * tiles per workgroup, the extra bins' start-up cost more than they
 * balanced.  Writes *out_P. */
int lbsa_auto_workgroups(int device, int32_t kv_dtype, int32_t q_len, int32_t num_kv_heads, int64_t total_tiles,
                         int32_t* out_P);

/* Layout and size of the task map for (batch, num_kv_heads, P). */
int lbsa_task_map_layout_get(int32_t batch, int32_t num_kv_heads, int32_t P,
                             lbsa_task_map_layout* out);
int lbsa_task_map_bytes(int32_t batch, int32_t num_kv_heads, int32_t P, size_t* out_bytes);

/* Layout and size of the split/combine workspace (partials). */
int lbsa_workspace_layout_get(int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t P, lbsa_workspace_layout* out);
int lbsa_workspace_bytes(int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t P, size_t* out_bytes);

/*
 * Assign: build the task map on the device (one launch, no host sync).
 * Source: vLLM post, "The solution: ..." bullet "Assign"; SGLang post,
 * "Scheduling around live KV work".
 *   seqlens_d          int32[batch] live KV lengths (device)
 *   num_workgroups     P >= 1, the split kernel's grid (see lbsa_default_workgroups)
 *   min_tiles_per_bin  F >= 1, or 0 for LBSA_DEFAULT_MIN_TILES
 *   task_map_d         caller buffer of >= lbsa_task_map_bytes bytes, 16-byte aligned
 * Bins: T = Hkv * sum_b ceil(L_b/64) tiles in head-major, batch-minor order;
 * K = min(P, max(1, floor(T/F))) active bins; the first T mod K bins hold
 * ceil(T/K) tiles, the rest floor(T/K); each maximal run of one (kv_head,
 * request) inside a bin is one descriptor.  Limits: (2*batch + Hkv*batch) <= 16382
 * (LDS of the single assign workgroup), batch * max_pages_per_seq * Hkv < 2^30.
 */
int lbsa_plan(const int32_t* seqlens_d, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
              int32_t page_size, int32_t max_pages_per_seq, int32_t num_workgroups,
              int32_t min_tiles_per_bin, void* task_map_d, size_t task_map_bytes, void* stream);

/*
 * Decode = split + combine with a task map from lbsa_plan (same batch,
 * num_heads, num_kv_heads and P).  Source: vLLM post, bullet "Compute and
 * combine"; SGLang post, "Scheduling around live KV work".
 *   q_len                     query tokens per request, 1 or 2 (multi-token decode)
 *   q_d, q_scale_d            query (bf16, or e4m3 codes + fp32 scales for fp8)
 *   k_cache_d, v_cache_d      paged caches, kv_dtype LBSA_KV_BF16 or LBSA_KV_FP8_E4M3
 *   k_scale_d, v_scale_d      fp32 scales (fp8 only, else NULL)
 *   page_table_d              int32 [batch][max_pages_per_seq]
 *   num_pages                 pages in each cache (page ids are checked against it)
 *   softmax_scale             multiplier of q.k (e.g. 1/sqrt(128))
 *   workspace_d               >= lbsa_workspace_bytes bytes, 256-byte aligned
 *   out_d                     bf16 [batch][q_len][num_heads][128]
 * The q/k/v/out dtypes follow kv_dtype: bf16 path = bf16 q, bf16 caches; fp8
 * path = e4m3 q with q_scale, e4m3 caches with k/v scales.  Output is bf16
 * (round to nearest even) in both.  A (kv_head, request) segment served by a
 * single descriptor needs no merge: the split kernel writes its output rows
 * itself and the combine leaves them alone, so lbsa_decode writes no partial
 * for such a segment (lbsa_decode_split, which has no output, writes them all).
 */
int lbsa_decode(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                const void* v_cache_d, const float* k_scale_d, const float* v_scale_d,
                int32_t kv_dtype, const int32_t* page_table_d, int32_t batch, int32_t q_len, int32_t num_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                int32_t max_pages_per_seq, int64_t num_pages, int32_t num_workgroups,
                float softmax_scale, const void* task_map_d, size_t task_map_bytes,
                void* workspace_d, size_t workspace_bytes, void* out_d, void* stream);

/*
 * lbsa_decode with no workspace argument, for callers that cannot allocate
 * device memory themselves (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split and combine kernels are
 * lbsa_decode's; their partials live in a static device array of
 * LBSA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates and frees nothing.
 *   Arguments: those of lbsa_decode minus workspace_d / workspace_bytes; the
 *   caller still owns q, the caches, the page table, the task map and out_d.
 *   Limit: lbsa_workspace_bytes(batch, q_len, num_heads, num_kv_heads, 128, P)
 *   must not exceed LBSA_NOALLOC_SCRATCH_BYTES, else LBSA_ERR_UNSUPPORTED and
 *   nothing is enqueued (16 MiB: e.g. batch 64 x 8 KV heads with P = 1024 at
 *   q_len 2).
 *   The array is shared by every call on one GPU and keeps the last call's
 *   partials: calls that overlap in time on one GPU (two streams, or two host
 *   threads) race on it and must be serialised by the caller.  Nothing in it
 *   needs to start at zero (every partial a call reads, it wrote first).
 * The first call on a device looks the array's device address up
 * (hipGetSymbolAddress); LBSA_ERR_HIP if that fails.
 */
#define LBSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int lbsa_decode_noalloc(const void* q_d, const float* q_scale_d, const void* k_cache_d, const void* v_cache_d,
                        const float* k_scale_d, const float* v_scale_d, int32_t kv_dtype,
                        const int32_t* page_table_d, int32_t batch, int32_t q_len, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t max_pages_per_seq,
                        int64_t num_pages, int32_t num_workgroups, float softmax_scale, const void* task_map_d,
                        size_t task_map_bytes, void* out_d, void* stream);

/* The split half of lbsa_decode alone: fills the workspace partials of every
 * descriptor (slot d = descriptor d), single-chunk segments included.  Same
 * arguments as lbsa_decode without out_d. */
int lbsa_decode_split(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                      const void* v_cache_d, const float* k_scale_d, const float* v_scale_d,
                      int32_t kv_dtype, const int32_t* page_table_d, int32_t batch, int32_t q_len,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t max_pages_per_seq, int64_t num_pages, int32_t num_workgroups,
                      float softmax_scale, const void* task_map_d, size_t task_map_bytes,
                      void* workspace_d, size_t workspace_bytes, void* stream);

/* The combine half of lbsa_decode alone: merges the workspace partials of each
 * (request, query token, query head) into out_d (bf16). */
int lbsa_decode_combine(int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t num_workgroups, const void* task_map_d, size_t task_map_bytes,
                        const void* workspace_d, size_t workspace_bytes, void* out_d,
                        void* stream);

/* Workspace bytes of the static baseline: batch * Hkv * num_splits partials. */
int lbsa_static_workspace_bytes(int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t num_splits, size_t* out_bytes);

/*
 * Static split-KV baseline (no task map): a grid of num_splits x batch x Hkv
 * workgroups; split s of request b covers tiles [floor(s*n_b/S), floor((s+1)*n_b/S))
 * of every KV head, followed by a fixed-S combine.  This is the "fixed number
 * of splits" static policy of the vLLM post, section "The challenge:
 * mixed-length decode in every batch".  Same tensors as lbsa_decode plus the
 * device lengths; workspace >= lbsa_static_workspace_bytes.
 */
int lbsa_decode_static(const void* q_d, const float* q_scale_d, const void* k_cache_d,
                       const void* v_cache_d, const float* k_scale_d, const float* v_scale_d,
                       int32_t kv_dtype, const int32_t* page_table_d, const int32_t* seqlens_d,
                       int32_t batch, int32_t q_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t page_size, int32_t max_pages_per_seq, int64_t num_pages,
                       int32_t num_splits, float softmax_scale, void* workspace_d,
                       size_t workspace_bytes, void* out_d, void* stream);

/*
 * Prefill / extend attention over the paged cache (vLLM post, Table 4:
 * prefill and extend shapes of the same backend).  The q_len new tokens of each
 * request are the last q_len of its seqlens[b] cached tokens (already written,
 * e.g. by lbsa_prologue); query i attends to tokens [0, seqlens[b] - q_len + i]
 * (causal), the same rule as multi-token decode.
 *   q_d            bf16 [batch][q_len][num_heads][128]
 *   k/v_cache_d    bf16 [num_pages][64][num_kv_heads][128]; kv_dtype must be
 *                  LBSA_KV_BF16 (LBSA_ERR_UNSUPPORTED for fp8)
 *   page_table_d   int32 [batch][max_pages_per_seq]; seqlens_d int32 [batch]
 *   out_d          bf16 [batch][q_len][num_heads][128]; a query that sees no
 *                  token (seqlens[b] < q_len) gives a zero row; a length outside
 *                  [0, max_pages_per_seq * 64] gives NaN rows for that request;
 *                  a page id outside [0, num_pages) is never dereferenced and
 *                  gives NaN rows for the queries that see that page
 * One launch, no workspace, no task map: every workgroup owns one (request,
 * KV head, block of query positions) and streams that KV head's pages itself;
 * the grid starts with the blocks that see the most tiles.  Alignment: q_d and
 * the caches 16 B, out_d 8 B, the int32 arrays 4 B (else
 * LBSA_ERR_INVALID_ARGUMENT, as for softmax_scale <= 0 or not finite).
 * q_len >= 1, any size; head_dim 128, page 64, group 8 as for decode.
 */
int lbsa_prefill(const void* q_d, const void* k_cache_d, const void* v_cache_d, int32_t kv_dtype,
                 const int32_t* page_table_d, const int32_t* seqlens_d, int32_t batch, int32_t q_len,
                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                 int32_t max_pages_per_seq, int64_t num_pages, float softmax_scale, void* out_d,
                 void* stream);

/*
 * Prefill, extend and decode rows on one task map (vLLM post, Table 4: one
 * backend over prefill, extend and decode shapes; the map of the section "The
 * solution: a per-step, load-balanced decode scheduler", bullet "Assign",
 * with a query-tile dimension).  Request b brings qlens[b] >= 1 new tokens,
 * the last qlens[b] of its seqlens[b] cached ones (1 for a decode row,
 * seqlens[b] for a prefill); query i attends to tokens [0, seqlens[b] -
 * qlens[b] + i].  Its queries form blocks of LBSA_QBLOCK positions, and a
 * segment is (KV head, request, query block) spanning the 64-token tiles its
 * last query sees: ceil(min(L, L - q + 16 (k + 1)) / 64) for block k.
 * Segments are walked head-major, batch-minor, query block innermost, and
 * binned with the decode budget, fill and spill (lbsa_plan).
 *   total_q        sum of qlens (host-side: the rows of the packed q and out);
 *                  the map and the launches are sized by it, and lbsa_plan_varlen
 *                  sets the error word when the device lengths disagree with it
 *   q_d / out_d    bf16 [total_q][num_heads][128], request b's queries at rows
 *                  [sum_{b' < b} qlens[b'], + qlens[b]) (packed, request order)
 *   map            lbsa_varlen_task_map_bytes(batch, num_kv_heads, P, total_q)
 *                  bytes: header (words as lbsa_plan's, plus 14 = query blocks
 *                  per KV head NQ, 15 = LBSA_QBLOCK), bin CSR, 32-byte
 *                  descriptors (kv_head, request, block, tile_begin, tile_end,
 *                  L, q, first packed row), per descriptor its partial slot,
 *                  the claim order (per group of bins, requests in walk order,
 *                  each from its last descriptor back), per segment
 *                  s = h * NQ + block (of all requests in order)
 *                  its first descriptor, chunk count and first partial slot,
 *                  per block its request and index, the prefixes of blocks and
 *                  of qlens, and the two length copies
 *                  (lbsa_varlen_task_map_layout_get)
 *   workspace      lbsa_varlen_workspace_bytes(num_heads, num_kv_heads, 128, P):
 *                  int32 counters (8 claim, then P arrival; cleared by every
 *                  call), padded to 256 bytes, then 2 P partial slots of
 *                  16 x 8 rows (position x head), fp32 LSE [2 P][128] then O
 *                  [2 P][128][128]; only a bin's first and last descriptors can
 *                  cut a segment, so slot 2 j + (0 first, 1 last)
 * lbsa_attend_varlen is two launches on the stream: a small kernel clears the
 * counters; persistent workgroups (as many as stay resident) claim the
 * descriptors of 8 groups of consecutive bins, one group per XCD, in the
 * map's claim order, and compute each descriptor's query block over its tiles
 * (MFMA, K/V through LDS), writing the bf16 rows of a segment it holds whole
 * and a partial otherwise; the workgroup that writes a cut segment's last
 * chunk merges its chunks into the output rows.  Calls that share a workspace
 * must not overlap.  The first lbsa_plan_varlen call in a process sets the assign
 * kernel's dynamic-LDS limit (a kernel attribute): make it before capturing the
 * calls in a graph.
 * Errors: shapes as lbsa_plan and lbsa_prefill (bf16 only); maps larger than
 * one assign workgroup's LDS give LBSA_ERR_UNSUPPORTED: 4 B + 10 NQ words over
 * 36 864 with 8 KV heads (NQ = batch + total_q / 24), about 88K query tokens.
 * A length or q out of range on the device sets the error word: every output
 * row is then NaN.  P (bins): lbsa_varlen_auto_workgroups, or
 * lbsa_varlen_default_workgroups (one bin per resident workgroup).
 */
#define LBSA_QBLOCK 24   /* 4 waves x 3 MFMA column blocks of 2 positions (x 8 heads) */
typedef struct {
    size_t header, bin_desc_begin, desc, desc_slot, claim_order, seg_first_desc, seg_num_chunks, seg_slot0,
        blk_req, blk_k, qbase, qstart, seqlens, qlens, total;
} lbsa_varlen_task_map_layout;
int lbsa_varlen_task_map_layout_get(int32_t batch, int32_t num_kv_heads, int32_t P, int64_t total_q,
                                    lbsa_varlen_task_map_layout* out);
int lbsa_varlen_task_map_bytes(int32_t batch, int32_t num_kv_heads, int32_t P, int64_t total_q, size_t* out_bytes);
int lbsa_varlen_workspace_bytes(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t P,
                                size_t* out_bytes);
int lbsa_varlen_default_workgroups(int device, int32_t* out_P);
/* P (bins) for a prefill / extend map from the host's copy of the q counts
 * (qlens_host: int32[batch], HOST memory): a quarter of the resident count when
 * the batch has at least 4 segments (Hkv x query blocks) per resident workgroup,
 * else the resident count.  The split kernel's workgroups claim descriptors, so
 * with many segments fewer bins only cut fewer of them: on MI355X the 8K extend
 * beside 63 decode rows and a q8k prefill took 2-4% less at a quarter of the
 * bins.  Errors: LBSA_ERR_INVALID_ARGUMENT for a NULL pointer or batch,
 * num_kv_heads < 1; LBSA_ERR_HIP when the device cannot be queried. */
int lbsa_varlen_auto_workgroups(int device, const int32_t* qlens_host, int32_t batch, int32_t num_kv_heads,
                                int32_t* out_P);
int lbsa_plan_varlen(const int32_t* seqlens_d, const int32_t* qlens_d, int32_t batch, int32_t num_heads,
                     int32_t num_kv_heads, int32_t page_size, int32_t max_pages_per_seq, int64_t total_q,
                     int32_t num_workgroups, int32_t min_tiles_per_bin, void* task_map_d, size_t task_map_bytes,
                     void* stream);
int lbsa_attend_varlen(const void* q_d, const void* k_cache_d, const void* v_cache_d, const int32_t* page_table_d,
                       int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t max_pages_per_seq, int64_t num_pages, int64_t total_q, int32_t num_workgroups,
                       float softmax_scale, const void* task_map_d, size_t task_map_bytes, void* workspace_d,
                       size_t workspace_bytes, void* out_d, void* stream);

/*
 * Split-bf16 router GEMM (SGLang post, section "Router GEMM: balancing routing
 * precision and throughput"): router scores from bf16 hidden states and fp32
 * router weights, run on bf16 MFMA with the weights' low mantissa bits kept.
 *
 * lbsa_router_split_weights, once per weight matrix:
 *   w_d        fp32 [n][k] (one row per expert)
 *   w_high_d   bf16, n * k elements: w truncated to bf16 (its low 16 bits dropped)
 *   w_low_d    bf16, n * k elements: (w - w_high) * 256 rounded to nearest even
 * so that w ~ w_high + w_low / 256 within 2^-16 |w|.  Both parts are stored
 * blocked for the GEMM's loads: element (e, c) (expert e, input feature c)
 * sits at index ((e / 16) * (k / 64) + c / 64) * 1024 + b * 512 + lane * 8 + i
 * with c % 64 = 16 g + 8 b + i and lane = 16 g + e % 16 (per 16 experts
 * and 64 features a 2 KiB block; each wave's load of a block half is one
 * contiguous 1 KiB read).
 *
 * lbsa_router_gemm, per call:
 *   x_d        bf16 [m][k] hidden states (m = 0 is a no-op)
 *   w_*_d      the two blocked parts from lbsa_router_split_weights
 *   scores_d   fp32 [m][n] = x w_high^T + (x w_low^T) / 256, fp32 accumulation
 *   workspace  >= lbsa_router_workspace_bytes(m, n, k) bytes, 16-byte aligned,
 *              any contents (0 bytes, and the pointer may be NULL, when k is
 *              not split): the fp32 partial scores of the parts of k.  Calls
 *              that share one workspace must not overlap in time.
 * Shapes: n a multiple of 16, k a multiple of 256 and at most 2^20 (else
 * LBSA_ERR_UNSUPPORTED); every pointer 16-byte aligned (else
 * LBSA_ERR_INVALID_ARGUMENT).  The scores are deterministic: the parts of a
 * split of k are added in a fixed order.  All buffers are the caller's; the
 * calls only enqueue kernels on the stream.
 */
int lbsa_router_split_weights(const float* w_d, int32_t n, int32_t k, void* w_high_d, void* w_low_d, void* stream);
int lbsa_router_workspace_bytes(int32_t m, int32_t n, int32_t k, size_t* out_bytes);
int lbsa_router_gemm(const void* x_d, const void* w_high_d, const void* w_low_d, int32_t m, int32_t n, int32_t k,
                     float* scores_d, void* workspace_d, size_t workspace_bytes, void* stream);

/*
 * Fused attention prologue: from the fused QKV projection of num_tokens tokens
 * to the decode path's inputs, in one launch.  Source: vLLM post, section "A
 * fused attention prologue"; SGLang post, the attention prologue section
 * (QK-Norm before RoPE, K and V written straight into the paged cache, in fp8
 * the query emitted as fp8 with a per-token, per-head scale).
 *   qkv_d            bf16 [num_tokens][(num_heads + 2 num_kv_heads) * 128]: per token the
 *                    query heads, then the key heads, then the value heads
 *   positions_d      int32 [num_tokens] position of each token in its sequence (RoPE)
 *   slot_mapping_d   int64 [num_tokens] cache slot page * 64 + row; a slot < 0 or
 *                    >= num_pages * 64 is not written (padding tokens)
 *   q_norm_weight_d, k_norm_weight_d   fp32 [128] RMSNorm weights (all query heads
 *                    share one, all KV heads the other)
 *   rope_theta, eps  RoPE base (> 1) and the RMSNorm epsilon (>= 0)
 *   kv_dtype         LBSA_KV_BF16: q_out bf16 [num_tokens][num_heads][128], bf16 caches;
 *                    LBSA_KV_FP8_E4M3: q_out e4m3 codes of the same shape plus
 *                    q_scale_out fp32 [num_tokens][num_heads], e4m3 caches plus
 *                    k_scale_d / v_scale_d fp32 [num_pages][num_kv_heads][64]
 *   k_cache_d, v_cache_d   [num_pages][64][num_kv_heads][128], updated in place
 * Per query and key head: y = x * w / sqrt(mean(x^2) + eps), then the pairs
 * (d, d + 64) rotate by pos * rope_theta^(-2d/128).  V is copied.  fp8: scale =
 * max|y| / 448 per token and head (1 for an all-zero head), codes rounded to
 * nearest even.  head_dim must be 128 and page_size 64 (else
 * LBSA_ERR_UNSUPPORTED); num_heads must be a multiple of num_kv_heads.
 * Alignment: qkv_d and the two weights 16 B; q_out_d, k_cache_d and v_cache_d
 * 16 B in bf16, 8 B in fp8; the rest their element size (else
 * LBSA_ERR_INVALID_ARGUMENT, as for a null pointer, theta <= 1 or eps < 0).
 * num_tokens = 0 is a no-op.  All buffers are the caller's; the call only
 * enqueues one kernel on the stream.
 */
int lbsa_prologue(const void* qkv_d, const int32_t* positions_d, const int64_t* slot_mapping_d,
                  const float* q_norm_weight_d, const float* k_norm_weight_d, double rope_theta,
                  float eps, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t page_size, int32_t kv_dtype, void* q_out_d,
                  float* q_scale_out_d, void* k_cache_d, void* v_cache_d, float* k_scale_d,
                  float* v_scale_d, int64_t num_pages, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LBSA_H */
