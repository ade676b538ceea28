/*
 * lbsa_oracle.c -- plain, slow, obviously-correct CPU oracle for
 * load-balanced paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library: every number format below is decoded from its
 * own definition here.
 *
 * Sources (the method is described on three web pages; cited by title and
 * section):
 *   [vLLM post]   "Tencent Hunyuan HPC-Ops in vLLM" (news.ainew.jp, English
 *                 text), section "The solution: a per-step, load-balanced
 *                 decode scheduler", bullets "Assign" and "Compute and
 *                 combine".
 *   [SGLang post] "HPC-Ops x SGLang" (Chinese), sections
 *                 "Attention: load balancing of variable-length decode" and
 *                 "Scheduling around live KV work".
 *
 * Readings taken where the pages are silent (each is also listed with its
 * reason in the design notes of the repository):
 *   R1  budget/spill: K = min(P, max(1, floor(T/F))) active bins; the first
 *       T mod K bins are filled to ceil(T/K) tiles, the rest to floor(T/K),
 *       in traversal order (fill-to-budget-then-spill with bin sizes that
 *       differ by at most one tile).
 *   R2  minimum-work floor F is a parameter (library default 2 tiles).
 *   R3  "heads" in the tile sum are KV heads; one task covers the whole GQA
 *       group of one KV head; query head hq reads KV head hq / (Hq/Hkv).
 *   R5  n_b = ceil(L_b / 64); tokens >= L_b are masked.
 *   R6  the per-bin terminator is represented as CSR offsets.
 *   R7  partials are normalised O (per query head, per dim) plus the
 *       natural-log LSE.
 *   R9  fp8 is OCP E4M3FN (bias 7, max 448, S.1111.111 is NaN, no inf).
 *   R10 K/V scales are per token per KV head (fp32), Q scales per request per
 *       query head; scale arrays are laid out [page][kv_head][slot].
 *   R11 L_b = 0 is allowed: no tiles, no chunks, output row 0, LSE -inf.
 *   R12 K/V caches are token-major [page][slot][kv_head][dim].
 *   M1  multi-token decode (q_len > 1, Hy3's MTP speculative layer in the
 *       vLLM post's model paragraph): the q_len new tokens of a request are
 *       the last q_len of its L_b cached tokens; query i (0-based) sits at
 *       position L_b - q_len + i and sees tokens [0, L_b - q_len + i], i.e.
 *       causal among the new tokens.  A query that sees no token gives 0.
 *       q is [B][q_len][Hq][D], q_scale [B][q_len][Hq], out like q; a
 *       descriptor's partial has one row per (query i, head g), row i*G + g.
 *   Q1  prefill / extend on the task map (the survey's query-tile dimension):
 *       request b brings q_b >= 1 new tokens, the last q_b of its L_b cached
 *       ones, query i seeing tokens [0, L_b - q_b + i] (M1 with a per-request
 *       q).  Its queries form blocks of QB consecutive positions; a segment is
 *       (kv_head, request, query block k) and spans the tiles its last query
 *       sees: ceil(min(L_b, L_b - q_b + QB (k + 1)) / 64).  Segments are walked
 *       head-major, batch-minor, query block innermost; budget, fill and spill
 *       are those of R1 over these tiles.  With q_b = 1 for every request this
 *       is the decode map.  Q and out are packed [sum q_b][Hq][D] in request
 *       order (row qstart_b + i); a partial has one row per (block position p,
 *       head g), row p*G + g, and positions past q_b are empty (0, -inf).
 *
 * Floating point is fp64 throughout; integers in the assign are int64.
 * Parity of every function here is pinned in tests/ against values that do
 * not come from this file (library routines, closed forms, brute force and
 * hand-derived examples).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_TILE 64

/* ------------------------------------------------------------------------ */
/* Number formats, each from its definition.                                 */
/* ------------------------------------------------------------------------ */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double mag;
    if (e == 0xFF)
        mag = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m / 128.0, -126);           /* subnormal */
    else
        mag = ldexp(1.0 + (double)m / 128.0, e - 127);  /* normal */
    return sign ? -mag : mag;
}

/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits,
 * no infinities, exponent=1111 with fraction=111 is NaN, max finite 448. */
double oracle_e4m3_value(uint8_t bits)
{
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        mag = NAN;
    else if (e == 0)
        mag = ldexp((double)m / 8.0, -6);              /* subnormal */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);     /* normal */
    return sign ? -mag : mag;
}

void oracle_bf16_values(const uint16_t* bits, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_value(bits[i]);
}

void oracle_e4m3_values(const uint8_t* bits, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_value(bits[i]);
}

/* ------------------------------------------------------------------------ */
/* Assign: the task-map builder.                                             */
/* ------------------------------------------------------------------------ */

/*
 * Header words (int32), shared layout with what the GPU map is compared on:
 *   0 T       total tiles over all (kv_head, request) segments
 *   1 K       active bins
 *   2 q       floor(T/K)
 *   3 r       T mod K
 *   4 Ndesc   descriptors emitted
 *   5 P       bins (= persistent workgroups)
 *   6 F       minimum-work floor (tiles)
 *   7 B       batch
 *   8 Hq      query heads
 *   9 Hkv     KV heads
 *  10 error   0 ok, 1 = some L_b < 0 or L_b > max_pages*64 (map is empty)
 *  11 N       tiles per KV head = sum_b n_b
 *  12 max_pages
 *  13 page_size (64)
 *  14,15 zero
 *
 * Descriptors are (kv_head, request, tile_begin, tile_end) with tile indices
 * local to the request.  Steps follow the pages' order:
 *   1. slice each live KV sequence into 64-token tiles;
 *   2. sum the tile counts over all KV heads and requests;
 *   3. derive the per-bin budget from total tiles / bins (reading R1, R2);
 *   4. walk the tiles head-major, batch-minor, filling the current bin up to
 *      its budget and then spilling into the next bin; each maximal run of
 *      tiles of one (kv_head, request) inside one bin is one descriptor
 *      ("one or more consecutive KV tiles");
 *   5. count the chunks of each (kv_head, request) for the combine.
 *
 * Returns 0, or -1 if an output capacity is too small / arguments invalid.
 */
int oracle_assign(const int32_t* seqlens, int32_t B, int32_t Hq, int32_t Hkv,
                  int32_t P, int32_t F, int32_t max_pages,
                  int32_t* header, int32_t* bin_desc_begin,
                  int32_t* desc, int64_t desc_cap,
                  int32_t* seg_first_desc, int32_t* seg_num_chunks)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || P <= 0 || F <= 0 || max_pages <= 0)
        return -1;
    if (Hq % Hkv != 0) return -1;

    int error = 0;
    for (int32_t b = 0; b < B; ++b)
        if (seqlens[b] < 0 || (int64_t)seqlens[b] > (int64_t)max_pages * OR_TILE)
            error = 1;

    /* Step 1: tiles per request. */
    int64_t* n = (int64_t*)calloc((size_t)B, sizeof(int64_t));
    int64_t N = 0;
    for (int32_t b = 0; b < B; ++b) {
        n[b] = error ? 0 : ((int64_t)seqlens[b] + OR_TILE - 1) / OR_TILE;
        N += n[b];
    }
    /* Step 2: total over all KV heads. */
    int64_t T = (int64_t)Hkv * N;

    /* Step 3: budget. */
    int64_t K = 0, q = 0, r = 0;
    if (T > 0) {
        int64_t by_floor = T / F;
        if (by_floor < 1) by_floor = 1;
        K = by_floor < P ? by_floor : P;
        q = T / K;
        r = T % K;
    }

    /* Step 4: walk tiles head-major, batch-minor; fill and spill. */
    for (int32_t j = 0; j <= P; ++j) bin_desc_begin[j] = -1;
    int64_t nd = 0;
    int64_t bin = 0, fill = 0;
    int open = 0;  /* is descriptor nd-1 still accepting tiles? */
    for (int32_t h = 0; h < Hkv; ++h) {
        for (int32_t b = 0; b < B; ++b) {
            for (int64_t t = 0; t < n[b]; ++t) {
                if (fill == 0) bin_desc_begin[bin] = (int32_t)nd;
                int extend = open && desc[4 * (nd - 1) + 0] == h &&
                             desc[4 * (nd - 1) + 1] == b &&
                             desc[4 * (nd - 1) + 3] == t;
                if (extend) {
                    desc[4 * (nd - 1) + 3] = (int32_t)(t + 1);
                } else {
                    if (nd >= desc_cap) { free(n); return -1; }
                    desc[4 * nd + 0] = h;
                    desc[4 * nd + 1] = b;
                    desc[4 * nd + 2] = (int32_t)t;
                    desc[4 * nd + 3] = (int32_t)(t + 1);
                    ++nd;
                    open = 1;
                }
                int64_t budget = (bin < r) ? q + 1 : q;
                if (++fill == budget) {  /* bin full: spill to the next */
                    ++bin;
                    fill = 0;
                    open = 0;
                }
            }
            open = 0;  /* a new request never extends the previous one */
        }
    }
    for (int64_t j = K; j <= P; ++j) bin_desc_begin[j] = (int32_t)nd;

    /* Step 5: chunk count and first chunk per (kv_head, request). */
    for (int64_t s = 0; s < (int64_t)Hkv * B; ++s) seg_num_chunks[s] = 0;
    for (int64_t d = 0; d < nd; ++d)
        seg_num_chunks[(int64_t)desc[4 * d + 0] * B + desc[4 * d + 1]] += 1;
    int64_t acc = 0;
    for (int64_t s = 0; s < (int64_t)Hkv * B; ++s) {
        seg_first_desc[s] = (int32_t)acc;
        acc += seg_num_chunks[s];
    }

    memset(header, 0, 16 * sizeof(int32_t));
    header[0] = (int32_t)T;
    header[1] = (int32_t)K;
    header[2] = (int32_t)q;
    header[3] = (int32_t)r;
    header[4] = (int32_t)nd;
    header[5] = P;
    header[6] = F;
    header[7] = B;
    header[8] = Hq;
    header[9] = Hkv;
    header[10] = error;
    header[11] = (int32_t)N;
    header[12] = max_pages;
    header[13] = OR_TILE;
    free(n);
    return 0;
}

/*
 * Assign with query blocks (reading Q1).  The same five steps as
 * oracle_assign, over segments (kv_head, request, query block):
 *   1. slice: query block k of request b spans n(b, k) =
 *      ceil(min(L_b, L_b - q_b + QB (k + 1)) / 64) tiles, for k < ceil(q_b / QB);
 *   2. T = sum of n(b, k) over every KV head, request and query block;
 *   3. budget from T and the bins (R1, R2);
 *   4. walk the tiles head-major, batch-minor, query block innermost, fill and
 *      spill; a maximal run of one segment's tiles inside one bin is a
 *      descriptor (kv_head, request, query_block, tile_begin, tile_end);
 *   5. chunk count and first chunk per segment, segment index
 *      s = h * NQ + (blocks of earlier requests) + k, NQ = sum_b ceil(q_b / QB).
 * Header as oracle_assign (word 11 N = tiles per KV head), plus 14 NQ and
 * 15 QB.  An L_b or q_b out of range (L_b < 0, L_b > max_pages * 64, q_b < 1,
 * q_b > L_b) sets the error word and empties the map.
 */
int oracle_assign_varlen(const int32_t* seqlens, const int32_t* qlens, int32_t B, int32_t Hq,
                         int32_t Hkv, int32_t P, int32_t F, int32_t max_pages, int32_t QB,
                         int32_t* header, int32_t* bin_desc_begin,
                         int32_t* desc, int64_t desc_cap,
                         int32_t* seg_first_desc, int32_t* seg_num_chunks, int64_t seg_cap)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || P <= 0 || F <= 0 || max_pages <= 0 || QB <= 0)
        return -1;
    if (Hq % Hkv != 0) return -1;

    int error = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t L = seqlens[b], q = qlens[b];
        if (L < 0 || L > (int64_t)max_pages * OR_TILE || q < 1 || q > L) error = 1;
    }

    /* Step 1: query blocks per request and the tiles of each block. */
    int64_t NQ = 0;
    int64_t* nq = (int64_t*)calloc((size_t)B, sizeof(int64_t));
    for (int32_t b = 0; b < B; ++b) {
        nq[b] = error ? 0 : ((int64_t)qlens[b] + QB - 1) / QB;
        NQ += nq[b];
    }
    if ((int64_t)Hkv * NQ > seg_cap) { free(nq); return -1; }
    int64_t* ntile = (int64_t*)calloc((size_t)(NQ > 0 ? NQ : 1), sizeof(int64_t));
    int64_t N = 0;
    {
        int64_t s = 0;
        for (int32_t b = 0; b < B; ++b)
            for (int64_t k = 0; k < nq[b]; ++k, ++s) {
                int64_t seen = (int64_t)seqlens[b] - qlens[b] + QB * (k + 1);
                if (seen > seqlens[b]) seen = seqlens[b];
                ntile[s] = (seen + OR_TILE - 1) / OR_TILE;
                N += ntile[s];
            }
    }
    /* Step 2: total over all KV heads. */
    int64_t T = (int64_t)Hkv * N;

    /* Step 3: budget. */
    int64_t K = 0, q = 0, r = 0;
    if (T > 0) {
        int64_t by_floor = T / F;
        if (by_floor < 1) by_floor = 1;
        K = by_floor < P ? by_floor : P;
        q = T / K;
        r = T % K;
    }

    /* Step 4: walk; fill and spill. */
    for (int32_t j = 0; j <= P; ++j) bin_desc_begin[j] = -1;
    int64_t nd = 0, bin = 0, fill = 0;
    int open = 0;
    for (int32_t h = 0; h < Hkv; ++h) {
        int64_t s = 0;
        for (int32_t b = 0; b < B; ++b) {
            for (int64_t k = 0; k < nq[b]; ++k, ++s) {
                for (int64_t t = 0; t < ntile[s]; ++t) {
                    if (fill == 0) bin_desc_begin[bin] = (int32_t)nd;
                    if (open) {
                        desc[5 * (nd - 1) + 4] = (int32_t)(t + 1);
                    } else {
                        if (nd >= desc_cap) { free(nq); free(ntile); return -1; }
                        desc[5 * nd + 0] = h;
                        desc[5 * nd + 1] = b;
                        desc[5 * nd + 2] = (int32_t)k;
                        desc[5 * nd + 3] = (int32_t)t;
                        desc[5 * nd + 4] = (int32_t)(t + 1);
                        ++nd;
                        open = 1;
                    }
                    int64_t budget = (bin < r) ? q + 1 : q;
                    if (++fill == budget) {  /* bin full: spill to the next */
                        ++bin;
                        fill = 0;
                        open = 0;
                    }
                }
                open = 0;  /* a new segment never extends the previous one */
            }
        }
    }
    for (int64_t j = K; j <= P; ++j) bin_desc_begin[j] = (int32_t)nd;

    /* Step 5: chunk count and first chunk per segment. */
    int64_t* qbase = (int64_t*)calloc((size_t)B + 1, sizeof(int64_t));
    for (int32_t b = 0; b < B; ++b) qbase[b + 1] = qbase[b] + nq[b];
    const int64_t S = (int64_t)Hkv * NQ;
    for (int64_t s = 0; s < S; ++s) seg_num_chunks[s] = 0;
    for (int64_t d = 0; d < nd; ++d)
        seg_num_chunks[(int64_t)desc[5 * d] * NQ + qbase[desc[5 * d + 1]] + desc[5 * d + 2]] += 1;
    int64_t acc = 0;
    for (int64_t s = 0; s < S; ++s) {
        seg_first_desc[s] = (int32_t)acc;
        acc += seg_num_chunks[s];
    }

    memset(header, 0, 16 * sizeof(int32_t));
    header[0] = (int32_t)T;
    header[1] = (int32_t)K;
    header[2] = (int32_t)q;
    header[3] = (int32_t)r;
    header[4] = (int32_t)nd;
    header[5] = P;
    header[6] = F;
    header[7] = B;
    header[8] = Hq;
    header[9] = Hkv;
    header[10] = error;
    header[11] = (int32_t)N;
    header[12] = max_pages;
    header[13] = OR_TILE;
    header[14] = (int32_t)NQ;
    header[15] = QB;
    free(nq);
    free(ntile);
    free(qbase);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention: the plain softmax definition over gathered paged K/V.          */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void* q;          /* [B][q_len][Hq][D]  bf16 bits (kv_dtype 0) or e4m3 bits (1) */
    const float* q_scale;   /* [B][q_len][Hq]     e4m3 only */
    const void* k_cache;    /* [pages][64][Hkv][D] */
    const void* v_cache;
    const float* k_scale;   /* [pages][Hkv][64]    e4m3 only */
    const float* v_scale;
    const int32_t* page_table; /* [B][max_pages] */
    const int32_t* seqlens;    /* [B] */
    int32_t kv_dtype;       /* 0 = bf16, 1 = e4m3fn */
    int32_t B, Hq, Hkv, D, max_pages, num_pages;
    double softmax_scale;
    int32_t q_len;          /* query tokens per request (M1), >= 1 */
    const int32_t* qlens;   /* Q1: per-request q_b, or NULL for q_len everywhere */
    const int32_t* qstart;  /* Q1: packed row of query 0 of request b (prefix of qlens), [B + 1] */
} oracle_inputs;

/* Element d of query i of request b, head hq. */
static int64_t q_of(const oracle_inputs* in, int64_t b)
{
    return in->qlens ? in->qlens[b] : in->q_len;
}

/* Row of query i of request b in q / out: [B][q_len] (M1) or packed (Q1). */
static int64_t q_row(const oracle_inputs* in, int64_t b, int64_t i)
{
    return in->qlens ? (int64_t)in->qstart[b] + i : b * in->q_len + i;
}

static double q_elem(const oracle_inputs* in, int64_t b, int64_t i, int64_t hq, int64_t d)
{
    const int64_t row = q_row(in, b, i) * in->Hq + hq;
    if (in->kv_dtype == 0) return oracle_bf16_value(((const uint16_t*)in->q)[row * in->D + d]);
    return oracle_e4m3_value(((const uint8_t*)in->q)[row * in->D + d]) * (double)in->q_scale[row];
}

/* M1: tokens [0, visible) of request b are seen by its query i. */
static int64_t visible(const oracle_inputs* in, int64_t b, int64_t i)
{
    const int64_t v = (int64_t)in->seqlens[b] - q_of(in, b) + 1 + i;
    return v > 0 ? v : 0;
}

static double kv_elem(const oracle_inputs* in, const void* cache, const float* scale,
                      int64_t page, int64_t slot, int64_t h, int64_t d)
{
    int64_t i = ((page * OR_TILE + slot) * in->Hkv + h) * in->D + d;
    if (in->kv_dtype == 0) return oracle_bf16_value(((const uint16_t*)cache)[i]);
    return oracle_e4m3_value(((const uint8_t*)cache)[i]) *
           (double)scale[(page * in->Hkv + h) * OR_TILE + slot];
}

/* Attention of query i, head hq of request b over its tokens [tok0, tok1)
 * (cut at what the query sees, M1).
 * out[D] = sum_t w_t v_t / sum_t w_t with w_t = exp(s_t - max s),
 * s_t = softmax_scale * <q, k_t>; *lse = max s + ln sum_t w_t.
 * An empty range gives out = 0 and lse = -inf.  Returns -1 on a bad page. */
static int attend_range(const oracle_inputs* in, int64_t b, int64_t i, int64_t hq,
                        int64_t tok0, int64_t tok1, double* out, double* lse,
                        double* qv, double* s)
{
    const int64_t D = in->D;
    const int64_t h = hq / (in->Hq / in->Hkv);
    if (tok1 > visible(in, b, i)) tok1 = visible(in, b, i);
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    if (tok1 <= tok0) { *lse = -INFINITY; return 0; }
    for (int64_t d = 0; d < D; ++d) qv[d] = q_elem(in, b, i, hq, d);

    double m = -INFINITY;
    for (int64_t t = tok0; t < tok1; ++t) {
        int64_t page = in->page_table[b * in->max_pages + t / OR_TILE];
        if (page < 0 || page >= in->num_pages) return -1;
        int64_t slot = t % OR_TILE;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += qv[d] * kv_elem(in, in->k_cache, in->k_scale, page, slot, h, d);
        s[t - tok0] = in->softmax_scale * dot;
        if (s[t - tok0] > m) m = s[t - tok0];
    }
    double wsum = 0.0;
    for (int64_t t = tok0; t < tok1; ++t) {
        int64_t page = in->page_table[b * in->max_pages + t / OR_TILE];
        int64_t slot = t % OR_TILE;
        double w = exp(s[t - tok0] - m);
        wsum += w;
        for (int64_t d = 0; d < D; ++d)
            out[d] += w * kv_elem(in, in->v_cache, in->v_scale, page, slot, h, d);
    }
    for (int64_t d = 0; d < D; ++d) out[d] /= wsum;
    *lse = m + log(wsum);
    return 0;
}

static int64_t max_len(const oracle_inputs* in)
{
    int64_t mx = 1;
    for (int32_t b = 0; b < in->B; ++b)
        if (in->seqlens[b] > mx) mx = in->seqlens[b];
    return mx;
}

/* Full attention for every (request, query, head): out [B][q_len][Hq][D],
 * lse [B][q_len][Hq].  Requests with L_b = 0 give zeros and -inf. */
int oracle_attention(const oracle_inputs* in, double* out, double* lse, int nthreads)
{
    const int64_t rows = (int64_t)in->B * in->q_len * in->Hq;
    const int64_t D = in->D;
    const int64_t L = max_len(in);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* qv = (double*)malloc((size_t)D * sizeof(double));
        double* s = (double*)malloc((size_t)L * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t row = 0; row < rows; ++row) {
            const int64_t b = row / ((int64_t)in->q_len * in->Hq);
            const int64_t i = row / in->Hq % in->q_len, hq = row % in->Hq;
            if (attend_range(in, b, i, hq, 0, in->seqlens[b], out + row * D, lse + row, qv, s))
                bad = 1;
        }
        free(qv);
        free(s);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/* Attention restricted to a subset of rows given as pairs (request, j) with
 * j = i * Hq + hq (query i, head hq); used to sample outputs of very large
 * batches. */
int oracle_attention_rows(const oracle_inputs* in, const int32_t* rows_bh, int64_t nrows,
                          double* out, double* lse, int nthreads)
{
    const int64_t D = in->D;
    const int64_t L = max_len(in);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* qv = (double*)malloc((size_t)D * sizeof(double));
        double* s = (double*)malloc((size_t)L * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t b = rows_bh[2 * i], qi = rows_bh[2 * i + 1] / in->Hq;
            const int64_t hq = rows_bh[2 * i + 1] % in->Hq;
            if (attend_range(in, b, qi, hq, 0, in->seqlens[b], out + i * D, lse + i, qv, s))
                bad = 1;
        }
        free(qv);
        free(s);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/* Per-descriptor partials: descriptor i = (h, b, t0, t1) covers tokens
 * [64 t0, min(64 t1, L_b)) of request b for the G query heads of KV head h
 * and each of the q_len queries (cut at what each sees, M1).
 * part_o [n][q_len * G][D] is the normalised partial output (row qi * G + g),
 * part_lse [n][q_len * G] its natural-log LSE (reading R7). */
int oracle_partials(const oracle_inputs* in, const int32_t* desc, int64_t ndesc,
                    double* part_o, double* part_lse, int nthreads)
{
    const int64_t D = in->D;
    const int64_t G = in->Hq / in->Hkv;
    const int64_t L = max_len(in);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* qv = (double*)malloc((size_t)D * sizeof(double));
        double* s = (double*)malloc((size_t)L * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < ndesc * in->q_len * G; ++i) {
            const int64_t di = i / (in->q_len * G), qi = i / G % in->q_len, g = i % G;
            const int64_t h = desc[4 * di], b = desc[4 * di + 1];
            const int64_t tok0 = (int64_t)desc[4 * di + 2] * OR_TILE;
            int64_t tok1 = (int64_t)desc[4 * di + 3] * OR_TILE;
            if (tok1 > in->seqlens[b]) tok1 = in->seqlens[b];
            if (attend_range(in, b, qi, h * G + g, tok0, tok1, part_o + i * D, part_lse + i, qv, s))
                bad = 1;
        }
        free(qv);
        free(s);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/* Q1: full attention of every packed query row: out [sum q_b][Hq][D], lse
 * [sum q_b][Hq] (in->qlens and in->qstart set). */
int oracle_attention_varlen(const oracle_inputs* in, double* out, double* lse, int nthreads)
{
    const int64_t D = in->D;
    const int64_t L = max_len(in);
    const int64_t rows = (int64_t)in->qstart[in->B] * in->Hq;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* qv = (double*)malloc((size_t)D * sizeof(double));
        double* s = (double*)malloc((size_t)L * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t row = 0; row < rows; ++row) {
            const int64_t t = row / in->Hq, hq = row % in->Hq;
            int64_t b = 0;
            while (in->qstart[b + 1] <= t) ++b;   /* the request that owns packed row t */
            if (attend_range(in, b, t - in->qstart[b], hq, 0, in->seqlens[b], out + row * D, lse + row, qv, s))
                bad = 1;
        }
        free(qv);
        free(s);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/* Q1: attention of selected packed rows given as pairs (t, hq): query row t of
 * q (request b with qstart[b] <= t < qstart[b + 1]), head hq. */
int oracle_attention_varlen_rows(const oracle_inputs* in, const int32_t* rows, int64_t nrows,
                                 double* out, double* lse, int nthreads)
{
    const int64_t D = in->D;
    const int64_t L = max_len(in);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* qv = (double*)malloc((size_t)D * sizeof(double));
        double* s = (double*)malloc((size_t)L * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t t = rows[2 * i], hq = rows[2 * i + 1];
            int64_t b = 0;
            while (in->qstart[b + 1] <= t) ++b;
            if (attend_range(in, b, t - in->qstart[b], hq, 0, in->seqlens[b], out + i * D, lse + i, qv, s))
                bad = 1;
        }
        free(qv);
        free(s);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/* Q1 partials: descriptor i = (h, b, k, t0, t1) covers tokens [64 t0,
 * min(64 t1, L_b)) of request b for the G query heads of KV head h and the QB
 * positions of query block k (each cut at what it sees).  part_o
 * [n][QB * G][D] (row p * G + g for query QB k + p), part_lse [n][QB * G];
 * positions at or past q_b give 0 and -inf. */
int oracle_partials_varlen(const oracle_inputs* in, const int32_t* desc, int64_t ndesc, int32_t QB,
                           double* part_o, double* part_lse, int nthreads)
{
    const int64_t D = in->D;
    const int64_t G = in->Hq / in->Hkv;
    const int64_t L = max_len(in);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* qv = (double*)malloc((size_t)D * sizeof(double));
        double* s = (double*)malloc((size_t)L * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < ndesc * QB * G; ++i) {
            const int64_t di = i / (QB * G), p = i / G % QB, g = i % G;
            const int64_t h = desc[5 * di], b = desc[5 * di + 1], k = desc[5 * di + 2];
            const int64_t qi = QB * k + p;
            if (qi >= q_of(in, b)) {
                for (int64_t d = 0; d < D; ++d) part_o[i * D + d] = 0.0;
                part_lse[i] = -INFINITY;
                continue;
            }
            const int64_t tok0 = (int64_t)desc[5 * di + 3] * OR_TILE;
            int64_t tok1 = (int64_t)desc[5 * di + 4] * OR_TILE;
            if (tok1 > in->seqlens[b]) tok1 = in->seqlens[b];
            if (attend_range(in, b, qi, h * G + g, tok0, tok1, part_o + i * D, part_lse + i, qv, s))
                bad = 1;
        }
        free(qv);
        free(s);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/* Combine: merge n partials (o_c [width], lse_c) of one row under the global
 * softmax normalisation: M = max lse_c, w_c = exp(lse_c - M),
 * out = sum w_c o_c / sum w_c, lse = M + ln sum w_c.  n = 0 (or all lse_c
 * -inf) gives zeros and -inf. */
void oracle_merge(const double* o, const double* lse, int64_t n, int64_t width,
                  double* out, double* out_lse)
{
    double M = -INFINITY;
    for (int64_t c = 0; c < n; ++c)
        if (lse[c] > M) M = lse[c];
    for (int64_t d = 0; d < width; ++d) out[d] = 0.0;
    if (M == -INFINITY) { *out_lse = -INFINITY; return; }
    double wsum = 0.0;
    for (int64_t c = 0; c < n; ++c) {
        double w = exp(lse[c] - M);
        wsum += w;
        for (int64_t d = 0; d < width; ++d) out[d] += w * o[c * width + d];
    }
    for (int64_t d = 0; d < width; ++d) out[d] /= wsum;
    *out_lse = M + log(wsum);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
