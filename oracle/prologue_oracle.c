/*
 * prologue_oracle.c -- plain, slow CPU oracle of the fused attention prologue
 * that produces the decode path's inputs: QK-Norm, then RoPE, then the Q
 * emitted as bf16 or as fp8 codes with a per-token-per-head scale, and K / V
 * written into the paged cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the test-suite does.  It shares no code with
 * the HIP library.
 *
 * Sources: the vLLM post (news.ainew.jp, "A fused attention prologue") and
 * the SGLang post (section "融合的Attention前奏"): starting from the fused
 * QKV projection, QK-Norm is applied before RoPE (the Hy3 order), K and V go
 * straight into the paged cache, and in fp8 the query leaves as fp8 codes with
 * one scale per token and head.
 *
 * Readings taken where the pages are silent (each is also listed with its
 * reason in the design notes of the repository):
 *   P1  QK-Norm is RMSNorm over head_dim, one weight vector of length D for
 *       all query heads and another for all KV heads:
 *       y_d = x_d * w_d / sqrt(mean_d(x_d^2) + eps).
 *   P2  RoPE rotates the pairs (d, d + D/2) (the "rotate half" layout) over
 *       the full head dimension with angle pos * theta^(-2d/D), d < D/2:
 *       y_d = x_d cos a - x_{d+D/2} sin a,  y_{d+D/2} = x_{d+D/2} cos a + x_d sin a.
 *   P3  fp8 (OCP e4m3fn) quantisation per token and head:
 *       scale = max|x| / 448 (1 when x is all zero), code = e4m3(x / scale)
 *       rounded to nearest, ties to the even code.
 *   P4  V is neither normalised nor rotated.
 *   P5  The fused projection row of a token is [Hq heads of Q][Hkv heads of
 *       K][Hkv heads of V], each head D contiguous values.
 *
 * Floating point is fp64 throughout.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

double oracle_bf16_value(uint16_t bits);   /* lbsa_oracle.c */
double oracle_e4m3_value(uint8_t bits);    /* lbsa_oracle.c */

/* P1: RMSNorm of n values. */
void oracle_rmsnorm(const double* x, const double* w, int n, double eps, double* y)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    const double r = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i) y[i] = x[i] * w[i] * r;
}

/* P2: rotate x (length D, even) in place for position pos. */
void oracle_rope(double* x, int D, double pos, double theta)
{
    const int h = D / 2;
    for (int d = 0; d < h; ++d) {
        const double a = pos * pow(theta, -2.0 * d / D);
        const double c = cos(a), s = sin(a);
        const double x0 = x[d], x1 = x[d + h];
        x[d] = x0 * c - x1 * s;
        x[d + h] = x1 * c + x0 * s;
    }
}

/* Nearest e4m3fn code to v (finite, |v| <= 448), ties to the even code: a
 * plain search over the 127 positive finite codes. */
static uint8_t e4m3_nearest(double v)
{
    const int neg = v < 0.0;
    const double a = fabs(v);
    int best = 0;
    double best_err = a;                        /* code 0 is +0 */
    for (int c = 1; c <= 0x7E; ++c) {           /* 0x7F is NaN */
        const double err = fabs(oracle_e4m3_value((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (neg && best ? 0x80 : 0));
}

/* P3: fp8 codes and scale of n values. */
void oracle_quant_e4m3(const double* x, int n, uint8_t* codes, double* scale)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) amax = fmax(amax, fabs(x[i]));
    const double s = amax > 0.0 ? amax / 448.0 : 1.0;
    for (int i = 0; i < n; ++i) {
        double v = x[i] / s;
        if (v > 448.0) v = 448.0;               /* only rounding of x / s can exceed it */
        if (v < -448.0) v = -448.0;
        codes[i] = e4m3_nearest(v);
    }
    *scale = s;
}

/* bf16 bits nearest to v (finite, |v| below the largest bf16), ties to even:
 * from the format's definition.  Positive bf16 values grow with their bit
 * pattern, so the largest one not above |v| is found by bisection over the
 * codes; then the nearer of it and the next one wins. */
uint16_t oracle_bf16_nearest(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    int lo = 0, hi = 0x7F7F;                    /* oracle_bf16_value(lo) <= a invariant */
    if (oracle_bf16_value((uint16_t)hi) <= a) return (uint16_t)(hi | sign);
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (oracle_bf16_value((uint16_t)mid) <= a) lo = mid; else hi = mid;
    }
    const double dl = a - oracle_bf16_value((uint16_t)lo), dh = oracle_bf16_value((uint16_t)hi) - a;
    const int r = (dl < dh || (dl == dh && (lo & 1) == 0)) ? lo : hi;
    return (uint16_t)(r | sign);
}

/*
 * The prologue of T tokens: q_out [T][Hq][D], k_out [T][Hkv][D], v_out
 * [T][Hkv][D] in fp64 (before any output rounding).  qkv holds bf16 bits,
 * [T][(Hq + 2 Hkv) D]; positions [T]; qw / kw [D].
 */
void oracle_prologue(const uint16_t* qkv, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                     const int32_t* positions, const double* qw, const double* kw, double theta,
                     double eps, double* q_out, double* k_out, double* v_out)
{
    const int64_t row = (int64_t)(Hq + 2 * Hkv) * D;
    double x[1024];
    if (D > 1024 || D % 2) return;
    for (int32_t t = 0; t < T; ++t) {
        const uint16_t* src = qkv + t * row;
        const double pos = (double)positions[t];
        for (int32_t h = 0; h < Hq + 2 * Hkv; ++h) {
            for (int32_t d = 0; d < D; ++d) x[d] = oracle_bf16_value(src[(int64_t)h * D + d]);
            if (h < Hq) {
                double* y = q_out + ((int64_t)t * Hq + h) * D;
                oracle_rmsnorm(x, qw, D, eps, y);
                oracle_rope(y, D, pos, theta);
            } else if (h < Hq + Hkv) {
                double* y = k_out + ((int64_t)t * Hkv + (h - Hq)) * D;
                oracle_rmsnorm(x, kw, D, eps, y);
                oracle_rope(y, D, pos, theta);
            } else {
                double* y = v_out + ((int64_t)t * Hkv + (h - Hq - Hkv)) * D;
                memcpy(y, x, sizeof(double) * D);
            }
        }
    }
}
