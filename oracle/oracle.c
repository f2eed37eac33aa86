/*
 * oracle.c -- plain CPU oracle of the compress-then-sparsify attention path.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's CPU-baseline leg
 * are the only callers. The GPU library shares no code, header, table or helper with this file,
 * and the product path never calls it.
 *
 * Arithmetic: fp64 for compression and attention; exact integers for indexer scores.
 * Nothing is blocked, fused or reordered beyond the definitions cited below.
 *
 * Sources (web pages, cited by title and section):
 *   [EXPL]  "DeepSeek V4 Architecture Explained: CSA, HCA, mHC and Muon"
 *           -- section "How compress-then-sparsify attention works", table "Key numbers".
 *   [LLMB]  "Inside DeepSeek-V4: How Hybrid Sparse Attention Slashes 1M Context Overhead by 90%"
 *           -- sections "1. Compressed Sparse Attention (CSA)", "2. Heavily Compressed
 *           Attention (HCA)".
 *   [BSWEN] "How DeepSeek V4 Handles 1M Token Context with Hybrid Attention"
 *           -- sections "Component 2: Multi-Level KV Compression",
 *           "Component 3: DeepSeek Sparse Attention (DSA)".
 * Number formats (public specifications the pages name only as "FP4" / "FP8" / "BF16"):
 *   OCP Microscaling Formats (MX) v1.0: FP4 E2M1 elements, E8M0 shared scales, blocks of 32.
 *   OCP 8-bit Floating Point (OFP8): E4M3 (bias 7, max 448, no infinities).
 *   bfloat16: the top 16 bits of an IEEE binary32, rounded to nearest even.
 *
 * Readings where the pages are silent (each one is listed with its reason in the design notes):
 *   R1 groups are the non-overlapping runs of m consecutive tokens [EXPL].
 *   R1b with a span of s > m tokens per entry at stride m [BSWEN], entry g pools the s tokens
 *       ending with the last token of group g (see oc_kv_compress_span).
 *   R2 the gate is one scalar logit per token: z_t = w.x_t + beta[t - g*m].
 *   R7 indexer heads are combined by a plain sum of per-head dot products.
 *   R8 top-k order is (score descending, index ascending); missing slots are -1.
 *   R9 compressed entry g is visible to position p once its group is complete:
 *      g < floor((p+1)/m).
 *   R10 the window is the w tokens [p-w+1, p] that have position >= 0.
 *   R12 the sink is one logit per head that enters the softmax denominator only.
 *   R13 the sparse / dense entries, the window and the sink share one softmax.
 *   R25 RoPE follows RoFormer's general form on the last R dims; a compressed entry sits at the
 *       position of the last token of its group (see oc_rope, oc_kv_compress_rope).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OC_OK 0
#define OC_EINVAL (-1)

/* element / row formats (values mirror the public ABI so tests can pass the same ints) */
#define OC_DT_F32 0
#define OC_DT_BF16 1
#define OC_FMT_ROW_F32 0
#define OC_FMT_ROW_E4M3_BF16 1
#define OC_FMT_FP4_E8M0 2

int oc_version(void) { return 1; }

#ifdef _OPENMP
#include <omp.h>
int oc_num_threads(void) { return omp_get_max_threads(); }
#else
int oc_num_threads(void) { return 1; }
#endif

/* ------------------------------------------------------------------------------------------ */
/* Rounding a real number onto a binary floating-point grid.                                   */
/* p = significand bits (including the implicit one), emin = smallest normal exponent.         */
/* Values below 2^emin fall on the subnormal grid, spaced 2^(emin-p+1). Ties go to even.       */
/* ------------------------------------------------------------------------------------------ */
static double round_to_grid(double v, int p, int emin) {
    if (v == 0.0 || !isfinite(v)) return v;
    int E;
    frexp(fabs(v), &E);          /* |v| = f * 2^E, f in [0.5, 1)  =>  floor(log2|v|) = E-1 */
    int e = E - 1;
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - p + 1);
    return nearbyint(v / quantum) * quantum; /* default rounding mode: to nearest, ties even */
}

/* ---- FP4 E2M1 (OCP MX v1.0): 1 sign, 2 exponent (bias 1), 1 mantissa bit. ------------------ */
double oc_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* nearest E2M1 code of v, ties to even, saturating at +-6 */
int oc_e2m1_encode(double v) {
    double r = round_to_grid(v, 2, 0);
    if (r > 6.0) r = 6.0;
    if (r < -6.0) r = -6.0;
    int s = (r < 0.0) || (r == 0.0 && signbit(r));
    double a = fabs(r);
    if (a == 0.0) return s << 3;
    int E;
    frexp(a, &E);
    int e = E - 1;
    int code;
    if (e < 0) code = 1;                                 /* 0.5: subnormal, m = 1 */
    else code = ((e + 1) << 1) | (int)((a / ldexp(1.0, e) - 1.0) * 2.0);
    return (s << 3) | code;
}

/* ---- E8M0 scale (OCP MX v1.0): 2^(byte-127); 255 is NaN. ---------------------------------- */
double oc_e8m0_value(int byte) { return byte == 255 ? NAN : ldexp(1.0, byte - 127); }

/* ---- OFP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa; 0x7F/0xFF are NaN; max 448. -------- */
double oc_e4m3_value(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* nearest E4M3 code, ties to even, saturating at +-448 (unit scale) */
int oc_e4m3_encode(double v) {
    double r = round_to_grid(v, 4, -6);
    if (r > 448.0) r = 448.0;
    if (r < -448.0) r = -448.0;
    int s = (r < 0.0) || (r == 0.0 && signbit(r));
    double a = fabs(r);
    int code;
    if (a == 0.0) code = 0;
    else {
        int E;
        frexp(a, &E);
        int e = E - 1;
        if (e < -6) code = (int)(a / ldexp(1.0, -9));                     /* subnormal */
        else code = ((e + 7) << 3) | (int)((a / ldexp(1.0, e) - 1.0) * 8.0);
    }
    return (s << 7) | code;
}

/* ---- bfloat16 ----------------------------------------------------------------------------- */
double oc_bf16_value(unsigned bits) {
    int s = (bits >> 15) & 1, e = (bits >> 7) & 255, m = bits & 127;
    double mag;
    if (e == 255) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0) mag = ldexp((double)m, -133);
    else mag = ldexp(1.0 + m / 128.0, e - 127);
    return s ? -mag : mag;
}

unsigned oc_bf16_encode(double v) {
    double r = round_to_grid(v, 8, -126);
    int s = (r < 0.0) || (r == 0.0 && signbit(r));
    double a = fabs(r);
    unsigned bits;
    if (a == 0.0) bits = 0;
    else if (a >= ldexp(1.0, 128)) bits = 255u << 7;                         /* overflow: inf */
    else {
        int E;
        frexp(a, &E);
        int e = E - 1;
        if (e < -126) bits = (unsigned)(a / ldexp(1.0, -133));
        else bits = ((unsigned)(e + 127) << 7) | (unsigned)((a / ldexp(1.0, e) - 1.0) * 128.0);
    }
    return (s << 15) | bits;
}

double oc_f32_value(const void* p) { float f; memcpy(&f, p, 4); return (double)f; }

/* ---- OCP MX v1.0 block conversion: shared exponent floor(log2 amax) - 2 (E2M1's largest
 *      exponent), elements rounded to nearest even and saturated. An all-zero block gets
 *      scale byte 127 (a reading: the specification leaves the zero block open). ------------- */
void oc_fp4_block_encode(const double* v, int n, unsigned char* codes, unsigned char* scale) {
    double amax = 0.0;
    for (int i = 0; i < n; i++) if (fabs(v[i]) > amax) amax = fabs(v[i]);
    int sexp;
    if (amax == 0.0) sexp = 0;
    else {
        int E;
        frexp(amax, &E);
        sexp = (E - 1) - 2;
        if (sexp < -127) sexp = -127;
        if (sexp > 127) sexp = 127;
    }
    *scale = (unsigned char)(sexp + 127);
    double x = ldexp(1.0, sexp);
    memset(codes, 0, (size_t)n / 2);
    for (int i = 0; i < n; i++) {
        int c = oc_e2m1_encode(v[i] / x);
        codes[i / 2] |= (unsigned char)(c << ((i & 1) ? 4 : 0)); /* element 2j in the low nibble */
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Row codecs for the cache layouts.                                                           */
/*   ROW_F32        : D little-endian binary32 values.                                         */
/*   ROW_E4M3_BF16  : (D-64) E4M3 bytes, then 64 bf16 values (the rotary part) -- the key     */
/*                    numbers table of [EXPL] stores rotary dimensions in BF16 and the rest    */
/*                    in FP8.                                                                  */
/*   FP4_E8M0       : D/2 bytes of E2M1 codes per row + D/32 E8M0 bytes per row (separate).    */
/* ------------------------------------------------------------------------------------------ */
int64_t oc_row_bytes(int fmt, int D) {
    if (fmt == OC_FMT_ROW_F32) return 4LL * D;
    if (fmt == OC_FMT_ROW_E4M3_BF16) return (int64_t)(D - 64) + 128;
    if (fmt == OC_FMT_FP4_E8M0) return D / 2;
    return -1;
}

static void decode_row(const unsigned char* row, const unsigned char* scales, int fmt, int D,
                       double* out) {
    if (fmt == OC_FMT_ROW_F32) {
        for (int d = 0; d < D; d++) out[d] = oc_f32_value(row + 4 * d);
    } else if (fmt == OC_FMT_ROW_E4M3_BF16) {
        int dn = D - 64;
        for (int d = 0; d < dn; d++) out[d] = oc_e4m3_value(row[d]);
        for (int d = 0; d < 64; d++) {
            unsigned bits = (unsigned)row[dn + 2 * d] | ((unsigned)row[dn + 2 * d + 1] << 8);
            out[dn + d] = oc_bf16_value(bits);
        }
    } else { /* FP4_E8M0 */
        for (int d = 0; d < D; d++) {
            int c = (row[d / 2] >> ((d & 1) ? 4 : 0)) & 15;
            out[d] = oc_e2m1_value(c) * oc_e8m0_value(scales[d / 32]);
        }
    }
}

static void encode_row(const double* v, int fmt, int D, unsigned char* row, unsigned char* scales) {
    if (fmt == OC_FMT_ROW_F32) {
        for (int d = 0; d < D; d++) { float f = (float)v[d]; memcpy(row + 4 * d, &f, 4); }
    } else if (fmt == OC_FMT_ROW_E4M3_BF16) {
        int dn = D - 64;
        for (int d = 0; d < dn; d++) row[d] = (unsigned char)oc_e4m3_encode(v[d]);
        for (int d = 0; d < 64; d++) {
            unsigned b = oc_bf16_encode(v[dn + d]);
            row[dn + 2 * d] = (unsigned char)(b & 255);
            row[dn + 2 * d + 1] = (unsigned char)(b >> 8);
        }
    } else {
        for (int b = 0; b < D / 32; b++) oc_fp4_block_encode(v + 32 * b, 32, row + 16 * b, scales + b);
    }
}

/* bulk helpers: tests use them to build identical device inputs for both sides */
int oc_encode_rows(const double* x, int64_t n_rows, int D, int fmt, unsigned char* rows,
                   unsigned char* scales) {
    int64_t rb = oc_row_bytes(fmt, D);
    if (rb <= 0 || (fmt == OC_FMT_FP4_E8M0 && D % 32) || (fmt == OC_FMT_ROW_E4M3_BF16 && D < 64))
        return OC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; r++)
        encode_row(x + r * D, fmt, D, rows + r * rb, scales ? scales + r * (D / 32) : NULL);
    return OC_OK;
}

int oc_decode_rows(const unsigned char* rows, const unsigned char* scales, int64_t n_rows, int D,
                   int fmt, double* out) {
    int64_t rb = oc_row_bytes(fmt, D);
    if (rb <= 0) return OC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; r++)
        decode_row(rows + r * rb, scales ? scales + r * (D / 32) : NULL, fmt, D, out + r * D);
    return OC_OK;
}

static double load_elem(const void* base, int dtype, int64_t i) {
    if (dtype == OC_DT_F32) return oc_f32_value((const unsigned char*)base + 4 * i);
    const unsigned char* p = (const unsigned char*)base + 2 * i;
    return oc_bf16_value((unsigned)p[0] | ((unsigned)p[1] << 8));
}

/* ------------------------------------------------------------------------------------------ */
/* kv_compress -- softmax-gated pooling of each group of m consecutive tokens' shared K=V row  */
/* into one entry, with a learned bias per position inside the group.                           */
/* [EXPL] "How compress-then-sparsify attention works": trainable compression weights, a       */
/* softmax over the group and learnable positional biases fold m tokens into one KV entry.     */
/* [LLMB] "1. Compressed Sparse Attention (CSA)": softmax-gated pooling, factor 4;             */
/* "2. Heavily Compressed Attention (HCA)": factor 128.                                        */
/*   z_t  = sum_c w_c x_{t,c} + beta[t - g m]          (R2)                                    */
/*   pi   = softmax over the group of z                                                        */
/*   c_g  = sum_t pi_t x_t                                                                     */
/* raw: [B][raw_seq_stride rows][D] (F32 or BF16); out: row format, out_seq_stride rows.      */
/* pre_out (nullable): fp64 c_g before encoding, [B][T/m][D].                                  */
/* pi_out  (nullable): fp64 group weights, [B][T/m][m].                                        */
/* ------------------------------------------------------------------------------------------ */
/* Entries of `span` tokens at stride m: [BSWEN] "Component 2: Multi-Level KV Compression" lists
 * a level that compresses 8 tokens into one entry with a stride of 4. Reading R1b: entry g pools
 * the span tokens that end with the last token of group g, [m(g+1) - span, m(g+1)); tokens before
 * the start of the buffer do not exist and are left out of the softmax; the positional bias is
 * indexed by the token's place in the span, 0 .. span-1. span = m is the non-overlapping case.
 * The first `skip` groups only provide context: their entries are neither computed nor written,
 * and entry g (g >= skip) goes to output row g - skip. */
/* ------------------------------------------------------------------------------------------ */
/* RoPE on the rotary dims of one row (reading R25).                                            */
/* [BSWEN] "Component 1: Shared Key-Value Vectors": keys and values are one shared vector and   */
/* an inverse RoPE restores its positional information; [EXPL] "Key numbers" (KV storage       */
/* precision row): each row keeps its rotary dims in BF16. The pages do not define the          */
/* rotation. The definition                                                                     */
/* used is RoFormer's (Su et al., "RoFormer: Enhanced Transformer with Rotary Position          */
/* Embedding", section 3.2, general form): the last R dims of the row form R/2 adjacent pairs   */
/* (2j, 2j+1), and at position p pair j turns counter-clockwise by the angle p * theta_j,       */
/* theta_j = base^(-2j/R):                                                                      */
/*   (a, b) -> (a cos(p theta_j) - b sin(p theta_j),  a sin(p theta_j) + b cos(p theta_j)).    */
/* The inverse turns each pair back by the same angle.                                          */
/* ------------------------------------------------------------------------------------------ */
static void rope_row(double* v, int D, int R, double p, double base, int inverse) {
    for (int j = 0; j < R / 2; j++) {
        double ang = p * pow(base, -2.0 * j / R);
        if (inverse) ang = -ang;
        double c = cos(ang), s = sin(ang);
        double* a = v + (D - R) + 2 * j;
        double x0 = a[0], x1 = a[1];
        a[0] = x0 * c - x1 * s;
        a[1] = x0 * s + x1 * c;
    }
}

/* x: [B][Q][H][D] (F32 or BF16); row (b, i, h) is at position pos[b] + i (the position rule of  */
/* the queries everywhere on the path). out: fp64 [B][Q][H][D], the rotated rows.               */
int oc_rope(const void* x, int dtype, int B, int Q, int H, int D, int R, const int64_t* pos,
            double base, int inverse, double* out) {
    if (!x || !pos || !out || B < 0 || Q < 0 || H <= 0 || D <= 0 || R < 2 || R % 2 || R > D ||
        !(base > 0.0) || isinf(base))
        return OC_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++) {
        for (int i = 0; i < Q; i++) {
            for (int h = 0; h < H; h++) {
                int64_t r = (((int64_t)b * Q + i) * H + h) * D;
                for (int d = 0; d < D; d++) out[r + d] = load_elem(x, dtype, r + d);
                rope_row(out + r, D, R, (double)(pos[b] + i), base, inverse);
            }
        }
    }
    return OC_OK;
}

/* Compression with RoPE (reading R25): the pooled entry c_g is rotated before it is encoded, at
 * the position of the last token of its group, tok_pos[b] + m(g+1) - 1 when raw's token 0 of
 * sequence b sits at tok_pos[b]. That is the token with which the group completes and the entry
 * becomes visible (R9), and it does not depend on the span. R = 0: no rotation. */
static int kv_compress_core(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B,
                            int64_t T, int D, int m, int span, int64_t skip, const float* w,
                            const float* beta, unsigned char* out_rows, int out_fmt,
                            int64_t out_seq_stride, unsigned char* out_scales,
                            const int64_t* tok_pos, int R, double base, double* pre_out,
                            double* pi_out) {
    if (!raw || !w || !beta || !out_rows || B <= 0 || T < 0 || D <= 0 || m <= 0 || T % m ||
        span < m || skip < 0 || skip > T / m)
        return OC_EINVAL;
    if (R != 0 && (!tok_pos || R < 2 || R % 2 || R > D || !(base > 0.0) || isinf(base)))
        return OC_EINVAL;
    if (out_fmt == OC_FMT_FP4_E8M0 && (D % 32 || !out_scales)) return OC_EINVAL;
    if (out_fmt == OC_FMT_ROW_E4M3_BF16 && D < 64) return OC_EINVAL;
    int64_t G = T / m - skip, rb = oc_row_bytes(out_fmt, D);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++) {
        for (int64_t go = 0; go < G; go++) {
            int64_t g = go + skip, first = m * (g + 1) - span; /* token of span position 0 */
            double* x = (double*)malloc(sizeof(double) * (size_t)span * D);
            double* z = (double*)malloc(sizeof(double) * (size_t)span);
            double* c = (double*)malloc(sizeof(double) * (size_t)D);
            double zmax = -INFINITY;
            for (int j = 0; j < span; j++) {
                z[j] = -INFINITY; /* a token before the buffer: weight 0 */
                if (first + j < 0) continue;
                double s = 0.0;
                for (int d = 0; d < D; d++) {
                    x[(int64_t)j * D + d] =
                        load_elem(raw, raw_dtype, ((int64_t)b * raw_seq_stride + first + j) * D + d);
                    s += (double)w[d] * x[(int64_t)j * D + d];
                }
                z[j] = s + (double)beta[j];
                if (z[j] > zmax) zmax = z[j];
            }
            double den = 0.0;
            for (int j = 0; j < span; j++) { z[j] = exp(z[j] - zmax); den += z[j]; }
            for (int j = 0; j < span; j++) z[j] /= den; /* z now holds pi */
            for (int d = 0; d < D; d++) {
                double s = 0.0;
                for (int j = 0; j < span; j++)
                    if (first + j >= 0) s += z[j] * x[(int64_t)j * D + d];
                c[d] = s;
            }
            if (R) rope_row(c, D, R, (double)(tok_pos[b] + m * (g + 1) - 1), base, 0);
            int64_t orow = (int64_t)b * out_seq_stride + go;
            encode_row(c, out_fmt, D, out_rows + orow * rb,
                       out_fmt == OC_FMT_FP4_E8M0 ? out_scales + orow * (D / 32) : NULL);
            if (pre_out) memcpy(pre_out + ((int64_t)b * G + go) * D, c, sizeof(double) * D);
            if (pi_out) memcpy(pi_out + ((int64_t)b * G + go) * span, z, sizeof(double) * span);
            free(x); free(z); free(c);
        }
    }
    return OC_OK;
}

int oc_kv_compress_span(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B, int64_t T,
                        int D, int m, int span, int64_t skip, const float* w, const float* beta,
                        unsigned char* out_rows, int out_fmt, int64_t out_seq_stride,
                        unsigned char* out_scales, double* pre_out, double* pi_out) {
    return kv_compress_core(raw, raw_dtype, raw_seq_stride, B, T, D, m, span, skip, w, beta,
                            out_rows, out_fmt, out_seq_stride, out_scales, NULL, 0, 0.0, pre_out,
                            pi_out);
}

int oc_kv_compress_rope(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B, int64_t T,
                        int D, int m, int span, int64_t skip, const float* w, const float* beta,
                        unsigned char* out_rows, int out_fmt, int64_t out_seq_stride,
                        unsigned char* out_scales, const int64_t* tok_pos, int R, double base,
                        double* pre_out, double* pi_out) {
    if (R == 0) return OC_EINVAL;
    return kv_compress_core(raw, raw_dtype, raw_seq_stride, B, T, D, m, span, skip, w, beta,
                            out_rows, out_fmt, out_seq_stride, out_scales, tok_pos, R, base,
                            pre_out, pi_out);
}

int oc_kv_compress(const void* raw, int raw_dtype, int64_t raw_seq_stride, int B, int64_t T, int D,
                   int m, const float* w, const float* beta, unsigned char* out_rows, int out_fmt,
                   int64_t out_seq_stride, unsigned char* out_scales, double* pre_out,
                   double* pi_out) {
    return oc_kv_compress_span(raw, raw_dtype, raw_seq_stride, B, T, D, m, m, 0, w, beta, out_rows,
                               out_fmt, out_seq_stride, out_scales, pre_out, pi_out);
}

/* ------------------------------------------------------------------------------------------ */
/* Indexer score of one compressed entry for one query, exact.                                 */
/* [EXPL]: the lightning indexer scores compressed indexer keys against low-rank indexer       */
/* queries; [LLMB] "1. CSA": the indexer works in FP4.  With R7 the score is                   */
/*   score = sum_h sum_blocks 2^(Eq+Ek-254) * sum_{i in block} e2m1(q_i) e2m1(k_i).            */
/* 2*e2m1 is an integer in [-12, 12], so each block sum is an integer times 2^(Eq+Ek-256),    */
/* and the whole score is an integer times a power of two: it is summed exactly here.         */
/* *exact_ok reports whether fp32 arithmetic in ANY summation order reproduces the value:     */
/* the sum of all |products| over the finest granularity is < 2^24, and every granularity and */
/* magnitude is inside the binary32 normal range.                                              */
/* ------------------------------------------------------------------------------------------ */
static int e2m1_twice[16];
static int e2m1_twice_ready = 0;

static void init_e2m1_twice(void) {
    if (e2m1_twice_ready) return;
    for (int c = 0; c < 16; c++) e2m1_twice[c] = (int)(2.0 * oc_e2m1_value(c));
    e2m1_twice_ready = 1;
}

static double exact_score(const unsigned char* qc, const unsigned char* qs, int HI, int dI,
                          const unsigned char* kc, const unsigned char* ks, int* exact_ok) {
    int nb = dI / 32, nt = HI * nb;
    long long I[64];
    long long Sabs[64];
    int E[64];
    int emin = 1 << 30, emax = -(1 << 30);
    for (int h = 0; h < HI; h++) {
        for (int b = 0; b < nb; b++) {
            long long s = 0, sa = 0;
            for (int i = 32 * b; i < 32 * b + 32; i++) {
                int cq = (qc[h * (dI / 2) + i / 2] >> ((i & 1) ? 4 : 0)) & 15;
                int ck = (kc[i / 2] >> ((i & 1) ? 4 : 0)) & 15;
                long long p = (long long)e2m1_twice[cq] * e2m1_twice[ck];
                s += p;
                sa += p < 0 ? -p : p;
            }
            int t = h * nb + b;
            I[t] = s;
            Sabs[t] = sa;
            E[t] = (int)qs[h * nb + b] + (int)ks[b]; /* value = I * 2^(E-256) */
            if (E[t] < emin) emin = E[t];
            if (E[t] > emax) emax = E[t];
        }
    }
    /* exact sum as a 128-bit integer in units of 2^(emin-256) */
    int ok = (emax - emin) <= 100;
    double score;
    if (ok) {
        __int128 tot = 0, tabs = 0;
        for (int t = 0; t < nt; t++) {
            tot += (__int128)I[t] << (E[t] - emin);
            tabs += (__int128)Sabs[t] << (E[t] - emin);
        }
        __int128 lim = (__int128)1 << 24;
        ok = tabs < lim && (emin - 256) >= -126 && (emax - 256 + 24) < 127;
        long double mag = (long double)(tot < 0 ? -tot : tot);
        score = (double)ldexpl(tot < 0 ? -mag : mag, emin - 256);
    } else {
        long double s = 0.0L;
        for (int t = 0; t < nt; t++) s += ldexpl((long double)I[t], E[t] - 256);
        score = (double)s;
    }
    if (exact_ok) *exact_ok = ok;
    return score;
}

typedef struct { double s; int64_t g; } scored_t;

/* R8: score descending, then index ascending */
static int cmp_scored(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->g < y->g) ? -1 : (x->g > y->g);
}

/* ------------------------------------------------------------------------------------------ */
/* index_topk -- [BSWEN] "Component 3": score all compressed entries, keep the top-k;          */
/* [LLMB] "1. CSA": the top 1,024 compressed blocks.                                           */
/* q_codes [B][Q][HI][dI/2], q_scales [B][Q][HI][dI/32];                                       */
/* k_codes [B][k_seq_stride][dI/2], k_scales [B][k_seq_stride][dI/32];                         */
/* pos[B]: position of query 0; query i sees g < min(floor((pos+i+1)/m), N)   (R9).           */
/* idx_out [B][Q][k]; score_out (nullable) [B][Q][k] fp64; exact_out (nullable) [B][Q]: 1 if   */
/* every visible entry met the fp32-exactness condition of exact_score.                        */
/* ------------------------------------------------------------------------------------------ */
int oc_index_topk(const unsigned char* q_codes, const unsigned char* q_scales, int HI, int dI,
                  const unsigned char* k_codes, const unsigned char* k_scales, int64_t k_seq_stride,
                  int64_t N, const int64_t* pos, int m, int B, int Q, int k, int32_t* idx_out,
                  double* score_out, int* exact_out) {
    if (!q_codes || !q_scales || !k_codes || !k_scales || !pos || !idx_out) return OC_EINVAL;
    if (HI <= 0 || HI > 16 || dI <= 0 || dI % 32 || dI > 128 || m <= 0 || B <= 0 || Q <= 0 ||
        k <= 0 || N < 0)
        return OC_EINVAL;
    init_e2m1_twice();
    int cb = dI / 2, sb = dI / 32;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; b++) {
        for (int i = 0; i < Q; i++) {
            int64_t nv = (pos[b] + i + 1) / m;
            if (nv > N) nv = N;
            if (nv < 0) nv = 0;
            scored_t* arr = (scored_t*)malloc(sizeof(scored_t) * (size_t)(nv > 0 ? nv : 1));
            const unsigned char* qc = q_codes + ((int64_t)b * Q + i) * HI * cb;
            const unsigned char* qs = q_scales + ((int64_t)b * Q + i) * HI * sb;
            int all_ok = 1;
            for (int64_t g = 0; g < nv; g++) {
                int ok;
                int64_t row = (int64_t)b * k_seq_stride + g;
                arr[g].s = exact_score(qc, qs, HI, dI, k_codes + row * cb, k_scales + row * sb, &ok);
                arr[g].g = g;
                all_ok &= ok;
            }
            qsort(arr, (size_t)nv, sizeof(scored_t), cmp_scored);
            int64_t base = ((int64_t)b * Q + i) * k;
            for (int j = 0; j < k; j++) {
                idx_out[base + j] = (j < nv) ? (int32_t)arr[j].g : -1;
                if (score_out) score_out[base + j] = (j < nv) ? arr[j].s : -INFINITY;
            }
            if (exact_out) exact_out[(int64_t)b * Q + i] = all_ok;
            free(arr);
        }
    }
    return OC_OK;
}

/* every visible entry's exact score for one (sequence, query): tests compare them one by one */
int oc_index_scores(const unsigned char* q_codes, const unsigned char* q_scales, int HI, int dI,
                    const unsigned char* k_codes, const unsigned char* k_scales, int64_t n,
                    double* scores, int* exact_ok) {
    if (HI <= 0 || HI > 16 || dI <= 0 || dI % 32 || dI > 128 || n < 0) return OC_EINVAL;
    init_e2m1_twice();
    int cb = dI / 2, sb = dI / 32;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n; g++)
        scores[g] = exact_score(q_codes, q_scales, HI, dI, k_codes + g * cb, k_scales + g * sb,
                                exact_ok ? exact_ok + g : NULL);
    return OC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Attention over a set of shared K=V rows plus a per-head sink, in fp64.                      */
/* [EXPL]: each query attends to its selected compressed entries and a small window of recent */
/* uncompressed tokens; the sink lets a head's weights total less than one; K and V are one   */
/* shared row per entry (shared-KV multi-query layout).  With R12/R13:                         */
/*   s_j = scale * q.y_j,  M = max(sigma, max_j s_j),                                          */
/*   den = e^(sigma-M) + sum_j e^(s_j-M),  out = sum_j e^(s_j-M) y_j / den,  lse = M + ln den. */
/* Without a sink the e^(sigma-M) term is absent. An empty row set with no sink gives out = 0 */
/* and lse = -inf (a convention: the pages do not reach this case).                            */
/* ------------------------------------------------------------------------------------------ */
static void attend_rows(const double* q, const double* Y, int64_t n, int D, int has_sink,
                        double sigma, double scale, double* out, double* lse) {
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double M = has_sink ? sigma : -INFINITY;
    for (int64_t j = 0; j < n; j++) {
        double acc = 0.0;
        for (int d = 0; d < D; d++) acc += q[d] * Y[j * D + d];
        s[j] = scale * acc;
        if (s[j] > M) M = s[j];
    }
    for (int d = 0; d < D; d++) out[d] = 0.0;
    if (M == -INFINITY) { *lse = -INFINITY; free(s); return; }
    double den = has_sink ? exp(sigma - M) : 0.0;
    for (int64_t j = 0; j < n; j++) {
        double p = exp(s[j] - M);
        den += p;
        for (int d = 0; d < D; d++) out[d] += p * Y[j * D + d];
    }
    for (int d = 0; d < D; d++) out[d] /= den;
    *lse = M + log(den);
    free(s);
}

/* shared driver of csa / hca: rows = list (CSA: selected entries; HCA: all visible entries)
 * + window rows [i, i+w-1] of the window buffer with position >= 0 (R10).                 */
static int attend_common(const void* q, int q_dtype, int H, int D, const unsigned char* cache,
                         int fmt, int64_t cache_seq_stride, int64_t N, const int32_t* idx, int k,
                         int m, const unsigned char* win, int64_t win_seq_stride, int w,
                         const int64_t* pos, const float* sink, double scale, int B, int Q,
                         double* out, double* lse) {
    int64_t rb = oc_row_bytes(fmt, D);
    if (!q || !cache || !pos || !out || !lse || H <= 0 || D <= 0 || B <= 0 || Q <= 0 || w < 0 ||
        rb <= 0 || fmt == OC_FMT_FP4_E8M0 || (w > 0 && !win))
        return OC_EINVAL;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; b++) {
        for (int i = 0; i < Q; i++) {
            int64_t p = pos[b] + i;
            /* compressed rows */
            int64_t nc = 0;
            int64_t* list;
            if (idx) {
                list = (int64_t*)malloc(sizeof(int64_t) * (size_t)(k > 0 ? k : 1));
                for (int j = 0; j < k; j++) {
                    int32_t g = idx[((int64_t)b * Q + i) * k + j];
                    if (g == -1) continue;
                    if (g < 0 || g >= N) { bad = 1; continue; }
                    list[nc++] = g;
                }
            } else {
                int64_t nv = (p + 1) / m;
                if (nv > N) nv = N;
                if (nv < 0) nv = 0;
                list = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nv > 0 ? nv : 1));
                for (int64_t g = 0; g < nv; g++) list[nc++] = g;
            }
            int64_t nrows = nc + w;
            double* Y = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1) * D);
            int64_t n = 0;
            for (int64_t j = 0; j < nc; j++)
                decode_row(cache + ((int64_t)b * cache_seq_stride + list[j]) * rb, NULL, fmt, D,
                           Y + (n++) * D);
            for (int r = i; r < i + w; r++) {
                int64_t rp = pos[b] - (w - 1) + r; /* position held by window row r */
                if (rp < 0) continue;
                decode_row(win + ((int64_t)b * win_seq_stride + r) * rb, NULL, fmt, D, Y + (n++) * D);
            }
            double* qv = (double*)malloc(sizeof(double) * (size_t)D);
            for (int h = 0; h < H; h++) {
                int64_t qo = (((int64_t)b * Q + i) * H + h) * D;
                for (int d = 0; d < D; d++) qv[d] = load_elem(q, q_dtype, qo + d);
                attend_rows(qv, Y, n, D, sink != NULL, sink ? (double)sink[h] : 0.0, scale,
                            out + qo, lse + ((int64_t)b * Q + i) * H + h);
            }
            free(qv); free(Y); free(list);
        }
    }
    return bad ? OC_EINVAL : OC_OK;
}

/* CSA: selected compressed entries (idx, -1 = empty slot) + window + sink.
 * [EXPL] "How compress-then-sparsify attention works"; [BSWEN] "Component 3". */
int oc_csa_attend(const void* q, int q_dtype, int H, int D, const unsigned char* cache, int fmt,
                  int64_t cache_seq_stride, int64_t N, const int32_t* idx, int k,
                  const unsigned char* win, int64_t win_seq_stride, int w, const int64_t* pos,
                  const float* sink, double scale, int B, int Q, double* out, double* lse) {
    if (!idx || k < 0) return OC_EINVAL;
    return attend_common(q, q_dtype, H, D, cache, fmt, cache_seq_stride, N, idx, k, 1, win,
                         win_seq_stride, w, pos, sink, scale, B, Q, out, lse);
}

/* HCA: every visible compressed entry (no selection) + window + sink.
 * [EXPL]: the same idea with a larger group and no sparse selection;
 * [LLMB] "2. HCA": dense attention over all 128x-compressed entries. */
int oc_hca_attend(const void* q, int q_dtype, int H, int D, const unsigned char* cache, int fmt,
                  int64_t cache_seq_stride, int64_t N, int m, const unsigned char* win,
                  int64_t win_seq_stride, int w, const int64_t* pos, const float* sink,
                  double scale, int B, int Q, double* out, double* lse) {
    if (m <= 0) return OC_EINVAL;
    return attend_common(q, q_dtype, H, D, cache, fmt, cache_seq_stride, N, NULL, 0, m, win,
                         win_seq_stride, w, pos, sink, scale, B, Q, out, lse);
}
