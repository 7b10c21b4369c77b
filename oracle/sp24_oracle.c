/*
 * sp24_oracle.c -- CPU oracle for 2:4 semi-structured sparsity.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * It is written to be read against the pages, not to be fast: plain loops,
 * fp64 arithmetic, OpenMP over output rows only.
 *
 * What it computes (sources: "2:4 Structured Sparsity Explained", sections
 * "How 2:4 sparsity works" and "How to make a model 2:4 sparse";
 * "Production 2:4 Structured Sparsity for LLMs", section "From Unstructured
 * Pruning to Hardware-Accelerable Sparsity"; the 2:4-versus-quantization
 * paper, section 2 "Sparse tensor cores"):
 *
 *   prune     in every group of 4 consecutive elements along the reduction
 *             axis K keep the 2 of largest magnitude, zero the other 2
 *             (ties between equal magnitudes go to the lower index);
 *   compress  keep the 2 values of each group (half the storage) plus a
 *             2-bit position 0..3 for each kept value;
 *   decompress  the inverse: kept values back in place, +0.0 elsewhere;
 *   GEMM      Y = X * W^T, computed as the plain dense product of the
 *             decompressed operand with the other operand, in fp64.
 *   audit     the layer-level manifest metrics of "Production 2:4 Structured
 *             Sparsity for LLMs" ("Audit Artifacts and Key Metrics"): layer
 *             counts, selection ratio and Sparse GPU-Time Coverage.
 *
 * Readings of points the pages leave open (each is also listed in the
 * design notes):
 *   - "magnitude" is compared as the integer value of the sign-stripped bit
 *     pattern (monotone in |x| for every non-NaN value; +0 and -0 tie; NaN
 *     ranks above Inf);
 *   - the two kept values are stored in ascending position order;
 *   - metadata: one 4-bit nibble per group, p0 | p1 << 2 with p0 < p1,
 *     packed little-endian 8 groups to a uint32 word, rows of ceil(K/32)
 *     words, unused high nibbles zero;
 *   - dropped positions decompress to +0.0 (bit pattern 0);
 *   - fp8 is OCP E4M3 ("e4m3fn": no Inf, 0x7F/0xFF are NaN, max 448) with one
 *     fp32 scale per row of each operand, applied to the fp64 result;
 *   - int8 is two's complement, its magnitude |x| (-128 ranks above 127),
 *     with per-row fp32 scales as for fp8;
 *   - fused online fp8 path: per-row scale max|x| / 448 and codes e4m3(x / s)
 *     rounded to nearest even and saturated at 448, both in fp32; pruning
 *     acts on the codes (quantize first, then prune);
 *   - fused online int8 path: per-row scale max|x| / 127 and codes
 *     int8(x / s), the quotient rounded to the nearest integer (ties to
 *     even) and saturated to [-127, 127], both in fp32; a NaN quotient codes
 *     to 0; pruning again acts on the codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_BF16 = 1, OR_E4M3 = 2, OR_F32 = 3, OR_I8 = 4 };
enum { OR_SPARSE_W = 0, OR_SPARSE_X = 1 };
enum { OR_OK = 0, OR_E_ARG = 1 };

/* ------------------------------------------------------------------ */
/* Number formats, decoded from their definitions.                      */
/* ------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                  /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);      /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* IEEE binary32: 1 sign, 8 exponent (bias 127), 23 fraction bits. */
static double decode_f32_bits(uint32_t u)
{
    int sign = (u >> 31) & 1;
    int e = (u >> 23) & 0xff;
    uint32_t f = u & 0x7fffff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -149);
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(0x800000u + f), e - 150);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32. */
double oracle_decode_bf16(uint16_t h) { return decode_f32_bits((uint32_t)h << 16); }

double oracle_decode_f32(uint32_t u) { return decode_f32_bits(u); }

/* OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN; largest finite value 448. */
double oracle_decode_e4m3(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xf;
    int f = b & 7;
    double v;
    if ((b & 0x7f) == 0x7f)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);                   /* subnormal: f/8 * 2^-6 */
    else
        v = ldexp((double)(8 + f), e - 10);         /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

static double decode_elem(int dt, const void *base, int64_t i)
{
    switch (dt) {
    case OR_F16:  return oracle_decode_f16(((const uint16_t *)base)[i]);
    case OR_BF16: return oracle_decode_bf16(((const uint16_t *)base)[i]);
    case OR_E4M3: return oracle_decode_e4m3(((const uint8_t *)base)[i]);
    case OR_F32:  return oracle_decode_f32(((const uint32_t *)base)[i]);
    case OR_I8:   return (double)((const int8_t *)base)[i];     /* two's complement */
    }
    return NAN;
}

/* Round-to-nearest-even encoders from fp64, written from the same format
 * definitions.  `man_bits` fraction bits, exponent bias `bias`, largest
 * biased exponent `emax_biased` for finite values.  Returns the magnitude
 * bits; the caller adds the sign.  rint() rounds half to even in the
 * default rounding mode, and every scaled value here is exact in fp64. */
static uint32_t encode_mag_rne(double a, int man_bits, int bias, int emax_biased)
{
    uint32_t inf_bits = (uint32_t)(emax_biased + 1) << man_bits;
    if (isinf(a))
        return inf_bits;
    int E;
    (void)frexp(a, &E);                     /* a in [2^(E-1), 2^E) */
    int e = E - 1;                          /* unbiased exponent */
    int emin = 1 - bias;                    /* smallest normal exponent */
    if (a == 0.0)
        return 0;
    if (e < emin) {
        /* subnormal range: units of 2^(emin - man_bits) */
        double q = rint(ldexp(a, man_bits - emin));
        return (uint32_t)q;                 /* q == 2^man_bits gives the smallest normal */
    }
    double q = rint(ldexp(a, man_bits - e)); /* in [2^man_bits, 2^(man_bits+1)] */
    if (q == ldexp(1.0, man_bits + 1)) {
        q = ldexp(1.0, man_bits);
        e += 1;
    }
    int be = e + bias;
    if (be > emax_biased)
        return inf_bits;
    return ((uint32_t)be << man_bits) | ((uint32_t)q - (1u << man_bits));
}

uint16_t oracle_encode_f16(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    return s | (uint16_t)encode_mag_rne(fabs(x), 10, 15, 30);
}

uint16_t oracle_encode_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    return s | (uint16_t)encode_mag_rne(fabs(x), 7, 127, 254);
}

/* OCP e4m3fn from fp64, round to nearest even, saturating: magnitudes at or
 * above the largest finite value 448 give 448 (the format has no infinity);
 * NaN gives the NaN pattern 0x7F.  Below 448 the rounding can reach 448 but
 * never the next step up (480, which would need a >= 464). */
uint8_t oracle_encode_e4m3(double x)
{
    if (isnan(x))
        return 0x7f;
    uint8_t s = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0)
        return s | 0x7e;
    return s | (uint8_t)encode_mag_rne(a, 3, 7, 15);
}

void oracle_decode_array(int dt, const void *src, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode_elem(dt, src, i);
}

void oracle_encode_array(int dt, const double *src, int64_t n, void *out)
{
    for (int64_t i = 0; i < n; ++i) {
        if (dt == OR_F16)
            ((uint16_t *)out)[i] = oracle_encode_f16(src[i]);
        else if (dt == OR_BF16)
            ((uint16_t *)out)[i] = oracle_encode_bf16(src[i]);
    }
}

/* ------------------------------------------------------------------ */
/* Pruning: the 2 largest magnitudes of each group of 4.                */
/* ------------------------------------------------------------------ */

static int elem_bytes(int dt)
{
    return dt == OR_E4M3 || dt == OR_I8 ? 1 : (dt == OR_F32 ? 4 : 2);
}

/* Raw bit pattern of element i. */
static uint32_t elem_bits(int dt, const void *base, int64_t i)
{
    if (dt == OR_E4M3 || dt == OR_I8)
        return ((const uint8_t *)base)[i];
    return ((const uint16_t *)base)[i];
}

/* Magnitude key: the bit pattern with the sign bit cleared (sign-magnitude
 * float formats), or |x| for two's complement int8 (-128 -> 128). */
static uint32_t magnitude_key(int dt, uint32_t bits)
{
    if (dt == OR_I8) {
        int v = (int8_t)(uint8_t)bits;
        return (uint32_t)(v < 0 ? -v : v);
    }
    return dt == OR_E4M3 ? (bits & 0x7f) : (bits & 0x7fff);
}

/* Element j beats element i when it is larger in magnitude, or equal in
 * magnitude and at a lower position. */
static int beats(const uint32_t key[4], int j, int i)
{
    return key[j] > key[i] || (key[j] == key[i] && j < i);
}

/* Keeps the elements that fewer than two others beat: exactly two of the
 * four, returned as p0 < p1. */
void oracle_select_pair(const uint32_t key[4], int *p0, int *p1)
{
    int kept[2], nk = 0;
    for (int i = 0; i < 4; ++i) {
        int beaten_by = 0;
        for (int j = 0; j < 4; ++j)
            if (j != i && beats(key, j, i))
                ++beaten_by;
        if (beaten_by < 2)
            kept[nk++] = i;
    }
    *p0 = kept[0];
    *p1 = kept[1];
}

int64_t oracle_meta_words_per_row(int64_t K) { return (K + 31) / 32; }

/* Compress rows x K (row stride ld_src elements) into values rows x K/2 and
 * meta rows x ceil(K/32). */
int oracle_prune_compress(int dt, int64_t rows, int64_t K, const void *src,
                          int64_t ld_src, void *values, uint32_t *meta)
{
    if (dt != OR_F16 && dt != OR_BF16 && dt != OR_E4M3 && dt != OR_I8)
        return OR_E_ARG;
    if (rows < 0 || K < 0 || K % 4 != 0 || ld_src < K)
        return OR_E_ARG;
    int eb = elem_bytes(dt);
    int64_t mw = oracle_meta_words_per_row(K);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const char *row = (const char *)src + (size_t)(r * ld_src) * eb;
        char *vrow = (char *)values + (size_t)(r * (K / 2)) * eb;
        uint32_t *mrow = meta + r * mw;
        for (int64_t w = 0; w < mw; ++w)
            mrow[w] = 0;
        for (int64_t g = 0; g < K / 4; ++g) {
            uint32_t key[4];
            for (int i = 0; i < 4; ++i)
                key[i] = magnitude_key(dt, elem_bits(dt, row, 4 * g + i));
            int p0, p1;
            oracle_select_pair(key, &p0, &p1);
            memcpy(vrow + (2 * g) * eb, row + (4 * g + p0) * eb, eb);
            memcpy(vrow + (2 * g + 1) * eb, row + (4 * g + p1) * eb, eb);
            uint32_t nibble = (uint32_t)p0 | ((uint32_t)p1 << 2);
            mrow[g / 8] |= nibble << (4 * (g % 8));
        }
    }
    return OR_OK;
}

/* Inverse of the above: all positions +0.0, then the first kept value at
 * its p0 and the second at its p1 (in that order). */
int oracle_decompress(int dt, int64_t rows, int64_t K, const void *values,
                      const uint32_t *meta, void *dst, int64_t ld_dst)
{
    if (dt != OR_F16 && dt != OR_BF16 && dt != OR_E4M3 && dt != OR_I8)
        return OR_E_ARG;
    if (rows < 0 || K < 0 || K % 4 != 0 || ld_dst < K)
        return OR_E_ARG;
    int eb = elem_bytes(dt);
    int64_t mw = oracle_meta_words_per_row(K);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        char *row = (char *)dst + (size_t)(r * ld_dst) * eb;
        const char *vrow = (const char *)values + (size_t)(r * (K / 2)) * eb;
        const uint32_t *mrow = meta + r * mw;
        memset(row, 0, (size_t)K * eb);
        for (int64_t g = 0; g < K / 4; ++g) {
            uint32_t nibble = (mrow[g / 8] >> (4 * (g % 8))) & 0xf;
            int p0 = nibble & 3, p1 = (nibble >> 2) & 3;
            memcpy(row + (4 * g + p0) * eb, vrow + (2 * g) * eb, eb);
            memcpy(row + (4 * g + p1) * eb, vrow + (2 * g + 1) * eb, eb);
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Per-row fp8 quantization (the fused online path).                   */
/* ------------------------------------------------------------------ */

/* Rows x K of f16 or bf16 (row stride ld_src elements) to e4m3 codes q
 * (rows x K, dense) and one fp32 scale per row (the 2:4-versus-quantization
 * paper, section 2 "Quantization": one scale per row; sections 3.5 and 4.2:
 * the online operand is quantized, pruned and compressed in one pass).  The
 * scale maps the row's largest magnitude to the largest finite e4m3 value:
 * s = max|x| / 448 (s = 1 for an all-zero row), and q = e4m3(x / s).  The
 * scale and the quotients are computed in fp32 (C float arithmetic, round
 * to nearest even), not fp64: they decide integer codes, and the GPU takes
 * the same decisions in the same precision.  Pruning then works on q, so
 * that the kept values are exactly what the GEMM consumes. */
int oracle_quantize_e4m3_rows(int dt, int64_t rows, int64_t K, const void *src, int64_t ld_src,
                              uint8_t *q, float *scales)
{
    if (dt != OR_F16 && dt != OR_BF16)
        return OR_E_ARG;
    if (rows < 0 || K < 0 || ld_src < K)
        return OR_E_ARG;
    int eb = elem_bytes(dt);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const char *row = (const char *)src + (size_t)(r * ld_src) * eb;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)decode_elem(dt, row, k);     /* exact: every f16/bf16 is a float */
            float a = fabsf(v);
            if (a > amax)
                amax = a;
        }
        float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        scales[r] = sc;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)decode_elem(dt, row, k);
            float t = v / sc;
            q[r * K + k] = oracle_encode_e4m3((double)t);
        }
    }
    return OR_OK;
}

/* The int8 code of an fp32 quotient: round to the nearest integer, ties to
 * even (the C default rounding mode of nearbyintf), then saturate to
 * [-127, 127], the symmetric int8 range; a NaN quotient (only from an
 * infinite scale meeting an infinite element) codes to 0. */
int8_t oracle_encode_i8(float t)
{
    if (isnan(t))
        return 0;
    float r = nearbyintf(t);
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

/* The same per-row quantization to symmetric int8 (the 2:4-versus-
 * quantization paper, section 2 "Quantization": one scale per row, and 4.2
 * "Speed": 2:4 with INT8): s = max|x| / 127 (s = 1 for an all-zero row), q =
 * int8(x / s), the scale and the quotients in fp32 as above; a NaN does not
 * count toward the maximum. */
int oracle_quantize_i8_rows(int dt, int64_t rows, int64_t K, const void *src, int64_t ld_src,
                            int8_t *q, float *scales)
{
    if (dt != OR_F16 && dt != OR_BF16)
        return OR_E_ARG;
    if (rows < 0 || K < 0 || ld_src < K)
        return OR_E_ARG;
    int eb = elem_bytes(dt);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const char *row = (const char *)src + (size_t)(r * ld_src) * eb;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf((float)decode_elem(dt, row, k));
            if (a > amax)
                amax = a;
        }
        float sc = amax > 0.0f ? amax / 127.0f : 1.0f;
        scales[r] = sc;
        for (int64_t k = 0; k < K; ++k)
            q[r * K + k] = oracle_encode_i8((float)decode_elem(dt, row, k) / sc);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* GEMM: R[i][n] = sum_k x[m_i][k] * w[n][k]  (* s_x[m_i] * s_w[n])     */
/* ------------------------------------------------------------------ */

/* Decoded dense rows: either read straight from a dense operand or
 * decompressed from (values, meta) first. */
static void dense_row_f64(int dt, int64_t K, const void *dense, int64_t r, double *out)
{
    int eb = elem_bytes(dt);
    const char *row = (const char *)dense + (size_t)(r * K) * eb;
    for (int64_t k = 0; k < K; ++k)
        out[k] = decode_elem(dt, row, k);
}

static void sparse_row_f64(int dt, int64_t K, const void *values, const uint32_t *meta,
                           int64_t r, double *out)
{
    int eb = elem_bytes(dt);
    char *tmp = (char *)malloc((size_t)K * eb);
    oracle_decompress(dt, 1, K, (const char *)values + (size_t)(r * (K / 2)) * eb,
                      meta + r * oracle_meta_words_per_row(K), tmp, K);
    for (int64_t k = 0; k < K; ++k)
        out[k] = decode_elem(dt, tmp, k);
    free(tmp);
}

/*
 * R (nm x N, fp64) for the X rows listed in mrows (nm of them).
 * x_vals/x_meta: when non-NULL, X is given compressed (the activation is
 * the sparse operand); otherwise X is the dense x_dense (M x K).
 * w_vals/w_meta: likewise for W (N x K).
 * scale_x[M], scale_w[N]: NULL, or fp32 scales multiplied into R in fp64.
 */
int oracle_gemm(int dt, int64_t M, int64_t N, int64_t K,
                const void *x_dense, const void *x_vals, const uint32_t *x_meta,
                const void *w_dense, const void *w_vals, const uint32_t *w_meta,
                const float *scale_x, const float *scale_w,
                const int64_t *mrows, int64_t nm, double *R)
{
    if (dt != OR_F16 && dt != OR_BF16 && dt != OR_E4M3 && dt != OR_I8)
        return OR_E_ARG;
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0 || nm < 0)
        return OR_E_ARG;
    if ((x_dense == NULL) == (x_vals == NULL) || (w_dense == NULL) == (w_vals == NULL))
        return OR_E_ARG;
    for (int64_t i = 0; i < nm; ++i)
        if (mrows[i] < 0 || mrows[i] >= M)
            return OR_E_ARG;

    double *xs = (double *)malloc(sizeof(double) * (size_t)(nm * K + 1));
    for (int64_t i = 0; i < nm; ++i) {
        if (x_vals)
            sparse_row_f64(dt, K, x_vals, x_meta, mrows[i], xs + i * K);
        else
            dense_row_f64(dt, K, x_dense, mrows[i], xs + i * K);
    }

    #pragma omp parallel
    {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)(K + 1));
        #pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            if (w_vals)
                sparse_row_f64(dt, K, w_vals, w_meta, n, wrow);
            else
                dense_row_f64(dt, K, w_dense, n, wrow);
            for (int64_t i = 0; i < nm; ++i) {
                const double *x = xs + i * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += x[k] * wrow[k];
                if (scale_x)
                    acc *= (double)scale_x[mrows[i]];
                if (scale_w)
                    acc *= (double)scale_w[n];
                R[i * N + n] = acc;
            }
        }
        free(wrow);
    }
    free(xs);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Layer-level audit metrics ("Production 2:4 Structured Sparsity for   */
/* LLMs", section "Audit Artifacts and Key Metrics"; playbook step 3).  */
/* ------------------------------------------------------------------ */

/*
 * n distinct layers, layer i standing for count[i] identical model layers.
 * Walks the model layer by layer:
 *   every layer is a candidate; eligible[i] marks the eligible ones;
 *   a layer runs sparse iff it is eligible and its choice is sparse;
 *   every other layer falls back to dense;
 *   its GPU time is t_sparse + t_compress when it runs sparse, else t_dense.
 * Then
 *   eligibility ratio        = eligible / candidate
 *   sparse selection ratio   = sparse / eligible
 *   Sparse GPU-Time Coverage = (time of the sparse layers) /
 *                              (time of every layer + other_time)
 * with 0 for a zero denominator.
 * counts_out: candidate, eligible, sparse, fallback.
 * ratios_out: eligibility, selection, sparse time, total time, coverage.
 */
int oracle_audit(int64_t n, const int *eligible, const int *sparse, const double *t_sparse,
                 const double *t_compress, const double *t_dense, const int64_t *count,
                 double other_time, int64_t *counts_out, double *ratios_out)
{
    if (n < 0)
        return OR_E_ARG;
    int64_t candidate = 0, n_eligible = 0, n_sparse = 0, n_dense = 0;
    double sparse_time = 0.0, all_time = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t c = 0; c < count[i]; ++c) {
            candidate += 1;
            if (eligible[i])
                n_eligible += 1;
            if (eligible[i] && sparse[i]) {
                n_sparse += 1;
                sparse_time += t_sparse[i] + t_compress[i];
                all_time += t_sparse[i] + t_compress[i];
            } else {
                n_dense += 1;
                all_time += t_dense[i];
            }
        }
    }
    all_time += other_time;
    counts_out[0] = candidate;
    counts_out[1] = n_eligible;
    counts_out[2] = n_sparse;
    counts_out[3] = n_dense;
    ratios_out[0] = candidate > 0 ? (double)n_eligible / (double)candidate : 0.0;
    ratios_out[1] = n_eligible > 0 ? (double)n_sparse / (double)n_eligible : 0.0;
    ratios_out[2] = sparse_time;
    ratios_out[3] = all_time;
    ratios_out[4] = all_time > 0.0 ? sparse_time / all_time : 0.0;
    return OR_OK;
}

/* Number of worker threads OpenMP will use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of worker threads of later calls (n >= 1), so that the CPU
 * baseline can be timed on all threads and on one. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}
