/*
 * CPU oracle for the tiled GEMM path.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the reference the HIP library is checked against.  It is plain
 * C, shares no header, helper or constant with the HIP library, and is only
 * ever loaded by the tests, by the smoke check and by the CPU-baseline leg of
 * the benchmark.  Nothing in the product path may call it.
 *
 * What it computes (the plain definition, written out):
 *
 *   C[i,j] = sum_{k=0..K-1} a(i,k) * b(k,j)             (k ascending, fp64)
 *   optionally  C[i,j] += bias[j]   then   C[i,j] = max(C[i,j], 0)
 *
 * where a, b and bias are the exact values of the fp16 / bf16 (or fp32) inputs.  The
 * unrounded fp64 value is returned as `ref` (tolerance check) and the same
 * value rounded ONCE to the output type, IEEE round-to-nearest-even, as
 * `ref_q` (bit-exact check).
 *
 * Sources on the pages:
 *  - the computation and its operands' strides: "Using Triton to optimise GEMM
 *    across chips" (yfxerp), section 2.1 (minimal GEMM kernel), and the Gluon
 *    page's matmul example (masked loads, fp32 accumulation);
 *  - fp16 output of an fp32 accumulator: FlagOS cross-chip page, section 3.1
 *    (baseline kernel casting the accumulator to fp16 on store);
 *  - fused bias + ReLU in the same block: yfxerp page, section 3.4;
 *  - accumulate in at least fp32: "Triton study notes", section 2.1.
 * The pages never state the rounding mode; round-to-nearest-even is taken
 * (the IEEE default).  ReLU of a non-positive value is +0.0.
 *
 * Grouped (MoE) variant: for expert e, rows offsets[e] .. offsets[e+1]-1 of X
 * are multiplied by W[e] (a K x N matrix), writing the same rows of Y.  The
 * yfxerp page, section 2.3, only says that an MoE layer chains dozens of
 * GEMMs; this packing (rows sorted by expert, exclusive prefix offsets) is the
 * plainest reading.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_F32 = 2 };

/* ---------------------------------------------------------------------------
 * Binary16 / bfloat16 / binary32 <-> double, from the IEEE 754 field
 * definitions.
 *   fp16 : 1 sign, 5 exponent (bias 15), 10 fraction bits
 *   bf16 : 1 sign, 8 exponent (bias 127), 7 fraction bits
 *   fp32 : 1 sign, 8 exponent (bias 127), 23 fraction bits
 * ------------------------------------------------------------------------- */
typedef struct {
    int frac_bits; /* p  */
    int exp_bits;
    int bias;
} orc_format;

static orc_format fmt_of(int dtype) {
    orc_format f;
    if (dtype == ORC_F16)      { f.frac_bits = 10; f.exp_bits = 5; f.bias = 15; }
    else if (dtype == ORC_F32) { f.frac_bits = 23; f.exp_bits = 8; f.bias = 127; }
    else                       { f.frac_bits = 7;  f.exp_bits = 8; f.bias = 127; }
    return f;
}

static double decode_fmt(uint64_t bits, orc_format f) {
    int sign = (int)((bits >> (f.frac_bits + f.exp_bits)) & 1u);
    uint64_t emask = (1u << f.exp_bits) - 1u;
    uint64_t e = (bits >> f.frac_bits) & emask;
    uint64_t frac = bits & ((1ull << f.frac_bits) - 1u);
    double v;
    if (e == emask) {
        v = frac ? NAN : INFINITY;
    } else if (e == 0) {
        /* subnormal: frac * 2^(1 - bias - p) */
        v = ldexp((double)frac, 1 - f.bias - f.frac_bits);
    } else {
        v = ldexp((double)((1ull << f.frac_bits) + frac), (int)e - f.bias - f.frac_bits);
    }
    return sign ? -v : v;
}

/* Round a double once to the target format, ties to even.  The value is
 * scaled by a power of two so that one unit in the last place becomes 1.0,
 * rounded with rint() (round-half-even under the default rounding mode) and
 * scaled back; both scalings are exact in double for every finite input of
 * the magnitudes reachable here. */
static uint64_t encode_fmt(double x, orc_format f) {
    int emax = f.bias;            /* largest unbiased exponent of a finite value */
    int emin = 1 - f.bias;        /* smallest normal exponent                   */
    uint64_t emask = (1u << f.exp_bits) - 1u;
    uint64_t sign = signbit(x) ? (1ull << (f.frac_bits + f.exp_bits)) : 0u;
    if (isnan(x)) {
        /* quiet NaN: exponent all ones, top fraction bit set */
        return sign | (emask << f.frac_bits) | (1ull << (f.frac_bits - 1));
    }
    double a = fabs(x);
    if (isinf(a)) return sign | (emask << f.frac_bits);
    if (a == 0.0) return sign;

    int e2;
    (void)frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1)            */
    int E = e2 - 1;               /* floor(log2 a)                          */
    if (E < emin) E = emin;       /* subnormal range shares emin's quantum */
    double quantum_exp = (double)(E - f.frac_bits);
    double n = rint(ldexp(a, -(int)quantum_exp)); /* integer number of quanta */
    double v = ldexp(n, (int)quantum_exp);        /* rounded magnitude        */

    if (v >= ldexp(1.0, emax + 1))                /* rounds past the largest finite */
        return sign | (emask << f.frac_bits);

    if (v < ldexp(1.0, emin)) {
        /* subnormal (or zero): fraction field = number of quanta at emin */
        return sign | (uint64_t)n;
    }
    int ev;
    (void)frexp(v, &ev);
    int Ev = ev - 1;
    double frac = ldexp(v, f.frac_bits - Ev) - ldexp(1.0, f.frac_bits);
    return sign | ((uint64_t)(Ev + f.bias) << f.frac_bits) | (uint64_t)frac;
}

double orc_decode(uint16_t bits, int dtype) { return decode_fmt(bits, fmt_of(dtype)); }
uint16_t orc_encode(double x, int dtype) { return (uint16_t)encode_fmt(x, fmt_of(dtype)); }
double orc_decode32(uint32_t bits) { return decode_fmt(bits, fmt_of(ORC_F32)); }
uint32_t orc_encode32(double x) { return (uint32_t)encode_fmt(x, fmt_of(ORC_F32)); }

void orc_decode32_array(const uint32_t* src, double* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_decode32(src[i]);
}

void orc_encode32_array(const double* src, uint32_t* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_encode32(src[i]);
}

void orc_decode_array(const uint16_t* src, double* dst, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_decode(src[i], dtype);
}

void orc_encode_array(const double* src, uint16_t* dst, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_encode(src[i], dtype);
}

/* Epilogue of one element: optional bias add, optional ReLU (to +0.0). */
static double epilogue(double acc, const uint16_t* bias, int64_t j, int dtype, int relu) {
    double v = acc;
    if (bias) v = v + orc_decode(bias[j], dtype);
    if (relu) v = (v > 0.0) ? v : 0.0;
    return v;
}

/* ---------------------------------------------------------------------------
 * Dense GEMM, full output.  A is M x K with row stride lda, B is K x N with row
 * stride ldb (elements; unit inner stride).  ref / ref_q are M x N, dense.
 * Rows are split across threads; each output element is still the k-ascending
 * fp64 sum, so the thread count does not change any result.
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t* A; const double* Bd; const uint16_t* bias;
    int64_t N, K, lda; int dtype, relu;
    double* ref; uint16_t* ref_q;
    int64_t row_begin, row_end;
} rows_job;

static void* rows_worker(void* p) {
    rows_job* j = (rows_job*)p;
    double* arow = (double*)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
    for (int64_t i = j->row_begin; i < j->row_end; ++i) {
        for (int64_t k = 0; k < j->K; ++k) arow[k] = orc_decode(j->A[i * j->lda + k], j->dtype);
        for (int64_t n = 0; n < j->N; ++n) acc[n] = 0.0;
        for (int64_t k = 0; k < j->K; ++k) {
            const double a = arow[k];
            const double* brow = j->Bd + k * j->N;
            for (int64_t n = 0; n < j->N; ++n) acc[n] += a * brow[n];
        }
        for (int64_t n = 0; n < j->N; ++n) {
            double v = epilogue(acc[n], j->bias, n, j->dtype, j->relu);
            if (j->ref) j->ref[i * j->N + n] = v;
            if (j->ref_q) j->ref_q[i * j->N + n] = orc_encode(v, j->dtype);
        }
    }
    free(arow);
    free(acc);
    return NULL;
}

static int run_rows(const uint16_t* A, const double* Bd, const uint16_t* bias,
                    int64_t M, int64_t N, int64_t K, int64_t lda, int dtype, int relu,
                    double* ref, uint16_t* ref_q, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = (int)(M > 0 ? M : 1);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    rows_job* jobs = (rows_job*)malloc(sizeof(rows_job) * (size_t)nthreads);
    int64_t per = (M + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        rows_job* j = &jobs[t];
        j->A = A; j->Bd = Bd; j->bias = bias; j->N = N; j->K = K; j->lda = lda;
        j->dtype = dtype; j->relu = relu; j->ref = ref; j->ref_q = ref_q;
        j->row_begin = t * per;
        j->row_end = (t + 1) * per < M ? (t + 1) * per : M;
        if (j->row_begin > j->row_end) j->row_begin = j->row_end;
        pthread_create(&th[t], NULL, rows_worker, j);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return 0;
}

static double* decode_matrix(const uint16_t* B, int64_t rows, int64_t cols, int64_t ld, int dtype) {
    double* d = (double*)malloc(sizeof(double) * (size_t)(rows * cols > 0 ? rows * cols : 1));
    if (!d) return NULL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) d[r * cols + c] = orc_decode(B[r * ld + c], dtype);
    return d;
}

int orc_gemm(const uint16_t* A, const uint16_t* B, const uint16_t* bias,
             int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
             int dtype, int relu, double* ref, uint16_t* ref_q, int nthreads) {
    if (M <= 0 || N <= 0) return 0;
    double* Bd = decode_matrix(B, K, N, ldb, dtype);
    if (!Bd) return -1;
    run_rows(A, Bd, bias, M, N, K, lda, dtype, relu, ref, ref_q, nthreads);
    free(Bd);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Dense GEMM at a list of (row, col) positions: one k-ascending fp64 dot
 * product per requested element.  Used where the full output is too large.
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t* A; const uint16_t* B; const uint16_t* bias;
    int64_t K, lda, ldb; int dtype, relu;
    const int64_t* rows; const int64_t* cols;
    double* ref; uint16_t* ref_q;
    int64_t begin, end;
} sample_job;

static void* sample_worker(void* p) {
    sample_job* j = (sample_job*)p;
    for (int64_t s = j->begin; s < j->end; ++s) {
        int64_t i = j->rows[s], c = j->cols[s];
        double acc = 0.0;
        for (int64_t k = 0; k < j->K; ++k)
            acc += orc_decode(j->A[i * j->lda + k], j->dtype) *
                   orc_decode(j->B[k * j->ldb + c], j->dtype);
        double v = epilogue(acc, j->bias, c, j->dtype, j->relu);
        if (j->ref) j->ref[s] = v;
        if (j->ref_q) j->ref_q[s] = orc_encode(v, j->dtype);
    }
    return NULL;
}

int orc_gemm_sampled(const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                     int64_t K, int64_t lda, int64_t ldb, int dtype, int relu,
                     const int64_t* rows, const int64_t* cols, int64_t count,
                     double* ref, uint16_t* ref_q, int nthreads) {
    if (count <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > count) nthreads = (int)count;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    sample_job* jobs = (sample_job*)malloc(sizeof(sample_job) * (size_t)nthreads);
    int64_t per = (count + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        sample_job* j = &jobs[t];
        j->A = A; j->B = B; j->bias = bias; j->K = K; j->lda = lda; j->ldb = ldb;
        j->dtype = dtype; j->relu = relu; j->rows = rows; j->cols = cols;
        j->ref = ref; j->ref_q = ref_q;
        j->begin = t * per;
        j->end = (t + 1) * per < count ? (t + 1) * per : count;
        if (j->begin > j->end) j->begin = j->end;
        pthread_create(&th[t], NULL, sample_worker, j);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Grouped GEMM (MoE).  offsets[0..E] are host int32 with offsets[0] = 0,
 * offsets[E] = T, nondecreasing.  X is T x K (row stride ldx); expert e's
 * weight W[e] starts at W + e * stride_we and is K x N with row stride ldw.
 * Y is T x N dense.
 * ------------------------------------------------------------------------- */
int orc_grouped_gemm(const uint16_t* X, const uint16_t* W, const int32_t* offsets,
                     int64_t E, int64_t N, int64_t K, int64_t ldx, int64_t stride_we,
                     int64_t ldw, int dtype, double* ref, uint16_t* ref_q, int nthreads) {
    for (int64_t e = 0; e < E; ++e) {
        int64_t r0 = offsets[e], r1 = offsets[e + 1];
        if (r1 <= r0) continue;
        double* Wd = decode_matrix(W + e * stride_we, K, N, ldw, dtype);
        if (!Wd) return -1;
        run_rows(X + r0 * ldx, Wd, NULL, r1 - r0, N, K, ldx, dtype, 0,
                 ref ? ref + r0 * N : NULL, ref_q ? ref_q + r0 * N : NULL, nthreads);
        free(Wd);
    }
    return 0;
}

/* Grouped GEMM at sampled (row, col) positions; the expert of a row is the e
 * with offsets[e] <= row < offsets[e+1]. */
int orc_grouped_sampled(const uint16_t* X, const uint16_t* W, const int32_t* offsets,
                        int64_t E, int64_t K, int64_t ldx, int64_t stride_we, int64_t ldw,
                        int dtype, const int64_t* rows, const int64_t* cols, int64_t count,
                        double* ref, uint16_t* ref_q) {
    for (int64_t s = 0; s < count; ++s) {
        int64_t i = rows[s], c = cols[s];
        int64_t e = -1;
        for (int64_t q = 0; q < E; ++q)
            if (offsets[q] <= i && i < offsets[q + 1]) { e = q; break; }
        if (e < 0) return -1;
        const uint16_t* We = W + e * stride_we;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += orc_decode(X[i * ldx + k], dtype) * orc_decode(We[k * ldw + c], dtype);
        if (ref) ref[s] = acc;
        if (ref_q) ref_q[s] = orc_encode(acc, dtype);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * GEMM of matrices already decoded to double (the fp32 path decodes with
 * orc_decode32_array): C[i,j] = sum_{k ascending} A[i,k] * B[k,j] in fp64,
 * A M x K, B K x N, both dense.  Full output, or the listed positions.
 * ------------------------------------------------------------------------- */
int orc_gemm_d(const double* A, const double* B, int64_t M, int64_t N, int64_t K, double* ref) {
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t n = 0; n < N; ++n) ref[i * N + n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = A[i * K + k];
            for (int64_t n = 0; n < N; ++n) ref[i * N + n] += a * B[k * N + n];
        }
    }
    return 0;
}

int orc_gemm_d_sampled(const double* A, const double* B, int64_t N, int64_t K, const int64_t* rows,
                       const int64_t* cols, int64_t count, double* ref) {
    for (int64_t s = 0; s < count; ++s) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += A[rows[s] * K + k] * B[k * N + cols[s]];
        ref[s] = acc;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * 2-D convolution (a GEMM consumer: the FlagOS cross-chip page, section 5.3,
 * lowers it to a GEMM through im2col).  The plain definition, cross-
 * correlation as deep-learning frameworks define it, over values already
 * decoded to double:
 *
 *   y[n,oh,ow,o] = sum_{kh, kw, c ascending} x[n, ih, iw, c] * w[kh, kw, c, o]
 *   ih = oh*sh - ph + kh*dh,  iw = ow*sw - pw + kw*dw
 *
 * with x taken as 0 where ih or iw falls outside the image (zero padding).
 * x is NHWC [Nb,H,W,C], w is [KH,KW,C,OC], y is [Nb,OH,OW,OC], all dense;
 * OH = (H + 2 ph - dh (KH - 1) - 1) / sh + 1 (floor), OW likewise.
 * Output rows are m = (n*OH + oh)*OW + ow; with `rows`/`cols` the listed
 * (m, o) positions only (count of them), else the full output.
 * ------------------------------------------------------------------------- */
static double conv_point(const double* x, const double* w, int64_t H, int64_t W, int64_t C, int64_t OC,
                         int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                         int64_t dw, int64_t n, int64_t oh, int64_t ow, int64_t o) {
    double acc = 0.0;
    for (int64_t kh = 0; kh < KH; ++kh) {
        const int64_t ih = oh * sh - ph + kh * dh;
        for (int64_t kw = 0; kw < KW; ++kw) {
            const int64_t iw = ow * sw - pw + kw * dw;
            const int inside = ih >= 0 && ih < H && iw >= 0 && iw < W;
            for (int64_t c = 0; c < C; ++c) {
                const double xv = inside ? x[((n * H + ih) * W + iw) * C + c] : 0.0;
                acc += xv * w[((kh * KW + kw) * C + c) * OC + o];
            }
        }
    }
    return acc;
}

int orc_conv2d_d(const double* x, const double* w, int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t OC,
                 int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                 const int64_t* rows, const int64_t* cols, int64_t count, double* y) {
    if (sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || KH < 1 || KW < 1) return 1;
    const int64_t OH = (H + 2 * ph - dh * (KH - 1) - 1) / sh + 1;
    const int64_t OW = (W + 2 * pw - dw * (KW - 1) - 1) / sw + 1;
    if (H + 2 * ph - dh * (KH - 1) - 1 < 0 || W + 2 * pw - dw * (KW - 1) - 1 < 0) return 2;
    if (rows) {
        for (int64_t s = 0; s < count; ++s) {
            const int64_t m = rows[s], n = m / (OH * OW), oh = (m / OW) % OH, ow = m % OW;
            y[s] = conv_point(x, w, H, W, C, OC, KH, KW, sh, sw, ph, pw, dh, dw, n, oh, ow, cols[s]);
        }
        return 0;
    }
    for (int64_t n = 0; n < Nb; ++n)
        for (int64_t oh = 0; oh < OH; ++oh)
            for (int64_t ow = 0; ow < OW; ++ow)
                for (int64_t o = 0; o < OC; ++o)
                    y[((n * OH + oh) * OW + ow) * OC + o] =
                        conv_point(x, w, H, W, C, OC, KH, KW, sh, sw, ph, pw, dh, dw, n, oh, ow, o);
    return 0;
}
