/*
 * CPU oracle for the tiled dense matrix-unit GEMM,  D = A*B + C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library.  The GPU library neither
 * links, includes nor calls it, and the two share no source, header, table or
 * helper.  Inputs reach both sides as the same raw element bits.
 *
 * What it computes is the plain definition of the product, over the exact
 * values of the stored inputs:
 *
 *     D[b](i,j) = round_out( sum_{k=0}^{K-1} A[b](i,k) * B[b](k,j) + C[b](i,j) )
 *
 *   - "Tensor Cores, CUTLASS and CuTe", section 2.1: one matrix instruction
 *     computes D = A*B + C with low-precision inputs and an fp32 (or int32)
 *     accumulator; section 4.1 states the 4096^3 bf16 problem (bf16 in, fp32
 *     accumulate, bf16 out) and section 4.3 rounds the accumulator to bf16
 *     with round-to-nearest-even in the epilogue.
 *   - "hgemm_mma_m16n8k16_mma2x4_warp4x4_kernel" walkthrough, section 1.1:
 *     C = A x B with row-major M x K and K x N inputs and an M x N output.
 *   - Layout-experiment post (KingOfEgg, RTX 5080), section 3: D = A x B + C
 *     with an fp32 accumulator as the floor for long accumulations.
 *
 * Floating-point inputs (fp16, bf16, fp32, and FP8 e4m3 -- "Tensor Cores,
 * CUTLASS and CuTe", section 2.1 lists e4m3 inputs with an fp32 accumulator,
 * section 6.5 the FP8 scaled GEMM) are decoded to exact fp64 values by
 * this file's own codecs; every product of two such values is exact in fp64,
 * and the products are summed in fp64 in increasing k.  C is added in fp64,
 * and the result is rounded ONCE, with IEEE round-to-nearest-even, directly
 * from fp64 to the output type (fp32, fp16 or bf16).  Integer (int8) inputs are
 * summed exactly in int64, C (int32) is added, and the result is narrowed to
 * int32 by two's-complement wrap-around.
 *
 * Optional fused epilogue ("Tensor Cores, CUTLASS and CuTe", section 5: the
 * scaled-mm epilogue multiplies the accumulator by a per-column and a per-row
 * scale before the bf16 conversion; section 7: the bias + ReLU / tanh-GELU
 * epilogue of the fused linear layer):
 *
 *     D[b](i,j) = round_out( act( rs[b](i) * cs[b](j) * P + bias[b](j) + C[b](i,j) ) )
 *
 * where P is the product sum above (for int8 inputs: the int32 accumulator,
 * i.e. the exact sum narrowed by wrap-around, then taken as a real number),
 * rs / cs / bias default to 1 / 1 / 0 when absent, and act is the identity,
 * ReLU (x > 0 ? x : +0) or the tanh form of GELU,
 * 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), evaluated through the
 * identity 0.5 (1 + tanh u) = 1 / (1 + e^(-2u)).  All of it is evaluated in
 * fp64 and rounded once.  int8 inputs may then have fp32, fp16 or bf16 output
 * (dequantisation); int32 output takes no epilogue.
 *
 * An "fp16 accumulate" request is the same computation with fp16 C and D: the
 * exact sum is rounded once to fp16 (no matrix instruction of the target chip
 * accumulates in fp16; the result is the best fp16 answer).
 *
 * Addressing (BLAS convention, element units):
 *   row-major X(r,c) at r*ld + c;   column-major X(r,c) at r + c*ld.
 *   A is logical M x K, B is logical K x N; C and D are row-major M x N.
 *   Batch b adds b*stride_* to each base.
 *
 * The file also holds the attention forward O = softmax(scale Q K^T) V (see
 * oracle_attention below), evaluated the same way: exact fp64 inputs, fp64
 * sums in index order, one rounding of each output.
 *
 * Parity pins for this file live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3, OR_I8 = 4, OR_I32 = 5, OR_E4M3 = 6 };
enum { OR_ROW = 0, OR_COL = 1 };
enum { OR_ACT_NONE = 0, OR_ACT_RELU = 1, OR_ACT_GELU_TANH = 2 };

/* ------------------------------------------------------------------ */
/* Codecs                                                              */
/* ------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 stored mantissa bits. */
double oracle_decode_f16(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^(1-15-10) */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25); /* (1024+m) * 2^(e-15-10) */
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits. */
double oracle_decode_bf16(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 7) & 0xff, m = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133); /* subnormal: m * 2^(1-127-7) */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x80), e - 134); /* (128+m) * 2^(e-127-7) */
    return s ? -v : v;
}

/* FP8 e4m3 (the pages' 8-bit input type; the "FN" form of the OCP 8-bit
 * formats): 1 sign, 4 exponent (bias 7), 3 stored mantissa bits, no
 * infinities; exponent and mantissa all ones is NaN, so the largest finite
 * value is 1.75 * 2^8 = 448. */
double oracle_decode_e4m3(uint8_t h)
{
    int s = (h >> 7) & 1, e = (h >> 3) & 0xf, m = h & 0x7;
    double v;
    if (e == 0xf && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* subnormal: m * 2^(1-7-3) */
    else
        v = ldexp((double)(m | 0x8), e - 10); /* (8+m) * 2^(e-7-3) */
    return s ? -v : v;
}

/*
 * Round x to the nearest value of a binary format with `man` stored mantissa
 * bits and `ex` exponent bits, ties to even, and return its bit pattern.
 * Overflow gives +-inf; NaN gives the positive quiet NaN with only the top
 * mantissa bit set.
 */
static uint64_t encode_rne(double x, int man, int ex)
{
    const uint64_t exp_all = (1ull << ex) - 1;
    const uint64_t sign_bit = (signbit(x) ? 1ull : 0ull) << (man + ex);
    if (isnan(x))
        return (exp_all << man) | (1ull << (man - 1));
    double a = fabs(x);
    if (isinf(a))
        return sign_bit | (exp_all << man);
    if (a == 0.0)
        return sign_bit;
    const int bias = (1 << (ex - 1)) - 1;
    const int emin = 1 - bias, emax = bias;
    int E;
    (void)frexp(a, &E);
    int e = E - 1; /* 2^e <= a < 2^(e+1) */
    if (e < emin)
        e = emin; /* subnormal range: fixed quantum 2^(emin-man) */
    /* a / 2^(e-man): a power-of-two scaling, exact in fp64. */
    double scaled = ldexp(a, man - e);
    double r = floor(scaled);
    double frac = scaled - r; /* exact: scaled < 2^(man+1) <= 2^24 */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    uint64_t n = (uint64_t)r;
    if (n == (1ull << (man + 1))) { /* rounded up into the next binade */
        n >>= 1;
        e += 1;
    }
    if (e > emax)
        return sign_bit | (exp_all << man);
    if (n < (1ull << man)) /* subnormal (only reachable with e == emin) */
        return sign_bit | n;
    return sign_bit | ((uint64_t)(e + bias) << man) | (n - (1ull << man));
}

uint16_t oracle_encode_f16(double x) { return (uint16_t)encode_rne(x, 10, 5); }
uint16_t oracle_encode_bf16(double x) { return (uint16_t)encode_rne(x, 7, 8); }
uint32_t oracle_encode_f32(double x) { return (uint32_t)encode_rne(x, 23, 8); }

/* Array forms, used by the tests to pin the codecs exhaustively. */
void oracle_decode_array(int type, const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = type == OR_F16 ? oracle_decode_f16(in[i]) : oracle_decode_bf16(in[i]);
}

void oracle_decode_array8(int type, const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = type == OR_E4M3 ? oracle_decode_e4m3(in[i]) : NAN;
}

void oracle_encode_array(int type, const double *in, void *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        if (type == OR_F16)
            ((uint16_t *)out)[i] = oracle_encode_f16(in[i]);
        else if (type == OR_BF16)
            ((uint16_t *)out)[i] = oracle_encode_bf16(in[i]);
        else
            ((uint32_t *)out)[i] = oracle_encode_f32(in[i]);
    }
}

/* ------------------------------------------------------------------ */
/* Element access                                                      */
/* ------------------------------------------------------------------ */

static double load_fp(const void *p, int type, int64_t idx)
{
    switch (type) {
    case OR_F16: return oracle_decode_f16(((const uint16_t *)p)[idx]);
    case OR_BF16: return oracle_decode_bf16(((const uint16_t *)p)[idx]);
    case OR_E4M3: return oracle_decode_e4m3(((const uint8_t *)p)[idx]);
    default: return (double)((const float *)p)[idx]; /* fp32 -> fp64 is exact */
    }
}

static int64_t load_int(const void *p, int type, int64_t idx)
{
    return type == OR_I8 ? (int64_t)((const int8_t *)p)[idx] : (int64_t)((const int32_t *)p)[idx];
}

/* Offset of logical element (r, c) of a matrix stored with leading dimension ld. */
static int64_t at(int layout, int64_t r, int64_t c, int64_t ld)
{
    return layout == OR_ROW ? r * ld + c : r + c * ld;
}

static void store_out(void *p, int type, int64_t idx, double v)
{
    switch (type) {
    case OR_F16: ((uint16_t *)p)[idx] = oracle_encode_f16(v); break;
    case OR_BF16: ((uint16_t *)p)[idx] = oracle_encode_bf16(v); break;
    default: ((uint32_t *)p)[idx] = oracle_encode_f32(v); break;
    }
}

static int32_t wrap_i32(int64_t v) { return (int32_t)(uint32_t)(uint64_t)v; }

/* ------------------------------------------------------------------ */
/* GEMM                                                                */
/* ------------------------------------------------------------------ */

typedef struct {
    int64_t M, N, K, batch;
    int in_type, out_type, layout_a, layout_b;
    const void *A; int64_t lda, stride_a;
    const void *B; int64_t ldb, stride_b;
    const void *C; int64_t ldc, stride_c;
    void *D; int64_t ldd, stride_d;
    /* epilogue (NULL / OR_ACT_NONE: absent) */
    const float *rs; int64_t stride_rs;
    const float *cs; int64_t stride_cs;
    const float *bias; int64_t stride_bias;
    int act;
    /* work split: rows [row_begin, row_end) of the flattened (batch*M) range */
    int64_t row_begin, row_end;
    int status;
} job_t;

static int is_fp_in(int t) { return t == OR_F16 || t == OR_BF16 || t == OR_F32 || t == OR_E4M3; }

static int check_args(const job_t *j)
{
    if (j->M < 0 || j->N < 0 || j->K < 0 || j->batch < 0)
        return 1;
    if (is_fp_in(j->in_type)) {
        if (j->out_type != OR_F16 && j->out_type != OR_BF16 && j->out_type != OR_F32)
            return 2;
    } else if (j->in_type == OR_I8) {
        if (j->out_type == OR_I32) {
            if (j->rs || j->cs || j->bias || j->act != OR_ACT_NONE)
                return 2; /* integer output takes no epilogue */
        } else if (j->out_type != OR_F16 && j->out_type != OR_BF16 && j->out_type != OR_F32) {
            return 2;
        }
    } else {
        return 2;
    }
    if (j->act < OR_ACT_NONE || j->act > OR_ACT_GELU_TANH)
        return 3;
    if ((j->layout_a != OR_ROW && j->layout_a != OR_COL) || (j->layout_b != OR_ROW && j->layout_b != OR_COL))
        return 3;
    return 0;
}

/* The epilogue on one value: p is the product sum (fp64, exact for int8). */
static double epilogue(const job_t *j, int64_t b, int64_t i, int64_t c, double p, double addend)
{
    double v = p;
    if (j->rs)
        v *= (double)j->rs[b * j->stride_rs + i];
    if (j->cs)
        v *= (double)j->cs[b * j->stride_cs + c];
    if (j->bias)
        v += (double)j->bias[b * j->stride_bias + c];
    v += addend;
    if (j->act == OR_ACT_RELU)
        v = v > 0.0 ? v : 0.0;
    else if (j->act == OR_ACT_GELU_TANH) {
        /* 0.5 (1 + tanh u) written as the equal 1 / (1 + e^(-2u)): the sum
         * 1 + tanh u cancels for strongly negative u, the quotient does not */
        const double u = sqrt(2.0 / acos(-1.0)) * (v + 0.044715 * v * v * v);
        v = v / (1.0 + exp(-2.0 * u));
    }
    return v;
}

/* One output row (b, i): the i-k-j order, accumulating a whole row at once. */
static void *gemm_rows(void *arg)
{
    job_t *j = (job_t *)arg;
    const int fp = is_fp_in(j->in_type);
    double *accf = fp ? (double *)calloc((size_t)(j->N ? j->N : 1), sizeof(double)) : NULL;
    int64_t *acci = fp ? NULL : (int64_t *)calloc((size_t)(j->N ? j->N : 1), sizeof(int64_t));
    if ((fp && !accf) || (!fp && !acci)) {
        j->status = 4;
        return NULL;
    }
    for (int64_t row = j->row_begin; row < j->row_end; ++row) {
        const int64_t b = row / j->M, i = row % j->M;
        const int64_t oa = b * j->stride_a, ob = b * j->stride_b;
        const int64_t oc = b * j->stride_c, od = b * j->stride_d;
        if (fp) {
            for (int64_t c = 0; c < j->N; ++c)
                accf[c] = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                const double a = load_fp(j->A, j->in_type, oa + at(j->layout_a, i, k, j->lda));
                for (int64_t c = 0; c < j->N; ++c)
                    accf[c] += a * load_fp(j->B, j->in_type, ob + at(j->layout_b, k, c, j->ldb));
            }
            for (int64_t c = 0; c < j->N; ++c) {
                const double addend = j->C ? load_fp(j->C, j->out_type, oc + i * j->ldc + c) : 0.0;
                store_out(j->D, j->out_type, od + i * j->ldd + c, epilogue(j, b, i, c, accf[c], addend));
            }
        } else {
            for (int64_t c = 0; c < j->N; ++c)
                acci[c] = 0;
            for (int64_t k = 0; k < j->K; ++k) {
                const int64_t a = load_int(j->A, OR_I8, oa + at(j->layout_a, i, k, j->lda));
                for (int64_t c = 0; c < j->N; ++c)
                    acci[c] += a * load_int(j->B, OR_I8, ob + at(j->layout_b, k, c, j->ldb));
            }
            for (int64_t c = 0; c < j->N; ++c) {
                if (j->out_type == OR_I32) {
                    int64_t v = acci[c];
                    if (j->C)
                        v += load_int(j->C, OR_I32, oc + i * j->ldc + c);
                    ((int32_t *)j->D)[od + i * j->ldd + c] = wrap_i32(v);
                } else { /* dequantisation: the int32 accumulator as a real number */
                    const double addend = j->C ? load_fp(j->C, j->out_type, oc + i * j->ldc + c) : 0.0;
                    store_out(j->D, j->out_type, od + i * j->ldd + c,
                              epilogue(j, b, i, c, (double)wrap_i32(acci[c]), addend));
                }
            }
        }
    }
    free(accf);
    free(acci);
    return NULL;
}

#define ORACLE_ARGS                                                                              \
    int64_t M, int64_t N, int64_t K, int64_t batch, int in_type, int out_type, int layout_a,     \
        int layout_b, const void *A, int64_t lda, int64_t stride_a, const void *B, int64_t ldb, \
        int64_t stride_b, const void *C, int64_t ldc, int64_t stride_c

#define EPILOGUE_ARGS                                                                          \
    const float *rs, int64_t stride_rs, const float *cs, int64_t stride_cs, const float *bias, \
        int64_t stride_bias, int act

static job_t make_job(ORACLE_ARGS)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.M = M; j.N = N; j.K = K; j.batch = batch;
    j.in_type = in_type; j.out_type = out_type; j.layout_a = layout_a; j.layout_b = layout_b;
    j.A = A; j.lda = lda; j.stride_a = stride_a;
    j.B = B; j.ldb = ldb; j.stride_b = stride_b;
    j.C = C; j.ldc = ldc; j.stride_c = stride_c;
    return j;
}

/*
 * Full product.  Returns 0 on success, nonzero for bad arguments or an
 * allocation failure.  Rows of the flattened (batch*M) range are split into
 * contiguous blocks over `nthreads` threads; each output element is computed
 * by one thread with the summation order stated above.
 */
int oracle_gemm_ex(ORACLE_ARGS, EPILOGUE_ARGS, void *D, int64_t ldd, int64_t stride_d, int nthreads)
{
    job_t base = make_job(M, N, K, batch, in_type, out_type, layout_a, layout_b, A, lda, stride_a,
                          B, ldb, stride_b, C, ldc, stride_c);
    base.D = D; base.ldd = ldd; base.stride_d = stride_d;
    base.rs = rs; base.stride_rs = stride_rs;
    base.cs = cs; base.stride_cs = stride_cs;
    base.bias = bias; base.stride_bias = stride_bias;
    base.act = act;
    int st = check_args(&base);
    if (st)
        return st;
    const int64_t rows = batch * M;
    if (rows == 0 || N == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > rows)
        nthreads = (int)rows;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return 4;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].row_begin = rows * t / nthreads;
        jobs[t].row_end = rows * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&tids[t], NULL, gemm_rows, &jobs[t]) != 0)
            jobs[t].status = -1; /* run it on this thread instead */
    gemm_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (jobs[t].status == -1) {
            jobs[t].status = 0;
            gemm_rows(&jobs[t]);
        } else {
            pthread_join(tids[t], NULL);
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status)
            st = jobs[t].status;
    free(jobs);
    free(tids);
    return st;
}

/*
 * Selected elements only: out[s] = D[b](i,j) for (b,i,j) = bij[3s..3s+2],
 * each a single k-ordered dot product (the same sum, in the same order, as
 * the full product) followed by the same epilogue.  `out` holds values of
 * out_type.  Used at sizes where the full product is too slow for a CPU.
 */
int oracle_gemm_at_ex(ORACLE_ARGS, EPILOGUE_ARGS, int64_t nsample, const int64_t *bij, void *out)
{
    job_t j = make_job(M, N, K, batch, in_type, out_type, layout_a, layout_b, A, lda, stride_a, B,
                       ldb, stride_b, C, ldc, stride_c);
    j.rs = rs; j.stride_rs = stride_rs;
    j.cs = cs; j.stride_cs = stride_cs;
    j.bias = bias; j.stride_bias = stride_bias;
    j.act = act;
    int st = check_args(&j);
    if (st)
        return st;
    for (int64_t s = 0; s < nsample; ++s) {
        const int64_t b = bij[3 * s], i = bij[3 * s + 1], c = bij[3 * s + 2];
        if (b < 0 || b >= batch || i < 0 || i >= M || c < 0 || c >= N)
            return 5;
        const int64_t oa = b * stride_a, ob = b * stride_b, oc = b * stride_c;
        if (is_fp_in(in_type)) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += load_fp(A, in_type, oa + at(layout_a, i, k, lda)) *
                       load_fp(B, in_type, ob + at(layout_b, k, c, ldb));
            double addend = 0.0;
            if (C)
                addend += load_fp(C, out_type, oc + i * ldc + c);
            store_out(out, out_type, s, epilogue(&j, b, i, c, acc, addend));
        } else {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += load_int(A, OR_I8, oa + at(layout_a, i, k, lda)) *
                       load_int(B, OR_I8, ob + at(layout_b, k, c, ldb));
            if (out_type == OR_I32) {
                if (C)
                    acc += load_int(C, OR_I32, oc + i * ldc + c);
                ((int32_t *)out)[s] = wrap_i32(acc);
            } else {
                const double addend = C ? load_fp(C, out_type, oc + i * ldc + c) : 0.0;
                store_out(out, out_type, s, epilogue(&j, b, i, c, (double)wrap_i32(acc), addend));
            }
        }
    }
    return 0;
}

/* The product without an epilogue. */
int oracle_gemm(ORACLE_ARGS, void *D, int64_t ldd, int64_t stride_d, int nthreads)
{
    return oracle_gemm_ex(M, N, K, batch, in_type, out_type, layout_a, layout_b, A, lda, stride_a, B, ldb,
                          stride_b, C, ldc, stride_c, NULL, 0, NULL, 0, NULL, 0, OR_ACT_NONE, D, ldd,
                          stride_d, nthreads);
}

int oracle_gemm_at(ORACLE_ARGS, int64_t nsample, const int64_t *bij, void *out)
{
    return oracle_gemm_at_ex(M, N, K, batch, in_type, out_type, layout_a, layout_b, A, lda, stride_a, B,
                             ldb, stride_b, C, ldc, stride_c, NULL, 0, NULL, 0, NULL, 0, OR_ACT_NONE,
                             nsample, bij, out);
}

/* ------------------------------------------------------------------ */
/* Attention forward                                                   */
/* ------------------------------------------------------------------ */

/*
 * O = softmax(scale * Q K^T) V, one batch slice at a time: the computation
 * whose two products the pages move onto the matrix units (layout-experiment
 * post, sections 1-2: S = QK^T and O = PV of a FlashAttention kernel, with the
 * elementwise exp taking S to P in between; "Tensor Cores, CUTLASS and CuTe",
 * part 3 section 2: the softmax of each row of S = QK^T needs that row's max
 * and sum, and P = softmax(S) feeds O = P V).
 *
 * Q is seq_q x d, K is seq_k x d, V is seq_k x dv, O is seq_q x dv, all
 * row-major with the given leading dimensions and batch strides (elements).
 * For query row i, in fp64 over the exact input values:
 *
 *     s_j = scale * sum_{t<d} Q(i,t) K(j,t)          (t in increasing order)
 *     m   = max_j s_j
 *     w_j = exp(s_j - m)                              (the largest weight is 1)
 *     O(i,c) = (sum_{j<seq_k} w_j V(j,c)) / (sum_{j<seq_k} w_j)
 *
 * rounded once to out_type.  Subtracting the row maximum does not change the
 * quotient; it keeps every exp at most 1.  seq_k == 0 leaves O undefined and is
 * rejected.
 */
typedef struct {
    int64_t batch, sq, sk, d, dv;
    int in_type, out_type;
    double scale;
    const void *Q; int64_t ldq, stride_q;
    const void *K; int64_t ldk, stride_k;
    const void *V; int64_t ldv, stride_v;
    void *O; int64_t ldo, stride_o;
    const int64_t *rows; /* selected (b, i) pairs, or NULL for all rows */
    int64_t begin, end;  /* work split over the row list */
    int status;
} att_t;

static void attention_row(const att_t *a, int64_t b, int64_t i, double *s, double *acc, int64_t out_row)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < a->sk; ++j) {
        double dot = 0.0;
        for (int64_t t = 0; t < a->d; ++t)
            dot += load_fp(a->Q, a->in_type, b * a->stride_q + i * a->ldq + t) *
                   load_fp(a->K, a->in_type, b * a->stride_k + j * a->ldk + t);
        s[j] = a->scale * dot;
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int64_t c = 0; c < a->dv; ++c)
        acc[c] = 0.0;
    for (int64_t j = 0; j < a->sk; ++j) {
        const double w = exp(s[j] - m);
        l += w;
        for (int64_t c = 0; c < a->dv; ++c)
            acc[c] += w * load_fp(a->V, a->in_type, b * a->stride_v + j * a->ldv + c);
    }
    for (int64_t c = 0; c < a->dv; ++c)
        store_out(a->O, a->out_type, out_row + c, acc[c] / l);
}

static void *attention_rows(void *arg)
{
    att_t *a = (att_t *)arg;
    double *s = (double *)malloc((size_t)a->sk * sizeof(double));
    double *acc = (double *)malloc((size_t)(a->dv ? a->dv : 1) * sizeof(double));
    if (!s || !acc) {
        a->status = 4;
        free(s);
        free(acc);
        return NULL;
    }
    for (int64_t r = a->begin; r < a->end; ++r) {
        int64_t b, i, out_row;
        if (a->rows) { /* selected rows: output row r of a dense [n][dv] array */
            b = a->rows[2 * r];
            i = a->rows[2 * r + 1];
            out_row = r * a->dv;
        } else {
            b = r / a->sq;
            i = r % a->sq;
            out_row = b * a->stride_o + i * a->ldo;
        }
        attention_row(a, b, i, s, acc, out_row);
    }
    free(s);
    free(acc);
    return NULL;
}

static int attention_run(att_t *base, int64_t nrows, int nthreads)
{
    if (base->batch < 0 || base->sq < 0 || base->sk <= 0 || base->d < 0 || base->dv < 0)
        return 1;
    if ((base->in_type != OR_F16 && base->in_type != OR_BF16 && base->in_type != OR_F32) ||
        (base->out_type != OR_F16 && base->out_type != OR_BF16 && base->out_type != OR_F32))
        return 2;
    if (nrows == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nrows)
        nthreads = (int)nrows;
    att_t *jobs = (att_t *)calloc((size_t)nthreads, sizeof(att_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return 4;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *base;
        jobs[t].begin = nrows * t / nthreads;
        jobs[t].end = nrows * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&tids[t], NULL, attention_rows, &jobs[t]) != 0)
            jobs[t].status = -1;
    attention_rows(&jobs[0]);
    int st = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (jobs[t].status == -1) {
            jobs[t].status = 0;
            attention_rows(&jobs[t]);
        } else {
            pthread_join(tids[t], NULL);
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status)
            st = jobs[t].status;
    free(jobs);
    free(tids);
    return st;
}

#define ATTENTION_ARGS                                                                              \
    int64_t batch, int64_t sq, int64_t sk, int64_t d, int64_t dv, int in_type, int out_type,          \
        double scale, const void *Q, int64_t ldq, int64_t stride_q, const void *K, int64_t ldk,       \
        int64_t stride_k, const void *V, int64_t ldv, int64_t stride_v

static att_t make_att(ATTENTION_ARGS)
{
    att_t a;
    memset(&a, 0, sizeof(a));
    a.batch = batch; a.sq = sq; a.sk = sk; a.d = d; a.dv = dv;
    a.in_type = in_type; a.out_type = out_type; a.scale = scale;
    a.Q = Q; a.ldq = ldq; a.stride_q = stride_q;
    a.K = K; a.ldk = ldk; a.stride_k = stride_k;
    a.V = V; a.ldv = ldv; a.stride_v = stride_v;
    return a;
}

/* Every row of O. */
int oracle_attention(ATTENTION_ARGS, void *O, int64_t ldo, int64_t stride_o, int nthreads)
{
    att_t a = make_att(batch, sq, sk, d, dv, in_type, out_type, scale, Q, ldq, stride_q, K, ldk, stride_k, V,
                       ldv, stride_v);
    a.O = O; a.ldo = ldo; a.stride_o = stride_o;
    return attention_run(&a, batch * sq, nthreads);
}

/* Selected rows: out[r][0..dv) = O[b](i, .) for (b, i) = rows[2r], rows[2r+1]. */
int oracle_attention_rows(ATTENTION_ARGS, int64_t nrows, const int64_t *rows, void *out, int nthreads)
{
    att_t a = make_att(batch, sq, sk, d, dv, in_type, out_type, scale, Q, ldq, stride_q, K, ldk, stride_k, V,
                       ldv, stride_v);
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= batch || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= sq)
            return 5;
    a.O = out; a.rows = rows;
    return attention_run(&a, nrows, nthreads);
}
