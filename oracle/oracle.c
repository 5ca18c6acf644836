/*
 * CPU oracle for the tiled GEMM  C[M,N] = epi( A[M,K] . B ).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU path.
 *
 * What it computes is the plain definition, not any tiled or pipelined form:
 *   C[i,j] = epi( sum_{k=0..K-1} dec(A[i,k]) * dec(B_e(k,j)) ),
 * summed in IEEE double, k ascending, where
 *   - B_e(k,j) = B[k,j] when B is stored [K,N] (the Pallas guide's Hopper
 *     matmul example multiplies [M,K] @ [K,N]), and B_e(k,j) = B[j,k] when B
 *     is stored [N,K] (the TileLang tutorial's matmul_auto, transpose_B=True);
 *   - dec() decodes an IEEE binary16 or bfloat16 pattern exactly;
 *   - epi() is the identity, or the tanh approximation of GELU,
 *     0.5 x (1 + tanh(0.7978845608 (x + 0.044715 x^3))), the function the
 *     XLA:GPU emitters page fuses in its loop-emitter example and the
 *     Triton lecture notes write in their GeLU kernel; the constants are
 *     the fp32 ones (sqrt(2/pi) and 0.044715), evaluated in double; or ReLU,
 *     max(x, 0), which the Triton lecture notes' matmul kernel applies to its
 *     accumulator before the store (Matmul section); zero of either sign
 *     maps to +0.
 * Output encodings (binary16, bfloat16, binary32) round the double result to
 * nearest, ties to even, straight from double (no double rounding).
 *
 * Build: gcc -O3 -ffp-contract=off -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 * (no -ffast-math and no FMA contraction: each product is rounded, then added,
 * and the k-ascending order of every sum is kept because IEEE addition is not
 * reassociated; vectorising over j does not change any single sum).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes used by this library's own interface */
enum { OR_F16 = 0, OR_BF16 = 1, OR_F32 = 2 };
/* B storage codes */
enum { OR_B_KN = 0, OR_B_NK = 1 };
/* epilogue codes */
enum { OR_EPI_NONE = 0, OR_EPI_GELU_TANH = 1, OR_EPI_RELU = 2 };

/* ---- exact decoders ------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1.f) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* f * 2^(1-127-7) */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);   /* (1.f) * 2^(e-127) */
    return sign ? -v : v;
}

static double decode(uint16_t bits, int dtype) {
    return dtype == OR_F16 ? oracle_decode_f16(bits) : oracle_decode_bf16(bits);
}

/* ---- round-to-nearest-even encoder -------------------------------------- */

/* Encode double x into a binary format with `fbits` fraction bits and
 * `ebits` exponent bits, rounding to nearest with ties to even.  Values whose
 * rounded magnitude exceeds the largest finite number become infinity. */
static uint32_t encode_rne(double x, int fbits, int ebits) {
    uint32_t sign = signbit(x) ? (1u << (fbits + ebits)) : 0u;
    uint32_t emax_field = (1u << ebits) - 1u;
    if (isnan(x)) return sign | (emax_field << fbits) | (1u << (fbits - 1));
    double a = fabs(x);
    if (isinf(a)) return sign | (emax_field << fbits);
    if (a == 0.0) return sign;
    int bias = (1 << (ebits - 1)) - 1;
    int emin = 1 - bias;
    int e;
    frexp(a, &e);          /* a = m * 2^e, 0.5 <= m < 1 */
    e -= 1;                /* now 1 <= a / 2^e < 2 */
    if (e < emin) e = emin;  /* subnormal range shares the quantum 2^(emin-fbits) */
    double q = ldexp(a, fbits - e);     /* a in units of the quantum (exact scaling) */
    double r = nearbyint(q);            /* default mode: nearest, ties to even */
    double one = ldexp(1.0, fbits);     /* 2^fbits: the implicit leading one */
    if (r >= 2.0 * one) {               /* rounded up into the next binade */
        r = one;
        e += 1;
    }
    if (r < one) {                      /* subnormal (only possible when e == emin) */
        return sign | (uint32_t)r;
    }
    int field = e + bias;
    if (field >= (int)emax_field) return sign | (emax_field << fbits);  /* overflow */
    return sign | ((uint32_t)field << fbits) | (uint32_t)(r - one);
}

uint16_t oracle_encode_f16(double x) { return (uint16_t)encode_rne(x, 10, 5); }
uint16_t oracle_encode_bf16(double x) { return (uint16_t)encode_rne(x, 7, 8); }
uint32_t oracle_encode_f32(double x) { return encode_rne(x, 23, 8); }

/* ---- GELU (tanh approximation) ------------------------------------------ */

/* 0.5 x (1 + tanh(u)), u = 0.7978845608 (x + 0.044715 x^3), with 1 + tanh(u) written
 * as 2 / (1 + exp(-2u)), which is the same number (tanh(u) = (1 - e^-2u)/(1 + e^-2u)).
 * Evaluated literally in double, 1 + tanh(u) cancels for u << 0: tanh(u) rounds next
 * to -1 and the sum keeps a few bits (8% relative error at x = -6.9, all of it by
 * x = -9).  The exp form has no cancellation.  exp(-2u) -> inf gives -0 for x < 0,
 * exp(-2u) -> 0 gives x. */
double oracle_gelu_tanh(double x) {
    const double u = 0.7978845608 * (x + 0.044715 * x * x * x);
    return 0.5 * x * (2.0 / (1.0 + exp(-2.0 * u)));
}

/* ---- ReLU ----------------------------------------------------------------- */

double oracle_relu(double x) { return x > 0.0 ? x : 0.0; }

/* ---- vector helpers for the Python side -------------------------------- */

void oracle_decode_array(const uint16_t* bits, int64_t n, int dtype, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = decode(bits[i], dtype);
}

/* out is uint16_t* for F16/BF16 and uint32_t* for F32 */
void oracle_encode_array(const double* x, int64_t n, int dtype, void* out) {
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == OR_F16) ((uint16_t*)out)[i] = oracle_encode_f16(x[i]);
        else if (dtype == OR_BF16) ((uint16_t*)out)[i] = oracle_encode_bf16(x[i]);
        else ((uint32_t*)out)[i] = oracle_encode_f32(x[i]);
    }
}

void oracle_gelu_array(const double* x, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_gelu_tanh(x[i]);
}

/* ---- the GEMM ------------------------------------------------------------ */

/*
 * Computes the rows listed in `rows` (or all M rows when rows == NULL, in
 * which case nrows must equal M) of C = epi(A . B_e) in double.
 *   A: M x K row-major 16-bit patterns; B: K x N (OR_B_KN) or N x K (OR_B_NK)
 *   row-major 16-bit patterns; out: nrows x N doubles, row r = C[rows[r], :].
 * Returns 0 on success, -1 on a bad argument, -2 when memory runs out.
 */
int oracle_gemm_rows(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                     int in_dtype, int b_layout, int epilogue, const int64_t* rows,
                     int64_t nrows, double* out) {
    if (M < 0 || N < 0 || K < 0 || nrows < 0) return -1;
    if (in_dtype != OR_F16 && in_dtype != OR_BF16) return -1;
    if (b_layout != OR_B_KN && b_layout != OR_B_NK) return -1;
    if (epilogue != OR_EPI_NONE && epilogue != OR_EPI_GELU_TANH && epilogue != OR_EPI_RELU)
        return -1;
    if (rows == NULL && nrows != M) return -1;
    if (rows != NULL)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nrows == 0 || N == 0) return 0;

    /* Decode B once into a K x N double array (B_e(k, j) at [k*N + j]). */
    double* Bd = (double*)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(double));
    if (!Bd) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            Bd[k * N + j] = decode(b_layout == OR_B_KN ? B[k * N + j] : B[j * K + k], in_dtype);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        double* c = out + r * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        /* i-k-j order: every c[j] still receives its K terms in ascending k. */
        for (int64_t k = 0; k < K; ++k) {
            double a = decode(A[i * K + k], in_dtype);
            const double* b = Bd + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
        if (epilogue == OR_EPI_GELU_TANH)
            for (int64_t j = 0; j < N; ++j) c[j] = oracle_gelu_tanh(c[j]);
        else if (epilogue == OR_EPI_RELU)
            for (int64_t j = 0; j < N; ++j) c[j] = oracle_relu(c[j]);
    }
    free(Bd);
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
