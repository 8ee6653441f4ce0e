/*
 * gemm_ref.c -- CPU oracle for C = A * B^T.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library.  The GPU product path never links it, and it shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes (the plain definition, written out):
 *   C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[j][k]
 * with A stored M x K row-major and B stored N x K row-major ("B transposed").
 *   - "Optimizing Blackwell matrix multiplication in Mojo (part 2)", section
 *     "Starting from the 4-line kernel": the naive kernel's inner product
 *     multiplies a[row, k] by b[col, k] with B held transposed (N x K), and
 *     section "Kernel 2: TMA and Tensor Core" lays B out row_major(N, K).
 *   - "Chapter 7: Writing custom kernels with Pallas", section 4.1 (tiled
 *     matmul with accumulator): C[i,j] is the sum over k of A[i,k] B[k,j];
 *     section 4.1' compares a bf16 kernel against float64 arithmetic on the
 *     same bf16 inputs, which is exactly what this file does.
 *
 * Arithmetic: each input is decoded exactly to double; every product of two
 * bf16, two f16 or two 8-bit float values is exact in double (at most 22
 * significant bits); the sum runs in increasing k with plain double additions
 * (built with -ffp-contract=off, no fast-math), so the only error is the fp64
 * summation.
 *
 * 8-bit inputs (OCP 8-bit floating point formats; the inputs are passed as
 * 16-bit words holding the code in the low byte): E4M3 has 1 sign, 4 exponent
 * (bias 7) and 3 fraction bits, no infinities, and S.1111.111 is NaN; E5M2 has
 * 1 sign, 5 exponent (bias 15) and 2 fraction bits with IEEE-style infinities
 * and NaNs.  Both have subnormals at the minimum exponent.
 *
 * Output rounding (used by the bit-exact tests): IEEE round-to-nearest-even
 * from the double value straight to the output format, overflow to +-Inf.
 *
 * 8-bit integer inputs ("Writing Mosaic GPU kernels with Pallas", section
 * "MMA (TensorCore)": int8 is the integer operand type, with an int32
 * accumulator) have their own entry points below: two's-complement bytes,
 * products and sums in int64, which is exact for every K below 2^49 (each
 * product is at most 2^14 in magnitude).  No rounding is involved.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_FP8_E4M3 = 3, ORC_FP8_E5M2 = 4 };

/* ---- exact decoders: 16-bit storage -> double ---------------------------- */

/* bfloat16 = the upper half of an IEEE binary32: 1 sign, 8 exponent, 7 fraction bits. */
static double decode_bf16(uint16_t h) {
    const int sign = h >> 15;
    const int e = (h >> 7) & 0xFF;
    const int f = h & 0x7F;
    double v;
    if (e == 0xFF) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -126 - 7);            /* subnormal: f * 2^-133 */
    } else {
        v = ldexp((double)(128 + f), e - 127 - 7); /* (1.f) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* IEEE binary16: 1 sign, 5 exponent, 10 fraction bits. */
static double decode_f16(uint16_t h) {
    const int sign = h >> 15;
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -14 - 10);             /* subnormal: f * 2^-24 */
    } else {
        v = ldexp((double)(1024 + f), e - 15 - 10); /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* OCP E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent 15 with
   fraction 7 is NaN, there is no infinity (largest finite: 448). */
static double decode_e4m3(uint16_t h) {
    if (h > 0xFF) return NAN;
    const int sign = h >> 7;
    const int e = (h >> 3) & 0xF;
    const int f = h & 0x7;
    double v;
    if (e == 0xF && f == 0x7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)f, -6 - 3);              /* subnormal: f * 2^-9 */
    } else {
        v = ldexp((double)(8 + f), e - 7 - 3);     /* (1.f) * 2^(e-7) */
    }
    return sign ? -v : v;
}

/* OCP E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits; exponent 31 is
   infinity (fraction 0) or NaN. */
static double decode_e5m2(uint16_t h) {
    if (h > 0xFF) return NAN;
    const int sign = h >> 7;
    const int e = (h >> 2) & 0x1F;
    const int f = h & 0x3;
    double v;
    if (e == 0x1F) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -14 - 2);             /* subnormal: f * 2^-16 */
    } else {
        v = ldexp((double)(4 + f), e - 15 - 2);    /* (1.f) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static int valid_in(int dtype) {
    return dtype == ORC_BF16 || dtype == ORC_F16 || dtype == ORC_FP8_E4M3 || dtype == ORC_FP8_E5M2;
}

static double decode(uint16_t h, int dtype) {
    switch (dtype) {
        case ORC_BF16: return decode_bf16(h);
        case ORC_FP8_E4M3: return decode_e4m3(h);
        case ORC_FP8_E5M2: return decode_e5m2(h);
        default: return decode_f16(h);
    }
}

/* ---- round-to-nearest-even from double ----------------------------------- */

/*
 * Round |x| (finite, > 0) to a binary format with `p` fraction bits and
 * minimum normal exponent `emin`.  Returns the rounded magnitude as a double
 * (exactly representable in the target).  nearbyint() rounds half to even in
 * the default rounding mode, and the scaling by a power of two is exact.
 */
static double rne_magnitude(double a, int p, int emin) {
    int e;
    frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) -> floor(log2 a) = e - 1 */
    int ex = e - 1;
    if (ex < emin) ex = emin;               /* subnormal range: fixed quantum */
    const double q = ldexp(1.0, ex - p);    /* spacing of representable values */
    return nearbyint(a / q) * q;
}

static uint16_t encode_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    const uint16_t s = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    /* largest finite bf16 is (2 - 2^-7) * 2^127; values at or beyond the
       midpoint to 2^128 round to infinity */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return s | 0x7F80;
    if (a == 0.0) return s;
    const double r = rne_magnitude(a, 7, -126);
    if (r == 0.0) return s;
    /* r is a bf16 value; assemble its fields */
    int e;
    const double m = frexp(r, &e); /* r = m * 2^e */
    int ex = e - 1;
    if (ex < -126) {               /* subnormal: r = f * 2^-133 */
        const int f = (int)ldexp(r, 133);
        return s | (uint16_t)f;
    }
    const int f = (int)ldexp(m * 2.0 - 1.0, 7);
    return s | (uint16_t)((ex + 127) << 7) | (uint16_t)f;
}

static uint16_t encode_f16(double x) {
    if (isnan(x)) return 0x7E00;
    const uint16_t s = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    /* largest finite f16 is 65504; the midpoint to 65536 (65520) and beyond
       round to infinity */
    if (a >= 65520.0) return s | 0x7C00;
    if (a == 0.0) return s;
    const double r = rne_magnitude(a, 10, -14);
    if (r == 0.0) return s;
    int e;
    const double m = frexp(r, &e);
    int ex = e - 1;
    if (ex < -14) {                /* subnormal: r = f * 2^-24 */
        const int f = (int)ldexp(r, 24);
        return s | (uint16_t)f;
    }
    const int f = (int)ldexp(m * 2.0 - 1.0, 10);
    return s | (uint16_t)((ex + 15) << 10) | (uint16_t)f;
}

/* ---- exported entry points ----------------------------------------------- */

int orc_version(void) { return 1; }

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Decode n 16-bit values to double. */
void orc_decode(const uint16_t* bits, int64_t n, int dtype, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = decode(bits[i], dtype);
}

/*
 * Round n doubles to the output format.  F32: out is uint32 bits of the
 * nearest float (C's conversion rounds to nearest even); F16/BF16: out is
 * uint16 bits.
 */
void orc_round(const double* x, int64_t n, int out_dtype, void* out) {
    if (out_dtype == ORC_F32) {
        uint32_t* o = (uint32_t*)out;
        for (int64_t i = 0; i < n; ++i) {
            const float f = (float)x[i];
            memcpy(&o[i], &f, 4);
        }
    } else {
        uint16_t* o = (uint16_t*)out;
        for (int64_t i = 0; i < n; ++i)
            o[i] = out_dtype == ORC_BF16 ? encode_bf16(x[i]) : encode_f16(x[i]);
    }
}

/* Exact value of every 16-bit pattern (f16, bf16, and the 8-bit formats in
   the low byte), filled from the decoders above once, when the library is
   loaded and before any call can run, so that the loops below index a table
   instead of re-decoding each operand and no call ever sees a table being
   filled. */
static double g_table[4][65536];
static const int g_table_dtype[4] = {ORC_F16, ORC_BF16, ORC_FP8_E4M3, ORC_FP8_E5M2};

__attribute__((constructor)) static void orc_fill_tables(void) {
    for (int t = 0; t < 4; ++t)
        for (int h = 0; h < 65536; ++h) g_table[t][h] = decode((uint16_t)h, g_table_dtype[t]);
}

static const double* table_for(int dtype) {
    const int t = dtype == ORC_BF16 ? 1 : (dtype == ORC_FP8_E4M3 ? 2 : (dtype == ORC_FP8_E5M2 ? 3 : 0));
    return g_table[t];
}

/* One output entry: the increasing-k fp64 dot product of row i of A and
   row j of stored B. */
static double dot_row(const uint16_t* a, const uint16_t* b, int64_t K, const double* tab) {
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += tab[a[k]] * tab[b[k]];
    return s;
}

static double norm_row(const uint16_t* a, int64_t K, const double* tab) {
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double v = tab[a[k]];
        s += v * v;
    }
    return sqrt(s);
}

/*
 * Full product.  C (M x N doubles), nA (M), nB (N) are caller-owned.
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad args.
 */
int orc_gemm_bt(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                int in_dtype, double* C, double* nA, double* nB, int nthreads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (!valid_in(in_dtype)) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const double* tab = table_for(in_dtype);
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        const uint16_t* a = A + i * K;
        for (int64_t j = 0; j < N; ++j) C[i * N + j] = dot_row(a, B + j * K, K, tab);
        if (nA) nA[i] = norm_row(a, K, tab);
    }
    if (nB) {
#pragma omp parallel for schedule(static)
        for (i = 0; i < N; ++i) nB[i] = norm_row(B + i * K, K, tab);
    }
    return 0;
}

/*
 * Selected entries only: out[t] = C[I[t]][J[t]] for t < n.  Used to check a
 * sample of a product too large to form whole on the CPU.
 */
int orc_gemm_bt_entries(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                        int in_dtype, const int64_t* I, const int64_t* J, int64_t n,
                        double* out, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || n < 0) return -1;
    if (!valid_in(in_dtype)) return -1;
    for (int64_t t = 0; t < n; ++t)
        if (I[t] < 0 || I[t] >= M || J[t] < 0 || J[t] >= N) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const double* tab = table_for(in_dtype);
    int64_t t;
#pragma omp parallel for schedule(dynamic, 64)
    for (t = 0; t < n; ++t) out[t] = dot_row(A + I[t] * K, B + J[t] * K, K, tab);
    return 0;
}

/* Row 2-norms of an R x K 16-bit matrix (for the tolerance bound). */
int orc_row_norms(const uint16_t* X, int64_t R, int64_t K, int in_dtype, double* out,
                  int nthreads) {
    if (R < 0 || K < 0) return -1;
    if (!valid_in(in_dtype)) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const double* tab = table_for(in_dtype);
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; ++r) out[r] = norm_row(X + r * K, K, tab);
    return 0;
}

/* ---- 8-bit integer inputs -------------------------------------------------- */

/* One output entry: the exact integer dot product of row i of A and row j of
   stored B. */
static int64_t dot_row_i8(const int8_t* a, const int8_t* b, int64_t K) {
    int64_t s = 0;
    for (int64_t k = 0; k < K; ++k) s += (int64_t)a[k] * (int64_t)b[k];
    return s;
}

/* Full product of int8 operands: C (M x N int64) is caller-owned.  Returns 0,
   or -1 on bad args. */
int orc_gemm_bt_i8(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K, int64_t* C,
                   int nthreads) {
    if (M < 0 || N < 0 || K < 0 || K >= ((int64_t)1 << 49)) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) C[i * N + j] = dot_row_i8(A + i * K, B + j * K, K);
    return 0;
}

/* Selected entries of an int8 product: out[t] = C[I[t]][J[t]] for t < n. */
int orc_gemm_bt_i8_entries(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K,
                           const int64_t* I, const int64_t* J, int64_t n, int64_t* out, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || n < 0 || K >= ((int64_t)1 << 49)) return -1;
    for (int64_t t = 0; t < n; ++t)
        if (I[t] < 0 || I[t] >= M || J[t] < 0 || J[t] >= N) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t t;
#pragma omp parallel for schedule(dynamic, 64)
    for (t = 0; t < n; ++t) out[t] = dot_row_i8(A + I[t] * K, B + J[t] * K, K);
    return 0;
}
