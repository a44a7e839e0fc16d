/*
 * Plain CPU oracle for the MXFP4 block-scaled GEMM
 *
 *     D[M,N] = bf16( alpha * A[M,K] * B[N,K]^T + beta * C[M,N] )
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * Sources (page title, then section):
 *   - "asm_f4gemm -- driving aiter's gfx950 MXFP4 GEMM code objects"
 *     (README of asm_f4gemm), top: the problem statement D = alpha*A*B^T +
 *     beta*C with bf16 D and MXFP4 A, B.
 *   - same page, "Data layouts", section "A -- activations": row-major
 *     [rows, K/2] bytes; byte i of a row holds element 2i in its low nibble
 *     and element 2i+1 in its high nibble; values are OCP E2M1
 *     {0, .5, 1, 1.5, 2, 3, 4, 6} with the sign in bit 3.
 *   - same page, "Data layouts", section "A_scale / B_scale": E8M0 is a bare
 *     biased exponent, value 2^(e-127), 0xFF is NaN, one scale per 32
 *     consecutive K elements of a row.
 *   - same page, "Verification": the reference is an f64-accumulate GEMM
 *     over the dequantized operands.
 *
 * Readings where the pages leave a step open (each is listed in the design doc):
 *   - E8M0 code 0x00: the page states the formula 2^(e-127) and, in the
 *     same sentence, "0 -> 2^-126".  The formula is used for every code
 *     below 0xFF, so 0x00 is 2^-127.
 *   - Output rounding is not stated; bf16 round-to-nearest-even is applied
 *     once, directly from the fp64 value (no detour through fp32).
 *   - beta == 0 means C is never read (C may be NULL).
 *   - C is bf16 with its own row stride ldc.
 *
 * Build: cc -O2 -ffp-contract=off -fPIC -shared mxfp4_oracle.c -lm
 * (no fast-math: every sum is formed in the order written, k ascending).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- element codes ---------------------------------------------------- */

/* E2M1 magnitudes indexed by the low three bits of the code; bit 3 is the
 * sign.  Values as listed in "Data layouts" / "A -- activations". */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1(unsigned code)
{
    double m = E2M1_MAGNITUDE[code & 7u];
    return (code & 8u) ? -m : m;
}

/* E8M0: 2^(e-127), 0xFF is NaN ("Data layouts" / "A_scale / B_scale"). */
double oracle_e8m0(unsigned e)
{
    e &= 0xFFu;
    if (e == 0xFFu)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* Code of element k of row r of a packed fp4x2 matrix whose rows are
 * ld fp4 elements (ld/2 bytes) apart: low nibble = even k. */
unsigned oracle_fp4_code(const uint8_t *X, int64_t ld, int64_t r, int64_t k)
{
    uint8_t byte = X[r * (ld / 2) + k / 2];
    return (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 0x0Fu);
}

/* Dequantized element: E2M1 value times the E8M0 scale of its 32-block. */
double oracle_mx_element(const uint8_t *X, int64_t ld, const uint8_t *SX,
                         int64_t lds, int64_t r, int64_t k)
{
    return oracle_e2m1(oracle_fp4_code(X, ld, r, k)) *
           oracle_e8m0(SX[r * lds + k / 32]);
}

/* ---- wider A formats ----------------------------------------------------- */

/*
 * "CDNA4 dense MFMA builtins", section "Mixed-precision with scaling": the
 * scaled matrix instructions take FP8 (E4M3), BF8 (E5M2), FP6 (E2M3),
 * FP6 (E3M2) and FP4 (E2M1) inputs, 8, 8, 6, 6 and 4 bits per element,
 * selected per operand.  The pages give the names and widths only; the
 * element encodings are those of the OCP Microscaling Formats v1.0
 * specification (section 5.3): sign in the top bit, then the exponent
 * field, then the mantissa field; exponent field 0 is subnormal
 * (0.m x 2^(1 - bias)); E4M3 has no infinities and NaN only at
 * exponent 1111 with mantissa 111; E5M2 is IEEE-like (exponent 11111:
 * infinity with mantissa 0, else NaN); the FP6 formats have no special
 * codes.
 *
 * Format ids here (the library's, not the instructions' codes):
 *   0 FP4 E2M1, 1 FP8 E4M3, 2 BF8 E5M2, 3 FP6 E2M3, 4 FP6 E3M2.
 *
 * Reading (the pages do not say how rows of these formats are laid out in
 * memory): a row of A is a little-endian bit stream of w-bit fields,
 * element k at bits [k*w, k*w + w).  For FP4 this is the low-nibble-first
 * byte order of "Data layouts"; for FP8 element k is byte k; for FP6 one
 * 32-element block is 24 bytes.
 */
int oracle_format_bits(int fmt)
{
    static const int bits[5] = {4, 8, 8, 6, 6};
    return (fmt >= 0 && fmt < 5) ? bits[fmt] : 0;
}

double oracle_decode(int fmt, unsigned code)
{
    if (fmt == 0)
        return oracle_e2m1(code & 0xFu);
    /* exponent bits, mantissa bits, bias */
    static const int EB[5] = {2, 4, 5, 2, 3}, MB[5] = {1, 3, 2, 3, 2}, BIAS[5] = {1, 7, 15, 1, 3};
    if (fmt < 1 || fmt > 4)
        return NAN;
    const int eb = EB[fmt], mb = MB[fmt], bias = BIAS[fmt];
    const unsigned s = (code >> (eb + mb)) & 1u;
    const unsigned e = (code >> mb) & ((1u << eb) - 1u);
    const unsigned m = code & ((1u << mb) - 1u);
    double v;
    if (fmt == 1 && e == 15u && m == 7u)
        return NAN;
    if (fmt == 2 && e == 31u)
        v = m == 0u ? INFINITY : NAN;
    else if (e == 0u)
        v = ldexp((double)m, 1 - bias - mb);
    else
        v = ldexp((double)((1u << mb) + m), (int)e - bias - mb);
    return s ? -v : v;
}

/* Code of element k of row r: bits [k*w, k*w + w) of the row's bytes,
 * little-endian; rows are ld_bytes apart. */
unsigned oracle_elem_code(const uint8_t *X, int64_t ld_bytes, int w, int64_t r, int64_t k)
{
    const int64_t bit = k * w;
    const uint8_t *p = X + r * ld_bytes + bit / 8;
    const int sh = (int)(bit % 8);
    unsigned v = p[0];
    if (sh + w > 8)
        v |= (unsigned)p[1] << 8;
    return (v >> sh) & ((1u << w) - 1u);
}

/* Dequantized element of a row of format fmt (rows ld_bytes apart). */
double oracle_mx_element_fmt(const uint8_t *X, int64_t ld_bytes, int fmt, const uint8_t *SX,
                             int64_t lds, int64_t r, int64_t k)
{
    return oracle_decode(fmt, oracle_elem_code(X, ld_bytes, oracle_format_bits(fmt), r, k)) *
           oracle_e8m0(SX[r * lds + k / 32]);
}

/* ---- bf16 --------------------------------------------------------------- */

double oracle_bf16_to_double(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Largest finite bf16: (2 - 2^-7) * 2^127. */
#define BF16_MAX_FINITE 3.3895313892515355e38

/* Round a double to the nearest bf16, ties to even, in one step.
 * bf16 has 8 significant bits; in the binade [2^E, 2^(E+1)) its spacing is
 * 2^(E-7); below 2^-126 the spacing stays 2^-133 (subnormals). */
uint16_t oracle_bf16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e;
    (void)frexp(a, &e);          /* a = f * 2^e with f in [0.5, 1) */
    int E = e - 1;               /* a in [2^E, 2^(E+1)) */
    if (E < -126)
        E = -126;
    double q = ldexp(1.0, E - 7);
    double r = nearbyint(a / q); /* default rounding mode: ties to even */
    double v = r * q;
    if (v > BF16_MAX_FINITE)
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)v;          /* exact: v has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (bits >> 16));
}

/* ---- the GEMM ------------------------------------------------------------ */

/*
 * Reference values for the sub-block rows[0..nrows) x cols[0..ncols) of D.
 *
 *   ref[ri*ncols+cj] = alpha * sum_k a(i,k) b(j,k) + beta * C[i,j]   (fp64)
 *   mag[ri*ncols+cj] = sum_k |a(i,k) b(j,k)|                         (fp64)
 *   dref[...]        = bf16_rne(ref)
 *
 * with i = rows[ri], j = cols[cj]; the sum runs over k = 0..K-1 ascending.
 * A is [M][lda/2] bytes, B is [N][ldb/2] bytes (both row-major, K-major;
 * with a_fmt != 0 A holds that format and its rows are lda * w / 8 bytes
 * apart, w its element width),
 * SA is [M][ldsa] bytes, SB is [N][ldsb] bytes, C is [M][ldc] bf16, or
 * float32 when c_f32 != 0 (the f32 bias of the asm_f4gemm README's
 * "C / bias" note; either way its value enters exactly, in fp64).
 * C is read only when beta != 0.  Any of mag/dref may be NULL.
 *
 * b_layout selects how B's codes are stored ("CDNA4 MFMA transpose load
 * builtins", opening section: an operand may be kept MN-major, B in
 * row-major [K][N] order, instead of K-major):
 *   0  B is [N][ldb/2] bytes, row j holding its K codes (K-major);
 *   1  B is [K][ldb/2] bytes, row k holding the codes of the N columns at
 *      that k (MN-major), element j of the row in the low nibble of byte j/2
 *      when j is even -- the same packing along the row as for K-major rows.
 * SB is [N][ldsb] (one scale per column j and 32-block of k) either way.
 * Returns 0, or -1 when scratch memory cannot be allocated.
 */
int oracle_mxgemm(int64_t K, int a_fmt,
                  const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                  const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb, int b_layout,
                  const void *C, int64_t ldc, int c_f32, double alpha, double beta,
                  const int64_t *rows, int64_t nrows,
                  const int64_t *cols, int64_t ncols,
                  double *ref, double *mag, uint16_t *dref)
{
    if (nrows <= 0 || ncols <= 0)
        return 0;
    double *a = (double *)malloc(sizeof(double) * (size_t)(nrows * (K > 0 ? K : 1)));
    double *b = (double *)malloc(sizeof(double) * (size_t)(ncols * (K > 0 ? K : 1)));
    if (!a || !b) {
        free(a);
        free(b);
        return -1;
    }
    /* Dequantize the rows of A and of B that the requested block needs. */
    const int64_t lda_bytes = lda * oracle_format_bits(a_fmt) / 8;
    for (int64_t ri = 0; ri < nrows; ++ri)
        for (int64_t k = 0; k < K; ++k)
            a[ri * K + k] = a_fmt == 0 ? oracle_mx_element(A, lda, SA, ldsa, rows[ri], k)
                                       : oracle_mx_element_fmt(A, lda_bytes, a_fmt, SA, ldsa, rows[ri], k);
    for (int64_t cj = 0; cj < ncols; ++cj)
        for (int64_t k = 0; k < K; ++k)
            b[cj * K + k] = b_layout == 0
                                ? oracle_mx_element(B, ldb, SB, ldsb, cols[cj], k)
                                : oracle_e2m1(oracle_fp4_code(B, ldb, k, cols[cj])) *
                                      oracle_e8m0(SB[cols[cj] * ldsb + k / 32]);

    for (int64_t ri = 0; ri < nrows; ++ri) {
        const double *ar = a + ri * K;
        for (int64_t cj = 0; cj < ncols; ++cj) {
            const double *bc = b + cj * K;
            double acc = 0.0, m = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = ar[k] * bc[k];
                acc += p;
                m += fabs(p);
            }
            double r = alpha * acc;
            if (beta != 0.0) {
                const int64_t ci = rows[ri] * ldc + cols[cj];
                r += beta * (c_f32 ? (double)((const float *)C)[ci]
                                   : oracle_bf16_to_double(((const uint16_t *)C)[ci]));
            }
            int64_t o = ri * ncols + cj;
            ref[o] = r;
            if (mag)
                mag[o] = m;
            if (dref)
                dref[o] = oracle_bf16_rne(r);
        }
    }
    free(a);
    free(b);
    return 0;
}

/* ---- FP16 GEMM ------------------------------------------------------------ */

/*
 * "CDNA4 MFMA transpose load builtins", "FP16 GEMM example": C = A * B with
 * A [M][K] fp16 row-major, B [K][N] fp16 row-major and fp32 C.  The
 * reference is the exact sum of the fp16 products in fp64, k ascending.
 * fp16 is IEEE binary16: sign, 5 exponent bits (bias 15), 10 fraction bits;
 * exponent 0 subnormal, 31 infinity or NaN.
 */
double oracle_f16_to_double(uint16_t h)
{
    const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* ref/mag for the sub-block rows[] x cols[]; lda, ldb in elements */
int oracle_f16_gemm(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                    const int64_t *rows, int64_t nrows, const int64_t *cols, int64_t ncols,
                    double *ref, double *mag)
{
    for (int64_t ri = 0; ri < nrows; ++ri)
        for (int64_t cj = 0; cj < ncols; ++cj) {
            double acc = 0.0, m = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = oracle_f16_to_double(A[rows[ri] * lda + k]) *
                                 oracle_f16_to_double(B[k * ldb + cols[cj]]);
                acc += p;
                m += fabs(p);
            }
            ref[ri * ncols + cj] = acc;
            if (mag)
                mag[ri * ncols + cj] = m;
        }
    return 0;
}

/* ---- exact mode ------------------------------------------------------------ */

/*
 * Exact value of sum_k a(i,k) b(j,k) for one (i, j), in integer arithmetic.
 *
 * Every E2M1 value is an integer multiple of 1/2 (2*|v| is one of
 * 0,1,2,3,4,6,8,12), so each product is (2a)(2b)/4 * 2^(sa+sb-254).  The
 * sum is held as a 128-bit integer in units of 2^(emin-256), where emin is
 * the smallest sa+sb over the K blocks.  Result: sum = *mant * 2^(*exp2).
 *
 * Returns 0 on success, 1 if a scale is NaN (0xFF), 2 if the spread of
 * exponents is too wide for 128-bit fixed point.
 */
static const int E2M1_TWICE[8] = {0, 1, 2, 3, 4, 6, 8, 12};

int oracle_dot_exact(int64_t K,
                     const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                     const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb,
                     int64_t i, int64_t j, __int128 *mant, int *exp2)
{
    int64_t nblk = K / 32;
    int emin = 1 << 20, emax = -(1 << 20);
    for (int64_t kb = 0; kb < nblk; ++kb) {
        int sa = SA[i * ldsa + kb], sb = SB[j * ldsb + kb];
        if (sa == 0xFF || sb == 0xFF)
            return 1;
        int s = sa + sb;
        if (s < emin) emin = s;
        if (s > emax) emax = s;
    }
    /* per block: 32 products of at most 144, i.e. < 2^13; whole sum < 2^13 * nblk */
    int guard = 13;
    for (int64_t n = nblk; n > 1; n >>= 1)
        ++guard;
    if ((emax - emin) + guard > 125)
        return 2;
    __int128 acc = 0;
    for (int64_t kb = 0; kb < nblk; ++kb) {
        int shift = SA[i * ldsa + kb] + SB[j * ldsb + kb] - emin;
        __int128 blk = 0;
        for (int64_t k = kb * 32; k < kb * 32 + 32; ++k) {
            unsigned ca = oracle_fp4_code(A, lda, i, k);
            unsigned cb = oracle_fp4_code(B, ldb, j, k);
            int p = E2M1_TWICE[ca & 7u] * E2M1_TWICE[cb & 7u];
            blk += ((ca ^ cb) & 8u) ? -p : p;
        }
        acc += blk * ((__int128)1 << shift);
    }
    *mant = acc;
    *exp2 = emin - 254 - 2; /* (2a)(2b)/4 and the two biases of 127 */
    return 0;
}

/* Round mant * 2^exp2 (exact) to bf16, ties to even. */
uint16_t oracle_bf16_rne_exact(__int128 mant, int exp2)
{
    uint16_t sign = 0;
    if (mant < 0) {
        sign = 0x8000u;
        mant = -mant;
    }
    if (mant == 0)
        return sign;
    unsigned __int128 u = (unsigned __int128)mant;
    int nbits = 0;
    for (unsigned __int128 t = u; t; t >>= 1)
        ++nbits;
    int E = nbits - 1 + exp2;  /* value in [2^E, 2^(E+1)) */
    int Eq = E < -126 ? -126 : E;
    int drop = (Eq - 7) - exp2; /* bits below the bf16 spacing 2^(Eq-7) */
    unsigned __int128 r;
    if (drop <= 0) {
        r = u << (-drop);
    } else if (drop >= 128) {
        r = 0; /* far below half of the smallest spacing */
    } else {
        unsigned __int128 q = u >> drop;
        unsigned __int128 rem = u - (q << drop);
        unsigned __int128 half = (unsigned __int128)1 << (drop - 1);
        if (rem > half || (rem == half && (q & 1)))
            ++q;
        r = q;
    }
    /* value = r * 2^(Eq-7) with r <= 256 */
    double v = ldexp((double)(uint64_t)r, Eq - 7);
    if (v > BF16_MAX_FINITE)
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)v;
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (bits >> 16));
}

/* The exact sum rounded once to fp64 (for comparing with the fp64 sum). */
double oracle_exact_to_double(__int128 mant, int exp2)
{
    /* split into two 64-bit halves; each conversion and the final add are
     * exact except for the single rounding of the add when the value needs
     * more than 53 bits */
    int neg = mant < 0;
    unsigned __int128 u = neg ? (unsigned __int128)(-mant) : (unsigned __int128)mant;
    uint64_t hi = (uint64_t)(u >> 64), lo = (uint64_t)u;
    double v;
    if (hi == 0) {
        v = (double)lo; /* one correctly rounded conversion */
    } else {
        /* reduce to 64 significant bits with a sticky bit, then convert */
        int nb = 0;
        for (unsigned __int128 t = u; t; t >>= 1)
            ++nb;
        int sh = nb - 64;
        unsigned __int128 q = u >> sh;
        int sticky = (u - (q << sh)) != 0;
        uint64_t q64 = (uint64_t)q | (uint64_t)sticky; /* bit 0 is far below bit 53 */
        v = ldexp((double)q64, sh);
    }
    v = ldexp(v, exp2);
    return neg ? -v : v;
}

/* Wrapper with plain types for foreign-function callers: the mantissa is
 * returned as two 64-bit halves (hi signed, lo unsigned). */
int oracle_dot_exact_parts(int64_t K,
                           const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                           const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb,
                           int64_t i, int64_t j,
                           int64_t *mant_hi, uint64_t *mant_lo, int *exp2,
                           double *as_double, uint16_t *as_bf16)
{
    __int128 m;
    int e;
    int rc = oracle_dot_exact(K, A, lda, SA, ldsa, B, ldb, SB, ldsb, i, j, &m, &e);
    if (rc)
        return rc;
    *mant_hi = (int64_t)(m >> 64);
    *mant_lo = (uint64_t)m;
    *exp2 = e;
    *as_double = oracle_exact_to_double(m, e);
    *as_bf16 = oracle_bf16_rne_exact(m, e);
    return 0;
}

/* ---- activation quantizer: bf16 -> MXFP4 ----------------------------------- */

/*
 * The pages define the two formats a quantizer produces (E2M1 codes and E8M0
 * scales, "Data layouts") but not how real-valued input is mapped onto them.
 * This follows the conversion rule of the OCP Microscaling Formats (MX) v1.0
 * specification, section 6.3 "Conversion of a vector of scalars to MX".
 * Readings (each also listed in the design doc):
 *   Q1 the scale exponent of a 32-block is X = floor(log2(max_i |v_i|)) - 2,
 *      2 being the largest E2M1 exponent (6 = 1.5 * 2^2), clamped to the E8M0
 *      range [-127, 127]; the scale code is X + 127.
 *   Q2 element i is v_i / 2^X rounded to the nearest E2M1 value, ties to the
 *      encoding whose mantissa bit is 0, magnitudes that round beyond 6 give 6;
 *      the sign is kept, so a negative value that rounds to zero is code 0x8.
 *   Q3 a block holding a NaN or an infinity gets scale 0xFF (NaN) and codes 0.
 *   Q4 an all-zero block gets the clamped exponent of Q1 (-127, code 0x00) and
 *      codes 0.
 * All arithmetic is exact in fp64 (bf16 inputs, power-of-two scaling).
 */

/* Q2: nearest E2M1 magnitude code by direct search over the eight values. */
static unsigned e2m1_nearest_code(double m)
{
    unsigned best = 0;
    double best_d = fabs(m - E2M1_MAGNITUDE[0]);
    for (unsigned c = 1; c < 8; ++c) {
        double d = fabs(m - E2M1_MAGNITUDE[c]);
        if (d < best_d || (d == best_d && (c & 1u) == 0u)) {
            best = c;
            best_d = d;
        }
    }
    return best; /* beyond 6 the nearest value is 6 (code 7): saturation */
}

/*
 * X is [M][ldx] bf16 (row-major); A receives [M][lda/2] bytes (lda in fp4
 * elements, element k of a row in the low nibble of byte k/2 when k is even),
 * S receives [M][lds] scale bytes.  K % 32 == 0.  Only the first K elements
 * of each row, the first K/2 bytes of each A row and the first K/32 bytes of
 * each S row are touched.
 */
void oracle_quantize_mxfp4(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                           uint8_t *A, int64_t lda, uint8_t *S, int64_t lds)
{
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t kb = 0; kb < K / 32; ++kb) {
            double v[32];
            double amax = 0.0;
            int special = 0;
            for (int i = 0; i < 32; ++i) {
                v[i] = oracle_bf16_to_double(X[r * ldx + kb * 32 + i]);
                if (isnan(v[i]) || isinf(v[i]))
                    special = 1;
                else if (fabs(v[i]) > amax)
                    amax = fabs(v[i]);
            }
            uint8_t *arow = A + r * (lda / 2) + kb * 16;
            if (special) { /* Q3 */
                S[r * lds + kb] = 0xFFu;
                memset(arow, 0, 16);
                continue;
            }
            int x = -127; /* Q4 for an all-zero block */
            if (amax > 0.0) {
                int e;
                (void)frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1) */
                x = (e - 1) - 2;       /* Q1 */
                if (x < -127)
                    x = -127;
                if (x > 127)
                    x = 127;
            }
            S[r * lds + kb] = (uint8_t)(x + 127);
            for (int i = 0; i < 32; i += 2) {
                unsigned c[2];
                for (int h = 0; h < 2; ++h) {
                    double s = ldexp(v[i + h], -x); /* exact */
                    c[h] = e2m1_nearest_code(fabs(s)) | (signbit(s) ? 8u : 0u);
                }
                arow[i / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}
