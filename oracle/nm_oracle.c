/*
 * nm_oracle.c -- plain, slow, obviously-correct CPU oracle for N:M
 * semi-structured sparse matrix-vector products.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the GPU library.
 *
 * What it follows (all pages are secondary write-ups of the SparseDecoding
 * preprint; the abstract is the authority):
 *   - "SparseDecoding: Decoding-Aware Pruning for Accurate and Efficient LLM
 *     Inference", Abstract: decoding is dominated by SpMV; the system axis is
 *     an N:M sparse matrix-vector kernel that indexes kept weights with a
 *     bitmask and walks them with a fixed step.
 *   - "SparseDecoding Makes LLM Pruning Aware of Generation", Key points: the
 *     same kernel (kept weights located by mask bits, groups at a constant
 *     stride in the packed values).
 *   - bedrocknews arXiv 2610.12327v1 article: N:M means a fixed count of
 *     zeros inside every small block, and the product is a sparse matrix
 *     times one vector.
 *
 * Readings of points the pages leave open (each is a choice, not a quote):
 *   - Exactly N values are stored per M-wide group along a row (the reduction
 *     axis); stored values may be zero.
 *   - The keep bitmap has one bit per dense column, row-major, least
 *     significant bit first: bit (c mod 8) of byte c/8 of a row marks column
 *     c as kept.  Values are stored in ascending column order; group g's
 *     values start at offset g*N of the row (fixed step).
 *   - Top-N selection compares exact magnitudes |w| (so -0 == +0); ties go
 *     to the lower column index; a NaN anywhere in a group is an error.
 *   - Products and sums are formed in double precision, ascending column
 *     order, then rounded once, to nearest-even, into the 16-bit format.
 *
 * Every function here is written from those definitions; none of it is
 * blocked, fused or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_OK = 0, ORC_BAD_ARG = 1, ORC_BAD_SHAPE = 2, ORC_BAD_MASK = 4, ORC_NONFINITE = 5 };
enum { ORC_FP16 = 0, ORC_BF16 = 1 };

/* ---- 16-bit float formats, decoded from their field definitions ---------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double orc_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* f * 2^-126 * 2^-7 */
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

double orc_to_double(uint16_t bits, int dtype)
{
    return dtype == ORC_FP16 ? orc_fp16_to_double(bits) : orc_bf16_to_double(bits);
}

/*
 * Round a double to the nearest value of a binary format with `fbits`
 * fraction bits and minimum normal exponent `emin` (ties to even), then
 * encode it.  Overflow goes to infinity.  Rounding straight from the double
 * avoids the double rounding of a detour through float.
 */
static uint16_t round_encode(double v, int fbits, int emin, int emax, int ebits)
{
    uint16_t sign = signbit(v) ? (uint16_t)(1u << 15) : 0;
    int bias = (1 << (ebits - 1)) - 1;
    uint16_t inf_bits = (uint16_t)(((1u << ebits) - 1) << fbits);
    if (isnan(v))
        return (uint16_t)(sign | inf_bits | (1u << (fbits - 1)));
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | inf_bits);
    int E;
    frexp(a, &E);                       /* a = m * 2^E, m in [0.5, 1): floor(log2 a) = E - 1 */
    int e = E - 1;
    if (e < emin)
        e = emin;                       /* subnormal range shares the ulp of the smallest binade */
    int q = e - fbits;                  /* exponent of one ulp at a */
    double scaled = ldexp(a, -q);       /* exact: only the exponent changes */
    double n = floor(scaled);
    double r = scaled - n;              /* exact fractional part */
    if (r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;
    /* n * 2^q is the rounded magnitude; n is in [0, 2^(fbits+1)]. */
    if (n >= ldexp(1.0, fbits + 1)) {   /* carried into the next binade */
        n = ldexp(1.0, fbits);
        q += 1;
    }
    if (n < ldexp(1.0, fbits))          /* subnormal (only possible when e == emin) */
        return (uint16_t)(sign | (uint16_t)n);
    int exp_field = q + fbits + bias;
    if (q + fbits > emax)
        return (uint16_t)(sign | inf_bits);
    return (uint16_t)(sign | (uint16_t)(exp_field << fbits) | (uint16_t)(n - ldexp(1.0, fbits)));
}

uint16_t orc_double_to_fp16(double v) { return round_encode(v, 10, -14, 15, 5); }
uint16_t orc_double_to_bf16(double v) { return round_encode(v, 7, -126, 127, 8); }

void orc_round_array(const double* y, int64_t n, int dtype, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == ORC_FP16 ? orc_double_to_fp16(y[i]) : orc_double_to_bf16(y[i]);
}

void orc_decode_array(const uint16_t* bits, int64_t n, int dtype, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_to_double(bits[i], dtype);
}

/* ---- shape rules ---------------------------------------------------------- */

static int check_nm(int64_t R, int64_t K, int N, int M)
{
    if (R < 0 || K < 0)
        return ORC_BAD_SHAPE;
    if (M != 4 && M != 8)
        return ORC_BAD_SHAPE;
    if (N < 1 || N >= M)
        return ORC_BAD_SHAPE;
    if (K % M != 0 || K % 8 != 0)
        return ORC_BAD_SHAPE;
    return ORC_OK;
}

/* ---- pack ----------------------------------------------------------------- */

/*
 * Choose the kept columns of one M-wide group.  keep != NULL: the kept
 * columns are the nonzero keep bytes and there must be exactly N of them.
 * keep == NULL: N times over, take the not-yet-chosen column of largest
 * |w|, scanning in ascending column order so the lowest index wins a tie.
 */
static int select_group(const uint16_t* w, const uint8_t* keep, int N, int M, int dtype, int* chosen)
{
    for (int j = 0; j < M; ++j)
        chosen[j] = 0;
    if (keep) {
        int count = 0;
        for (int j = 0; j < M; ++j)
            if (keep[j] != 0) {
                chosen[j] = 1;
                ++count;
            }
        return count == N ? ORC_OK : ORC_BAD_MASK;
    }
    double mag[8];
    for (int j = 0; j < M; ++j) {
        double v = orc_to_double(w[j], dtype);
        if (isnan(v))
            return ORC_NONFINITE;
        mag[j] = fabs(v);
    }
    for (int t = 0; t < N; ++t) {
        int best = -1;
        for (int j = 0; j < M; ++j) {
            if (chosen[j])
                continue;
            if (best < 0 || mag[j] > mag[best])
                best = j;
        }
        chosen[best] = 1;
    }
    return ORC_OK;
}

/*
 * W [R][K] 16-bit words, keep [R][K] bytes or NULL.
 * values [R][K*N/M] 16-bit words, masks [R][K/8] bytes.
 * All groups are checked before anything is written, so on error the
 * outputs are untouched.
 */
int orc_pack(const uint16_t* W, const uint8_t* keep, int64_t R, int64_t K, int N, int M, int dtype,
             uint16_t* values, uint8_t* masks)
{
    int st = check_nm(R, K, N, M);
    if (st != ORC_OK)
        return st;
    if (dtype != ORC_FP16 && dtype != ORC_BF16)
        return ORC_BAD_ARG;
    int chosen[8];
    int64_t G = K / M;
    int worst = ORC_OK;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t g = 0; g < G; ++g) {
            st = select_group(W + r * K + g * M, keep ? keep + r * K + g * M : NULL, N, M, dtype, chosen);
            if (st == ORC_NONFINITE)
                return st;
            if (st != ORC_OK)
                worst = st;
        }
    if (worst != ORC_OK)
        return worst;

    int64_t vrow = K / M * N;
    for (int64_t r = 0; r < R; ++r) {
        uint8_t* mrow = masks + r * (K / 8);
        uint16_t* vout = values + r * vrow;
        memset(mrow, 0, (size_t)(K / 8));
        for (int64_t g = 0; g < G; ++g) {
            select_group(W + r * K + g * M, keep ? keep + r * K + g * M : NULL, N, M, dtype, chosen);
            int64_t next = g * N;                     /* fixed step: group g starts at g*N */
            for (int j = 0; j < M; ++j) {
                if (!chosen[j])
                    continue;
                int64_t c = g * M + j;
                mrow[c / 8] |= (uint8_t)(1u << (c % 8));
                vout[next++] = W[r * K + c];
            }
        }
    }
    return ORC_OK;
}

/* ---- expand --------------------------------------------------------------- */

/*
 * Rebuild the dense pruned matrix: column c of row r holds the k-th value of
 * its group when bit c is set (k = set bits below c inside the group), else
 * +0.  A group whose popcount is not N is a malformed packed matrix.
 */
int orc_expand(const uint16_t* values, const uint8_t* masks, int64_t R, int64_t K, int N, int M, uint16_t* Wt)
{
    int st = check_nm(R, K, N, M);
    if (st != ORC_OK)
        return st;
    int64_t G = K / M;
    int64_t vrow = G * N;
    for (int64_t r = 0; r < R; ++r) {
        const uint8_t* mrow = masks + r * (K / 8);
        for (int64_t g = 0; g < G; ++g) {
            int k = 0;
            for (int j = 0; j < M; ++j) {
                int64_t c = g * M + j;
                int bit = (mrow[c / 8] >> (c % 8)) & 1;
                if (bit) {
                    if (k >= N)
                        return ORC_BAD_MASK;
                    Wt[r * K + c] = values[r * vrow + g * N + k];
                    ++k;
                } else {
                    Wt[r * K + c] = 0;
                }
            }
            if (k != N)
                return ORC_BAD_MASK;
        }
    }
    return ORC_OK;
}

/* ---- products ------------------------------------------------------------- */

/*
 * y[b][r] = sum_c Wd[r][c] * x[b][c] and A[b][r] = sum_c |Wd[r][c] * x[b][c]|,
 * in double, ascending c, for rows r in [r0, r1).  Wd is a dense 16-bit row
 * source given as a callback-free pair: either a full dense matrix (W) or a
 * packed one expanded row by row.
 */
static void dense_rows(const uint16_t* Wrow, int64_t K, int dtype, const uint16_t* x, int B,
                       int64_t r, int64_t R, double* y, double* A, double* wbuf)
{
    for (int64_t c = 0; c < K; ++c)
        wbuf[c] = orc_to_double(Wrow[c], dtype);
    for (int b = 0; b < B; ++b) {
        double s = 0.0, sa = 0.0;
        for (int64_t c = 0; c < K; ++c) {
            double p = wbuf[c] * orc_to_double(x[b * K + c], dtype);   /* exact: 16-bit * 16-bit fits a double */
            s += p;
            sa += fabs(p);
        }
        y[b * R + r] = s;
        if (A)
            A[b * R + r] = sa;
    }
}

/* Dense GEMV over rows [r0, r1): W [R][K], x [B][K], y and A [B][R] (double). */
int orc_gemv_rows(const uint16_t* W, int64_t R, int64_t K, int dtype, const uint16_t* x, int B,
                  int64_t r0, int64_t r1, double* y, double* A)
{
    if (R < 0 || K < 0 || B < 1 || r0 < 0 || r1 > R || r0 > r1)
        return ORC_BAD_SHAPE;
    double* wbuf = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!wbuf)
        return ORC_BAD_ARG;
    for (int64_t r = r0; r < r1; ++r)
        dense_rows(W + r * K, K, dtype, x, B, r, R, y, A, wbuf);
    free(wbuf);
    return ORC_OK;
}

int orc_gemv(const uint16_t* W, int64_t R, int64_t K, int dtype, const uint16_t* x, int B, double* y, double* A)
{
    return orc_gemv_rows(W, R, K, dtype, x, B, 0, R, y, A);
}

/*
 * Sparse product over rows [r0, r1): expand each packed row to dense (the
 * definition of what the packed matrix means), then form the dense product.
 */
int orc_spmv_rows(const uint16_t* values, const uint8_t* masks, int64_t R, int64_t K, int N, int M, int dtype,
                  const uint16_t* x, int B, int64_t r0, int64_t r1, double* y, double* A)
{
    int st = check_nm(R, K, N, M);
    if (st != ORC_OK)
        return st;
    if (B < 1 || r0 < 0 || r1 > R || r0 > r1)
        return ORC_BAD_SHAPE;
    int64_t vrow = K / M * N;
    uint16_t* row = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(K > 0 ? K : 1));
    double* wbuf = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!row || !wbuf) {
        free(row);
        free(wbuf);
        return ORC_BAD_ARG;
    }
    for (int64_t r = r0; r < r1; ++r) {
        st = orc_expand(values + r * vrow, masks + r * (K / 8), 1, K, N, M, row);
        if (st != ORC_OK)
            break;
        dense_rows(row, K, dtype, x, B, r, R, y, A, wbuf);
    }
    free(row);
    free(wbuf);
    return st;
}

int orc_spmv(const uint16_t* values, const uint8_t* masks, int64_t R, int64_t K, int N, int M, int dtype,
             const uint16_t* x, int B, double* y, double* A)
{
    return orc_spmv_rows(values, masks, R, K, N, M, dtype, x, B, 0, R, y, A);
}

/* ---- gated-MLP epilogue --------------------------------------------------------
 * The decoder MLP of the model families the pages evaluate (Llama-3.1,
 * Llama-3.3, Qwen3) is SiLU-gated: h = SiLU(W_gate x) * (W_up x) elementwise,
 * SiLU(t) = t * sigmoid(t) = t / (1 + e^-t).  The pages do not describe the
 * layer; this is the definition written out, applied to the exact double
 * sums that orc_spmv / orc_gemv return.
 */
double orc_silu(double t)
{
    return t / (1.0 + exp(-t));
}

void orc_swiglu(const double* g, const double* u, int64_t n, double* h)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = orc_silu(g[i]) * u[i];
}

/* ---- decoding-aware calibration ---------------------------------------------
 * "SparseDecoding: Decoding-Aware Pruning ..." (Abstract) and "SparseDecoding
 * Makes LLM Pruning Aware of Generation" (Key points; section on why fixed-text
 * calibration misses): the pruning objective is built from the layer inputs
 * seen while the dense model generates, prefill excluded, and it is
 * Hessian-guided.  The pages give no formula.  Readings taken here:
 *   - the Hessian of a linear layer's squared output error is H = sum_t x_t x_t^T
 *     over its input rows x_t (up to a constant factor, which changes no
 *     decision); only rows marked as decode steps enter the sum;
 *   - the N:M keep-mask keeps, per group, the N columns of largest saliency
 *     w^2 * H_jj (the optimal-brain-surgeon saliency with H taken diagonal),
 *     ties to the lower column, like the magnitude rule.
 */

/* H[i][j] += sum over decode rows t of x[t][i] * x[t][j] (row-major K x K),
 * and A[i][j] += the same sum of |x[t][i] * x[t][j]|.  decode == NULL means
 * every row is a decode step. */
int orc_calib_accumulate(const uint16_t* X, const uint8_t* decode, int64_t T, int64_t K, int dtype, double* H,
                         double* A)
{
    if (T < 0 || K < 0 || (dtype != ORC_FP16 && dtype != ORC_BF16))
        return ORC_BAD_ARG;
    double* row = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!row)
        return ORC_BAD_ARG;
    for (int64_t t = 0; t < T; ++t) {
        if (decode && !decode[t])
            continue;                                   /* prefill row: excluded */
        for (int64_t i = 0; i < K; ++i)
            row[i] = orc_to_double(X[t * K + i], dtype);
        for (int64_t i = 0; i < K; ++i)
            for (int64_t j = 0; j < K; ++j) {
                double p = row[i] * row[j];             /* exact: two 16-bit significands */
                H[i * K + j] += p;
                A[i * K + j] += fabs(p);
            }
    }
    free(row);
    return ORC_OK;
}

/* The order used to rank saliencies and row losses: every number above NaN
 * (-inf included), numbers by value (-0 equal to +0), all NaNs equal. */
static int rank_above(double a, double b)
{
    if (isnan(a))
        return 0;
    return isnan(b) || a > b;
}

static int rank_equal(double a, double b)
{
    if (isnan(a) || isnan(b))
        return isnan(a) && isnan(b);
    return a == b;
}

/* keep[r][c] = 1 for the N columns of each M-group of row r with the largest
 * saliency w^2 * h[c], 0 elsewhere; equal saliencies go to the lower column.
 * h holds the Hessian diagonal (fp32 values, passed exactly as doubles).  The
 * saliency is formed exactly in double (w^2 has at most 22 significant bits,
 * h 24).  A NaN saliency ranks below every number, -inf included; NaNs
 * rank equal among themselves (lower column first). */
int orc_calib_keep(const uint16_t* W, const double* h, int64_t R, int64_t K, int N, int M, int dtype, uint8_t* keep)
{
    int st = check_nm(R, K, N, M);
    if (st != ORC_OK)
        return st;
    if (dtype != ORC_FP16 && dtype != ORC_BF16)
        return ORC_BAD_ARG;
    double sal[8];
    int taken[8];
    for (int64_t r = 0; r < R; ++r)
        for (int64_t g = 0; g < K / M; ++g) {
            for (int j = 0; j < M; ++j) {
                int64_t c = g * M + j;
                double w = orc_to_double(W[r * K + c], dtype);
                double s = w * w * h[c];
                sal[j] = s;
                taken[j] = 0;
                keep[r * K + c] = 0;
            }
            for (int k = 0; k < N; ++k) {
                int best = -1;
                for (int j = 0; j < M; ++j)
                    if (!taken[j] && (best < 0 || rank_above(sal[j], sal[best])))
                        best = j;
                taken[best] = 1;
                keep[r * K + g * M + best] = 1;
            }
        }
    return ORC_OK;
}

/* ---- hybrid sparse + dense rows ----------------------------------------------
 * The Spense abstract on the fifth page (thelatestinai.com page for arXiv
 * 2610.02598) splits a weight matrix into a 2:4-sparse region and a dense
 * region and stresses choosing the dense region well; it gives neither the
 * region's shape nor the rule.  Readings taken here: the dense region is a
 * set of whole rows (output channels), and the rows kept dense are those
 * whose pruning loses most, the loss of a row being
 *     L_r = sum over its pruned columns c of w[r][c]^2 * h[c]
 * (the diagonal saliency of the calibration reading, h = 1 without one).
 * The pruned columns are those the keep-mask drops, or, without one, those
 * top-N by magnitude drops (the nm_pack rule).
 */

/* L_r for every row: groups in column order, and within a group the pruned
 * columns in ascending order; each term (w*w)*h is exact in double and the
 * running sum is rounded once per term.  h == NULL means h = 1. */
int orc_hybrid_row_loss(const uint16_t* W, const uint8_t* keep, const double* h, int64_t R, int64_t K, int N, int M,
                        int dtype, double* loss)
{
    int st = check_nm(R, K, N, M);
    if (st != ORC_OK)
        return st;
    if (dtype != ORC_FP16 && dtype != ORC_BF16)
        return ORC_BAD_ARG;
    int chosen[8];
    for (int64_t r = 0; r < R; ++r) {
        double l = 0.0;
        for (int64_t g = 0; g < K / M; ++g) {
            const uint16_t* w = W + r * K + g * M;
            st = select_group(w, keep ? keep + r * K + g * M : NULL, N, M, dtype, chosen);
            if (st != ORC_OK)
                return st;
            for (int j = 0; j < M; ++j) {
                if (chosen[j])
                    continue;
                double v = orc_to_double(w[j], dtype);
                double hv = h ? h[g * M + j] : 1.0;
                double term = v * v * hv;
                l = l + term;
            }
        }
        loss[r] = l;
    }
    return ORC_OK;
}

/* flags[r] = 1 for the n_dense rows of largest loss (a NaN loss below every
 * number, -inf included), the lower row first among equals; 0 for the others. */
int orc_hybrid_select(const double* loss, int64_t R, int64_t n_dense, uint8_t* flags)
{
    if (R < 0 || n_dense < 0 || n_dense > R)
        return ORC_BAD_SHAPE;
    for (int64_t r = 0; r < R; ++r) {
        int64_t above = 0;
        for (int64_t s = 0; s < R; ++s)
            if (rank_above(loss[s], loss[r]) || (rank_equal(loss[s], loss[r]) && s < r))
                ++above;
        flags[r] = above < n_dense ? 1 : 0;
    }
    return ORC_OK;
}
