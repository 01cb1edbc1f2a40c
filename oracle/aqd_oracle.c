/*
 * CPU oracle for the additive-codebook decode linear  (TEST INFRASTRUCTURE)
 * =========================================================================
 *
 * A plain, slow, double-precision reference of what the decode-time linear
 * of Drop-by-Drop computes.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * links, loads or calls it, and it shares no code, header, table or helper
 * with the HIP library.
 *
 * Source: "Multi-Bitwidth Quantization for LLMs Using Additive Codebooks"
 * (Drop-by-Drop), cited by section below.
 *
 *   y[n][i] = s_i * sum_c What_k[i][c] * xrot[n][c]
 *   What_k[i][8j + t] = sum_{m < k} C_m[ codes[i][j][m] ][t]
 *   xrot = (1/sqrt(b)) * blockdiag(H_b, ..., H_b) * x
 *
 * - Section 3.2 (AQLM): a weight row is split into groups of g consecutive
 *   inputs; each group is the sum of one codeword from each codebook, the
 *   codeword picked by that group's index into the codebook; the row is the
 *   concatenation of its d_in/g group sums along the input dimension.
 * - Section 5: at inference the weights are dequantized from a prefix of the
 *   first k <= M codebooks; the optional block-wise Walsh-Hadamard rotation.
 * - Section 6 "Experimental Setup" / "Method Definitions": g = 8, 8-bit codes
 *   (2^8 = 256 codewords per codebook).
 * - Appendix "Estimating Model Size": fp16 codebooks [M][2^B][g], B-bit
 *   codes, one fp16 scale per output row; the storage formula.
 *
 * Readings where the pages leave a step open (each is a choice made here):
 *   - the scale multiplies the whole output row and one scale serves every k;
 *   - the rotation is orthonormal: H_b / sqrt(b) with H_b the Sylvester
 *     (natural-order) Walsh-Hadamard matrix, H[r][c] = (-1)^popcount(r & c),
 *     applied to contiguous aligned blocks of b inputs, no random signs
 *     (the signed variant below is a separate entry, R = H_b diag(eps)/sqrt(b));
 *   - codeword element t multiplies input 8j + t.
 *
 * Everything here is the definition written out: the Hadamard product is a
 * dense O(b^2) sum per block (not a fast transform), Wk is reconstructed
 * explicitly element by element, and the product is an ascending-index dot
 * product in double.  Rows are independent, so the OpenMP split over rows
 * gives bit-identical results for any thread count.
 *
 * Parity pins live in the test suite (closed forms, invariants, brute force,
 * the storage worked example).  Parity unpinned: nothing in this file is
 * left without a pin; the GPU's fp32 summation order is compared by
 * tolerance only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 8
#define ORACLE_CODEWORDS 256

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_F32 = 2 };

/* ---------------------------------------------------------------------------
 * Number formats (IEEE binary16 and bfloat16), exact decode and
 * round-to-nearest-even encode from double.
 * ------------------------------------------------------------------------- */

double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                  /* zero / subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);      /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int f = h & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                 /* zero / subnormal */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);      /* 1.f * 2^(e-127) */
    return sign ? -v : v;
}

/* Round |v| to a binary format with `mant` stored fraction bits, exponent
 * bias `bias` and all-ones exponent `emax_field` reserved for inf/nan.
 * Returns the magnitude bits (no sign). */
static uint32_t encode_mag(double a, int mant, int bias, int emax_field)
{
    const int emin = 1 - bias;                      /* smallest normal exponent */
    int ex;
    double q;
    if (a == 0.0)
        return 0;
    frexp(a, &ex);                                  /* a = f * 2^ex, f in [0.5, 1) */
    ex -= 1;                                        /* a in [2^ex, 2^(ex+1)) */
    if (ex < emin) {
        /* subnormal: integer multiples of 2^(emin - mant) */
        q = nearbyint(ldexp(a, mant - emin));
        return (uint32_t)q;                         /* q == 2^mant lands on the smallest normal */
    }
    q = nearbyint(ldexp(a, mant - ex));             /* in [2^mant, 2^(mant+1)] */
    if (q >= ldexp(1.0, mant + 1)) {
        q = ldexp(1.0, mant);
        ex += 1;
    }
    if (ex + bias >= emax_field)
        return (uint32_t)emax_field << mant;        /* overflow -> infinity */
    return ((uint32_t)(ex + bias) << mant) | (uint32_t)(q - ldexp(1.0, mant));
}

uint16_t oracle_f64_to_f16(double v)
{
    if (isnan(v))
        return 0x7E00;
    uint16_t s = signbit(v) ? 0x8000 : 0;
    return s | (uint16_t)encode_mag(fabs(v), 10, 15, 31);
}

uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t s = signbit(v) ? 0x8000 : 0;
    return s | (uint16_t)encode_mag(fabs(v), 7, 127, 255);
}

/* Decode n 16-bit patterns (dtype ORACLE_F16 or ORACLE_BF16) or n float32
 * values (ORACLE_F32, `src` read as float) into doubles. */
int oracle_decode(const void *src, int dtype, int64_t n, double *out)
{
    int64_t i;
    if (dtype == ORACLE_F16) {
        const uint16_t *h = (const uint16_t *)src;
        for (i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
    } else if (dtype == ORACLE_BF16) {
        const uint16_t *h = (const uint16_t *)src;
        for (i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(h[i]);
    } else if (dtype == ORACLE_F32) {
        const float *f = (const float *)src;
        for (i = 0; i < n; ++i) out[i] = (double)f[i];
    } else {
        return -1;
    }
    return 0;
}

/* Encode n doubles to fp16 / bf16 bit patterns, round to nearest even. */
int oracle_encode(const double *v, int dtype, int64_t n, uint16_t *out)
{
    int64_t i;
    if (dtype == ORACLE_F16) {
        for (i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(v[i]);
    } else if (dtype == ORACLE_BF16) {
        for (i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(v[i]);
    } else {
        return -1;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Block Walsh-Hadamard rotation (section 5: block-wise Walsh-Hadamard
 * rotation; applied online to the activation at inference, section 6
 * "DbyD vs. SOTA comparison").
 * ------------------------------------------------------------------------- */

static int popcount32(uint32_t v)
{
    int c = 0;
    while (v) {
        c += (int)(v & 1u);
        v >>= 1;
    }
    return c;
}

static int valid_block(int32_t b)
{
    return b >= 1 && b <= 4096 && (b & (b - 1)) == 0;
}

/* H[r*b + c] = (-1)^popcount(r & c): the Sylvester-order Hadamard matrix. */
int oracle_hadamard(int32_t b, int32_t *H)
{
    if (!valid_block(b))
        return -1;
    for (int32_t r = 0; r < b; ++r)
        for (int32_t c = 0; c < b; ++c)
            H[(int64_t)r * b + c] = (popcount32((uint32_t)(r & c)) & 1) ? -1 : 1;
    return 0;
}

/* out[n][beta*b + r] = b^(-1/2) * sum_c H[r][c] * x[n][beta*b + c]
 * x, out: [batch][d_in] doubles; b must divide d_in.  Dense product per block. */
int oracle_rotate(const double *x, int64_t batch, int64_t d_in, int32_t b, double *out)
{
    if (!valid_block(b) || d_in % b != 0 || batch < 0)
        return -1;
    int32_t *H = (int32_t *)malloc(sizeof(int32_t) * (size_t)b * (size_t)b);
    if (!H)
        return -2;
    oracle_hadamard(b, H);
    const double inv = 1.0 / sqrt((double)b);
    const int64_t nblk = d_in / b;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < batch * nblk; ++t) {
        const int64_t n = t / nblk, beta = t % nblk;
        const double *xb = x + n * d_in + beta * b;
        double *ob = out + n * d_in + beta * b;
        for (int32_t r = 0; r < b; ++r) {
            double acc = 0.0;
            for (int32_t c = 0; c < b; ++c)
                acc += (double)H[(int64_t)r * b + c] * xb[c];
            ob[r] = acc * inv;
        }
    }
    free(H);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Randomized block Hadamard rotation R = (1/sqrt(b)) H_b diag(eps), the
 * variant of "ApexQuant: calibration-free elastic quantization" (section 3,
 * the randomized Hadamard transform named after Eq. 2).  The sign pattern is a
 * bit mask: eps_c = -1 when bit (c mod 8) of byte signs[c / 8] is set, +1
 * otherwise; one pattern serves every row of the batch.
 * ------------------------------------------------------------------------- */

/* eps[c] = -1.0 or +1.0 from the bit mask, c in [0, d_in). */
int oracle_sign_vector(const uint8_t *signs, int64_t d_in, double *eps)
{
    if (d_in < 0 || (d_in > 0 && !signs))
        return -1;
    for (int64_t c = 0; c < d_in; ++c)
        eps[c] = ((signs[c / 8] >> (c % 8)) & 1u) ? -1.0 : 1.0;
    return 0;
}

/* out[n][beta*b + r] = b^(-1/2) * sum_c H[r][c] * eps[beta*b + c] * x[n][beta*b + c]
 * x, out: [batch][d_in] doubles; b must divide d_in.  Dense product per block. */
int oracle_rotate_signed(const double *x, const uint8_t *signs, int64_t batch, int64_t d_in, int32_t b,
                         double *out)
{
    if (!valid_block(b) || d_in % b != 0 || batch < 0)
        return -1;
    int32_t *H = (int32_t *)malloc(sizeof(int32_t) * (size_t)b * (size_t)b);
    double *eps = (double *)malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
    if (!H || !eps) {
        free(H);
        free(eps);
        return -2;
    }
    oracle_hadamard(b, H);
    if (oracle_sign_vector(signs, d_in, eps) != 0) {
        free(H);
        free(eps);
        return -1;
    }
    const double inv = 1.0 / sqrt((double)b);
    const int64_t nblk = d_in / b;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < batch * nblk; ++t) {
        const int64_t n = t / nblk, beta = t % nblk;
        const double *xs = x + n * d_in + beta * b;
        const double *es = eps + beta * b;
        double *os = out + n * d_in + beta * b;
        for (int32_t r = 0; r < b; ++r) {
            double acc = 0.0;
            for (int32_t c = 0; c < b; ++c)
                acc += (double)H[(int64_t)r * b + c] * (es[c] * xs[c]);
            os[r] = acc * inv;
        }
    }
    free(H);
    free(eps);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Additive-codebook reconstruction (section 3.2, prefix of k codebooks per
 * section 5).
 * codes:     [d_out][d_in/8][M] uint8 (row i, group j, codebook m)
 * codebooks: [M][256][8] doubles (decoded fp16)
 * scales:    [d_out] doubles (decoded fp16), or NULL for no scale
 * ------------------------------------------------------------------------- */

static int check_layer(int64_t d_out, int64_t d_in, int32_t M, int32_t k)
{
    if (d_out < 0 || d_in < 0 || d_in % ORACLE_GROUP != 0)
        return -1;
    if (M < 1 || k < 1 || k > M)
        return -1;
    return 0;
}

/* Row i of s_i * What_k into w[0..d_in). */
static void reconstruct_row(const uint8_t *codes, const double *codebooks, const double *scales,
                            int64_t i, int64_t d_in, int32_t M, int32_t k, double *w)
{
    const int64_t G = d_in / ORACLE_GROUP;
    const double s = scales ? scales[i] : 1.0;
    for (int64_t j = 0; j < G; ++j) {
        for (int t = 0; t < ORACLE_GROUP; ++t) {
            double g = 0.0;
            for (int32_t m = 0; m < k; ++m) {
                const uint8_t c = codes[(i * G + j) * M + m];
                g += codebooks[((int64_t)m * ORACLE_CODEWORDS + c) * ORACLE_GROUP + t];
            }
            w[j * ORACLE_GROUP + t] = s * g;
        }
    }
}

/* W[d_out][d_in] = s_i * What_k[i][c], explicitly. */
int oracle_reconstruct(const uint8_t *codes, const double *codebooks, const double *scales,
                       int64_t d_out, int64_t d_in, int32_t M, int32_t k, double *W)
{
    if (check_layer(d_out, d_in, M, k))
        return -1;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < d_out; ++i)
        reconstruct_row(codes, codebooks, scales, i, d_in, M, k, W + i * d_in);
    return 0;
}

/* y[n][i] = sum_c (s_i * What_k[i][c]) * xrot[n][c], ascending c.
 * xrot: [batch][d_in] doubles (already rotated); y: [batch][d_out].
 * Each row of Wk is reconstructed explicitly into a per-thread buffer. */
int oracle_linear(const uint8_t *codes, const double *codebooks, const double *scales,
                  int64_t d_out, int64_t d_in, int32_t M, int32_t k,
                  const double *xrot, int64_t batch, double *y)
{
    if (check_layer(d_out, d_in, M, k) || batch < 0)
        return -1;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
        if (!w) {
#pragma omp atomic write
            err = -2;
        } else {
            int64_t i;
#pragma omp for schedule(static)
            for (i = 0; i < d_out; ++i) {
                reconstruct_row(codes, codebooks, scales, i, d_in, M, k, w);
                for (int64_t n = 0; n < batch; ++n) {
                    const double *xr = xrot + n * d_in;
                    double acc = 0.0;
                    for (int64_t c = 0; c < d_in; ++c)
                        acc += w[c] * xr[c];
                    y[n * d_out + i] = acc;
                }
            }
            free(w);
        }
    }
    return err;
}

/* The whole decode linear from the raw activation: rotate, then multiply. */
int oracle_forward(const uint8_t *codes, const double *codebooks, const double *scales,
                   int64_t d_out, int64_t d_in, int32_t M, int32_t k,
                   const double *x, int64_t batch, int32_t b, double *y)
{
    if (check_layer(d_out, d_in, M, k) || batch < 0)
        return -1;
    double *xr = (double *)malloc(sizeof(double) * (size_t)(batch * d_in > 0 ? batch * d_in : 1));
    if (!xr)
        return -2;
    int rc = oracle_rotate(x, batch, d_in, b, xr);
    if (rc == 0)
        rc = oracle_linear(codes, codebooks, scales, d_out, d_in, M, k, xr, batch, y);
    free(xr);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Packed code layout.  Plane-major, so the codes of the first k codebooks are
 * a prefix of the buffer (section 5: the first k codebooks are a
 * self-contained lower bitwidth).  Inside a plane the codes sit in 1 KiB
 * tiles of 16 rows x 64 groups, tiles ordered by group tile then row tile,
 * bytes inside a tile ordered by group then row; rows and groups beyond the
 * layer are zero padding.  This tile order is the library's storage format
 * (the pages fix only the prefix property), written out from its definition:
 *   packed[m*P + (jt*R + it)*1024 + l*16 + r] = codes[16*it + r][64*jt + l][m]
 * ------------------------------------------------------------------------- */

#define ORACLE_TILE_ROWS 16
#define ORACLE_TILE_GROUPS 64

static int64_t tiles_r(int64_t d_out) { return (d_out + ORACLE_TILE_ROWS - 1) / ORACLE_TILE_ROWS; }
static int64_t tiles_g(int64_t G) { return (G + ORACLE_TILE_GROUPS - 1) / ORACLE_TILE_GROUPS; }

int64_t oracle_packed_bytes(int64_t d_out, int64_t G, int32_t M)
{
    return (int64_t)M * tiles_r(d_out) * tiles_g(G) * ORACLE_TILE_ROWS * ORACLE_TILE_GROUPS;
}

static int64_t packed_offset(int64_t i, int64_t j, int32_t m, int64_t R, int64_t P)
{
    const int64_t it = i / ORACLE_TILE_ROWS, r = i % ORACLE_TILE_ROWS;
    const int64_t jt = j / ORACLE_TILE_GROUPS, l = j % ORACLE_TILE_GROUPS;
    return (int64_t)m * P + (jt * R + it) * (ORACLE_TILE_ROWS * ORACLE_TILE_GROUPS) + l * ORACLE_TILE_ROWS + r;
}

int oracle_pack_codes(const uint8_t *codes, int64_t d_out, int64_t G, int32_t M, uint8_t *packed)
{
    if (d_out < 0 || G < 0 || M < 1)
        return -1;
    const int64_t R = tiles_r(d_out);
    const int64_t P = R * tiles_g(G) * ORACLE_TILE_ROWS * ORACLE_TILE_GROUPS;
    memset(packed, 0, (size_t)(P * M));
    for (int32_t m = 0; m < M; ++m)
        for (int64_t i = 0; i < d_out; ++i)
            for (int64_t j = 0; j < G; ++j)
                packed[packed_offset(i, j, m, R, P)] = codes[(i * G + j) * M + m];
    return 0;
}

int oracle_unpack_codes(const uint8_t *packed, int64_t d_out, int64_t G, int32_t M, uint8_t *codes)
{
    if (d_out < 0 || G < 0 || M < 1)
        return -1;
    const int64_t R = tiles_r(d_out);
    const int64_t P = R * tiles_g(G) * ORACLE_TILE_ROWS * ORACLE_TILE_GROUPS;
    for (int64_t i = 0; i < d_out; ++i)
        for (int64_t j = 0; j < G; ++j)
            for (int32_t m = 0; m < M; ++m)
                codes[(i * G + j) * M + m] = packed[packed_offset(i, j, m, R, P)];
    return 0;
}

/* ---------------------------------------------------------------------------
 * Storage (appendix "Estimating Model Size"): bits of codebooks, codes and
 * scales of one layer; bits per parameter = total / (d_out * d_in).
 * ------------------------------------------------------------------------- */

double oracle_storage_bits(int64_t d_out, int64_t d_in, int32_t g, int32_t M, int32_t B)
{
    const double codebooks = (double)g * (double)M * ldexp(1.0, B) * 16.0;
    const double codes = (double)d_out * ((double)d_in / (double)g) * (double)B * (double)M;
    const double scales = (double)d_out * 16.0;
    return codebooks + codes + scales;
}

double oracle_bits_per_param(int64_t d_out, int64_t d_in, int32_t g, int32_t M, int32_t B)
{
    return oracle_storage_bits(d_out, d_in, g, M, B) / ((double)d_out * (double)d_in);
}

/* ---------------------------------------------------------------------------
 * Encode side: greedy residual code assignment for fixed codebooks.
 *
 * Section 3.2 defines the decoder (a group is the sum of one codeword from
 * each codebook) and section 5 the prefix order (codebook 1 first).  The
 * pages do not include AQLM's search for the codes (its appendix is not on
 * them), so this is a stated stand-in that respects the prefix order: for
 * every group of 8 target values, codebook m = 0, 1, ..., M-1 in turn picks
 * the codeword nearest (squared Euclidean distance) to the residual that the
 * earlier codebooks left, and the residual loses that codeword.
 *
 * The target is the weight group already rotated and divided by its row
 * scale.  The pages fix no precision for this search; the decision is an
 * index, so it is taken in float32 with one fixed operation order, which the
 * GPU encoder follows too:
 *     e_t = r_t - C[c][t]  (float),  d = fmaf(e_t, e_t, d) for t = 0..7 from d = 0,
 * the smallest d wins and equal d go to the lower index; then r_t = r_t - C[c*][t].
 * codebooks are the fp16 codebooks decoded exactly; codes: [d_out][G][M].
 * ------------------------------------------------------------------------- */
int oracle_encode_greedy(const float *target, const uint16_t *codebooks, int64_t d_out, int64_t d_in, int32_t M,
                         uint8_t *codes)
{
    if (d_out < 0 || d_in < 0 || d_in % ORACLE_GROUP != 0 || M < 1)
        return -1;
    const int64_t G = d_in / ORACLE_GROUP;
    float *cbf = (float *)malloc(sizeof(float) * (size_t)M * ORACLE_CODEWORDS * ORACLE_GROUP);
    if (!cbf)
        return -2;
    for (int64_t e = 0; e < (int64_t)M * ORACLE_CODEWORDS * ORACLE_GROUP; ++e)
        cbf[e] = (float)oracle_f16_to_f64(codebooks[e]);
    int64_t q;
#pragma omp parallel for schedule(static)
    for (q = 0; q < d_out * G; ++q) {
        float r[ORACLE_GROUP];
        for (int t = 0; t < ORACLE_GROUP; ++t)
            r[t] = target[q * ORACLE_GROUP + t];
        for (int32_t m = 0; m < M; ++m) {
            const float *cm = cbf + (int64_t)m * ORACLE_CODEWORDS * ORACLE_GROUP;
            int best = 0;
            float best_d = 0.0f;
            for (int c = 0; c < ORACLE_CODEWORDS; ++c) {
                float d = 0.0f;
                for (int t = 0; t < ORACLE_GROUP; ++t) {
                    const float e = r[t] - cm[c * ORACLE_GROUP + t];
                    d = fmaf(e, e, d);
                }
                if (c == 0 || d < best_d) {
                    best = c;
                    best_d = d;
                }
            }
            codes[q * M + m] = (uint8_t)best;
            for (int t = 0; t < ORACLE_GROUP; ++t)
                r[t] = r[t] - cm[best * ORACLE_GROUP + t];
        }
    }
    free(cbf);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Threading control for the timing leg and the determinism pin.
 * ------------------------------------------------------------------------- */

int oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
