/*
 * kvarn_oracle.c -- plain, slow CPU oracle for the KVarN KV-cache tile codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or constant generator with the
 * HIP kernels.
 *
 * Everything is computed in IEEE binary64 with plain loops, in the order the
 * method is described, and rounding happens only where the stored format
 * demands it (FP8 E4M3 scales, FP16 zero-points, integer codes).
 *
 * Sources (web pages about arXiv 2606.03458, "KVarN: Variance-Normalized
 * KV-Cache Quantization Mitigates Error Accumulation in Reasoning Tasks"):
 *   [review]     dimensionstp.github.io "KVarN ... Review", sections 2-2, 3-2
 *   [paperlayer] paperlayer.ai summary of arXiv 2606.03458v1, sections
 *                2 Preliminaries, 3 Methods, 4 Experiments, D Experimental
 *                details, H Variance Normalization Algorithm, I KVarN
 *                Dequantization Overhead
 *   [agihunt]    agihunt.info paper note (pipeline and storage paragraph)
 *   [pheeree]    pheeree.github.io blog on KVarN, "core three points" part 3
 *                and part 2 (error decomposition, equation 3)
 *
 * Readings taken where the pages are silent (each is also listed in the design
 * notes of the repository):
 *   - tile = 128 tokens x 128 channels, token-major (channels contiguous);
 *   - rotation H = Sylvester-order Walsh-Hadamard matrix scaled by 1/sqrt(128),
 *     applied over the channel (head_dim) axis of every token;
 *   - normalisation: T iterations (T = 8 by default) of
 *       channel step  c_j = std_i( Y_ij / r_i )      (std over the 128 tokens)
 *       token step    r_i = std_j( Y_ij / c_j )      (std over the 128 channels)
 *     starting from r = 1; std is the centred population std (divide by 128);
 *     a degenerate std (at most 2^-16 times the RMS of the matrix normalised
 *     in that step) is replaced by that RMS;
 *   - K: groups are channels (s1, z per channel), s2 = r per token;
 *     V: groups are tokens  (s1, z per token),   s2 = c per channel;
 *   - s2 gets a power-of-two gauge (divide by 2^k, k = frexp exponent of its
 *     mean), then FP8 E4M3 (OCP "FN" variant) round-to-nearest-even, saturating
 *     at 448, floored at 2^-9;
 *   - Zn = Y / s2 broadcast over the group axis; per group mn = min, mx = max;
 *     s1 = max(FP8(( mx - mn ) / L), 2^-9) with L = 2^bits - 1;
 *     z  = FP16 round-to-nearest-even of mn, saturated at +-65504;
 *   - code = clamp( round-half-even( (Zn - z) / s1 ), 0, L );
 *   - dequant: K  Yh_ij = s2_i * (code_ij * s1_j + z_j)
 *              V  Yh_ij = s2_j * (code_ij * s1_i + z_i),   Xh = Yh * H.
 *
 * Packed record of one tile (bits b in {2, 4}), contiguous bytes:
 *   [0, 2048*b)            codes.  Row r is index r of the s2 axis (K: token r,
 *                          V: channel r), position p its group index (K:
 *                          channel p, V: token p).  With n = r/8, i = r%8 the
 *                          code sits at
 *                            b = 2: byte 1024*(i/2) + 16*(16*(p/32) + n)
 *                                        + 8*(i%2) + (p%32)/4,  bit 2*(p%4)
 *                            b = 4: byte 1024*i + 16*(16*((p/16)%4) + n)
 *                                        + 8*(p/64) + (p%16)/2, bit 4*(p%2)
 *                          (the order in which the decode kernel's matrix
 *                          instructions consume them; a reading of the pages,
 *                          which fix only the bit count)
 *   [2048*b, +128)         s1, FP8 E4M3, indexed by group
 *   [2048*b + 128, +128)   s2, FP8 E4M3, indexed by the other axis
 *   [2048*b + 256, +256)   z, FP16 little-endian, indexed by group
 *   total 2048*b + 512 bytes: 4608 for b = 2 (2.25 bits per element), 8704 for
 *   b = 4 ([paperlayer] section D: two FP8 scales and one FP16 zero-point per
 *   128-element group on top of the codes).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define N 128
#define NN (N * N)

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2 };
enum { AX_K = 0, AX_V = 1 };

/* ------------------------------------------------------------------------- */
/* Number formats, written from their public definitions.                      */
/* ------------------------------------------------------------------------- */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double kvo_bf16_decode(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double kvo_f16_decode(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

/* OCP 8-bit floating point, E4M3 ("FN": no infinities, S.1111.111 is NaN):
 * 1 sign, 4 exponent (bias 7), 3 fraction bits, largest finite 448. */
double kvo_fp8_decode(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(m + 8), e - 10);
    return s ? -v : v;
}

/* Round a non-negative double to the nearest integer, ties to even. */
static double rne_int(double q)
{
    double f = floor(q);
    double d = q - f;
    if (d > 0.5)
        return f + 1.0;
    if (d < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* Round |v| onto a binary grid with `mant` fraction bits and smallest normal
 * exponent `emin` (subnormals below it), ties to even.  Returns the rounded
 * magnitude (no saturation). */
static double grid_round(double a, int mant, int emin)
{
    if (a == 0.0)
        return 0.0;
    int E;
    frexp(a, &E);           /* a = m * 2^E, m in [0.5, 1) */
    int e = E - 1;          /* floor(log2 a) */
    if (e < emin)
        e = emin;
    double quantum = ldexp(1.0, e - mant);
    return rne_int(a / quantum) * quantum;
}

/* FP8 E4M3 value nearest to v (ties to even), saturating at +-448. */
double kvo_fp8_round(double v)
{
    if (isnan(v))
        return v;
    double a = grid_round(fabs(v), 3, -6);
    if (a > 448.0)
        a = 448.0;
    return signbit(v) ? -a : a;
}

/* Bit pattern of a value that is exactly representable in FP8 E4M3. */
uint8_t kvo_fp8_bits(double v)
{
    uint8_t s = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7F;
    if (a == 0.0)
        return s;
    int E;
    frexp(a, &E);
    int e = E - 1;
    if (e < -6)
        return s | (uint8_t)(a / ldexp(1.0, -9));
    int mant = (int)(a / ldexp(1.0, e - 3)) - 8;
    return s | (uint8_t)(((e + 7) << 3) | mant);
}

uint8_t kvo_fp8_encode(double v) { return kvo_fp8_bits(kvo_fp8_round(v)); }

/* FP16 value nearest to v (ties to even), saturating at +-65504. */
double kvo_f16_round(double v)
{
    if (isnan(v))
        return v;
    double a = grid_round(fabs(v), 10, -14);
    if (a > 65504.0)
        a = 65504.0;
    return signbit(v) ? -a : a;
}

uint16_t kvo_f16_bits(double v)
{
    uint16_t s = (v < 0 || (v == 0 && signbit(v))) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7E00;
    if (a == 0.0)
        return s;
    int E;
    frexp(a, &E);
    int e = E - 1;
    if (e < -14)
        return s | (uint16_t)(a / ldexp(1.0, -24));
    int mant = (int)(a / ldexp(1.0, e - 10)) - 1024;
    return s | (uint16_t)(((e + 15) << 10) | mant);
}

uint16_t kvo_f16_encode(double v) { return kvo_f16_bits(kvo_f16_round(v)); }

/* ------------------------------------------------------------------------- */
/* Record layout                                                              */
/* ------------------------------------------------------------------------- */

size_t kvo_record_bytes(int bits) { return (bits == 2 || bits == 4) ? (size_t)(2048 * bits + 512) : 0; }

static size_t off_s1(int bits) { return (size_t)2048 * bits; }
static size_t off_s2(int bits) { return (size_t)2048 * bits + 128; }
static size_t off_z(int bits) { return (size_t)2048 * bits + 256; }

/* Bit offset of the code of token t, channel c (layout in the header above). */
static size_t code_bit(int bits, int axis, int t, int c)
{
    int r = axis == AX_K ? t : c, p = axis == AX_K ? c : t;
    int n = r / 8, i = r % 8;
    size_t byte;
    if (bits == 2)
        byte = (size_t)1024 * (i / 2) + 16 * (16 * (p / 32) + n) + 8 * (i % 2) + (p % 32) / 4;
    else
        byte = (size_t)1024 * i + 16 * (16 * ((p / 16) % 4) + n) + 8 * (p / 64) + (p % 16) / 2;
    return 8 * byte + (size_t)(bits == 2 ? 2 * (p % 4) : 4 * (p % 2));
}

static void put_code(uint8_t *rec, int bits, int axis, int t, int c, int code)
{
    size_t bit = code_bit(bits, axis, t, c);
    rec[bit / 8] |= (uint8_t)(code << (bit % 8));
}

static int get_code(const uint8_t *rec, int bits, int axis, int t, int c)
{
    size_t bit = code_bit(bits, axis, t, c);
    return (rec[bit / 8] >> (bit % 8)) & ((1 << bits) - 1);
}

static double rec_s1(const uint8_t *rec, int bits, int g) { return kvo_fp8_decode(rec[off_s1(bits) + g]); }
static double rec_s2(const uint8_t *rec, int bits, int g) { return kvo_fp8_decode(rec[off_s2(bits) + g]); }
static double rec_z(const uint8_t *rec, int bits, int g)
{
    const uint8_t *p = rec + off_z(bits) + 2 * g;
    return kvo_f16_decode((uint16_t)(p[0] | (p[1] << 8)));
}

/* ------------------------------------------------------------------------- */
/* Rotation: normalised Walsh-Hadamard matrix over head_dim                    */
/* [review] section 2-2 and 3-2(2); [paperlayer] section 2 Preliminaries and   */
/* appendix A (head-wise block-diagonal transform of block size = head size).  */
/* ------------------------------------------------------------------------- */

static int popcount7(int v)
{
    int n = 0;
    while (v) {
        n += v & 1;
        v >>= 1;
    }
    return n;
}

/* H_ij = (-1)^popcount(i & j) / sqrt(128), Sylvester (natural) order. */
void kvo_hadamard(double *h)
{
    double s = 1.0 / sqrt((double)N);
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j)
            h[i * N + j] = (popcount7(i & j) & 1) ? -s : s;
}

/* out[t][k] = sum_j in[t][j] * H[j][k]: the plain matrix product. */
static void rotate_rows(const double *in, double *out, const double *h)
{
    for (int t = 0; t < N; ++t)
        for (int k = 0; k < N; ++k) {
            double acc = 0.0;
            for (int j = 0; j < N; ++j)
                acc += in[t * N + j] * h[j * N + k];
            out[t * N + k] = acc;
        }
}

/* ------------------------------------------------------------------------- */
/* Dual-axis standard-deviation normalisation (Sinkhorn-Knopp style)           */
/* [review] 3-2(3); [paperlayer] 3 Methods, 4 Experiments (eight iterations),  */
/* H Variance Normalization Algorithm; [agihunt] pipeline paragraph.          */
/* ------------------------------------------------------------------------- */

/* Centred population standard deviation of n values, two-pass. */
static double pstd(const double *v, int n)
{
    double m = 0.0;
    for (int i = 0; i < n; ++i)
        m += v[i];
    m /= n;
    double s = 0.0;
    for (int i = 0; i < n; ++i)
        s += (v[i] - m) * (v[i] - m);
    return sqrt(s / n);
}

/* A std is degenerate when it is at most 2^-16 times the root-mean-square of
 * the whole matrix being normalised in that step (or below 2^-60); it is then
 * replaced by that RMS (by 1 when the RMS itself is below 2^-60).  Exactly
 * cancelling rotations leave rounding noise where exact arithmetic has zeros;
 * the relative floor keeps such noise from being normalised up. */
#define DEGENERATE_REL 1.52587890625e-05 /* 2^-16 */
#define DEGENERATE_ABS 8.673617379884035e-19 /* 2^-60 */

static double guarded(double sd, double rms)
{
    if (sd > DEGENERATE_REL * rms && sd >= DEGENERATE_ABS)
        return sd;
    return rms >= DEGENERATE_ABS ? rms : 1.0;
}

/* r (per token, length 128) and c (per channel) after n_iter iterations. */
void kvo_sinkhorn(const double *y, int n_iter, double *r, double *c)
{
    double col[N], row[N];
    for (int i = 0; i < N; ++i)
        r[i] = 1.0, c[i] = 1.0;
    for (int it = 0; it < n_iter; ++it) {
        double ss = 0.0;                        /* channel step on Y_ij / r_i */
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j)
                ss += (y[i * N + j] / r[i]) * (y[i * N + j] / r[i]);
        double rms = sqrt(ss / NN);
        for (int j = 0; j < N; ++j) {
            for (int i = 0; i < N; ++i)
                col[i] = y[i * N + j] / r[i];
            c[j] = guarded(pstd(col, N), rms);
        }
        ss = 0.0;                               /* token step on Y_ij / c_j */
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j)
                ss += (y[i * N + j] / c[j]) * (y[i * N + j] / c[j]);
        rms = sqrt(ss / NN);
        for (int i = 0; i < N; ++i) {
            for (int j = 0; j < N; ++j)
                row[j] = y[i * N + j] / c[j];
            r[i] = guarded(pstd(row, N), rms);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Input access                                                               */
/* ------------------------------------------------------------------------- */

static double load_elem(const void *x, int dtype, int64_t idx)
{
    switch (dtype) {
    case DT_F16:
        return kvo_f16_decode(((const uint16_t *)x)[idx]);
    case DT_BF16:
        return kvo_bf16_decode(((const uint16_t *)x)[idx]);
    default:
        return (double)((const float *)x)[idx];
    }
}

static void load_tile(const void *x, int dtype, int64_t base, int64_t token_stride, double *out)
{
    for (int t = 0; t < N; ++t)
        for (int c = 0; c < N; ++c)
            out[t * N + c] = load_elem(x, dtype, base + (int64_t)t * token_stride + c);
}

static int64_t tile_base(int64_t i, int64_t tile_stride, const int64_t *tile_off)
{
    return tile_off ? tile_off[i] : i * tile_stride;
}

/* Rotated tile Y = X H (or Y = X when rotate == 0). */
static void rotated_tile(const void *x, int dtype, int64_t base, int64_t token_stride, int rotate,
                         const double *h, double *y)
{
    double *xt = (double *)malloc(sizeof(double) * NN);
    load_tile(x, dtype, base, token_stride, xt);
    if (rotate)
        rotate_rows(xt, y, h);
    else
        memcpy(y, xt, sizeof(double) * NN);
    free(xt);
}

/* Element (i, j) of the tile is in group grp(i, j) and carries s2 index sidx(i, j). */
static int grp(int axis, int i, int j) { return axis == AX_K ? j : i; }
static int sidx(int axis, int i, int j) { return axis == AX_K ? i : j; }

/* ------------------------------------------------------------------------- */
/* Quantisation of one tile                                                   */
/* ------------------------------------------------------------------------- */

/* Power-of-two gauge and FP8 second scale from the non-group-axis factors g. */
static void second_scale(const double *g_in, double *g_pre, double *s2)
{
    double mean = 0.0;
    for (int i = 0; i < N; ++i)
        mean += g_in[i];
    mean /= N;
    int k;
    frexp(mean, &k);
    for (int i = 0; i < N; ++i) {
        g_pre[i] = ldexp(g_in[i], -k);
        double v = kvo_fp8_round(g_pre[i]);
        s2[i] = (v < ldexp(1.0, -9)) ? ldexp(1.0, -9) : v;
    }
}

/* Group min/max of Zn = Y / s2 and the FP8 / FP16 group metadata. */
static void group_meta(const double *y, int axis, int bits, const double *s2, double *s1_pre, double *z_pre,
                       double *s1, double *z)
{
    const double L = (double)((1 << bits) - 1);
    for (int g = 0; g < N; ++g) {
        double mn = INFINITY, mx = -INFINITY;
        for (int k = 0; k < N; ++k) {
            int i = axis == AX_K ? k : g, j = axis == AX_K ? g : k;
            double zn = y[i * N + j] / s2[sidx(axis, i, j)];
            if (zn < mn)
                mn = zn;
            if (zn > mx)
                mx = zn;
        }
        s1_pre[g] = (mx - mn) / L;
        z_pre[g] = mn;
        double q = kvo_fp8_round(s1_pre[g]);
        s1[g] = (q < ldexp(1.0, -9)) ? ldexp(1.0, -9) : q;
        z[g] = kvo_f16_round(mn);
    }
}

static int rtn_code(double zn, double z, double s1, int bits, double *t_out)
{
    const int L = (1 << bits) - 1;
    double t = (zn - z) / s1;
    if (t_out)
        *t_out = t;
    double q = (t < 0) ? -rne_int(-t) : rne_int(t);
    if (q < 0)
        q = 0;
    if (q > L)
        q = L;
    return (int)q;
}

static void write_meta(uint8_t *rec, int bits, const double *s1, const double *s2, const double *z)
{
    for (int g = 0; g < N; ++g) {
        rec[off_s1(bits) + g] = kvo_fp8_bits(s1[g]);
        rec[off_s2(bits) + g] = kvo_fp8_bits(s2[g]);
        uint16_t zb = kvo_f16_bits(z[g]);
        rec[off_z(bits) + 2 * g] = (uint8_t)(zb & 0xFF);
        rec[off_z(bits) + 2 * g + 1] = (uint8_t)(zb >> 8);
    }
}

static void quantize_one(const double *y, int bits, int axis, int n_iter, uint8_t *rec, double *g_pre_out,
                         double *s1_pre_out, double *z_pre_out)
{
    double r[N], c[N], g_pre[N], s2[N], s1_pre[N], z_pre[N], s1[N], z[N];
    kvo_sinkhorn(y, n_iter, r, c);
    second_scale(axis == AX_K ? r : c, g_pre, s2);
    group_meta(y, axis, bits, s2, s1_pre, z_pre, s1, z);
    memset(rec, 0, kvo_record_bytes(bits));
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            int gi = grp(axis, i, j);
            double zn = y[i * N + j] / s2[sidx(axis, i, j)];
            put_code(rec, bits, axis, i, j, rtn_code(zn, z[gi], s1[gi], bits, NULL));
        }
    write_meta(rec, bits, s1, s2, z);
    if (g_pre_out)
        memcpy(g_pre_out, g_pre, sizeof g_pre);
    if (s1_pre_out)
        memcpy(s1_pre_out, s1_pre, sizeof s1_pre);
    if (z_pre_out)
        memcpy(z_pre_out, z_pre, sizeof z_pre);
}

static int bad_common(int bits, int axis, int dtype)
{
    return !(bits == 2 || bits == 4) || !(axis == AX_K || axis == AX_V) || dtype < 0 || dtype > 2;
}

/*
 * Quantise n_tiles tiles.  Tile i starts at element tile_off[i] (or
 * i * tile_stride when tile_off is NULL); token t, channel c of it is element
 * base + t * token_stride + c of x.  records receives n_tiles * record_bytes.
 * Optional per-tile outputs (NULL to skip): g_pre[n][128] gauge-fixed second
 * scale before FP8 rounding, s1_pre / z_pre[n][128] group values before
 * rounding, y_out[n][128*128] the rotated tile.  Returns 0 or -1.
 */
int kvo_quantize_tiles(const void *x, int dtype, int64_t n_tiles, int64_t tile_stride, int64_t token_stride,
                       const int64_t *tile_off, int bits, int axis, int n_iter, int rotate, uint8_t *records,
                       double *g_pre, double *s1_pre, double *z_pre, double *y_out)
{
    if (bad_common(bits, axis, dtype) || n_tiles < 0 || n_iter < 0)
        return -1;
    double h[NN];
    kvo_hadamard(h);
    size_t pb = kvo_record_bytes(bits);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_tiles; ++i) {
        double *y = (double *)malloc(sizeof(double) * NN);
        rotated_tile(x, dtype, tile_base(i, tile_stride, tile_off), token_stride, rotate, h, y);
        quantize_one(y, bits, axis, n_iter, records + i * pb, g_pre ? g_pre + i * N : NULL,
                     s1_pre ? s1_pre + i * N : NULL, z_pre ? z_pre + i * N : NULL);
        if (y_out)
            memcpy(y_out + i * NN, y, sizeof(double) * NN);
        free(y);
    }
    return 0;
}

/*
 * Group values before rounding when the FP8 second scale is the one given in
 * s2_bytes[n][128] (for example the one another implementation chose).
 */
int kvo_group_meta_given_s2(const void *x, int dtype, int64_t n_tiles, int64_t tile_stride, int64_t token_stride,
                            const int64_t *tile_off, int bits, int axis, int rotate, const uint8_t *s2_bytes,
                            double *s1_pre, double *z_pre)
{
    if (bad_common(bits, axis, dtype) || n_tiles < 0)
        return -1;
    double h[NN];
    kvo_hadamard(h);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_tiles; ++i) {
        double *y = (double *)malloc(sizeof(double) * NN);
        double s2[N], s1[N], z[N];
        rotated_tile(x, dtype, tile_base(i, tile_stride, tile_off), token_stride, rotate, h, y);
        for (int g = 0; g < N; ++g)
            s2[g] = kvo_fp8_decode(s2_bytes[i * N + g]);
        group_meta(y, axis, bits, s2, s1_pre + i * N, z_pre + i * N, s1, z);
        free(y);
    }
    return 0;
}

/*
 * Codes (one byte each, [n][128 tokens][128 channels]) and the unrounded
 * t = (Zn - z) / s1 the oracle obtains when s1, s2 and z are taken from the
 * metadata part of the given records.
 */
int kvo_codes_given_meta(const void *x, int dtype, int64_t n_tiles, int64_t tile_stride, int64_t token_stride,
                         const int64_t *tile_off, int bits, int axis, int rotate, const uint8_t *records,
                         uint8_t *codes, double *t_out)
{
    if (bad_common(bits, axis, dtype) || n_tiles < 0)
        return -1;
    double h[NN];
    kvo_hadamard(h);
    size_t pb = kvo_record_bytes(bits);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < n_tiles; ++n) {
        const uint8_t *rec = records + n * pb;
        double *y = (double *)malloc(sizeof(double) * NN);
        rotated_tile(x, dtype, tile_base(n, tile_stride, tile_off), token_stride, rotate, h, y);
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j) {
                int gi = grp(axis, i, j);
                double zn = y[i * N + j] / rec_s2(rec, bits, sidx(axis, i, j));
                double t;
                int code = rtn_code(zn, rec_z(rec, bits, gi), rec_s1(rec, bits, gi), bits, &t);
                codes[n * NN + i * N + j] = (uint8_t)code;
                if (t_out)
                    t_out[n * NN + i * N + j] = t;
            }
        free(y);
    }
    return 0;
}

/* Codes of packed records, unpacked to one byte per element [n][128 tokens][128 channels]. */
int kvo_unpack_codes(const uint8_t *records, int64_t n_tiles, int bits, int axis, uint8_t *codes)
{
    if (!(bits == 2 || bits == 4) || !(axis == AX_K || axis == AX_V) || n_tiles < 0)
        return -1;
    size_t pb = kvo_record_bytes(bits);
    for (int64_t n = 0; n < n_tiles; ++n)
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j)
                codes[n * NN + i * N + j] = (uint8_t)get_code(records + n * pb, bits, axis, i, j);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Dequantisation ([paperlayer] 3 Methods: one extra multiply per element;    */
/* I KVarN Dequantization Overhead: per-row second scale s2)                  */
/* ------------------------------------------------------------------------- */

static void dequant_one(const uint8_t *rec, int bits, int axis, int rotate, const double *h, double *out)
{
    double *yh = (double *)malloc(sizeof(double) * NN);
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            int gi = grp(axis, i, j);
            yh[i * N + j] = rec_s2(rec, bits, sidx(axis, i, j)) *
                            (get_code(rec, bits, axis, i, j) * rec_s1(rec, bits, gi) + rec_z(rec, bits, gi));
        }
    if (rotate)
        rotate_rows(yh, out, h); /* H is symmetric and orthogonal: its own inverse */
    else
        memcpy(out, yh, sizeof(double) * NN);
    free(yh);
}

int kvo_dequantize_tiles(const uint8_t *records, int64_t n_tiles, int bits, int axis, int rotate, double *out)
{
    if (!(bits == 2 || bits == 4) || !(axis == AX_K || axis == AX_V) || n_tiles < 0)
        return -1;
    double h[NN];
    kvo_hadamard(h);
    size_t pb = kvo_record_bytes(bits);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_tiles; ++i)
        dequant_one(records + i * pb, bits, axis, rotate, h, out + i * NN);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Single-query decode attention over the packed cache                       */
/* ------------------------------------------------------------------------- */

/*
 * q[b][hq][128] FP16; out[b][hq][128] float64.  For sequence b and KV head
 * h = hq / (n_q_heads / n_kv_heads) (at most 64 query heads per KV head), the
 * keys and values attended over are, in this order (the order does not change
 * the result):
 *   the n_sink FP16 sink tokens  k_sink[b][h][0 .. n_sink),
 *   the packed body: tile j < min(n_tiles[b], max_tiles) is record
 *     idx = block_table ? block_table[row] : row,  row = (b * n_kv_heads + h) * max_tiles + j
 *     of k_rec (K layout, bits_k) and v_rec (V layout, bits_v), dequantised
 *     exactly (binary64), with or without the inverse rotation as written,
 *   the FP16 recent tokens  k_recent[b][h][0 .. min(n_recent[b], recent_cap)).
 * The windows are the FP16 sink and trailing regions around the quantised body
 * (paperlayer.ai summary, appendix D: S = 128, R = 128); NULL window pointers
 * mean no window.  Then  s_t = sm_scale * q . k_t,  p = softmax(s),
 * out = sum_t p_t v_t.  A sequence with no tokens gets a zero output.
 */
int kvo_decode_attn(const uint16_t *q, const uint8_t *k_rec, const uint8_t *v_rec, const int32_t *block_table,
                    const int32_t *n_tiles, int64_t batch, int n_q_heads, int n_kv_heads, int max_tiles, int bits_k,
                    int bits_v, int rotate, double sm_scale, const uint16_t *k_sink, const uint16_t *v_sink,
                    int n_sink, const uint16_t *k_recent, const uint16_t *v_recent, const int32_t *n_recent,
                    int recent_cap, double *out)
{
    if (batch < 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0 ||
        n_q_heads / n_kv_heads > 64 || max_tiles < 0 || kvo_record_bytes(bits_k) == 0 ||
        kvo_record_bytes(bits_v) == 0 || n_sink < 0 || recent_cap < 0)
        return -1;
    if (k_sink == NULL || v_sink == NULL)
        n_sink = 0;
    if (k_recent == NULL || v_recent == NULL || n_recent == NULL)
        recent_cap = 0;
    double h[NN];
    kvo_hadamard(h);
    const int gs = n_q_heads / n_kv_heads; /* query heads sharing one KV head */
    const size_t pk = kvo_record_bytes(bits_k), pv = kvo_record_bytes(bits_v);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < batch; ++b)
        for (int kvh = 0; kvh < n_kv_heads; ++kvh) {
            int nt = n_tiles[b] < max_tiles ? n_tiles[b] : max_tiles;
            if (nt < 0)
                nt = 0;
            int nr = recent_cap > 0 ? n_recent[b] : 0;
            nr = nr < 0 ? 0 : (nr > recent_cap ? recent_cap : nr);
            const int64_t ntok = (int64_t)n_sink + (int64_t)nt * N + nr;
            double *o = out + (b * n_q_heads + (int64_t)kvh * gs) * N;
            for (int u = 0; u < gs * N; ++u)
                o[u] = 0.0;
            if (ntok == 0)
                continue;
            double *kall = (double *)malloc(sizeof(double) * (size_t)ntok * N);
            double *vall = (double *)malloc(sizeof(double) * (size_t)ntok * N);
            double *s = (double *)malloc(sizeof(double) * (size_t)ntok);
            int64_t u = 0;
            for (int t = 0; t < n_sink; ++t, ++u)
                for (int d = 0; d < N; ++d) {
                    const int64_t e = (((int64_t)b * n_kv_heads + kvh) * n_sink + t) * N + d;
                    kall[u * N + d] = kvo_f16_decode(k_sink[e]);
                    vall[u * N + d] = kvo_f16_decode(v_sink[e]);
                }
            for (int j = 0; j < nt; ++j, u += N) {
                int64_t row = (b * n_kv_heads + kvh) * (int64_t)max_tiles + j;
                int64_t idx = block_table ? block_table[row] : row;
                dequant_one(k_rec + idx * pk, bits_k, AX_K, rotate, h, kall + u * N);
                dequant_one(v_rec + idx * pv, bits_v, AX_V, rotate, h, vall + u * N);
            }
            for (int t = 0; t < nr; ++t, ++u)
                for (int d = 0; d < N; ++d) {
                    const int64_t e = (((int64_t)b * n_kv_heads + kvh) * recent_cap + t) * N + d;
                    kall[u * N + d] = kvo_f16_decode(k_recent[e]);
                    vall[u * N + d] = kvo_f16_decode(v_recent[e]);
                }
            for (int g = 0; g < gs; ++g) {
                double qd[N];
                for (int d = 0; d < N; ++d)
                    qd[d] = kvo_f16_decode(q[(b * n_q_heads + (int64_t)kvh * gs + g) * N + d]);
                /* scores, then softmax with the maximum subtracted */
                double m = -INFINITY;
                for (int64_t t = 0; t < ntok; ++t) {
                    double acc = 0.0;
                    for (int d = 0; d < N; ++d)
                        acc += qd[d] * kall[t * N + d];
                    s[t] = sm_scale * acc;
                    if (s[t] > m)
                        m = s[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < ntok; ++t) {
                    s[t] = exp(s[t] - m);
                    l += s[t];
                }
                for (int64_t t = 0; t < ntok; ++t)
                    for (int d = 0; d < N; ++d)
                        o[g * N + d] += s[t] * vall[t * N + d];
                for (int d = 0; d < N; ++d)
                    o[g * N + d] /= l;
            }
            free(kall);
            free(vall);
            free(s);
        }
    return 0;
}

/* Threads OpenMP will use for the parallel loops above. */
#ifdef _OPENMP
#include <omp.h>
int kvo_num_threads(void) { return omp_get_max_threads(); }
#else
int kvo_num_threads(void) { return 1; }
#endif
