/*
 * Plain CPU oracle for the randomized-Hadamard + Lloyd-Max codecs.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark may load this file. The product library never links,
 * includes or calls it, and shares no code, header or table with it.
 *
 * Sources (cited by page title and the construct on the page):
 *   [TQ3]   "ComfyUI-TurboQuant: tq3_core.py" (TurboQuant 3-bit KV codec).
 *   [ORBIT] "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py"
 *           (OrbitQuant weight-only backend).
 *
 * Arithmetic is IEEE binary32 with round-to-nearest-even, as on both pages
 * (the TQ3 page upcasts with .float(); the OrbitQuant page works on an fp32
 * weight). Build with -O2 -ffp-contract=off and no fast-math so that every
 * product and sum is rounded exactly once, in the order written here.
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *   - L2 norm order: the pages call torch.norm, whose summation order is not
 *     specified. Here the sum of squares is the pairwise tree that first adds
 *     neighbours (j, j^1), then (j, j^2), ..., i.e. recursive doubling over
 *     the index bits from bit 0 upward. For the OrbitQuant row norm the tree
 *     runs inside each Hadamard block and the block sums are then added left
 *     to right.
 *   - Scalar constants (1/sqrt(128), 1e-8, 1e-10, codebook values, d^-0.5) are
 *     Python doubles that torch rounds to float32 before the fp32 operation,
 *     so each is written here as a double literal cast to float.
 *   - Post-transform scaling: the FWHT stages run first, the 1/sqrt(n)
 *     multiply comes after the last stage, exactly as both pages write it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TQ3_N 128
#define TQ3_PACKED 48
#define TQ3_RECORD 56

/* [TQ3] TQ3_CENTROIDS / TQ3_BOUNDARIES tables: the 8-level codebook and its 7
 * decision boundaries, entered as printed (doubles rounded to fp32). */
static float tq3_centroid(int k) {
    static const double c[8] = {-0.9816, -0.6168, -0.3479, -0.1129,
                                0.1129, 0.3479, 0.6168, 0.9816};
    return (float)c[k];
}
static float tq3_boundary(int k) {
    static const double b[7] = {-0.7992, -0.4824, -0.2304, 0.0,
                                0.2304, 0.4824, 0.7992};
    return (float)b[k];
}

/* Sum of squares by the canonical pairwise tree over a power-of-two run
 * (n <= 65536). */
static float sumsq_pairwise(const float* v, int n) {
    float small[128] = {0.0f};
    float* s = n <= 128 ? small : (float*)malloc((size_t)n * sizeof(float));
    for (int j = 0; j < n; ++j) s[j] = v[j] * v[j];
    for (int w = 1; w < n; w *= 2)
        for (int j = 0; j < n; j += 2 * w) s[j] = s[j] + s[j + w];
    const float r = s[0];
    if (s != small) free(s);
    return r;
}

/* [TQ3] _fwht_inplace and [ORBIT] _fwht: butterfly stages with half-width
 * h = 1, 2, 4, ..., n/2; each stage replaces the pair (v[j], v[j+h]) -- j
 * with bit log2(h) clear -- by (sum, difference). No normalisation here. */
static void fwht_stages(float* v, int n) {
    for (int h = 1; h < n; h *= 2)
        for (int base = 0; base < n; base += 2 * h)
            for (int j = base; j < base + h; ++j) {
                float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

static void fwht_scaled(float* v, int64_t rows, int n, float k) {
    for (int64_t r = 0; r < rows; ++r) {
        float* p = v + r * n;
        fwht_stages(p, n);
        for (int j = 0; j < n; ++j) p[j] = p[j] * k;
    }
}

/* [TQ3] _fwht_inplace including its final multiply by 1.0/sqrt(n) (a double
 * rounded to fp32), applied to `rows` consecutive runs of n floats
 * (n a power of two, 2..4096). */
void orc_fwht(float* v, int64_t rows, int n) {
    fwht_scaled(v, rows, n, (float)(1.0 / sqrt((double)n)));
}

/* [ORBIT] _fwht: the same stages, then a multiply by h ** -0.5 (Python's
 * power of a double, rounded to fp32). */
void orc_fwht_orbit(float* v, int64_t rows, int n) {
    fwht_scaled(v, rows, n, (float)pow((double)n, -0.5));
}

/* [TQ3] _quantize_to_indices: searchsorted on the ascending boundaries with
 * the default left side, i.e. the number of boundaries strictly below x. */
static int tq3_bucket(float x) {
    int idx = 0;
    for (int k = 0; k < 7; ++k)
        if (tq3_boundary(k) < x) idx++;
    return idx;
}

/* Bucket indices of given normalised values (for the tie-rule pins). */
void orc_tq3_bucketize(const float* xs, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)tq3_bucket(xs[i]);
}

/* The two tables as the oracle holds them (8 centroids, 7 boundaries). */
void orc_tq3_tables(float* centroids, float* boundaries) {
    for (int k = 0; k < 8; ++k) centroids[k] = tq3_centroid(k);
    for (int k = 0; k < 7; ++k) boundaries[k] = tq3_boundary(k);
}

/* LSB-first bitstream: value j occupies bits bits*j .. bits*j+bits-1, bit t
 * of the value at stream bit bits*j+t, stream bit q at bit q%8 of byte q/8.
 * For 3-bit values this is the layout of [TQ3] _pack_3bit (groups of eight
 * indices form a little-endian 24-bit word). */
void orc_pack_lsb(const uint8_t* codes, int64_t count, int bits, uint8_t* out) {
    int64_t nbytes = (count * bits + 7) / 8;
    memset(out, 0, (size_t)nbytes);
    for (int64_t j = 0; j < count; ++j)
        for (int t = 0; t < bits; ++t)
            if ((codes[j] >> t) & 1) {
                int64_t q = j * bits + t;
                out[q / 8] |= (uint8_t)(1u << (q % 8));
            }
}

void orc_unpack_lsb(const uint8_t* packed, int64_t count, int bits, uint8_t* codes) {
    for (int64_t j = 0; j < count; ++j) {
        int v = 0;
        for (int t = 0; t < bits; ++t) {
            int64_t q = j * bits + t;
            v |= ((packed[q / 8] >> (q % 8)) & 1) << t;
        }
        codes[j] = (uint8_t)v;
    }
}

/* [ORBIT] pack_codes / unpack_codes: the flat bitstream written most
 * significant bit first. Value j's bit (bits-1-t) sits at stream bit bits*j+t,
 * and stream bit q is bit 7-(q%8) of byte q/8; the tail is zero-padded. */
void orc_pack_msb(const uint8_t* codes, int64_t count, int bits, uint8_t* out) {
    int64_t nbytes = (count * bits + 7) / 8;
    memset(out, 0, (size_t)nbytes);
    for (int64_t j = 0; j < count; ++j)
        for (int t = 0; t < bits; ++t)
            if ((codes[j] >> (bits - 1 - t)) & 1) {
                int64_t q = j * bits + t;
                out[q / 8] |= (uint8_t)(0x80u >> (q % 8));
            }
}

void orc_unpack_msb(const uint8_t* packed, int64_t count, int bits, uint8_t* codes) {
    for (int64_t j = 0; j < count; ++j) {
        int v = 0;
        for (int t = 0; t < bits; ++t) {
            int64_t q = j * bits + t;
            v = (v << 1) | ((packed[q / 8] >> (7 - (q % 8))) & 1);
        }
        codes[j] = (uint8_t)v;
    }
}

/* ---------------------------------------------------------------- TQ3 --- */

/* One 128-vector through [TQ3] tq3_quantize, steps 1-6 of its docstring.
 * post_flip != 0 applies the sign flips after the transform instead of before
 * it: the broken ordering the page's change note measures on constant blocks.
 * It exists only so a test can reproduce that measurement. */
static void tq3_quantize_one(const float* x, const float* signs, int post_flip,
                             uint8_t* rec) {
    float u[TQ3_N];
    uint8_t idx[TQ3_N];
    /* Step 1: L2 normalise; the norm is clamped below at 1e-8. */
    float n = sqrtf(sumsq_pairwise(x, TQ3_N));
    const float nmin = (float)1e-8;
    if (n < nmin) n = nmin;
    for (int j = 0; j < TQ3_N; ++j) u[j] = x[j] / n;
    /* Steps 2-3: sign flips, then the normalised 128-point FWHT. */
    if (!post_flip)
        for (int j = 0; j < TQ3_N; ++j) u[j] = u[j] * signs[j];
    orc_fwht(u, 1, TQ3_N);
    if (post_flip)
        for (int j = 0; j < TQ3_N; ++j) u[j] = u[j] * signs[j];
    /* Step 4: absmax scale, clamped below at 1e-8. */
    float scale = 0.0f;
    for (int j = 0; j < TQ3_N; ++j) {
        float a = fabsf(u[j]);
        if (a > scale) scale = a;
    }
    if (scale < nmin) scale = nmin;
    /* Step 5: 8-level codebook index per coefficient. */
    for (int j = 0; j < TQ3_N; ++j) idx[j] = (uint8_t)tq3_bucket(u[j] / scale);
    /* Step 6: 48 bytes of indices, then the fp32 norm and scale
     * (3.5 bits per value: 48 + 4 + 4 = 56 bytes). */
    orc_pack_lsb(idx, TQ3_N, 3, rec);
    memcpy(rec + TQ3_PACKED, &n, 4);
    memcpy(rec + TQ3_PACKED + 4, &scale, 4);
}

/* [TQ3] tq3_dequantize for one record: centroid lookup, times scale, the
 * normalised FWHT (its own inverse), the sign flips, times the norm. */
static void tq3_dequantize_one(const uint8_t* rec, const float* signs,
                               int post_flip, float* y) {
    uint8_t idx[TQ3_N];
    float n, scale;
    orc_unpack_lsb(rec, TQ3_N, 3, idx);
    memcpy(&n, rec + TQ3_PACKED, 4);
    memcpy(&scale, rec + TQ3_PACKED + 4, 4);
    for (int j = 0; j < TQ3_N; ++j) y[j] = tq3_centroid(idx[j]) * scale;
    if (post_flip)
        for (int j = 0; j < TQ3_N; ++j) y[j] = y[j] * signs[j];
    orc_fwht(y, 1, TQ3_N);
    if (!post_flip)
        for (int j = 0; j < TQ3_N; ++j) y[j] = y[j] * signs[j];
    for (int j = 0; j < TQ3_N; ++j) y[j] = y[j] * n;
}

static void set_threads(int threads) {
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
}

/* x: n_vec rows of 128 fp32 (row-major, contiguous). signs: 128 values of
 * +1/-1. rec: n_vec * 56 bytes. */
void orc_tq3_quantize(const float* x, int64_t n_vec, const float* signs,
                      int post_flip, uint8_t* rec, int threads) {
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n_vec; ++v)
        tq3_quantize_one(x + v * TQ3_N, signs, post_flip, rec + v * TQ3_RECORD);
}

void orc_tq3_dequantize(const uint8_t* rec, int64_t n_vec, const float* signs,
                        int post_flip, float* y, int threads) {
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n_vec; ++v)
        tq3_dequantize_one(rec + v * TQ3_RECORD, signs, post_flip, y + v * TQ3_N);
}

/* Normalised values before bucketing, for boundary-distance accounting:
 * xs[v*128 + j] is coefficient j of vector v divided by its scale. */
void orc_tq3_scaled_coeffs(const float* x, int64_t n_vec, const float* signs,
                           float* xs, int threads) {
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n_vec; ++v) {
        const float* xv = x + v * TQ3_N;
        float u[TQ3_N];
        float n = sqrtf(sumsq_pairwise(xv, TQ3_N));
        const float nmin = (float)1e-8;
        if (n < nmin) n = nmin;
        for (int j = 0; j < TQ3_N; ++j) u[j] = (xv[j] / n) * signs[j];
        orc_fwht(u, 1, TQ3_N);
        float scale = 0.0f;
        for (int j = 0; j < TQ3_N; ++j) {
            float a = fabsf(u[j]);
            if (a > scale) scale = a;
        }
        if (scale < nmin) scale = nmin;
        for (int j = 0; j < TQ3_N; ++j) xs[v * TQ3_N + j] = u[j] / scale;
    }
}

/* ------------------------------------------------------------ OrbitQuant --- */

/* [ORBIT] hadamard_block_size: the largest power of two dividing d. */
int64_t orc_block_size(int64_t d) { return d & (-d); }

/* [ORBIT] rpbh_forward on one row: gather by the permutation, multiply by the
 * Rademacher signs, then the normalised FWHT on every h-block. */
static void rpbh_forward_row(const float* w, int64_t d, int64_t h,
                             const int64_t* perm, const int8_t* signs, float* y) {
    for (int64_t j = 0; j < d; ++j) y[j] = w[perm[j]] * (float)signs[j];
    orc_fwht_orbit(y, d / h, (int)h);
}

/* [ORBIT] rpbh_inverse on one row: normalised FWHT per block, times the
 * signs, then gather with the inverse permutation. */
static void rpbh_inverse_row(const float* y, int64_t d, int64_t h,
                             const int64_t* inv_perm, const int8_t* signs,
                             float* z, float* out) {
    memcpy(z, y, (size_t)d * sizeof(float));
    orc_fwht_orbit(z, d / h, (int)h);
    for (int64_t j = 0; j < d; ++j) z[j] = z[j] * (float)signs[j];
    for (int64_t j = 0; j < d; ++j) out[j] = z[inv_perm[j]];
}

void orc_rpbh_forward(const float* w, int64_t rows, int64_t d,
                      const int64_t* perm, const int8_t* signs, float* y,
                      int threads) {
    const int64_t h = orc_block_size(d);
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        rpbh_forward_row(w + r * d, d, h, perm, signs, y + r * d);
}

void orc_rpbh_inverse(const float* y, int64_t rows, int64_t d,
                      const int64_t* inv_perm, const int8_t* signs, float* out,
                      int threads) {
    const int64_t h = orc_block_size(d);
    set_threads(threads);
#pragma omp parallel
    {
        float* z = (float*)malloc((size_t)d * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            rpbh_inverse_row(y + r * d, d, h, inv_perm, signs, z, out + r * d);
        free(z);
    }
}

/* Row L2 norm of a rotated row: pairwise tree inside each h-block, then the
 * block sums left to right, then the square root. */
static float row_norm(const float* y, int64_t d, int64_t h) {
    float total = 0.0f;
    for (int64_t b = 0; b < d / h; ++b) {
        float s = sumsq_pairwise(y + b * h, (int)h);
        total = (b == 0) ? s : total + s;
    }
    return sqrtf(total);
}

/* [ORBIT] _quantize_rows: rotate, take row norms, divide by (norm + 1e-10),
 * bucket against the codebook midpoints (count of edges strictly below),
 * pack. codebook: 2^bits ascending fp32 values (already scaled by d^-0.5).
 * msb_first selects the page's pack_codes layout (1) or the LSB-first
 * stream (0). packed receives rows*d*bits/8 bytes; norms receives rows. */
void orc_orbit_quantize(const float* w, int64_t rows, int64_t d, int bits,
                        const int64_t* perm, const int8_t* signs,
                        const float* codebook, int msb_first, uint8_t* packed,
                        float* norms, int threads) {
    const int64_t h = orc_block_size(d);
    const int levels = 1 << bits;
    float edges[15];
    for (int k = 0; k + 1 < levels; ++k)
        edges[k] = (codebook[k] + codebook[k + 1]) / 2.0f;
    const float eps = (float)1e-10;
    const int64_t row_bytes = d * bits / 8;
    set_threads(threads);
#pragma omp parallel
    {
        float* y = (float*)malloc((size_t)d * sizeof(float));
        uint8_t* codes = (uint8_t*)malloc((size_t)d);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            rpbh_forward_row(w + r * d, d, h, perm, signs, y);
            float n = row_norm(y, d, h);
            float denom = n + eps;
            for (int64_t j = 0; j < d; ++j) {
                float u = y[j] / denom;
                int c = 0;
                for (int k = 0; k + 1 < levels; ++k)
                    if (edges[k] < u) c++;
                codes[j] = (uint8_t)c;
            }
            /* rows stay byte-aligned because d*bits is a multiple of 8
             * whenever h >= 8 */
            if (msb_first)
                orc_pack_msb(codes, d, bits, packed + r * row_bytes);
            else
                orc_pack_lsb(codes, d, bits, packed + r * row_bytes);
            norms[r] = n;
        }
        free(y);
        free(codes);
    }
}

/* [ORBIT] _dequantize_rotated (rotated_only != 0): W' = codebook[code] times
 * the row norm. [ORBIT] dequantize (rotated_only == 0): W' then rpbh_inverse. */
void orc_orbit_dequantize(const uint8_t* packed, const float* norms,
                          int64_t rows, int64_t d, int bits,
                          const int64_t* inv_perm, const int8_t* signs,
                          const float* codebook, int msb_first, int rotated_only,
                          float* out, int threads) {
    const int64_t h = orc_block_size(d);
    const int64_t row_bytes = d * bits / 8;
    set_threads(threads);
#pragma omp parallel
    {
        float* y = (float*)malloc((size_t)d * sizeof(float));
        float* z = (float*)malloc((size_t)d * sizeof(float));
        uint8_t* codes = (uint8_t*)malloc((size_t)d);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            if (msb_first)
                orc_unpack_msb(packed + r * row_bytes, d, bits, codes);
            else
                orc_unpack_lsb(packed + r * row_bytes, d, bits, codes);
            for (int64_t j = 0; j < d; ++j) y[j] = codebook[codes[j]] * norms[r];
            if (rotated_only)
                memcpy(out + r * d, y, (size_t)d * sizeof(float));
            else
                rpbh_inverse_row(y, d, h, inv_perm, signs, z, out + r * d);
        }
        free(y);
        free(z);
        free(codes);
    }
}

/* Unit directions before bucketing, for boundary-distance accounting. */
void orc_orbit_unit(const float* w, int64_t rows, int64_t d,
                    const int64_t* perm, const int8_t* signs, float* unit,
                    float* norms, int threads) {
    const int64_t h = orc_block_size(d);
    const float eps = (float)1e-10;
    set_threads(threads);
#pragma omp parallel
    {
        float* y = (float*)malloc((size_t)d * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            rpbh_forward_row(w + r * d, d, h, perm, signs, y);
            float n = row_norm(y, d, h);
            float denom = n + eps;
            for (int64_t j = 0; j < d; ++j) unit[r * d + j] = y[j] / denom;
            norms[r] = n;
        }
        free(y);
    }
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
