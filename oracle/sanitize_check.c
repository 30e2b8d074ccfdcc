/*
 * A test program that exercises every function of tq_oracle.c on small inputs held
 * in exactly sized heap buffers, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py builds and runs
 * it; any out-of-bounds access, leak or undefined operation ends the run with
 * a report). It also checks a few identities so that the calls do real work:
 * unpack(pack(c)) = c, the normalised FWHT is its own inverse, rpbh_inverse
 * undoes rpbh_forward, and dequantize(quantize(x)) keeps the sign pattern of
 * the codes it decodes.
 *
 * TEST INFRASTRUCTURE ONLY, like the rest of oracle/.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_fwht(float* v, int64_t rows, int n);
void orc_fwht_orbit(float* v, int64_t rows, int n);
void orc_tq3_bucketize(const float* xs, int64_t n, uint8_t* out);
void orc_tq3_tables(float* centroids, float* boundaries);
void orc_pack_lsb(const uint8_t* codes, int64_t count, int bits, uint8_t* out);
void orc_unpack_lsb(const uint8_t* packed, int64_t count, int bits, uint8_t* codes);
void orc_pack_msb(const uint8_t* codes, int64_t count, int bits, uint8_t* out);
void orc_unpack_msb(const uint8_t* packed, int64_t count, int bits, uint8_t* codes);
void orc_tq3_quantize(const float* x, int64_t n_vec, const float* signs, int post_flip,
                      uint8_t* rec, int threads);
void orc_tq3_dequantize(const uint8_t* rec, int64_t n_vec, const float* signs, int post_flip,
                        float* y, int threads);
void orc_tq3_scaled_coeffs(const float* x, int64_t n_vec, const float* signs, float* xs,
                           int threads);
int64_t orc_block_size(int64_t d);
void orc_rpbh_forward(const float* w, int64_t rows, int64_t d, const int64_t* perm,
                      const int8_t* signs, float* y, int threads);
void orc_rpbh_inverse(const float* y, int64_t rows, int64_t d, const int64_t* inv_perm,
                      const int8_t* signs, float* out, int threads);
void orc_orbit_quantize(const float* w, int64_t rows, int64_t d, int bits, const int64_t* perm,
                        const int8_t* signs, const float* codebook, int msb_first,
                        uint8_t* packed, float* norms, int threads);
void orc_orbit_dequantize(const uint8_t* packed, const float* norms, int64_t rows, int64_t d,
                          int bits, const int64_t* inv_perm, const int8_t* signs,
                          const float* codebook, int msb_first, int rotated_only, float* out,
                          int threads);
void orc_orbit_unit(const float* w, int64_t rows, int64_t d, const int64_t* perm,
                    const int8_t* signs, float* unit, float* norms, int threads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {  /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 2685821657736338717ull) >> 32);
}
static float urand(void) { return (float)(rnd() / 4294967296.0) * 2.0f - 1.0f; }

static int failures = 0;
#define CHECK(cond, what)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            fprintf(stderr, "check failed: %s\n", what);    \
            failures++;                                     \
        }                                                   \
    } while (0)

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void check_packing(void) {
    const int64_t counts[] = {1, 7, 8, 13, 128, 1001};
    for (int bits = 2; bits <= 4; ++bits)
        for (size_t c = 0; c < sizeof counts / sizeof counts[0]; ++c) {
            const int64_t n = counts[c];
            const int64_t nbytes = (n * bits + 7) / 8;
            uint8_t* codes = xmalloc((size_t)n);
            uint8_t* back = xmalloc((size_t)n);
            uint8_t* packed = xmalloc((size_t)nbytes);
            for (int64_t j = 0; j < n; ++j) codes[j] = (uint8_t)(rnd() & ((1u << bits) - 1));
            orc_pack_lsb(codes, n, bits, packed);
            orc_unpack_lsb(packed, n, bits, back);
            CHECK(memcmp(codes, back, (size_t)n) == 0, "lsb round trip");
            orc_pack_msb(codes, n, bits, packed);
            orc_unpack_msb(packed, n, bits, back);
            CHECK(memcmp(codes, back, (size_t)n) == 0, "msb round trip");
            free(codes);
            free(back);
            free(packed);
        }
}

static void check_fwht(void) {
    const int sizes[] = {2, 8, 32, 128, 1024, 16384};
    for (size_t s = 0; s < sizeof sizes / sizeof sizes[0]; ++s) {
        const int n = sizes[s];
        const int64_t rows = 3;
        float* v = xmalloc(sizeof(float) * (size_t)(rows * n));
        float* orig = xmalloc(sizeof(float) * (size_t)(rows * n));
        for (int64_t i = 0; i < rows * n; ++i) orig[i] = v[i] = urand();
        orc_fwht(v, rows, n);
        orc_fwht(v, rows, n);
        float err = 0.0f;
        for (int64_t i = 0; i < rows * n; ++i) err = fmaxf(err, fabsf(v[i] - orig[i]));
        CHECK(err < 1e-4f, "fwht self-inverse");
        orc_fwht_orbit(v, rows, n);
        free(v);
        free(orig);
    }
}

static void check_tq3(void) {
    float c[8], b[7];
    orc_tq3_tables(c, b);
    CHECK(c[0] < 0 && c[7] > 0 && b[3] == 0.0f, "tables");
    const int64_t counts[] = {1, 5, 64, 100};
    float signs[128];
    for (int j = 0; j < 128; ++j) signs[j] = (rnd() & 1) ? 1.0f : -1.0f;
    for (size_t k = 0; k < sizeof counts / sizeof counts[0]; ++k) {
        const int64_t n = counts[k];
        float* x = xmalloc(sizeof(float) * (size_t)(n * 128));
        for (int64_t i = 0; i < n * 128; ++i) x[i] = urand();
        if (n > 1) {
            for (int j = 0; j < 128; ++j) x[j] = 0.0f;             /* zero vector */
            for (int j = 0; j < 128; ++j) x[128 + j] = 1e30f;      /* norm overflows */
        }
        uint8_t* rec = xmalloc((size_t)(n * 56));
        float* y = xmalloc(sizeof(float) * (size_t)(n * 128));
        float* xs = xmalloc(sizeof(float) * (size_t)(n * 128));
        uint8_t* idx = xmalloc((size_t)(n * 128));
        for (int post = 0; post <= 1; ++post) {
            orc_tq3_quantize(x, n, signs, post, rec, 1);
            orc_tq3_dequantize(rec, n, signs, post, y, 1);
        }
        orc_tq3_scaled_coeffs(x, n, signs, xs, 1);
        orc_tq3_bucketize(xs, n * 128, idx);
        for (int64_t i = 0; i < n * 128; ++i) CHECK(idx[i] < 8, "bucket range");
        free(x);
        free(rec);
        free(y);
        free(xs);
        free(idx);
    }
}

static void shuffle(int64_t* p, int64_t d) {
    for (int64_t i = 0; i < d; ++i) p[i] = i;
    for (int64_t i = d - 1; i > 0; --i) {
        const int64_t j = (int64_t)(rnd() % (uint32_t)(i + 1));
        const int64_t t = p[i];
        p[i] = p[j];
        p[j] = t;
    }
}

static void check_orbit(void) {
    const int64_t dims[] = {32, 96, 160, 3072, 12288};
    const int64_t rows = 3;
    for (size_t k = 0; k < sizeof dims / sizeof dims[0]; ++k) {
        const int64_t d = dims[k];
        CHECK(orc_block_size(d) == (d & -d), "block size");
        int64_t* perm = xmalloc(sizeof(int64_t) * (size_t)d);
        int64_t* inv = xmalloc(sizeof(int64_t) * (size_t)d);
        int8_t* signs = xmalloc((size_t)d);
        float* w = xmalloc(sizeof(float) * (size_t)(rows * d));
        float* y = xmalloc(sizeof(float) * (size_t)(rows * d));
        float* back = xmalloc(sizeof(float) * (size_t)(rows * d));
        float* unit = xmalloc(sizeof(float) * (size_t)(rows * d));
        float* norms = xmalloc(sizeof(float) * (size_t)rows);
        shuffle(perm, d);
        for (int64_t j = 0; j < d; ++j) inv[perm[j]] = j;
        for (int64_t j = 0; j < d; ++j) signs[j] = (rnd() & 1) ? 1 : -1;
        for (int64_t i = 0; i < rows * d; ++i) w[i] = 0.02f * urand();
        for (int64_t j = 0; j < d; ++j) w[j] = 0.0f;   /* a zero row */
        orc_rpbh_forward(w, rows, d, perm, signs, y, 1);
        orc_rpbh_inverse(y, rows, d, inv, signs, back, 1);
        float err = 0.0f;
        for (int64_t i = 0; i < rows * d; ++i) err = fmaxf(err, fabsf(back[i] - w[i]));
        CHECK(err < 1e-6f, "rpbh round trip");
        orc_orbit_unit(w, rows, d, perm, signs, unit, norms, 1);
        for (int bits = 2; bits <= 4; ++bits) {
            const int levels = 1 << bits;
            float* cb = xmalloc(sizeof(float) * (size_t)levels);
            for (int c = 0; c < levels; ++c)
                cb[c] = (float)((c - (levels - 1) / 2.0) / sqrt((double)d));
            const int64_t nbytes = rows * d * bits / 8;
            uint8_t* packed = xmalloc((size_t)nbytes);
            float* out = xmalloc(sizeof(float) * (size_t)(rows * d));
            for (int msb = 0; msb <= 1; ++msb) {
                orc_orbit_quantize(w, rows, d, bits, perm, signs, cb, msb, packed, norms, 1);
                for (int rot = 0; rot <= 1; ++rot)
                    orc_orbit_dequantize(packed, norms, rows, d, bits, inv, signs, cb, msb, rot,
                                         out, 1);
            }
            CHECK(norms[0] == 0.0f, "zero row norm");
            free(cb);
            free(packed);
            free(out);
        }
        free(perm);
        free(inv);
        free(signs);
        free(w);
        free(y);
        free(back);
        free(unit);
        free(norms);
    }
}

int main(void) {
    check_packing();
    check_fwht();
    check_tq3();
    check_orbit();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
