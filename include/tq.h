/*
 * libtq -- randomized-Hadamard + Lloyd-Max vector codecs for AMD MI355X (gfx950).
 *
 * Two codecs share one shape: a randomized Hadamard rotation, a Lloyd-Max
 * codebook quantiser and bit packing, plus the inverse.
 *
 *   TQ3     the 3-bit KV-vector codec of the page "ComfyUI-TurboQuant:
 *           tq3_core.py" (module docstring, tq3_quantize, tq3_dequantize):
 *           each 128-float vector becomes a 56-byte record.
 *   Orbit   the weight codec of the page "zerogpu-sdxlTrainer:
 *           toolkit/util/orbit_quant.py" (rpbh_forward, _quantize_rows,
 *           _dequantize_rotated, dequantize): permutation + signs + block
 *           Hadamard, per-row norms, 2/3/4-bit Gaussian Lloyd-Max codes.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device memory owned by the caller; the
 *     library never allocates, frees or synchronises. Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream) and runs asynchronously.
 *   - Pointers named "host" are read during the call only.
 *   - A count of zero is a successful no-op.
 *   - Every argument is checked before anything is launched; on a non-zero
 *     return nothing was enqueued. tq_status_str() names each code.
 *   - Results are bit-for-bit deterministic: fixed operation order, no atomics.
 *   - Arithmetic is IEEE fp32, round to nearest even, with the operation order
 *     fixed by the library (see each function). Inputs holding NaN or Inf are
 *     outside the contract.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
    TQ_OK = 0,
    TQ_ERR_NULL = 1,    /* a required pointer is NULL                       */
    TQ_ERR_SHAPE = 2,   /* negative count, bad stride, d not a multiple of h */
    TQ_ERR_DTYPE = 3,   /* unknown dtype code                               */
    TQ_ERR_BITS = 4,    /* bits not in {2, 3, 4}                            */
    TQ_ERR_BLOCK = 5,   /* h = d & -d below 32, or d above 16384            */
    TQ_ERR_ALIGN = 6,   /* pointer or stride breaks the stated alignment    */
    TQ_ERR_LAUNCH = 7,  /* the HIP runtime refused the launch               */
    TQ_ERR_ARG = 8,     /* other invalid argument (flag value, codebook)    */
    TQ_ERR_SCRATCH = 9  /* sizes exceed the library-held scratch            */
};

/* ---- element types ----------------------------------------------------- */
enum {
    TQ_F32 = 0,   /* IEEE binary32                              */
    TQ_BF16 = 1,  /* bfloat16; widened exactly, narrowed by RNE */
    TQ_F16 = 2    /* IEEE binary16; widened exactly, narrowed by RNE */
};

/* ---- bit order of packed OrbitQuant codes --------------------------------- */
enum {
    TQ_MSB_FIRST = 0, /* the page's pack_codes layout: code j's most significant
                         bit at stream bit bits*j, stream bit q = bit 7-(q%8)
                         of byte q/8                                         */
    TQ_LSB_FIRST = 1  /* code j's bit t at stream bit bits*j+t, stream bit q =
                         bit q%8 of byte q/8                                 */
};

#define TQ3_DIM 128          /* elements per TQ3 vector                      */
#define TQ3_RECORD_BYTES 56  /* 48 bytes of 3-bit indices + fp32 norm + scale */

/*
 * tq3_quantize -- "tq3_core.py", tq3_quantize (docstring steps 1-6).
 *
 * For each of n_vec vectors v (128 elements at x + v*x_row_stride):
 *   norm   = max(sqrt(sum of squares), 1e-8); the sum is the pairwise tree
 *            that adds neighbours (j, j^1), then (j, j^2), ..., (j, j^64);
 *   u_j    = x_j / norm;  w_j = u_j * s_j  (s_j = -1 where sign bit j is set);
 *   y      = FWHT_128(w) (stages with half-width 1, 2, ..., 64, each pair
 *            becoming (a + b, a - b)), then times fp32(1/sqrt(128));
 *   scale  = max(max_j |y_j|, 1e-8);
 *   idx_j  = number of TQ3 boundaries b_k (fp32 of -0.7992, -0.4824, -0.2304,
 *            0, 0.2304, 0.4824, 0.7992) with b_k < y_j / scale.
 * Record v (56 bytes at records + 56*v): bytes 0..47 hold idx_j at stream
 * bits 3j..3j+2 (LSB-first; stream bit q = bit q%8 of byte q/8), bytes 48..51
 * the fp32 norm, 52..55 the fp32 scale, little-endian.
 *
 *   x            device, n_vec rows of x_dtype; 16-byte aligned; x_row_stride
 *                in elements, >= 128, a multiple of 8 (16 bytes).
 *   x_dtype      TQ_F32, TQ_BF16 or TQ_F16.
 *   sign_mask    host, 16 bytes: bit j (bit j%8 of byte j/8) set <=> s_j = -1.
 *                The TQ3 page draws s from a CPU generator seeded with 42.
 *   records      device, n_vec * 56 bytes, 8-byte aligned.
 */
int tq3_quantize(const void* x, int x_dtype, int64_t n_vec, int64_t x_row_stride,
                 const uint8_t* sign_mask, uint8_t* records, void* stream);

/*
 * tq3_dequantize -- "tq3_core.py", tq3_dequantize.
 *
 * For each record: c_j = C[idx_j] * scale (C = fp32 of the printed centroids
 * -0.9816, -0.6168, -0.3479, -0.1129, 0.1129, 0.3479, 0.6168, 0.9816), the
 * same FWHT and 1/sqrt(128) multiply as above (the normalised transform is its
 * own inverse), times s_j, times norm. fp32 results, narrowed by RNE when
 * y_dtype is TQ_BF16 or TQ_F16.
 *
 *   records      device, n_vec * 56 bytes, 8-byte aligned.
 *   sign_mask    host, 16 bytes, as for tq3_quantize.
 *   y            device, n_vec rows of y_dtype, 16-byte aligned; y_row_stride
 *                in elements, >= 128, a multiple of 8.
 */
int tq3_dequantize(const uint8_t* records, int64_t n_vec, const uint8_t* sign_mask,
                   void* y, int y_dtype, int64_t y_row_stride, void* stream);

/*
 * tq3_quantize_split / tq3_dequantize_split -- "tq3_core.py", tq3_quantize and
 * tq3_dequantize in the page's own storage layout: the dict it returns keeps
 * the indices, the norms and the scales as three tensors ("packed" uint8
 * [..., 48], "norms" and "scales" fp32 [...]) rather than one record.
 *
 * Same arithmetic, same index bytes and the same fp32 values as tq3_quantize /
 * tq3_dequantize; vector v's fields live at packed + 48*v, norms[v] and
 * scales[v] instead of at records + 56*v.
 *
 *   x, x_dtype, x_row_stride, y, y_dtype, y_row_stride, sign_mask
 *                as for tq3_quantize / tq3_dequantize.
 *   packed       device, n_vec * 48 bytes, 4-byte aligned.
 *   norms        device, n_vec fp32, 4-byte aligned.
 *   scales       device, n_vec fp32, 4-byte aligned.
 */
int tq3_quantize_split(const void* x, int x_dtype, int64_t n_vec, int64_t x_row_stride,
                       const uint8_t* sign_mask, uint8_t* packed, float* norms,
                       float* scales, void* stream);
int tq3_dequantize_split(const uint8_t* packed, const float* norms, const float* scales,
                         int64_t n_vec, const uint8_t* sign_mask, void* y, int y_dtype,
                         int64_t y_row_stride, void* stream);

/*
 * orbit_quantize_weight -- "orbit_quant.py", _quantize_rows with the buffers
 * of OrbitQuantizer.quantize_.
 *
 * For each of `rows` rows of the fp32 weight W (d elements each, contiguous):
 *   y_j     = W[perm_j] * signs_j, then on every block of h = d & -d elements
 *             the FWHT stages above, then times fp32(h ** -0.5);
 *   norm    = sqrt(s), s = pairwise-tree sums of y^2 inside each block (as
 *             for TQ3), added block by block from left to right;
 *   u_j     = y_j / (norm + fp32(1e-10));
 *   code_j  = number of edges e_k < u_j, e_k = (codebook[k] + codebook[k+1])/2
 *             in fp32.
 * Codes are packed in `bit_order` into rows of d*bits/8 bytes.
 *
 *   W            device, rows x d fp32, row-major, 16-byte aligned.
 *   d            input features, at most 16384 (one row is held on chip by
 *                one block of up to 16 waves); h = d & -d must be at least
 *                32 (the page skips layers with h < 32).
 *   bits         2, 3 or 4.
 *   perm         device, d int32, a permutation of 0..d-1; 16-byte aligned.
 *   signs        device, d int8, each +1 or -1; 16-byte aligned.
 *   codebook     host, 2^bits fp32 values in ascending order (the page's
 *                Gaussian Lloyd-Max codebook times d ** -0.5; see
 *                orbit_make_codebook).
 *   bit_order    TQ_MSB_FIRST (the page's layout) or TQ_LSB_FIRST.
 *   packed       device, rows * d * bits / 8 bytes, 16-byte aligned.
 *   row_norms    device, rows fp32.
 */
int orbit_quantize_weight(const float* W, int64_t rows, int64_t d, int bits,
                          const int32_t* perm, const int8_t* signs,
                          const float* codebook, int bit_order, uint8_t* packed,
                          float* row_norms, void* stream);

/*
 * orbit_dequantize -- "orbit_quant.py", _dequantize_rotated and dequantize.
 *
 *   rotated_only = 1: W'[r, j] = codebook[code_j] * norm_r (the rotated-basis
 *                     weight that the page's forward multiplies with P x).
 *   rotated_only = 0: W' as above, then per block the FWHT and h ** -0.5
 *                     multiply, times signs_j, then out[r, j] = z[inv_perm_j]
 *                     (the original-basis weight).
 *
 *   packed, row_norms   device, as written by orbit_quantize_weight.
 *   inv_perm            device, d int32, the inverse of perm, 16-byte aligned
 *                       (used when rotated_only = 0; may be NULL otherwise).
 *   signs               device, d int8, 16-byte aligned (may be NULL when
 *                       rotated_only = 1).
 *   codebook            host, 2^bits fp32.
 *   W_out               device, rows x d of out_dtype (TQ_F32, TQ_BF16 or
 *                       TQ_F16), 16-byte aligned.
 */
int orbit_dequantize(const uint8_t* packed, const float* row_norms, int64_t rows,
                     int64_t d, int bits, const int32_t* inv_perm,
                     const int8_t* signs, const float* codebook, int bit_order,
                     int rotated_only, void* W_out, int out_dtype, void* stream);

/*
 * orbit_rotate -- the forward rotation of activation rows ("zerogpu-
 * sdxlTrainer: toolkit/util/orbit_quant.py", rpbh_forward as
 * OrbitQuantizer.forward applies it to x): x_rot[r, j] = FWHT-blocks of
 * (x[r, perm_j] * signs_j), times fp32(h^-1/2), h = d & -d, in the page's
 * stage order, bit-identical to rpbh_forward evaluated on tensors of dtype:
 * for TQ_BF16 / TQ_F16 every stage's sums and differences and the final
 * products are computed in fp32 and rounded to that format (nearest even).
 *   x, x_rot    device, rows x d of dtype (TQ_F32, TQ_BF16, TQ_F16),
 *               row-major, 16-byte aligned.
 *   perm, signs device, int32 [d] and int8 [d] (+-1), 16-byte aligned.
 * Same limits on d as orbit_quantize_weight (TQ_ERR_BLOCK otherwise).
 */
int orbit_rotate(const void* x, int dtype, int64_t rows, int64_t d, const int32_t* perm,
                 const int8_t* signs, void* x_rot, void* stream);

/*
 * orbit_linear -- the forward's matmul ("orbit_quant.py",
 * OrbitQuantizer.forward: F.linear(x_rot, W', bias)) with the rotated-basis
 * weight W' of _dequantize_rotated decoded on the fly from the packed codes:
 *     y[i, o] = sum_j x_rot[i, j] W'[o, j] + bias[o].
 * dtype TQ_F32: W'[o, j] = codebook[code_{o,j}] * row_norms[o] in fp32, the
 *   sum on fp32 matrix cores.
 * dtype TQ_BF16 / TQ_F16 (the page's forward on activations of that dtype):
 *   W'[o, j] = round(round(codebook[code]) * round(row_norms[o])), each
 *   round to the dtype (nearest even); the sum on bf16 / fp16 matrix cores
 *   with fp32 accumulation; y = round(sum + bias).
 * The summation order is the library's (the page leaves it to the BLAS):
 * results agree with the definition to fp32 accumulation error (plus the
 * output's rounding for bf16 / fp16).
 *   x_rot       device, m x d_in of dtype, row-major, 16-byte aligned.
 *   packed      device, d_out rows of d_in * bits / 8 bytes (the layout
 *               orbit_quantize_weight writes), 16-byte aligned.
 *   row_norms   device, fp32 [d_out].
 *   codebook    host, 2^bits ascending fp32; bit_order as for the codec.
 *   bias        device [d_out] of dtype, or NULL.
 *   y           device, m x d_out of dtype, row-major.
 * d_in must be a positive multiple of 32 (TQ_ERR_SHAPE otherwise).
 */
int orbit_linear(const void* x_rot, int dtype, int64_t m, int64_t d_in, const uint8_t* packed,
                 const float* row_norms, int64_t d_out, int bits, const float* codebook,
                 int bit_order, const void* bias, void* y, void* stream);

/*
 * The same two steps of the forward ("orbit_quant.py", OrbitQuantizer.forward:
 * rpbh_forward, then F.linear with W') with the rotated activations passed in
 * the operand layout of the library's bf16 / fp16 matrix-core tiles, so the
 * linear layer loads them straight into registers (a layout of this library,
 * not of the page). The values are those of orbit_rotate, and
 * orbit_linear_tiled(orbit_rotate_tiled(x)) equals orbit_linear(orbit_rotate(x))
 * bit for bit.
 *
 * Tiled layout of an m x d matrix (d a multiple of 32): rows padded to
 * mp = 16 * ceil(m / 16); the 16 x 32 block of row tile t (rows 16 t ..) and
 * column chunk kc (columns 32 kc ..) is 1024 bytes at byte offset
 * (t * (d / 32) + kc) * 1024; inside it, the 16 bytes at l * 16 (l = 0..63)
 * hold row 16 t + l % 16, columns 32 kc + 8 (l / 16) .. + 7, in column order.
 * orbit_tiled_bytes(m, d) = mp * d * 2 (0 for d not a positive multiple of
 * 32, d > 16384 or m out of range).
 *
 * orbit_rotate_tiled -- orbit_rotate into that layout; the pad rows are
 *   written as zeros. dtype TQ_BF16 or TQ_F16 (TQ_ERR_DTYPE otherwise); x as
 *   for orbit_rotate; x_tiled device, orbit_tiled_bytes(rows, d) bytes,
 *   16-byte aligned. Same limits on d as orbit_rotate.
 * orbit_linear_tiled -- orbit_linear with x_rot in that layout (its m rows;
 *   the pad rows are read, their outputs not written). dtype TQ_BF16 or
 *   TQ_F16; 64 <= d_in < 2^22, a multiple of 32 (TQ_ERR_SHAPE otherwise);
 *   the other arguments as for orbit_linear.
 */
size_t orbit_tiled_bytes(int64_t m, int64_t d);
int orbit_rotate_tiled(const void* x, int dtype, int64_t rows, int64_t d, const int32_t* perm,
                       const int8_t* signs, void* x_tiled, void* stream);
int orbit_linear_tiled(const void* x_tiled, int dtype, int64_t m, int64_t d_in,
                       const uint8_t* packed, const float* row_norms, int64_t d_out, int bits,
                       const float* codebook, int bit_order, const void* bias, void* y,
                       void* stream);

/*
 * tq3_decode_attention -- one decode step of attention over a KV cache whose
 * K and V vectors are TQ3 records ("ComfyUI-TurboQuant: tq3_core.py": TQ3 is
 * a KV-cache codec; attention reads the vectors tq3_dequantize reconstructs).
 * For each query head h, with j = h / (n_q_heads / n_kv_heads):
 *     s_t = softmax_scale * <q_h, Khat_{t,j}>,  p = softmax(s),
 *     out_h = sum_t p_t Vhat_{t,j},
 * where Khat, Vhat are the tq3_dequantize reconstructions. The kernels never
 * reconstruct a vector: they score and accumulate in the rotated domain and
 * rotate each output back once; results agree with the definition to fp32
 * rounding, not bit for bit.
 *   q            device, n_q_heads x 128 of q_dtype (TQ_F32, TQ_BF16, TQ_F16),
 *                16-byte aligned.
 *   k_records,   device, n_tokens x n_kv_heads records of 56 bytes, token
 *   v_records    major (record t * n_kv_heads + j is token t of KV head j),
 *                8-byte aligned.
 *   n_tokens     >= 1, <= 2^31, and n_tokens x n_kv_heads <= 2^31.
 *   n_q_heads / n_kv_heads must be 1, 2, 4 or 8 (1 <= n_kv_heads <= 65535).
 *   sign_mask    host, 16 bytes, the mask the records were written with.
 *   workspace    device, at least tq3_attention_workspace_bytes(n_tokens,
 *                n_q_heads, n_kv_heads) bytes, 16-byte aligned; scratch for
 *                the per-chunk partial results, overwritten.
 *   out          device, n_q_heads x 128 of out_dtype (TQ_F32, TQ_BF16 or
 *                TQ_F16), 16-byte aligned.
 * Returns TQ_ERR_SHAPE for bad counts or head ratios, TQ_ERR_ARG for a short
 * workspace or a non-finite scale.
 */
int tq3_decode_attention(const void* q, int q_dtype, int n_q_heads,
                         const uint8_t* k_records, const uint8_t* v_records,
                         int64_t n_tokens, int n_kv_heads, const uint8_t* sign_mask,
                         float softmax_scale, void* workspace, size_t workspace_bytes,
                         void* out, int out_dtype, void* stream);

/* Workspace bytes tq3_decode_attention needs for these sizes (0 if invalid). */
size_t tq3_attention_workspace_bytes(int64_t n_tokens, int n_q_heads, int n_kv_heads);

/*
 * tq3_decode_attention_noalloc -- tq3_decode_attention for callers that cannot
 * allocate device memory or own a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. Same arguments,
 * arithmetic and results (bit for bit) as tq3_decode_attention, without the
 * workspace: the per-chunk partial results go to a library-held array of
 * tq3_attention_noalloc_max_bytes() = 16 MiB per GPU (a static device
 * array, one copy on each GPU the library runs on, held until the process
 * ends). The call allocates nothing.
 *   Sizes whose partial results need more than that array
 *   (tq3_attention_workspace_bytes(n_tokens, n_q_heads, n_kv_heads) > 16 MiB;
 *   at most about 4 MiB up to 8192 query heads, whatever the token count, so
 *   only sizes beyond about 31,000 query heads) return TQ_ERR_SCRATCH and
 *   enqueue nothing.
 *   Every call on a GPU shares that GPU's array: two calls that overlap in
 *   time on one GPU (on different streams, or from different threads without
 *   ordering) race and give undefined results. Calls ordered on one stream
 *   are safe; each call writes every partial it later reads, so nothing has
 *   to be cleared between calls.
 *   The first call on a device looks up that device's copy of the array
 *   (TQ_ERR_LAUNCH if the runtime cannot).
 */
int tq3_decode_attention_noalloc(const void* q, int q_dtype, int n_q_heads,
                                 const uint8_t* k_records, const uint8_t* v_records,
                                 int64_t n_tokens, int n_kv_heads, const uint8_t* sign_mask,
                                 float softmax_scale, void* out, int out_dtype, void* stream);

/* Bytes of the library-held scratch of tq3_decode_attention_noalloc (16 MiB). */
size_t tq3_attention_noalloc_max_bytes(void);

/* Bytes per TQ3 record: 48 + 4 + 4 = 56 ("tq3_core.py", tq3_memory_bytes). */
size_t tq3_record_bytes(void);

/* Largest power of two dividing d ("orbit_quant.py", hadamard_block_size);
 * returns 0 for d <= 0. */
int64_t orbit_block_size(int64_t d);

/*
 * tq_gaussian_lloyd_max -- host-side codebook ("orbit_quant.py",
 * gaussian_lloyd_max): 2^bits levels for the standard normal, started at the
 * quantiles of (k + 1/2) / 2^bits, `iters` Lloyd iterations in fp64 (edges at
 * centroid midpoints, centroids at the conditional means of their cells), no
 * early stop. Writes 2^bits ascending doubles to `out` (host). bits in [1, 8],
 * iters >= 0.
 */
int tq_gaussian_lloyd_max(int bits, int iters, double* out);

/*
 * orbit_make_codebook -- host-side: the codebook OrbitQuantizer.quantize_
 * builds for input dimension d: fp32(LM_k) * fp32(d ** -0.5) in fp32, with
 * LM from tq_gaussian_lloyd_max(bits, 200). Writes 2^bits floats to `out`.
 */
int orbit_make_codebook(int bits, int64_t d, float* out);

/* Human-readable name of a status code (static string). */
const char* tq_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
