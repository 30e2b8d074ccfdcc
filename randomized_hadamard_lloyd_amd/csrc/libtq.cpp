// C-ABI entry points of libtq: argument checks, launch geometry, and the
// host-side Gaussian Lloyd-Max codebook. Declarations and contracts are in
// include/tq.h.
#include "tq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "tq_kernels.h"

namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

// Compute units of the current device (queried once per device).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  });
  return g_cu_count[dev];
}

bool valid_dtype(int dt) { return dt == TQ_F32 || dt == TQ_BF16 || dt == TQ_F16; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launched(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH; }

constexpr int64_t kMaxVectors = (int64_t)1 << 40;
// Longest OrbitQuant row: one 1024-thread block holds it on chip.
constexpr int64_t kMaxOrbitD = 16384;

// ---- Gaussian Lloyd-Max (fp64), the procedure of the OrbitQuant page ----

double std_normal_cdf(double t) { return 0.5 * (1.0 + std::erf(t / std::sqrt(2.0))); }

double std_normal_pdf(double t) {
  if (std::isinf(t)) return 0.0;
  return std::exp(-t * t / 2.0) / std::sqrt(2.0 * M_PI);
}

// Quantile of the standard normal: bisection on the CDF written through erfc
// (accurate in both tails), run until the bracket stops shrinking.
double std_normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 2000; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    const double c = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (c < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

}  // namespace

extern "C" {

size_t tq3_record_bytes(void) { return TQ3_RECORD_BYTES; }

int64_t orbit_block_size(int64_t d) { return d > 0 ? (d & -d) : 0; }

const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_NULL: return "null pointer";
    case TQ_ERR_SHAPE: return "invalid shape or stride";
    case TQ_ERR_DTYPE: return "invalid dtype";
    case TQ_ERR_BITS: return "bits must be 2, 3 or 4";
    case TQ_ERR_BLOCK: return "Hadamard block d & -d below 32, or d above 16384";
    case TQ_ERR_ALIGN: return "misaligned pointer or stride";
    case TQ_ERR_LAUNCH: return "kernel launch failed";
    case TQ_ERR_ARG: return "invalid argument";
    case TQ_ERR_SCRATCH:
      return "sizes need more partial results than the library's 16 MiB attention scratch holds";
    default: return "unknown status";
  }
}

int tq3_quantize(const void* x, int x_dtype, int64_t n_vec, int64_t x_row_stride,
                 const uint8_t* sign_mask, uint8_t* records, void* stream) {
  if (!valid_dtype(x_dtype)) return TQ_ERR_DTYPE;
  if (n_vec < 0 || n_vec > kMaxVectors) return TQ_ERR_SHAPE;
  if (x_row_stride < TQ3_DIM || x_row_stride % 8 != 0 || x_row_stride > ((int64_t)1 << 24))
    return TQ_ERR_SHAPE;
  if (n_vec == 0) return TQ_OK;
  if (!x || !sign_mask || !records) return TQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(records, 8)) return TQ_ERR_ALIGN;
  tq::SignMask m;
  std::memcpy(m.w, sign_mask, sizeof(m.w));  // little-endian host
  return launched(tq::launch_tq3_quantize(x, x_dtype, n_vec, x_row_stride, m, records, cu_count(),
                                          static_cast<hipStream_t>(stream)));
}

int tq3_dequantize(const uint8_t* records, int64_t n_vec, const uint8_t* sign_mask, void* y,
                   int y_dtype, int64_t y_row_stride, void* stream) {
  if (!valid_dtype(y_dtype)) return TQ_ERR_DTYPE;
  if (n_vec < 0 || n_vec > kMaxVectors) return TQ_ERR_SHAPE;
  if (y_row_stride < TQ3_DIM || y_row_stride % 8 != 0 || y_row_stride > ((int64_t)1 << 24))
    return TQ_ERR_SHAPE;
  if (n_vec == 0) return TQ_OK;
  if (!records || !sign_mask || !y) return TQ_ERR_NULL;
  if (!aligned(y, 16) || !aligned(records, 8)) return TQ_ERR_ALIGN;
  tq::SignMask m;
  std::memcpy(m.w, sign_mask, sizeof(m.w));
  return launched(tq::launch_tq3_dequantize(records, n_vec, m, y, y_dtype, y_row_stride, cu_count(),
                                            static_cast<hipStream_t>(stream)));
}

int tq3_quantize_split(const void* x, int x_dtype, int64_t n_vec, int64_t x_row_stride,
                       const uint8_t* sign_mask, uint8_t* packed, float* norms, float* scales,
                       void* stream) {
  if (!valid_dtype(x_dtype)) return TQ_ERR_DTYPE;
  if (n_vec < 0 || n_vec > kMaxVectors) return TQ_ERR_SHAPE;
  if (x_row_stride < TQ3_DIM || x_row_stride % 8 != 0 || x_row_stride > ((int64_t)1 << 24))
    return TQ_ERR_SHAPE;
  if (n_vec == 0) return TQ_OK;
  if (!x || !sign_mask || !packed || !norms || !scales) return TQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(packed, 4) || !aligned(norms, 4) || !aligned(scales, 4))
    return TQ_ERR_ALIGN;
  tq::SignMask m;
  std::memcpy(m.w, sign_mask, sizeof(m.w));
  return launched(tq::launch_tq3_quantize_split(x, x_dtype, n_vec, x_row_stride, m, packed, norms,
                                                scales, cu_count(),
                                                static_cast<hipStream_t>(stream)));
}

int tq3_dequantize_split(const uint8_t* packed, const float* norms, const float* scales,
                         int64_t n_vec, const uint8_t* sign_mask, void* y, int y_dtype,
                         int64_t y_row_stride, void* stream) {
  if (!valid_dtype(y_dtype)) return TQ_ERR_DTYPE;
  if (n_vec < 0 || n_vec > kMaxVectors) return TQ_ERR_SHAPE;
  if (y_row_stride < TQ3_DIM || y_row_stride % 8 != 0 || y_row_stride > ((int64_t)1 << 24))
    return TQ_ERR_SHAPE;
  if (n_vec == 0) return TQ_OK;
  if (!packed || !norms || !scales || !sign_mask || !y) return TQ_ERR_NULL;
  if (!aligned(y, 16) || !aligned(packed, 4) || !aligned(norms, 4) || !aligned(scales, 4))
    return TQ_ERR_ALIGN;
  tq::SignMask m;
  std::memcpy(m.w, sign_mask, sizeof(m.w));
  return launched(tq::launch_tq3_dequantize_split(packed, norms, scales, n_vec, m, y, y_dtype,
                                                  y_row_stride, cu_count(),
                                                  static_cast<hipStream_t>(stream)));
}

// Shared checks of the OrbitQuant entry points; fills the kernel's codebook.
static int orbit_check(int64_t rows, int64_t d, int bits, const float* codebook, int bit_order,
                       tq::OrbitCodebook* cb) {
  if (bits < 2 || bits > 4) return TQ_ERR_BITS;
  if (rows < 0 || rows > kMaxVectors || d <= 0) return TQ_ERR_SHAPE;
  const int64_t h = d & -d;
  if (h < 32 || d > kMaxOrbitD) return TQ_ERR_BLOCK;
  if (bit_order != TQ_MSB_FIRST && bit_order != TQ_LSB_FIRST) return TQ_ERR_ARG;
  if (!codebook) return TQ_ERR_NULL;
  const int levels = 1 << bits;
  for (int k = 0; k < levels; ++k) {
    if (!std::isfinite(codebook[k])) return TQ_ERR_ARG;
    if (k > 0 && !(codebook[k] > codebook[k - 1])) return TQ_ERR_ARG;
    cb->cb[k] = codebook[k];
  }
  for (int k = levels; k < 16; ++k) cb->cb[k] = codebook[levels - 1];
  // fp32 midpoints of neighbours, as the page's _quantize_rows forms them
  for (int k = 0; k < 15; ++k)
    cb->edge[k] = (k + 1 < levels) ? (codebook[k] + codebook[k + 1]) / 2.0f : INFINITY;
  // Exactly symmetric codebooks (the Gaussian Lloyd-Max ones are) let the
  // kernels compare |u| against the positive edges only.
  bool sym = true;
  for (int k = 0; k < levels; ++k) sym = sym && codebook[k] == -codebook[levels - 1 - k];
  cb->sym = sym && cb->edge[levels / 2 - 1] == 0.0f;
  for (int i = 0; i < 7; ++i) {
    const int k = levels / 2 + i;
    uint32_t b = 0;
    if (k < levels - 1) std::memcpy(&b, &cb->edge[k], 4);
    cb->th[i] = 2u * b;
  }
  return TQ_OK;
}

int orbit_quantize_weight(const float* W, int64_t rows, int64_t d, int bits,
                          const int32_t* perm, const int8_t* signs, const float* codebook,
                          int bit_order, uint8_t* packed, float* row_norms, void* stream) {
  tq::OrbitCodebook cb;
  const int st = orbit_check(rows, d, bits, codebook, bit_order, &cb);
  if (st != TQ_OK) return st;
  if (rows == 0) return TQ_OK;
  if (!W || !perm || !signs || !packed || !row_norms) return TQ_ERR_NULL;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(perm, 16) || !aligned(signs, 16) ||
      !aligned(row_norms, 4))
    return TQ_ERR_ALIGN;
  return launched(tq::launch_orbit_quantize(W, rows, d, bits, perm, signs, cb,
                                            bit_order == TQ_LSB_FIRST, packed, row_norms, cu_count(),
                                            static_cast<hipStream_t>(stream)));
}

int orbit_dequantize(const uint8_t* packed, const float* row_norms, int64_t rows, int64_t d,
                     int bits, const int32_t* inv_perm, const int8_t* signs,
                     const float* codebook, int bit_order, int rotated_only, void* W_out,
                     int out_dtype, void* stream) {
  tq::OrbitCodebook cb;
  const int st = orbit_check(rows, d, bits, codebook, bit_order, &cb);
  if (st != TQ_OK) return st;
  if (!valid_dtype(out_dtype)) return TQ_ERR_DTYPE;
  if (rotated_only != 0 && rotated_only != 1) return TQ_ERR_ARG;
  if (rows == 0) return TQ_OK;
  if (!packed || !row_norms || !W_out) return TQ_ERR_NULL;
  if (!rotated_only && (!inv_perm || !signs)) return TQ_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(W_out, 16) || !aligned(row_norms, 4) ||
      (!rotated_only && (!aligned(inv_perm, 16) || !aligned(signs, 16))))
    return TQ_ERR_ALIGN;
  return launched(tq::launch_orbit_dequantize(packed, row_norms, rows, d, bits, inv_perm, signs,
                                              cb, bit_order == TQ_LSB_FIRST, rotated_only,
                                              W_out, out_dtype, cu_count(),
                                              static_cast<hipStream_t>(stream)));
}

int orbit_rotate(const void* x, int dtype, int64_t rows, int64_t d, const int32_t* perm,
                 const int8_t* signs, void* x_rot, void* stream) {
  if (!valid_dtype(dtype)) return TQ_ERR_DTYPE;
  if (rows < 0 || rows > kMaxVectors || d <= 0) return TQ_ERR_SHAPE;
  const int64_t h = d & -d;
  if (h < 32 || d > kMaxOrbitD) return TQ_ERR_BLOCK;
  if (rows == 0) return TQ_OK;
  if (!x || !perm || !signs || !x_rot) return TQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x_rot, 16) || !aligned(perm, 16) || !aligned(signs, 16))
    return TQ_ERR_ALIGN;
  return launched(tq::launch_orbit_rotate(x, dtype, rows, d, perm, signs, x_rot, 0, cu_count(),
                                          static_cast<hipStream_t>(stream)));
}

size_t orbit_tiled_bytes(int64_t rows, int64_t d) {
  if (rows < 0 || rows > kMaxVectors || d < 32 || d % 32 != 0 || d > kMaxOrbitD) return 0;
  return (size_t)((rows + 15) / 16 * 16) * (size_t)d * 2;
}

int orbit_rotate_tiled(const void* x, int dtype, int64_t rows, int64_t d, const int32_t* perm,
                       const int8_t* signs, void* x_tiled, void* stream) {
  if (dtype != TQ_BF16 && dtype != TQ_F16) return TQ_ERR_DTYPE;
  if (rows < 0 || rows > kMaxVectors || d <= 0) return TQ_ERR_SHAPE;
  const int64_t h = d & -d;
  if (h < 32 || d > kMaxOrbitD) return TQ_ERR_BLOCK;
  if (rows == 0) return TQ_OK;
  if (!x || !perm || !signs || !x_tiled) return TQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x_tiled, 16) || !aligned(perm, 16) || !aligned(signs, 16))
    return TQ_ERR_ALIGN;
  return launched(tq::launch_orbit_rotate(x, dtype, rows, d, perm, signs, x_tiled, 1, cu_count(),
                                          static_cast<hipStream_t>(stream)));
}

int orbit_linear(const void* x_rot, int dtype, int64_t m, int64_t d_in, const uint8_t* packed,
                 const float* row_norms, int64_t d_out, int bits, const float* codebook,
                 int bit_order, const void* bias, void* y, void* stream) {
  if (!valid_dtype(dtype)) return TQ_ERR_DTYPE;
  if (bits < 2 || bits > 4) return TQ_ERR_BITS;
  if (m < 0 || m > kMaxVectors || d_in < 32 || d_in % 32 != 0 || d_in > ((int64_t)1 << 24) ||
      d_out < 1 || d_out > ((int64_t)1 << 31))
    return TQ_ERR_SHAPE;
  if (m > ((int64_t)65535 * 128)) return TQ_ERR_SHAPE;  // grid rows
  if ((m + 127) / 128 * ((d_out + 127) / 128) > ((int64_t)1 << 30) ||
      (m + 255) / 256 * ((d_out + 63) / 64) > ((int64_t)1 << 30))
    return TQ_ERR_SHAPE;  // 128 x 128 or 256 x 64 tiles of a one-dimensional grid
  tq::OrbitCodebook cb;
  // the weight codec's codebook checks, at a block size that always passes
  const int st = orbit_check(1, 32, bits, codebook, bit_order, &cb);
  if (st != TQ_OK) return st;
  if (m == 0) return TQ_OK;
  if (!x_rot || !packed || !row_norms || !y) return TQ_ERR_NULL;
  const int es = dtype == TQ_F32 ? 4 : 2;
  if (!aligned(x_rot, 16) || !aligned(packed, 16) || !aligned(row_norms, 4) ||
      !aligned(y, es) || (bias && !aligned(bias, es)))
    return TQ_ERR_ALIGN;
  if (dtype != TQ_F32)
    return launched(tq::launch_orbit_linear_lp(x_rot, dtype, m, d_in, packed, row_norms, d_out,
                                               bits, cb, bit_order == TQ_LSB_FIRST, bias, y, 0,
                                               static_cast<hipStream_t>(stream)));
  return launched(tq::launch_orbit_linear(static_cast<const float*>(x_rot), m, d_in, packed,
                                          row_norms, d_out, bits, cb, bit_order == TQ_LSB_FIRST,
                                          static_cast<const float*>(bias), static_cast<float*>(y),
                                          static_cast<hipStream_t>(stream)));
}

int orbit_linear_tiled(const void* x_tiled, int dtype, int64_t m, int64_t d_in,
                       const uint8_t* packed, const float* row_norms, int64_t d_out, int bits,
                       const float* codebook, int bit_order, const void* bias, void* y,
                       void* stream) {
  if (dtype != TQ_BF16 && dtype != TQ_F16) return TQ_ERR_DTYPE;
  if (bits < 2 || bits > 4) return TQ_ERR_BITS;
  // the tall tiles: 64 <= d_in < 2^22 (32-bit fragment offsets inside a block)
  if (m < 0 || m > kMaxVectors || d_in < 64 || d_in % 32 != 0 || d_in >= ((int64_t)1 << 22) ||
      d_out < 1 || d_out > ((int64_t)1 << 31))
    return TQ_ERR_SHAPE;
  if ((m + 255) / 256 * ((d_out + 63) / 64) > ((int64_t)1 << 30)) return TQ_ERR_SHAPE;
  tq::OrbitCodebook cb;
  const int st = orbit_check(1, 32, bits, codebook, bit_order, &cb);
  if (st != TQ_OK) return st;
  if (m == 0) return TQ_OK;
  if (!x_tiled || !packed || !row_norms || !y) return TQ_ERR_NULL;
  if (!aligned(x_tiled, 16) || !aligned(packed, 16) || !aligned(row_norms, 4) || !aligned(y, 2) ||
      (bias && !aligned(bias, 2)))
    return TQ_ERR_ALIGN;
  return launched(tq::launch_orbit_linear_lp(x_tiled, dtype, m, d_in, packed, row_norms, d_out,
                                             bits, cb, bit_order == TQ_LSB_FIRST, bias, y, 1,
                                             static_cast<hipStream_t>(stream)));
}

static bool attn_shape_ok(int64_t n_tok, int hq, int hkv) {
  // hkv <= 65535: a lane's byte offset within a piece of 256 tokens' records
  // is 32-bit; n_tok * hkv <= 2^31: the (chunk, KV head) blocks fit a 1D grid
  if (n_tok < 1 || n_tok > ((int64_t)1 << 31) || hkv < 1 || hkv > 65535 || hq < hkv ||
      hq % hkv != 0 || n_tok * hkv > ((int64_t)1 << 31))
    return false;
  const int g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

size_t tq3_attention_workspace_bytes(int64_t n_tokens, int n_q_heads, int n_kv_heads) {
  if (!attn_shape_ok(n_tokens, n_q_heads, n_kv_heads)) return 0;
  return tq::tq3_attention_ws_floats(n_tokens, n_q_heads, n_kv_heads) * sizeof(float);
}

int tq3_decode_attention(const void* q, int q_dtype, int n_q_heads, const uint8_t* k_records,
                         const uint8_t* v_records, int64_t n_tokens, int n_kv_heads,
                         const uint8_t* sign_mask, float softmax_scale, void* workspace,
                         size_t workspace_bytes, void* out, int out_dtype, void* stream) {
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype)) return TQ_ERR_DTYPE;
  if (!attn_shape_ok(n_tokens, n_q_heads, n_kv_heads)) return TQ_ERR_SHAPE;
  if (!std::isfinite(softmax_scale)) return TQ_ERR_ARG;
  if (!q || !k_records || !v_records || !sign_mask || !workspace || !out) return TQ_ERR_NULL;
  if (workspace_bytes < tq3_attention_workspace_bytes(n_tokens, n_q_heads, n_kv_heads))
    return TQ_ERR_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, 16) || !aligned(k_records, 8) ||
      !aligned(v_records, 8))
    return TQ_ERR_ALIGN;
  tq::SignMask m;
  std::memcpy(m.w, sign_mask, sizeof(m.w));
  return launched(tq::launch_tq3_attention(q, q_dtype, n_q_heads, k_records, v_records, n_tokens,
                                           n_kv_heads, m, softmax_scale,
                                           static_cast<float*>(workspace), out, out_dtype,
                                           static_cast<hipStream_t>(stream)));
}

size_t tq3_attention_noalloc_max_bytes(void) { return tq::kAttnScratchBytes; }

int tq3_decode_attention_noalloc(const void* q, int q_dtype, int n_q_heads,
                                 const uint8_t* k_records, const uint8_t* v_records,
                                 int64_t n_tokens, int n_kv_heads, const uint8_t* sign_mask,
                                 float softmax_scale, void* out, int out_dtype, void* stream) {
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype)) return TQ_ERR_DTYPE;
  if (!attn_shape_ok(n_tokens, n_q_heads, n_kv_heads)) return TQ_ERR_SHAPE;
  if (!std::isfinite(softmax_scale)) return TQ_ERR_ARG;
  if (!q || !k_records || !v_records || !sign_mask || !out) return TQ_ERR_NULL;
  if (tq3_attention_workspace_bytes(n_tokens, n_q_heads, n_kv_heads) > tq::kAttnScratchBytes)
    return TQ_ERR_SCRATCH;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_records, 8) || !aligned(v_records, 8))
    return TQ_ERR_ALIGN;
  float* ws = nullptr;
  if (tq::attention_scratch(&ws) != hipSuccess || !ws) return TQ_ERR_LAUNCH;
  tq::SignMask m;
  std::memcpy(m.w, sign_mask, sizeof(m.w));
  return launched(tq::launch_tq3_attention(q, q_dtype, n_q_heads, k_records, v_records, n_tokens,
                                           n_kv_heads, m, softmax_scale, ws, out, out_dtype,
                                           static_cast<hipStream_t>(stream)));
}

int tq_gaussian_lloyd_max(int bits, int iters, double* out) {
  if (bits < 1 || bits > 8) return TQ_ERR_BITS;
  if (iters < 0) return TQ_ERR_ARG;
  if (!out) return TQ_ERR_NULL;
  const int levels = 1 << bits;
  double c[256], lo[256], hi[256];
  for (int k = 0; k < levels; ++k) c[k] = std_normal_quantile((k + 0.5) / levels);
  for (int it = 0; it < iters; ++it) {
    lo[0] = -INFINITY;
    hi[levels - 1] = INFINITY;
    for (int k = 0; k + 1 < levels; ++k) {
      const double e = (c[k] + c[k + 1]) / 2.0;
      hi[k] = e;
      lo[k + 1] = e;
    }
    for (int k = 0; k < levels; ++k)
      c[k] = (std_normal_pdf(lo[k]) - std_normal_pdf(hi[k])) /
             (std_normal_cdf(hi[k]) - std_normal_cdf(lo[k]));
  }
  std::memcpy(out, c, sizeof(double) * levels);
  return TQ_OK;
}

int orbit_make_codebook(int bits, int64_t d, float* out) {
  if (bits < 2 || bits > 4) return TQ_ERR_BITS;
  if (d <= 0) return TQ_ERR_SHAPE;
  if (!out) return TQ_ERR_NULL;
  double lm[16];
  const int st = tq_gaussian_lloyd_max(bits, 200, lm);
  if (st != TQ_OK) return st;
  const float s = (float)std::pow((double)d, -0.5);
  for (int k = 0; k < (1 << bits); ++k) out[k] = (float)lm[k] * s;
  return TQ_OK;
}

}  // extern "C"
