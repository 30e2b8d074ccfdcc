// Launch interface between the C-ABI layer (libtq.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// 128-bit TQ3 sign mask passed by value: bit j of the vector (bit j%32 of
// w[j/32]) set means element j is negated.
struct SignMask {
  uint32_t w[4];
};

// Vectors one 256-thread TQ3 block handles per grid-stride iteration
// (a 4-lane quad owns one vector).
constexpr int kTq3VecPerBlock = 64;

// Launchers take the device's compute-unit count `cus`: grids hold as many
// blocks as the CUs keep resident at once (from the occupancy of the exact
// kernel instantiation), never more than there is work for, and the kernels'
// grid-stride loops spread the rest evenly.
hipError_t launch_tq3_quantize(const void* x, int dt, int64_t n_vec, int64_t stride,
                               const SignMask& m, uint8_t* rec, int cus, hipStream_t s);
hipError_t launch_tq3_dequantize(const uint8_t* rec, int64_t n_vec, const SignMask& m,
                                 void* y, int dt, int64_t stride, int cus, hipStream_t s);
// The same codec with the record's fields in three arrays: indices [n, 48],
// norms [n], scales [n].
hipError_t launch_tq3_quantize_split(const void* x, int dt, int64_t n_vec, int64_t stride,
                                     const SignMask& m, uint8_t* packed, float* norms,
                                     float* scales, int cus, hipStream_t s);
hipError_t launch_tq3_dequantize_split(const uint8_t* packed, const float* norms,
                                       const float* scales, int64_t n_vec, const SignMask& m,
                                       void* y, int dt, int64_t stride, int cus, hipStream_t s);

// OrbitQuant weight codec.
struct OrbitCodebook {
  float cb[16];     // 2^bits ascending centroids
  float edge[15];   // fp32 midpoints of neighbours
  // Set when cb[k] == -cb[2^bits - 1 - k] for every k: the edges are then
  // symmetric with the middle one exactly 0, and th[i] = 2 * bits(e) for the
  // positive edges e in ascending order (see the bucketize comment).
  int sym;
  uint32_t th[7];
};

hipError_t launch_orbit_quantize(const float* W, int64_t rows, int64_t d, int bits,
                                 const int32_t* perm, const int8_t* signs,
                                 const OrbitCodebook& cb, int lsb_first, uint8_t* packed,
                                 float* norms, int cus, hipStream_t s);
hipError_t launch_orbit_linear(const float* x, int64_t M, int64_t K, const uint8_t* packed,
                               const float* norms, int64_t N, int bits, const OrbitCodebook& cb,
                               int lsb_first, const float* bias, float* y, hipStream_t s);
// The same on bf16 / fp16 activations (dt = DT_BF16 or DT_F16): x, bias and y
// of that format, W' products rounded to it, bf16 / fp16 matrix cores.
// tiled: x is in the fragment layout of launch_orbit_rotate's tiled form
// (64 <= K < 2^22).
hipError_t launch_orbit_linear_lp(const void* x, int dt, int64_t M, int64_t K,
                                  const uint8_t* packed, const float* norms, int64_t N, int bits,
                                  const OrbitCodebook& cb, int lsb_first, const void* bias,
                                  void* y, int tiled, hipStream_t s);
// tiled (bf16 / fp16): xrot in the fragment layout of the tiled linear layer
hipError_t launch_orbit_rotate(const void* x, int dt, int64_t rows, int64_t d,
                               const int32_t* perm, const int8_t* signs, void* xrot, int tiled,
                               int cus, hipStream_t s);
hipError_t launch_orbit_dequantize(const uint8_t* packed, const float* norms, int64_t rows,
                                   int64_t d, int bits, const int32_t* inv_perm,
                                   const int8_t* signs, const OrbitCodebook& cb,
                                   int lsb_first, int rotated_only, void* out, int dt,
                                   int cus, hipStream_t s);
// Decode attention over TQ3 records: the token chunk per block and the number
// of chunks, both fixed by (n_tok, hkv, query heads per KV head) so that the
// caller can size the workspace before the call.
struct AttnPlan {
  int64_t chunk, nchunk;
};
AttnPlan tq3_attention_plan(int64_t n_tok, int hkv, int g);
size_t tq3_attention_ws_floats(int64_t n_tok, int hq, int hkv);
hipError_t launch_tq3_attention(const void* q, int qdt, int hq, const uint8_t* k,
                                const uint8_t* v, int64_t n_tok, int hkv, const SignMask& m,
                                float softmax_scale, float* ws, void* out, int odt,
                                hipStream_t s);
// Bytes of the library-held attention scratch (one array per GPU) and its
// device address on the current device, looked up once per device.
constexpr size_t kAttnScratchBytes = (size_t)16 << 20;
hipError_t attention_scratch(float** ptr);

// Blocks of `kernel` that one CU keeps resident with `block` threads and
// `shm` bytes of dynamic LDS (at least 1).
template <typename K>
inline int resident_blocks_per_cu(K kernel, int block, size_t shm) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, shm) != hipSuccess || n < 1)
    n = 1;
  return n;
}
inline int grid_size(int64_t need_blocks, int cus, int per_cu) {
  const int64_t cap = (int64_t)(cus > 0 ? cus : 1) * per_cu;
  return (int)(need_blocks < cap ? need_blocks : cap);
}


}  // namespace tq
