// The linear layer of the OrbitQuant runtime forward on bf16 / fp16
// activations for gfx950 -- "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py",
// OrbitQuantizer.forward: with x of dtype bf16 or fp16 the page forms
// W' = codebook.to(dtype)[code] * row_norms.to(dtype) (each product rounded
// to the dtype) and F.linear(x_rot, W', bias) in that dtype. Here W' never
// reaches HBM: each block turns its W' rows into a table of the 2^bits
// values each row can take (the same rounded products), decodes its tile of
// codes through that table into LDS, and multiplies on bf16 / fp16 matrix
// cores (v_mfma_f32_16x16x32_{bf16,f16}) with fp32 accumulation; the bias is
// added in fp32 and the sum rounded to the dtype once.
//
// Tiling. A 256-thread block owns a 128 x 128 tile of y; its four waves sit
// in a 2 x 2 grid and each owns 64 x 64 outputs as 4 x 4 MFMA tiles. K
// advances 32 per step through two LDS buffers (one barrier per step): while
// the matrix cores work on one, the next step's x_rot rows and codes are
// loaded and written to the other. LDS rows hold 32 elements padded to 40
// (80 bytes), so the 16-byte operand reads of eight consecutive lanes fall in
// distinct banks.
//
// MFMA operand layout (checked on the device): lane l supplies
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e = 0..7, i.e.
// 16 contiguous bytes of an x_rot row and of a W' row; result register r of
// lane l is D[4 (l / 16) + r][l % 16].
#include "orbit_codes.h"
#include "tq_common.h"
#include "tq_kernels.h"

namespace tq {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));

// fp32 -> the format's bit pattern (nearest even), and back.
template <int DT>
__device__ __forceinline__ uint32_t lp_bits(float v) {
  if constexpr (DT == DT_BF16) return __builtin_bit_cast(uint16_t, (__bf16)v);
  else return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <int DT>
__device__ __forceinline__ float lp_float(uint32_t b) {
  if constexpr (DT == DT_BF16) return as_f(b << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

template <int DT>
__device__ __forceinline__ f32x4v mfma_lp(u32x4v a, u32x4v b, f32x4v c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a),
                                                   __builtin_bit_cast(bf16x8v, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8v, a),
                                                  __builtin_bit_cast(f16x8v, b), c, 0, 0, 0);
}

constexpr int kLpBM = 128, kLpBN = 128, kLpBK = 32;
constexpr int kLpRow = 40;  // padded LDS row (elements)

template <int DT, int BITS, bool LSB>
__global__ __launch_bounds__(256) void orbit_linear_lp_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const float* __restrict__ norms, int64_t N, OrbitCodebook cb,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  constexpr int L = 1 << BITS;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kLpBM * kLpRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kLpBN * kLpRow];
  __shared__ uint16_t tbl[kLpBN][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * kLpBM, n0 = (int64_t)blockIdx.x * kLpBN;

  // This thread decodes 16 codes of W' row bn per step (half bh of the 32).
  const int bn = tid >> 1, bh = tid & 1;
  const bool nvalid = n0 + bn < N;
  const int64_t row_bytes = K * BITS / 8;
  const uint8_t* prow = packed + (nvalid ? n0 + bn : 0) * row_bytes;
  {
    // row bn's table: round(round(codebook[c]) * round(norm)); rows past N
    // get zeros
    const float nl = nvalid ? lp_float<DT>(lp_bits<DT>(norms[n0 + bn])) : 0.0f;
#pragma unroll
    for (int c = 0; c < L; c += 2) {
      const int cc = c + bh;
      tbl[bn][cc] = (uint16_t)lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[cc])) * nl);
    }
  }

  // The next step's operands: two 16-byte pieces of x_rot rows per thread
  // (piece f: row f / 4, elements 8 (f % 4) .. + 7) and 16 codes. Rows past
  // M re-read row m0 (unconditional loads) and are zeroed when staged.
  u32x4v av[2];
  uint64_t raw;
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = tid + 256 * i;
      const int64_t mr = m0 + (f >> 2) < M ? m0 + (f >> 2) : m0;
      av[i] = *reinterpret_cast<const u32x4v*>(x + mr * K + k0 + 8 * (f & 3));
    }
    raw = load_codes<BITS>(prow + (k0 / 16 + bh) * (2 * BITS));
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = tid + 256 * i;
      const bool mv = m0 + (f >> 2) < M;
      const u32x4v z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4v*>(&As[buf][(f >> 2) * kLpRow + 8 * (f & 3)]) = mv ? av[i] : z;
    }
    uint32_t code[16];
    unpack16<BITS, LSB>(raw, code);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = (uint32_t)tbl[bn][code[2 * i]] | ((uint32_t)tbl[bn][code[2 * i + 1]] << 16);
    u32x4v* dst = reinterpret_cast<u32x4v*>(&Bs[buf][bn * kLpRow + 16 * bh]);
    dst[0] = u32x4v{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4v{w[4], w[5], w[6], w[7]};
  };

  f32x4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

  fetch(0);
  __syncthreads();  // tables
  stage(0);
  __syncthreads();
  int buf = 0;
  for (int64_t k0 = 0; k0 < K; k0 += kLpBK) {
    const bool more = k0 + kLpBK < K;
    if (more) fetch(k0 + kLpBK);
    u32x4v a[4], b[4];
    const int koff = 8 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const u32x4v*>(
          &As[buf][(wm * 64 + 16 * i + (lane & 15)) * kLpRow + koff]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const u32x4v*>(
          &Bs[buf][(wn * 64 + 16 * j + (lane & 15)) * kLpRow + koff]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_lp<DT>(a[i], b[j], acc[i][j]);
    if (more) stage(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // y = round(acc + bias)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 64 + 16 * j + (lane & 15);
    if (n >= N) continue;
    const float bv = bias ? lp_float<DT>(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
        if (m < M) y[m * N + n] = (uint16_t)lp_bits<DT>(acc[i][j][r] + bv);
      }
  }
}

template <int DT, int BITS, bool LSB>
hipError_t launch_lp(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                     const float* norms, int64_t N, const OrbitCodebook& cb, const void* bias,
                     void* y, hipStream_t s) {
  const dim3 grid((unsigned)((N + kLpBN - 1) / kLpBN), (unsigned)((M + kLpBM - 1) / kLpBM));
  orbit_linear_lp_kernel<DT, BITS, LSB><<<grid, 256, 0, s>>>(
      static_cast<const uint16_t*>(x), M, K, packed, norms, N, cb,
      static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y));
  return hipGetLastError();
}

template <int DT>
hipError_t launch_lp_bits(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                          const float* norms, int64_t N, int bits, const OrbitCodebook& cb,
                          int lsb_first, const void* bias, void* y, hipStream_t s) {
#define TQ_LP(B, O) launch_lp<DT, B, O>(x, M, K, packed, norms, N, cb, bias, y, s)
  if (lsb_first) {
    if (bits == 2) return TQ_LP(2, true);
    if (bits == 3) return TQ_LP(3, true);
    return TQ_LP(4, true);
  }
  if (bits == 2) return TQ_LP(2, false);
  if (bits == 3) return TQ_LP(3, false);
  return TQ_LP(4, false);
#undef TQ_LP
}

}  // namespace

hipError_t launch_orbit_linear_lp(const void* x, int dt, int64_t M, int64_t K,
                                  const uint8_t* packed, const float* norms, int64_t N, int bits,
                                  const OrbitCodebook& cb, int lsb_first, const void* bias,
                                  void* y, hipStream_t s) {
  if (dt == DT_BF16)
    return launch_lp_bits<DT_BF16>(x, M, K, packed, norms, N, bits, cb, lsb_first, bias, y, s);
  return launch_lp_bits<DT_F16>(x, M, K, packed, norms, N, bits, cb, lsb_first, bias, y, s);
}

}  // namespace tq
