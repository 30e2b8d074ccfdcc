// The linear layer of the OrbitQuant runtime forward for gfx950 --
// "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py", OrbitQuantizer.forward:
// y = x_rot W'^T + bias, where W' = codebook[code] * row_norm is the
// rotated-basis weight of _dequantize_rotated. W' is never materialised in
// HBM: each block decodes its tile of codes into LDS and multiplies on fp32
// matrix cores (v_mfma_f32_16x16x4_f32). Each W' entry is the same fp32
// product the page forms (codebook value times row norm, rounded once).
//
// Tiling. A 256-thread block owns a BM x 128 tile of y; its four waves sit in
// a WM x WN grid and each owns (BM / WM) x (128 / WN) outputs as 16 x 16
// MFMA tiles. K advances 32 per step: x_rot[BM][32] is staged in LDS with
// rows padded to 36 floats, and W'^T[32][128] with rows padded to 144 floats
// (both pads make the MFMA operand reads conflict-free); thread t decodes
// 16 codes of W' row t % 128 per step.
//
// MFMA operand layout (v_mfma_f32_16x16x4_f32, checked on the device): lane
// l supplies A[l % 16][l / 16] and B[l / 16][l % 16]; result register r of
// lane l is D[4 (l / 16) + r][l % 16].
#include "orbit_codes.h"
#include "tq_common.h"
#include "tq_kernels.h"

namespace tq {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kBN = 128;      // output columns (W' rows) per block
constexpr int kBK = 32;       // K per step
constexpr int kArow = 36;     // padded LDS row of the x_rot tile
constexpr int kBrow = 144;    // padded LDS row of the W'^T tile

template <int BITS, bool LSB, int BM, int WM>
__global__ __launch_bounds__(256) void orbit_linear_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const float* __restrict__ norms, int64_t N, OrbitCodebook cb,
    const float* __restrict__ bias, float* __restrict__ y) {
  constexpr int WN = 4 / WM;
  constexpr int TM = BM / WM / 16, TN = kBN / WN / 16;
  __shared__ __attribute__((aligned(16))) float As[BM * kArow];
  __shared__ __attribute__((aligned(16))) float Bs[kBK * kBrow];
  __shared__ float cbs[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  int tx, ty;
  if (!xcd_tile((int)((N + kBN - 1) / kBN), (int)((M + BM - 1) / BM), tx, ty)) return;
  const int64_t m0 = (int64_t)ty * BM, n0 = (int64_t)tx * kBN;
  if (tid < 16) cbs[tid] = cb.cb[tid];

  // this thread's W' row and half of each K step
  const int bn = tid & (kBN - 1), bh = tid >> 7;
  const bool nvalid = n0 + bn < N;
  const float nrm = nvalid ? norms[n0 + bn] : 0.0f;
  const int64_t row_bytes = K * BITS / 8;
  const uint8_t* prow = packed + (nvalid ? n0 + bn : 0) * row_bytes;

  f32x4v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();  // cbs

  // The next K step's operands are loaded into registers while the current
  // one is multiplied.
  constexpr int NA = BM * 8 / 256;  // float4 of the x_rot tile per thread
  f32x4v av[NA];
  uint64_t raw;
  // Unconditional loads (rows past M re-read row m0) keep the loop free of
  // divergent branches; those rows are zeroed when they are staged.
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int f = tid + 256 * i;
      const int row = f >> 3, c4 = f & 7;
      const int64_t mr = m0 + row < M ? m0 + row : m0;
      av[i] = *reinterpret_cast<const f32x4v*>(x + mr * K + k0 + 4 * c4);
    }
    raw = load_codes<BITS>(prow + (k0 / 16 + bh) * (2 * BITS));
  };
  fetch(0);
  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    // x_rot tile: BM rows x 32 floats as float4 (8 per row)
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int f = tid + 256 * i;
      const float z = m0 + (f >> 3) < M ? 1.0f : 0.0f;
      *reinterpret_cast<f32x4v*>(&As[(f >> 3) * kArow + 4 * (f & 7)]) = av[i] * z;
    }
    // W'^T tile: 16 codes of row bn, K positions k0 + 16 bh .. + 15
    {
      uint32_t code[16];
      unpack16<BITS, LSB>(raw, code);
#pragma unroll
      for (int i = 0; i < 16; ++i) Bs[(16 * bh + i) * kBrow + bn] = cbs[code[i]] * nrm;
    }
    __syncthreads();
    if (k0 + kBK < K) fetch(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 4; ++kk) {
      float a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = As[(wm * (BM / WM) + 16 * i + (lane & 15)) * kArow + 4 * kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = Bs[(4 * kk + (lane >> 4)) * kBrow + wn * (kBN / WN) + 16 * j + (lane & 15)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // y = acc + bias
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = n0 + wn * (kBN / WN) + 16 * j + (lane & 15);
    if (n >= N) continue;
    const float bv = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * (BM / WM) + 16 * i + 4 * (lane >> 4) + r;
        if (m < M) y[m * N + n] = acc[i][j][r] + bv;
      }
  }
}

// Few rows (decode-sized batches up to 256 rows): one 16 x 32 tile of y per
// block. The four waves split K four ways, each staging its own operands in
// LDS (no block barrier inside the loop) with the next K step's loads in
// flight; the partial tiles are added in LDS at the end in a fixed order.
// Many small blocks keep every CU busy and shorten each block's chain of K
// steps. (Measured alternatives that were slower: eight waves per block,
// loads two and four steps ahead, operands decoded straight into registers
// in the MFMA layout.)
constexpr int kSmallWaves = 4;
template <int BITS, bool LSB>
__global__ __launch_bounds__(64 * kSmallWaves) void orbit_linear_small_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const float* __restrict__ norms, int64_t N, OrbitCodebook cb,
    const float* __restrict__ bias, float* __restrict__ y) {
  constexpr int KS = kSmallWaves, BNs = 32, kBsRow = 48;  // rows of 32 padded to 48
  __shared__ __attribute__((aligned(16))) float As[KS][16 * kArow];
  __shared__ __attribute__((aligned(16))) float Bs[KS][kBK * kBsRow];
  __shared__ float red[KS][16][BNs + 1];
  __shared__ float cbs[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * 16, n0 = (int64_t)blockIdx.x * BNs;
  if (tid < 16) cbs[tid] = cb.cb[tid];
  const int bn = lane & 31, bh = lane >> 5;
  const bool nvalid = n0 + bn < N;
  const float nrm = nvalid ? norms[n0 + bn] : 0.0f;
  const int64_t row_bytes = K * BITS / 8;
  const uint8_t* prow = packed + (nvalid ? n0 + bn : 0) * row_bytes;
  float* as = As[wave];
  float* bs = Bs[wave];
  f32x4v acc[2] = {f32x4v{0.0f, 0.0f, 0.0f, 0.0f}, f32x4v{0.0f, 0.0f, 0.0f, 0.0f}};
  __syncthreads();  // cbs
  const int64_t ksteps = K / kBK;
  const int64_t kb = ksteps * wave / KS, ke = ksteps * (wave + 1) / KS;
  // x_rot: 16 rows x 32 floats = 128 float4, two per lane, loaded one K step
  // ahead with the codes (unconditional loads: rows past M re-read row m0 and
  // are zeroed when staged, keeping the loop free of divergent branches)
  f32x4v av[2];
  uint64_t raw = 0;
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = lane + 64 * i;
      const int row = f >> 3, c4 = f & 7;
      const int64_t mr = m0 + row < M ? m0 + row : m0;
      av[i] = *reinterpret_cast<const f32x4v*>(x + mr * K + k0 + 4 * c4);
    }
    raw = load_codes<BITS>(prow + (k0 / 16 + bh) * (2 * BITS));
  };
  if (kb < ke) fetch(kb * kBK);
  for (int64_t ks = kb; ks < ke; ++ks) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = lane + 64 * i;
      const float z = m0 + (f >> 3) < M ? 1.0f : 0.0f;
      *reinterpret_cast<f32x4v*>(&as[(f >> 3) * kArow + 4 * (f & 7)]) = av[i] * z;
    }
    {
      uint32_t code[16];
      unpack16<BITS, LSB>(raw, code);
#pragma unroll
      for (int i = 0; i < 16; ++i) bs[(16 * bh + i) * kBsRow + bn] = cbs[code[i]] * nrm;
    }
    __builtin_amdgcn_wave_barrier();
    if (ks + 1 < ke) fetch((ks + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 4; ++kk) {
      const float a = as[(lane & 15) * kArow + 4 * kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float b = bs[(4 * kk + (lane >> 4)) * kBsRow + 16 * j + (lane & 15)];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * (lane >> 4) + r][16 * j + (lane & 15)] = acc[j][r];
  __syncthreads();
  for (int e = tid; e < 16 * BNs; e += 64 * KS) {
    const int rr = e / BNs, cc = e % BNs;
    const int64_t m = m0 + rr, n = n0 + cc;
    if (m < M && n < N) {
      float v = red[0][rr][cc];
#pragma unroll
      for (int w = 1; w < KS; ++w) v = v + red[w][rr][cc];
      y[m * N + n] = v + (bias ? bias[n] : 0.0f);
    }
  }
}

template <int BITS, bool LSB, int BM, int WM>
hipError_t launch_lin(const float* x, int64_t M, int64_t K, const uint8_t* packed,
                      const float* norms, int64_t N, const OrbitCodebook& cb, const float* bias,
                      float* y, hipStream_t s) {
  const unsigned grid = xcd_grid((N + kBN - 1) / kBN, (M + BM - 1) / BM);
  orbit_linear_kernel<BITS, LSB, BM, WM><<<grid, 256, 0, s>>>(x, M, K, packed, norms, N, cb,
                                                               bias, y);
  return hipGetLastError();
}

template <int BITS, bool LSB>
hipError_t launch_lin_m(const float* x, int64_t M, int64_t K, const uint8_t* packed,
                        const float* norms, int64_t N, const OrbitCodebook& cb,
                        const float* bias, float* y, hipStream_t s) {
  // up to 256 rows: 16 x 32 tiles with K split over the waves (enough blocks
  // to fill the chip); beyond, 128 x 128 tiles
  if (M <= 256) {
    const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + 15) / 16));
    orbit_linear_small_kernel<BITS, LSB><<<grid, 64 * kSmallWaves, 0, s>>>(x, M, K, packed, norms, N, cb,
                                                             bias, y);
    return hipGetLastError();
  }
  return launch_lin<BITS, LSB, 128, 2>(x, M, K, packed, norms, N, cb, bias, y, s);
}

}  // namespace

hipError_t launch_orbit_linear(const float* x, int64_t M, int64_t K, const uint8_t* packed,
                               const float* norms, int64_t N, int bits, const OrbitCodebook& cb,
                               int lsb_first, const float* bias, float* y, hipStream_t s) {
#define TQ_L(B, O) launch_lin_m<B, O>(x, M, K, packed, norms, N, cb, bias, y, s)
  if (lsb_first) {
    if (bits == 2) return TQ_L(2, true);
    if (bits == 3) return TQ_L(3, true);
    return TQ_L(4, true);
  }
  if (bits == 2) return TQ_L(2, false);
  if (bits == 3) return TQ_L(3, false);
  return TQ_L(4, false);
#undef TQ_L
}

}  // namespace tq
