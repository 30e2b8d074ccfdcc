// The linear layer of the OrbitQuant runtime forward on bf16 / fp16
// activations for gfx950 -- "zerogpu-sdxlTrainer: toolkit/util/orbit_quant.py",
// OrbitQuantizer.forward: with x of dtype bf16 or fp16 the page forms
// W' = codebook.to(dtype)[code] * row_norms.to(dtype) (each product rounded
// to the dtype) and F.linear(x_rot, W', bias) in that dtype. Here W' never
// reaches HBM: each block turns its W' rows into a table of the values each
// row can take (the same rounded products; for 2- and 3-bit codes a table of
// code pairs), decodes its codes through that table and multiplies on bf16 /
// fp16 matrix cores (v_mfma_f32_16x16x32_{bf16,f16}) with fp32
// accumulation; the bias is added in fp32 and the sum rounded to the dtype
// once. Three kernels: tall 256 x 64 tiles for batches of more than 64 rows,
// square 128 x 128 tiles for the shapes the tall ones do not take (K = 32,
// or rows too long for their 32-bit offsets), and one for decode-sized
// batches of up to 64 rows (see each kernel's comment).
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
typedef uint16_t u16x2v __attribute__((ext_vector_type(2)));

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

constexpr int kLpBM = 128, kLpBN = 128, kLpBK = 64;
constexpr int kLpRow = 72;  // padded LDS row (elements)
constexpr int kLpRing = 4;  // K steps whose global loads are in flight
constexpr size_t kLpSmallLds = 64 * 1024;  // the few-rows kernel's LDS ceiling
#ifndef TQ_LP_WIDE_MIN
#define TQ_LP_WIDE_MIN 32  // above this many rows the few-rows blocks take 32 W' rows
#endif

// Many rows, square tiles (K = 32, or K of 2^22 and more). A 256-thread
// block owns a 128 x 128 tile of y; its four waves sit
// in a 2 x 2 grid and each owns 64 x 64 outputs as 4 x 4 MFMA tiles. K
// advances 64 per step through one set of LDS tiles (two barriers per step),
// while the global loads of the next four steps are in flight in a register
// ring. LDS rows hold 64 elements padded to 72 (144 bytes), so the 16-byte
// operand reads of eight consecutive lanes fall in distinct banks.

template <int DT, int BITS, bool LSB>
__global__ __launch_bounds__(256) void orbit_linear_lp_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const float* __restrict__ norms, int64_t N, OrbitCodebook cb,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  constexpr int L = 1 << BITS;
  // 2- and 3-bit codes decode through a table of code pairs (one dword per
  // pair, both rounded products); 4-bit codes, whose pair table would not
  // fit, through a table of single values.
  constexpr bool PAIRS = BITS <= 3;
  // dwords per row's table, padded by one so that rows start in different banks
  constexpr int TW = (PAIRS ? L * L : L / 2) + 1;
  __shared__ __attribute__((aligned(16))) uint16_t As[kLpBM * kLpRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kLpBN * kLpRow];
  __shared__ uint32_t tbw[kLpBN * TW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tx, ty;
  if (!xcd_tile((int)((N + kLpBN - 1) / kLpBN), (int)((M + kLpBM - 1) / kLpBM), tx, ty)) return;
  const int64_t m0 = (int64_t)ty * kLpBM, n0 = (int64_t)tx * kLpBN;

  // This thread decodes 32 codes of W' row bn per step (half bh of the 64).
  const int bn = tid >> 1, bh = tid & 1;
  const bool nvalid = n0 + bn < N;
  const int64_t row_bytes = K * BITS / 8;
  const uint8_t* prow = packed + (nvalid ? n0 + bn : 0) * row_bytes;
  uint16_t* t16 = reinterpret_cast<uint16_t*>(tbw) + bn * 2 * TW;
  {
    // row bn's table of round(round(codebook[c]) * round(norm)) (zeros for
    // rows past N), split between the row's two threads
    const float nl = nvalid ? lp_float<DT>(lp_bits<DT>(norms[n0 + bn])) : 0.0f;
    if constexpr (PAIRS) {
      for (int e = bh; e < L * L; e += 2) {
        const int a = LSB ? e % L : e / L, b = LSB ? e / L : e % L;
        tbw[bn * TW + e] = lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[a])) * nl) |
                           (lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[b])) * nl) << 16);
      }
    } else {
#pragma unroll
      for (int c = 0; c < L; c += 2) {
        const int cc = c + bh;
        t16[cc] = (uint16_t)lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[cc])) * nl);
      }
    }
  }

  // Per step, four 16-byte pieces of x_rot rows per thread (piece f: row
  // f / 8, elements 8 (f % 8) .. + 7) and 32 codes. Rows past M re-read row
  // m0 (their outputs are never stored). When K is an odd multiple of 32 the
  // last step's upper half re-reads the lower half and is zeroed in x_rot.
  const int64_t steps = (K + kLpBK - 1) / kLpBK;
  u32x4v av[kLpRing][4];
  uint64_t raw[kLpRing][2];
  // Piece i of this thread: row tid / 8 + 32 i of the tile, elements
  // 8 (tid % 8) .. + 7 of the step; `upper` marks the step's second half.
  const bool upper = (tid & 7) >= 4;
  const uint16_t* xp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t mr = m0 + (tid >> 3) + 32 * i;
    xp[i] = x + (mr < M ? mr : m0) * K + 8 * (tid & 7);
  }
  auto fetch = [&](int u, int64_t st) {
    const int64_t s = st < steps ? st : steps - 1;
    const int64_t k0 = s * kLpBK;
    const bool hv = k0 + 32 < K;
    const int64_t ka = hv || !upper ? k0 : k0 - 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) av[u][i] = *reinterpret_cast<const u32x4v*>(xp[i] + ka);
    const int64_t cg = k0 / 16 + (hv ? 2 * bh : 0);  // 16-code group
#pragma unroll
    for (int q = 0; q < 2; ++q) raw[u][q] = load_codes<BITS>(prow + (cg + q) * (2 * BITS));
  };
  auto stage = [&](int u, int64_t st) {
    if (st * kLpBK + 32 >= K) {
      // a half step: zeros in the upper half
      if (upper) {
#pragma unroll
        for (int i = 0; i < 4; ++i) av[u][i] = u32x4v{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4v*>(&As[((tid >> 3) + 32 * i) * kLpRow + 8 * (tid & 7)]) = av[u][i];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t w[8];
      if constexpr (PAIRS) {
        uint32_t pi[8];
        pairs16<BITS, LSB>(raw[u][q], pi);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = tbw[bn * TW + pi[e]];
      } else {
        uint32_t code[16];
        unpack16<BITS, LSB>(raw[u][q], code);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          w[e] = (uint32_t)t16[code[2 * e]] | ((uint32_t)t16[code[2 * e + 1]] << 16);
      }
      u32x4v* dst = reinterpret_cast<u32x4v*>(&Bs[bn * kLpRow + 32 * bh + 16 * q]);
      dst[0] = u32x4v{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4v{w[4], w[5], w[6], w[7]};
    }
  };

  f32x4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int u = 0; u < kLpRing; ++u) fetch(u, u);
  __syncthreads();  // tables
  // Step st stages ring slot st % 4 into the LDS tiles, refills the slot
  // with step st + 4 and multiplies; one set of tiles, two barriers a step.
  for (int64_t s0 = 0; s0 < steps; s0 += kLpRing) {
#pragma unroll
    for (int u = 0; u < kLpRing; ++u) {
      const int64_t st = s0 + u;
      if (st < steps) {
        stage(u, st);
        fetch(u, st + kLpRing);
        asm volatile("" ::: "memory");  // the refill stays a full ring ahead
        __syncthreads();
        const int koff = 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4v a[4], b[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const u32x4v*>(
                &As[(wm * 64 + 16 * i + (lane & 15)) * kLpRow + 32 * kk + koff]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            b[j] = *reinterpret_cast<const u32x4v*>(
                &Bs[(wn * 64 + 16 * j + (lane & 15)) * kLpRow + 32 * kk + koff]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_lp<DT>(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
      }
    }
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

// Many rows, tall tiles. A 256-thread block owns a 256 x 64 tile of y and
// wave w the rows 64 w .. 64 w + 63 of it (4 x 4 MFMA tiles). The block's 64
// W' rows are decoded once per 64-wide K step into an LDS tile that all four
// waves read, so each decoded element feeds 256 output rows: the decode's
// VALU work, which does not overlap the MFMAs, costs half as much per MFMA as
// in the square tiles. The decoded tile is double-buffered (one barrier per
// step); codes load two steps ahead. No two waves share an x_rot row: each
// wave loads its own 64 rows with coalesced 16-byte loads one step ahead and
// passes them through a private LDS tile into the MFMA layout, without a
// barrier. Tables of single values (pairs for 2-bit codes) and unpadded,
// XOR-swizzled tiles keep the block at 52 KB of LDS, so three blocks (twelve
// waves) share a CU.
//
// Tile layout: row r holds 64 elements as eight 16-byte chunks; chunk c sits
// in slot c ^ ((r / 2) % 8). The MFMA operand reads (16 consecutive rows, one
// chunk) then cover all 64 banks once per 16 lanes.
//
// TILED: x_rot comes in the MFMA fragment layout orbit_rotate_tiled writes
// (1 KB per 16 rows x 32 columns, lane l's 16 bytes at l * 16: row l % 16,
// columns 8 (l / 16) .. + 7), so each wave loads its operands straight into
// registers, whole cache lines per load, and x_rot never passes through LDS.
// Each step's two halves load half a step apart (the next step's first half
// at the start of a step, its second half once the first half's MFMAs are
// issued): 159-166 VGPRs, three waves per SIMD. The LDS left free also holds
// pair tables for 3-bit codes (one table read per two codes; 68.7 -> 58.1 us
// at 512 rows of the 12288 x 3072 layer). Unrolling three steps to rotate the
// fragment registers instead of copying them spilled and ran 2.5x slower.
constexpr int kTallBM = 256, kTallBN = 64;

// One v_bfe_u32 per 3-bit field (left to itself the compiler shifts and
// masks in two instructions to fold the table's element size in).
__device__ __forceinline__ uint32_t bfe3(uint32_t v, int off) {
  uint32_t r;
  asm("v_bfe_u32 %0, %1, %2, 3" : "=v"(r) : "v"(v), "i"(off));
  return r;
}

__device__ __forceinline__ int tall_off(int r, int c) {  // byte offset of (row, chunk)
  return r * 128 + ((c ^ (r >> 1)) & 7) * 16;
}

// KS = 2 (one row band of at most 256 rows and an even step count): eight
// waves, waves 4 kh .. 4 kh + 3 taking the steps kh S/2 .. (kh + 1) S/2 - 1
// of the same tile in lockstep, each half with its own tile buffers; the
// second half's accumulators are then added to the first half's through LDS
// (first half + second half: a fixed order). Half the dependent steps per
// wave, where a lone row band leaves the CUs one block each.
template <int DT, int BITS, bool LSB, bool TILED, int KS = 1>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(KS == 2 ? 2 : 3))) void
orbit_linear_lp_tall_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                            const uint8_t* __restrict__ packed, const float* __restrict__ norms,
                            int64_t N, OrbitCodebook cb, const uint16_t* __restrict__ bias,
                            uint16_t* __restrict__ y) {
  constexpr int L = 1 << BITS;
  // pair tables for 2-bit codes, and for 3-bit ones when x_rot does not take
  // LDS (TILED): one read per two codes, already the packed dword
  constexpr bool PAIRS = BITS == 2 || (TILED && BITS == 3);
  // dwords per row's table, padded by one so that rows start in different banks
  constexpr int TW = (PAIRS ? L * L : L / 2) + 1;
  static_assert(KS == 1 || KS == 2, "one or two halves of the steps");
  // x_rot staging (per wave) and, for KS = 2, the second half's accumulators
  constexpr int AS_BYTES = TILED ? 16 : 4 * KS * 64 * 128;
  constexpr int RED_BYTES = KS == 2 ? 16 * 4 * 256 * 4 : 0;
  __shared__ __attribute__((aligned(16))) char As_[AS_BYTES > RED_BYTES ? AS_BYTES : RED_BYTES];
  __shared__ __attribute__((aligned(16))) char Bs_[KS][2][kTallBN * 128];
  __shared__ uint32_t tbw[kTallBN * TW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 3, kh = wave >> 2;  // the wave's 64 rows; its half of the steps
  char (*Bs)[kTallBN * 128] = Bs_[kh];
  int tx, ty;
  if (!xcd_tile((int)((N + kTallBN - 1) / kTallBN), (int)((M + kTallBM - 1) / kTallBM), tx, ty))
    return;
  const int64_t m0 = (int64_t)ty * kTallBM, n0 = (int64_t)tx * kTallBN;

  // This thread decodes codes 16 bq .. 16 bq + 15 of each step (of its
  // half) of W' row bn.
  const int bn = (tid & 255) >> 2, bq = tid & 3;
  const bool nvalid = n0 + bn < N;
  const int64_t row_bytes = K * BITS / 8;
  const uint8_t* prow = packed + (nvalid ? n0 + bn : 0) * row_bytes;
  uint16_t* t16 = reinterpret_cast<uint16_t*>(tbw) + bn * 2 * TW;
  if (kh == 0) {  // one half builds the tables (KS = 2)
    // row bn's table of round(round(codebook[c]) * round(norm)) (zeros for
    // rows past N), split between the row's four threads
    const float nl = nvalid ? lp_float<DT>(lp_bits<DT>(norms[n0 + bn])) : 0.0f;
    if constexpr (PAIRS) {
      for (int e = bq; e < L * L; e += 4) {
        const int a = LSB ? e % L : e / L, b = LSB ? e / L : e % L;
        tbw[bn * TW + e] = lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[a])) * nl) |
                           (lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[b])) * nl) << 16);
      }
    } else {
      for (int c = bq; c < L; c += 4)
        t16[c] = (uint16_t)lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[c])) * nl);
    }
  }

  // x_rot: piece p of this lane is row 8 p + lane / 8 of the wave's 64, chunk
  // lane % 8 of the step (byte offsets from the block's first row at the
  // step's column; rows past M re-read row m0 and are never stored).
  // TILED: piece p = 2 i + h is the fragment of row tile 4 wave + i (tiles
  // past the last one re-read it), half h of the step.
  const char* xblk = reinterpret_cast<const char*>(x + m0 * K);
  uint32_t xoff[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if constexpr (TILED) {
      const int64_t last_t = (M + 15) / 16 - 1 - m0 / 16;
      const int64_t t = 4 * wv + (p >> 1) < last_t ? 4 * wv + (p >> 1) : last_t;
      xoff[p] = (uint32_t)(((t * (K / 32) + (p & 1)) * 64 + lane) * 16);
    } else {
      const int64_t r = 64 * wv + 8 * p + (lane >> 3);
      xoff[p] = (uint32_t)(((m0 + r < M ? r : 0) * K + 8 * (lane & 7)) * 2);
    }
  }
  const int64_t steps = (K + 63) / 64;
  // K is a multiple of 32 (and at least 64): when it is an odd one, the last
  // step's window starts 32 columns early, so that its second half holds the
  // last 32 columns, and the MFMAs skip its first half.
  const bool half_last = (K & 63) != 0;
  const int64_t last = steps - 1;
  // this wave's steps: s0 .. s0 + sh - 1 (KS = 2: half of them)
  const int64_t sh = KS == 2 ? steps / 2 : steps;
  const int64_t s0 = KS == 2 ? kh * sh : 0;
  const int64_t s_end = s0 + sh - 1;
  auto kbase = [&](int64_t st) { return st * 64 - (half_last && st == last ? 32 : 0); };
  auto fetch_x = [&](u32x4v (&xv)[8], int64_t st) {
    const char* b = TILED ? xblk + (kbase(st) / 32) * 1024 : xblk + kbase(st) * 2;
#pragma unroll
    for (int p = 0; p < 8; ++p) xv[p] = *reinterpret_cast<const u32x4v*>(b + xoff[p]);
  };
  // TILED: the four fragments of one half step
  auto fetch_half = [&](u32x4v (&xv)[4], int64_t st, int h) {
    const char* b = xblk + (kbase(st) / 32) * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = *reinterpret_cast<const u32x4v*>(b + xoff[2 * i + h]);
  };
  auto stage_x = [&](const u32x4v (&xv)[8]) {
#pragma unroll
    for (int p = 0; p < 8; ++p)
      *reinterpret_cast<u32x4v*>(As_ + (TILED ? 0 : wave) * (64 * 128) +
                                 tall_off(8 * p + (lane >> 3), lane & 7)) =
          xv[p];
  };
  auto fetch_c = [&](int64_t st) -> uint64_t {
    return load_codes<BITS>(prow + (kbase(st) / 16 + bq) * (2 * BITS));
  };
  // The 16 decoded elements of one step: chunks 2 bq, 2 bq + 1 of row bn.
  auto decode = [&](uint64_t raw, int buf) {
    uint32_t w[8];
    if constexpr (PAIRS) {
      uint32_t pi[8];
      pairs16<BITS, LSB>(raw, pi);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = tbw[bn * TW + pi[e]];
    } else {
      uint32_t code[16];
      const uint32_t lo = (uint32_t)raw, hi = (uint32_t)(raw >> 32);
      if constexpr (BITS == 3 && !LSB) {
        // the two 24-bit groups of 8 codes, bytes reversed so that the
        // earliest code sits in the top bits
        const uint32_t g0 = __builtin_amdgcn_perm(0u, lo, 0x0c000102u);
        const uint32_t g1 = __builtin_amdgcn_perm(hi, lo, 0x0c030405u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          code[i] = bfe3(g0, 21 - 3 * i);
          code[8 + i] = bfe3(g1, 21 - 3 * i);
        }
      } else if constexpr (BITS == 4) {
        // byte b: codes 2 b and 2 b + 1 (the earlier one in the high nibble
        // for MSB-first)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t wd = i < 8 ? lo : hi;
          const int sh = 8 * ((i >> 1) & 3) + (LSB ? 4 * (i & 1) : 4 - 4 * (i & 1));
          code[i] = __builtin_amdgcn_ubfe(wd, sh, 4);
        }
      } else {
        unpack16<BITS, LSB>(raw, code);
      }
      // two 16-bit table reads per dword, the second into the upper half
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u16x2v v;
        v.x = t16[code[2 * e]];
        v.y = t16[code[2 * e + 1]];
        w[e] = __builtin_bit_cast(uint32_t, v);
      }
    }
    *reinterpret_cast<u32x4v*>(&Bs[buf][tall_off(bn, 2 * bq)]) = u32x4v{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4v*>(&Bs[buf][tall_off(bn, 2 * bq + 1)]) =
        u32x4v{w[4], w[5], w[6], w[7]};
  };

  f32x4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4v xa[8];  // TILED: the current step's fragments
  if constexpr (TILED) {
    fetch_x(xa, s0);
  } else {
    u32x4v xv[8];
    fetch_x(xv, s0);
    stage_x(xv);
  }
  const uint64_t craw0 = fetch_c(s0);
  uint64_t cr = fetch_c(sh > 1 ? s0 + 1 : s0);
  __syncthreads();  // tables
  decode(craw0, 0);
  __syncthreads();  // the tile of step 0
  // operand reads: row 16 t + lane % 16 of a tile, chunk 4 kk + lane / 16
  const int orow = lane & 15, ochk = lane >> 4;
  // One step: multiply the tile of step st (both halves, or only the second
  // on a half step) while the next step's x_rot and the codes two steps ahead
  // load and the next step's tile is decoded into the other buffer.
  auto step_staged = [&](int64_t st, bool first_half, bool more) {
    u32x4v xv[8];
    uint64_t cn = 0;
    if (more) {
      fetch_x(xv, st + 1);
      cn = fetch_c(st + 2 <= s_end ? st + 2 : s_end);
    }
    // keeps those loads here, a whole step ahead of their use
    asm volatile("" ::: "memory");
    const char* at = As_ + wave * (64 * 128);
    const char* bt = Bs[(st - s0) & 1];
    u32x4v a[4], b[4];
    if (first_half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4v*>(&at[tall_off(16 * i + orow, ochk)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4v*>(&bt[tall_off(16 * j + orow, ochk)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_lp<DT>(a[i], b[j], acc[i][j]);
    }
    if (more) {
      decode(cr, (int)((st + 1 - s0) & 1));
      cr = cn;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const u32x4v*>(&at[tall_off(16 * i + orow, 4 + ochk)]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const u32x4v*>(&bt[tall_off(16 * j + orow, 4 + ochk)]);
    // this wave's next x_rot tile, after its last read of this one (a wave's
    // LDS accesses complete in order)
    if (more) stage_x(xv);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_lp<DT>(a[i], b[j], acc[i][j]);
    if (more) __syncthreads();
  };
  // The same with the fragments in registers: the same MFMAs on the same
  // operands, in the same order.
  auto step_tiled = [&](int64_t st, bool first_half, bool more) {
    u32x4v xn[4], xh[4];
    uint64_t cn = 0;
    if (more) {
      fetch_half(xn, st + 1, 0);
      cn = fetch_c(st + 2 <= s_end ? st + 2 : s_end);
    }
    asm volatile("" ::: "memory");
    const char* bt = Bs[(st - s0) & 1];
    u32x4v b[4];
    if (first_half) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4v*>(&bt[tall_off(16 * j + orow, ochk)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_lp<DT>(xa[2 * i], b[j], acc[i][j]);
    }
    if (more) {
      fetch_half(xh, st + 1, 1);
      decode(cr, (int)((st + 1 - s0) & 1));
      cr = cn;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const u32x4v*>(&bt[tall_off(16 * j + orow, 4 + ochk)]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_lp<DT>(xa[2 * i + 1], b[j], acc[i][j]);
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xa[2 * i] = xn[i];
        xa[2 * i + 1] = xh[i];
      }
      __syncthreads();
    }
  };
  for (int64_t st = s0; st < s_end; ++st) {
    if constexpr (TILED) step_tiled(st, true, true);
    else step_staged(st, true, true);
  }
  const bool fh = !(half_last && s_end == last);
  if constexpr (TILED) step_tiled(s_end, fh, false);
  else step_staged(s_end, fh, false);

  if constexpr (KS == 2) {
    // the second half's tiles -> LDS (over the x_rot staging, which every
    // wave is done with), then added to the first half's
    float* red = reinterpret_cast<float*>(As_);  // [tile][reg][wave of the half][lane]
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((i * 4 + j) * 4 + r) * 256 + wv * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i][j][r] = acc[i][j][r] + red[((i * 4 + j) * 4 + r) * 256 + wv * 64 + lane];
  }

  // y = round(acc + bias)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + 16 * j + (lane & 15);
    if (n >= N) continue;
    const float bv = bias ? lp_float<DT>(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 64 * wv + 16 * i + 4 * (lane >> 4) + r;
        if (m < M) y[m * N + n] = (uint16_t)lp_bits<DT>(acc[i][j][r] + bv);
      }
  }
}

// Few rows (up to 64): a block owns 16 W' rows (one MFMA column tile) and
// all MT 16-row tiles of x_rot; its four waves take every fourth K step of
// 32 and add their partial tiles in LDS at the end, in a fixed order.
//
// The block's codes (16 rows, contiguous in memory) are first copied into LDS
// in one coalesced sweep: read straight from HBM in the MFMA's order, each
// wave would touch 16 rows 1 row apart per step, a comb of short pieces over
// the whole weight that reopens every DRAM page many times. In LDS each row
// is padded by one dword so that the 16 rows a step reads start in 16
// different banks. x_rot (small,
// shared by every block, L2-resident) goes straight into registers in the
// MFMA layout: lane l reads 16 bytes of row 16 t + l % 16 at K offset
// 8 (l / 16), and the 8 codes of W' row l % 16 at the same offset become its
// B operand through a per-row table of code pairs: entry (a, b) holds the
// two rounded products for codes a then b as one packed dword, so one LDS
// read yields two operand elements. A ring of four K steps keeps the next
// four steps' loads in flight while one is multiplied.
template <int DT, int BITS, bool LSB, int MT, int NTL>
__global__ __launch_bounds__(256) void orbit_linear_lp_small_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const float* __restrict__ norms, int64_t N, OrbitCodebook cb,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  constexpr int L = 1 << BITS;
  // Tables of code pairs (one dword holds both rounded products), except for
  // 4-bit codes in two-tile blocks, whose pair tables would not fit beside
  // the codes: those use 16-bit single values.
  constexpr bool PAIRS = BITS <= 3 || NTL == 1;
  constexpr int P = PAIRS ? L * L : L;  // entries per row
  constexpr int RING = 4;
  constexpr int NR = 16 * NTL;  // W' rows of the block
  extern __shared__ __attribute__((aligned(16))) uint32_t lsm[];
  const int row_bytes = (int)(K * BITS / 8);
  const int row_dw = row_bytes / 4 + 1;       // padded LDS row, dwords
  const int code_words = (NR * row_dw + 3) / 4 * 4;
  uint32_t* codes = lsm;
  uint32_t* ptab = lsm + code_words;
  // the partial tiles reuse the code rows once every wave is done with them
  float* red = reinterpret_cast<float*>(lsm);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * NR;

  // the block's code rows -> LDS (rows past N are left unset: their table
  // entries are zero)
  {
    const int nrows = N - n0 < NR ? (int)(N - n0) : NR;
    const int rw = row_bytes / 4;  // dwords per row (a row is a multiple of 4 bytes)
    const uint32_t* src = reinterpret_cast<const uint32_t*>(packed + n0 * row_bytes);
    for (int c = tid; c < rw; c += 256) {
#pragma unroll
      for (int h = 0; h < NTL; ++h) {
        uint32_t v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = 16 * h + r < nrows ? src[(16 * h + r) * rw + c] : 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) codes[(16 * h + r) * row_dw + c] = v[r];
      }
    }
  }
  // Pair tables of the block's rows (zeros past N). Entry index: the pair's
  // bits as they sit in the stream -- (a << BITS) | b for MSB-first (code a
  // first), a | (b << BITS) for LSB-first.
  uint16_t* stab = reinterpret_cast<uint16_t*>(ptab);
  for (int e = tid; e < NR * P; e += 256) {
    const int r = e / P, pr = e % P;
    const int64_t n = n0 + r;
    const float nl = n < N ? lp_float<DT>(lp_bits<DT>(norms[n])) : 0.0f;
    if constexpr (PAIRS) {
      const int a = LSB ? pr % L : pr / L, b = LSB ? pr / L : pr % L;
      const float wa = lp_float<DT>(lp_bits<DT>(cb.cb[a])) * nl;
      const float wb = lp_float<DT>(lp_bits<DT>(cb.cb[b])) * nl;
      ptab[e] = lp_bits<DT>(wa) | (lp_bits<DT>(wb) << 16);
    } else {
      stab[e] = (uint16_t)lp_bits<DT>(lp_float<DT>(lp_bits<DT>(cb.cb[pr])) * nl);
    }
  }

  const int j = lane >> 4;          // K group of 8 inside a step
  const int nr = lane & 15;         // W' row inside each 16-row tile of the block
  const uint8_t* crow[NTL];
  const uint32_t* tb[NTL];
  const uint16_t* ts[NTL];
#pragma unroll
  for (int h = 0; h < NTL; ++h) {
    crow[h] = reinterpret_cast<const uint8_t*>(codes + (16 * h + nr) * row_dw);
    tb[h] = ptab + (16 * h + nr) * P;
    ts[h] = stab + (16 * h + nr) * P;
  }
  const uint16_t* xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = 16 * t + nr < M ? 16 * t + nr : M - 1;
    xr[t] = x + m * K + 8 * j;
  }
  // This lane's group (group j of a step's four) from the staged row: BITS = 3
  // takes the two dwords its 3 bytes straddle (inside the step's 12 bytes).
  const int glo = (3 * j) >> 2, ghi = glo + 1 < 3 ? glo + 1 : 2, gsh = 8 * ((3 * j) & 3);
  auto group = [&](int h, int s) -> uint32_t {
    const uint8_t* g = crow[h] + s * (4 * BITS);
    if constexpr (BITS == 4) {
      return reinterpret_cast<const uint32_t*>(g)[j];
    } else if constexpr (BITS == 2) {
      return reinterpret_cast<const uint16_t*>(g)[j];
    } else {
      const uint32_t* d = reinterpret_cast<const uint32_t*>(g);
      return __builtin_amdgcn_alignbit(d[ghi], d[glo], gsh) & 0xffffffu;
    }
  };
  // the group's 4 code pairs in stream order -> 4 packed operand dwords
  auto decode = [&](int h, uint32_t g, u32x4v& b) {
    uint32_t w = g;
    if constexpr (!LSB) {
      if constexpr (BITS == 4) w = __builtin_bswap32(g);
      else if constexpr (BITS == 3) w = (g >> 16) | (g & 0xff00u) | ((g & 0xffu) << 16);
      else w = ((g & 0xffu) << 8) | (g >> 8);
    }
    if constexpr (PAIRS) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t idx = LSB ? (w >> (2 * BITS * p)) & (P - 1)
                                 : (w >> (BITS * (6 - 2 * p))) & (P - 1);
        b[p] = tb[h][idx];
      }
    } else {
      // 4-bit codes: code e of the group at nibble e (LSB-first) or 7 - e
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e0 = 2 * p, e1 = 2 * p + 1;
        const uint32_t c0 = (w >> (4 * (LSB ? e0 : 7 - e0))) & 15u;
        const uint32_t c1 = (w >> (4 * (LSB ? e1 : 7 - e1))) & 15u;
        b[p] = (uint32_t)ts[h][c0] | ((uint32_t)ts[h][c1] << 16);
      }
    }
  };

  f32x4v acc[MT][NTL];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int h = 0; h < NTL; ++h) acc[t][h] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  const int steps = (int)(K / 32);
  // Wave w takes steps w, w + 4, ... (nw of them, possibly none when K has
  // fewer than four steps); ring slot u holds the x_rot operands of its step
  // i + u. Loads past the wave's last step re-read that step (step 0 for a
  // wave without steps) and are never used.
  const int nw = steps > wave ? (steps - wave + 3) >> 2 : 0;
  const int s_last = nw > 0 ? wave + 4 * (nw - 1) : 0;
  u32x4v ar[RING][MT];
  auto fetch = [&](int u, int i) {
    const int s = i < nw ? wave + 4 * i : s_last;
#pragma unroll
    for (int t = 0; t < MT; ++t) ar[u][t] = *reinterpret_cast<const u32x4v*>(xr[t] + 32 * s);
  };
  auto step = [&](int u, int i) {
#pragma unroll
    for (int h = 0; h < NTL; ++h) {
      u32x4v b;
      decode(h, group(h, wave + 4 * i), b);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t][h] = mfma_lp<DT>(ar[u][t], b, acc[t][h]);
    }
  };
#pragma unroll
  for (int u = 0; u < RING; ++u) fetch(u, u);
  __syncthreads();  // codes and pair tables
  int i = 0;
  for (; i + RING <= nw; i += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      step(u, i + u);
      fetch(u, i + u + RING);
      // keep the refill here, a full ring ahead of its use (the scheduler
      // would otherwise sink every refill to the end of the iteration)
      asm volatile("" ::: "memory");
    }
  }
#pragma unroll
  for (int u = 0; u < RING - 1; ++u)
    if (i + u < nw) step(u, i + u);

  // partial tiles -> LDS (over the code rows, once every wave is done with
  // them); wave-ordered sums; bias; one rounding
  constexpr int TT = MT * NTL;  // output tiles
  __syncthreads();
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int h = 0; h < NTL; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[wave * TT * 256 + ((t * NTL + h) * 4 + r) * 64 + lane] = acc[t][h][r];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    const int v = tid + 256 * q;  // ((t * NTL + h) * 4 + r) * 64 + lane'
    const float sum = ((red[v] + red[TT * 256 + v]) + red[2 * TT * 256 + v]) + red[3 * TT * 256 + v];
    const int ln = v & 63, r = (v >> 6) & 3, th = v >> 8;
    const int t = th / NTL, h = th % NTL;
    const int64_t m = 16 * t + 4 * (ln >> 4) + r;
    const int64_t nn = n0 + 16 * h + (ln & 15);
    if (m < M && nn < N) {
      const float bv = bias ? lp_float<DT>(bias[nn]) : 0.0f;
      y[m * N + nn] = (uint16_t)lp_bits<DT>(sum + bv);
    }
  }
}

// LDS bytes of the small kernel: the block's codes, pair tables, partials.
inline size_t lp_small_lds(int64_t K, int bits, int mt, int ntl) {
  const int64_t row_dw = K * bits / 32 + 1;
  const size_t code_bytes = (size_t)((16 * ntl * row_dw + 3) / 4 * 16);
  const size_t red_bytes = (size_t)4 * mt * ntl * 256 * 4;
  const size_t table = bits <= 3 || ntl == 1 ? (size_t)(1 << (2 * bits)) * 4 : (size_t)(1 << bits) * 2;
  return (code_bytes > red_bytes ? code_bytes : red_bytes) + (size_t)16 * ntl * table;
}

template <int DT, int BITS, bool LSB>
hipError_t launch_lp(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                     const float* norms, int64_t N, const OrbitCodebook& cb, const void* bias,
                     void* y, bool tiled, hipStream_t s) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* bp = static_cast<const uint16_t*>(bias);
  uint16_t* yp = static_cast<uint16_t*>(y);
  // One row band above the few-rows range (65..256 rows) with an even step
  // count: the steps split between two halves of an 8-wave block (the grid
  // then holds N / 64 blocks, fewer than the CUs).
  const int64_t tsteps = (K + 63) / 64;
  const bool split = M > 64 && M <= kTallBM && tsteps % 2 == 0;
  if (tiled) {  // x_rot in the fragment layout: the tall tiles at every M (64 <= K < 2^22)
    const unsigned grid = xcd_grid((N + kTallBN - 1) / kTallBN, (M + kTallBM - 1) / kTallBM);
    if (split)
      orbit_linear_lp_tall_kernel<DT, BITS, LSB, true, 2><<<grid, 512, 0, s>>>(
          xp, M, K, packed, norms, N, cb, bp, yp);
    else
      orbit_linear_lp_tall_kernel<DT, BITS, LSB, true><<<grid, 256, 0, s>>>(
          xp, M, K, packed, norms, N, cb, bp, yp);
    return hipGetLastError();
  }
  const int mt = (int)((M + 15) / 16);
  // Above 32 rows a block takes two 16-row tiles of W' (when they fit in LDS):
  // every block reads all of x_rot, and that read then serves twice the
  // outputs.
  const int ntl = M > TQ_LP_WIDE_MIN && lp_small_lds(K, BITS, mt, 2) <= kLpSmallLds ? 2 : 1;
  if (M <= 64 && lp_small_lds(K, BITS, mt, ntl) <= kLpSmallLds) {
    const dim3 grid((unsigned)((N + 16 * ntl - 1) / (16 * ntl)));
    const size_t shm = lp_small_lds(K, BITS, mt, ntl);
#define TQ_SM(T, H) orbit_linear_lp_small_kernel<DT, BITS, LSB, T, H><<<grid, 256, shm, s>>>( \
    xp, M, K, packed, norms, N, cb, bp, yp)
    if (M <= 16) TQ_SM(1, 1);
    else if (M <= 32) TQ_SM(2, 1);
    else if (ntl == 1) { if (M <= 48) TQ_SM(3, 1); else TQ_SM(4, 1); }
    else if (M <= 48) TQ_SM(3, 2);
    else TQ_SM(4, 2);
#undef TQ_SM
    return hipGetLastError();
  }
  // Tall tiles for every batch above the few-rows range (measured faster
  // than the square tiles from 65 rows on: even a lone row of tiles fills
  // twice as many CUs), unless K is a single half step or so large that the
  // lanes' 32-bit x_rot offsets could overflow.
  if (K >= 64 && K < ((int64_t)1 << 22)) {
    const unsigned grid = xcd_grid((N + kTallBN - 1) / kTallBN, (M + kTallBM - 1) / kTallBM);
    if (split)
      orbit_linear_lp_tall_kernel<DT, BITS, LSB, false, 2><<<grid, 512, 0, s>>>(
          xp, M, K, packed, norms, N, cb, bp, yp);
    else
      orbit_linear_lp_tall_kernel<DT, BITS, LSB, false><<<grid, 256, 0, s>>>(
          xp, M, K, packed, norms, N, cb, bp, yp);
    return hipGetLastError();
  }
  const unsigned grid = xcd_grid((N + kLpBN - 1) / kLpBN, (M + kLpBM - 1) / kLpBM);
  orbit_linear_lp_kernel<DT, BITS, LSB><<<grid, 256, 0, s>>>(xp, M, K, packed, norms, N, cb, bp,
                                                             yp);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_lp_bits(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                          const float* norms, int64_t N, int bits, const OrbitCodebook& cb,
                          int lsb_first, const void* bias, void* y, bool tiled, hipStream_t s) {
#define TQ_LP(B, O) launch_lp<DT, B, O>(x, M, K, packed, norms, N, cb, bias, y, tiled, s)
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
                                  void* y, int tiled, hipStream_t s) {
  if (dt == DT_BF16)
    return launch_lp_bits<DT_BF16>(x, M, K, packed, norms, N, bits, cb, lsb_first, bias, y,
                                   tiled != 0, s);
  return launch_lp_bits<DT_F16>(x, M, K, packed, norms, N, bits, cb, lsb_first, bias, y,
                                tiled != 0, s);
}

}  // namespace tq
