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

// One tile of rows (up to 16). A block owns 16 W' rows and the single
// 16-row tile of x_rot; its four waves take every fourth K step of 32 and add
// their partial tiles in LDS at the end, in a fixed order. The block's 16
// code rows (contiguous in memory) are copied to LDS in one coalesced sweep,
// each row padded by a dword so that the 16 rows a step reads start in
// different banks, next to a per-row table of code pairs: entry (a, b) holds
// the two fp32 products codebook[a] * norm and codebook[b] * norm, so one
// 8-byte LDS read yields two operand values (4-bit codes use a table of
// single products). x_rot (small, shared by every
// block, L2-resident) goes straight into registers, four steps ahead. The K
// order inside a step is permuted (the MFMA sums over it): in the step's e-th
// MFMA, lane l supplies x_rot and W' at column 8 (l / 16) + e, so each lane
// reads 8 consecutive values of one x_rot row and decodes 8 consecutive
// codes of one W' row.
constexpr size_t kFewLds = 64 * 1024;  // LDS ceiling of the one-tile kernel

// Tables: code pairs (two fp32 products, 8 bytes) for 2- and 3-bit codes;
// single products for 4-bit codes, whose 256-pair tables (32 KB a block)
// would leave room for fewer blocks.
constexpr bool few_pairs(int bits) { return bits <= 3; }
inline size_t few_lds(int64_t K, int bits) {  // codes, tables, partials
  const int64_t row_dw = K * bits / 32 + 1;
  const size_t table = few_pairs(bits) ? (size_t)(1 << (2 * bits)) * 8 : (size_t)(1 << bits) * 4;
  return (size_t)((16 * row_dw + 3) / 4 * 16) + 16 * table + (size_t)4 * 256 * 4;
}

template <int BITS, bool LSB>
__global__ __launch_bounds__(256) void orbit_linear_few_kernel(
    const float* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const float* __restrict__ norms, int64_t N, OrbitCodebook cb,
    const float* __restrict__ bias, float* __restrict__ y) {
  constexpr int L = 1 << BITS;
  constexpr bool PAIRS = few_pairs(BITS);
  constexpr int P = PAIRS ? L * L : L;  // table entries per row
  constexpr int RING = 4;
  extern __shared__ __attribute__((aligned(16))) uint32_t lsm[];
  const int row_bytes = (int)(K * BITS / 8);
  const int row_dw = row_bytes / 4 + 1;       // padded LDS row, dwords
  const int code_words = (16 * row_dw + 3) / 4 * 4;
  uint32_t* codes = lsm;
  float2* ptab = reinterpret_cast<float2*>(lsm + code_words);
  float* stab = reinterpret_cast<float*>(lsm + code_words);
  float* red = PAIRS ? reinterpret_cast<float*>(ptab + 16 * P) : stab + 16 * P;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * 16;

  // the block's code rows -> LDS (rows past N are left unset: their table
  // entries are zero)
  {
    const int nrows = N - n0 < 16 ? (int)(N - n0) : 16;
    const int rw = row_bytes / 4;  // dwords per row (a row is a multiple of 4 bytes)
    const uint32_t* src = reinterpret_cast<const uint32_t*>(packed + n0 * row_bytes);
    for (int c = tid; c < rw; c += 256) {
      uint32_t v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = r < nrows ? src[r * rw + c] : 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) codes[r * row_dw + c] = v[r];
    }
  }
  // Pair tables of the block's 16 rows (zeros past N). Entry index: the
  // pair's bits as they sit in the stream -- (a << BITS) | b for MSB-first
  // (code a first), a | (b << BITS) for LSB-first.
  for (int e = tid; e < 16 * P; e += 256) {
    const int r = e / P, pr = e % P;
    const int64_t n = n0 + r;
    const float nl = n < N ? norms[n] : 0.0f;
    if constexpr (PAIRS) {
      const int a = LSB ? pr % L : pr / L, b = LSB ? pr / L : pr % L;
      ptab[e] = make_float2(cb.cb[a] * nl, cb.cb[b] * nl);
    } else {
      stab[e] = cb.cb[pr] * nl;
    }
  }

  const int j = lane >> 4;          // group of 8 columns inside a step
  const int nr = lane & 15;         // W' row inside the block, and x_rot row
  const uint8_t* crow = reinterpret_cast<const uint8_t*>(codes + nr * row_dw);
  const float2* tb = ptab + nr * P;
  const float* ts = stab + nr * P;
  const float* xr = x + (nr < M ? nr : M - 1) * K + 8 * j;  // rows past M: never stored
  // This lane's group of 8 codes (group j of a step's four) from the staged
  // row: BITS = 3 takes the two dwords its 3 bytes straddle.
  const int glo = (3 * j) >> 2, ghi = glo + 1 < 3 ? glo + 1 : 2, gsh = 8 * ((3 * j) & 3);
  auto group = [&](int s) -> uint32_t {
    const uint8_t* g = crow + s * (4 * BITS);
    if constexpr (BITS == 4) {
      return reinterpret_cast<const uint32_t*>(g)[j];
    } else if constexpr (BITS == 2) {
      return reinterpret_cast<const uint16_t*>(g)[j];
    } else {
      const uint32_t* d = reinterpret_cast<const uint32_t*>(g);
      return __builtin_amdgcn_alignbit(d[ghi], d[glo], gsh) & 0xffffffu;
    }
  };
  // the group's 4 code pairs in stream order -> its 8 W' values
  auto decode = [&](uint32_t g, float (&b)[8]) {
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
        const float2 v = tb[idx];
        b[2 * p] = v.x;
        b[2 * p + 1] = v.y;
      }
    } else {
      // 4-bit: code e of the group at nibble e (LSB-first) or 7 - e
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = ts[(w >> (4 * (LSB ? e : 7 - e))) & 15u];
    }
  };

  f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int steps = (int)(K / 32);
  // Wave w takes steps w, w + 4, ... (nw of them, possibly none); ring slot
  // u holds the x_rot values of its step i + u. Loads past the wave's last
  // step re-read that step (step 0 for a wave without steps), never used.
  const int nw = steps > wave ? (steps - wave + 3) >> 2 : 0;
  const int s_last = nw > 0 ? wave + 4 * (nw - 1) : 0;
  f32x4v ar[RING][2];
  auto fetch = [&](int u, int i) {
    const int s = i < nw ? wave + 4 * i : s_last;
    ar[u][0] = *reinterpret_cast<const f32x4v*>(xr + 32 * s);
    ar[u][1] = *reinterpret_cast<const f32x4v*>(xr + 32 * s + 4);
  };
  auto step = [&](int u, int i) {
    float b[8];
    decode(group(wave + 4 * i), b);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[u][e >> 2][e & 3], b[e], acc, 0, 0, 0);
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
      // keep the refill here, a full ring ahead of its use
      asm volatile("" ::: "memory");
    }
  }
#pragma unroll
  for (int u = 0; u < RING - 1; ++u)
    if (i + u < nw) step(u, i + u);

  // partial tiles -> LDS; wave-ordered sums; bias
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave * 256 + r * 64 + lane] = acc[r];
  __syncthreads();
  {
    const int v = tid;  // r * 64 + lane'
    const float sum = ((red[v] + red[256 + v]) + red[512 + v]) + red[768 + v];
    const int ln = v & 63, r = v >> 6;
    const int64_t m = 4 * (ln >> 4) + r;
    const int64_t nn = n0 + (ln & 15);
    if (m < M && nn < N) y[m * N + nn] = sum + (bias ? bias[nn] : 0.0f);
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
  // up to 16 rows: one tile of rows per block, codes staged in LDS with pair
  // tables (while they fit in 64 KB of LDS); up to 256 rows: 16 x 32 tiles
  // with K split over the waves (enough blocks to fill the chip); beyond,
  // 128 x 128 tiles
  if (M <= 16 && few_lds(K, BITS) <= kFewLds) {
    orbit_linear_few_kernel<BITS, LSB><<<(unsigned)((N + 15) / 16), 256, few_lds(K, BITS), s>>>(
        x, M, K, packed, norms, N, cb, bias, y);
    return hipGetLastError();
  }
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
