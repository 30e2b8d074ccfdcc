// OrbitQuant weight-codec kernels for gfx950 -- "zerogpu-sdxlTrainer:
// toolkit/util/orbit_quant.py": rpbh_forward, _quantize_rows,
// _dequantize_rotated, dequantize.
//
// Work mapping. One block of NT = ceil(d / 1024) waves owns one weight row
// at a time; wave w holds the row's elements [1024 w, 1024 w + 1024) as 64
// chunks of 16, one chunk per lane (see lane_chunk for which lane holds
// which). Element j = 16 c + i of chunk c: index bits 0-3 are register bits,
// bits 4-9 chunk bits inside the wave, bits 10-13 the wave (d <= 16384:
// up to 16 waves, a 1024-thread block). FWHT stages run in the order 1, 2,
// 4, ..., h/2: in registers for bits 0-3; across lanes without LDS for bits
// 4-9 (DPP fmac with the lazy lane sign described in tq3.hip for bits 4-7,
// permlane16/32 swaps for bits 8 and 9); across waves through LDS for bits
// 10-13. The row norm's sum of squares follows the same bit order inside
// each h-block (1024-element tile sums meet in LDS and go through the rest
// of the pairwise tree); block sums are then added left to right.
//
// NT = 1..4 are compiled for their exact wave count (256-thread launch
// bounds); NT = 0 takes the wave count from the block size at run time, for
// rows of 4097..16384 elements. Rows of up to 512 elements share a wave in
// all three kernels: 64 / (d / 16) rows side by side.
#include <atomic>

#include "orbit_codes.h"
#include "tq_common.h"
#include "tq_kernels.h"

namespace tq {

namespace {

constexpr int kMaxD = 16384;     // longest row: 16 waves of 1024 elements
constexpr int kMaxBlocks = kMaxD / 32;  // d / h with h >= 32

// Waves of a block: NT, or for NT = 0 the block's own size.
template <int NT>
__device__ __forceinline__ int block_waves() {
  if constexpr (NT > 0) return NT;
  else return (int)(blockDim.x >> 6);
}

// Stage class of a kernel instantiation, from h = d & -d: 0 for h < 1024,
// 1 for h = 1024 (every in-wave stage runs, known at compile time), 2 for
// h > 1024 (also stages across waves, with a second LDS buffer). Class 2
// needs d to be a multiple of 2048: an even wave count (or the run-time one).
inline int stage_class(int log2h) { return log2h < 10 ? 0 : log2h == 10 ? 1 : 2; }

// Sum of squares of a row from its partial sums in LDS: for h <= 1024 one
// value per h-block, added left to right; for h > 1024 one value per
// 1024-element tile, combined by the pairwise tree inside each block (tiles
// 2k and 2k + 1 first) before the block sums are added left to right.
template <int TPB>
__device__ __forceinline__ float tiles_then_blocks(const float* bsum, int nblk) {
  float total = 0.0f;
  for (int bi = 0; bi < nblk; ++bi) {
    float t[TPB];
#pragma unroll
    for (int k = 0; k < TPB; ++k) t[k] = bsum[bi * TPB + k];
#pragma unroll
    for (int w = 1; w < TPB; w *= 2)
#pragma unroll
      for (int k = 0; k < TPB; k += 2 * w) t[k] = t[k] + t[k + w];
    total = bi == 0 ? t[0] : total + t[0];
  }
  return total;
}
template <bool SPAN>
__device__ __forceinline__ float row_sumsq(const float* bsum, int log2h, int nblk) {
  if (!SPAN || log2h <= 10) {
    float total = bsum[0];
    for (int bi = 1; bi < nblk; ++bi) total = total + bsum[bi];
    return total;
  }
  // tiles per block (2..16) as a compile-time count: the tree is straight
  // adds instead of sixteen guarded ones per block
  switch (log2h - 10) {
    case 1: return tiles_then_blocks<2>(bsum, nblk);
    case 2: return tiles_then_blocks<4>(bsum, nblk);
    case 3: return tiles_then_blocks<8>(bsum, nblk);
    default: return tiles_then_blocks<16>(bsum, nblk);
  }
}
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Chunk position (within its wave's 64 chunks) held by physical lane l.
// The register-only cross-lane exchanges pair lane l with l ^ 1 and l ^ 2
// (DPP quad_perm), l ^ 7 (row_half_mirror), l ^ 15 (row_mirror), l ^ 16 and
// l ^ 32 (permlane16/32 swap). Lane l holds chunk L(l) for the GF(2)-linear
// L that maps 1, 2, 7, 15, 16, 32 to 1, 2, 4, 8, 16, 32, so each of those
// exchanges pairs exactly the chunks whose indices differ in one bit.
__device__ __forceinline__ int lane_chunk(int l) {
  return (l & 0x33) ^ ((l & 4) ? 7 : 0) ^ ((l & 8) ? 12 : 0);
}

// DPP controls of the exchanges on chunk bits 0..3.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane ^ 7
constexpr int kDppMirror = 0x140;      // row_mirror: lane ^ 15

// v + (the value of the lane holding the chunk that differs in bit S):
// DPP for bits 0..3, ds_swizzle (lane ^ 16 inside 32) and ds_bpermute
// (lane ^ 32) for bits 4 and 5. (A permlane swap of a value with itself is
// not used here: hipcc folds the pair of results into one.)
template <int S>
__device__ __forceinline__ float lane_sum(float v) {
  const int iv = __builtin_bit_cast(int, v);
  int o;
  if constexpr (S < 4) {
    constexpr int ctrl = S == 0 ? kDppXor1 : S == 1 ? kDppXor2 : S == 2 ? kDppHalfMirror : kDppMirror;
    o = __builtin_amdgcn_mov_dpp(iv, ctrl, 0xF, 0xF, false);
  } else if constexpr (S == 4) {
    o = __builtin_amdgcn_ds_swizzle(iv, (16 << 10) | 0x1F);
  } else {
    o = __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2, iv);
  }
  return v + __builtin_bit_cast(float, o);
}

// Rounding of fp32 values to the activation format (RD = DT_BF16 or DT_F16;
// DT_F32: none), nearest even, back in fp32 registers. Torch evaluates each
// elementwise operation on bf16 / fp16 tensors in fp32 and rounds the result
// to the tensor's format; the rotation of such activations repeats that
// after every butterfly stage and after the scaling. The rounding is odd
// (round(-v) = -round(v)), so it commutes with the lazy lane sign.
template <int RD>
__device__ __forceinline__ void round_pair(float& a, float& b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  if constexpr (RD == DT_BF16) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
    a = as_f(w << 16);
    b = as_f(w & 0xffff0000u);
  } else if constexpr (RD == DT_F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const f2 r = __builtin_convertvector(__builtin_convertvector(v, h2), f2);
    a = r[0];
    b = r[1];
  }
}
template <int RD>
__device__ __forceinline__ void round16(float (&y)[16]) {
  if constexpr (RD != DT_F32) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) round_pair<RD>(y[i], y[i + 1]);
  }
}

// Butterflies on chunk bit 4 or 5 for 16 registers, exact signs: a swap
// gives a lower-row lane (own, partner) of register a and an upper-row lane
// (partner, own) of register b; sum and difference are then the lower
// result of a / upper result of b where they are, and a second swap returns
// the other two to the lanes that own them.
template <int S, int RD = DT_F32>
__device__ __forceinline__ void swap_stage(float (&y)[16]) {
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t a = as_u(y[i]), b = as_u(y[i + 1]);
    const auto p = S == 4 ? __builtin_amdgcn_permlane16_swap(a, b, false, false)
                          : __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const float lo = as_f(p[0]), hi = as_f(p[1]);
    float fs = lo + hi, fd = lo - hi;
    round_pair<RD>(fs, fd);
    const uint32_t sm = as_u(fs), df = as_u(fd);
    const auto r = S == 4 ? __builtin_amdgcn_permlane16_swap(sm, df, false, false)
                          : __builtin_amdgcn_permlane32_swap(sm, df, false, false);
    y[i] = as_f(r[0]);
    y[i + 1] = as_f(r[1]);
  }
}

// Per-lane constants of the cross-lane stages: on chunk bits 0..3 the lane
// holding the upper chunk of a pair computes own - partner = -(a - b), and
// the sign is applied once at the end (sigma); bits 4, 5 use exact signs.
struct LaneCx {
  float c[4];
  float sigma;
};
__device__ __forceinline__ LaneCx lane_cx(int lc, int log2h) {
  LaneCx x;
#pragma unroll
  for (int k = 0; k < 4; ++k) x.c[k] = ((lc >> k) & 1) ? -1.0f : 1.0f;
  const int lazy = log2h - 4 < 4 ? log2h - 4 : 4;  // chunk bits inside a block, up to 4
  x.sigma = (__builtin_popcount(lc & ((1 << lazy) - 1)) & 1) ? -1.0f : 1.0f;
  return x;
}

// Full FWHT stage sequence for one wave's 64 x 16 elements in blocks of
// h = 2^log2h (32 <= h <= 1024 inside the wave), without the final scaling
// and with the lazy sign sigma still to apply. FULL: h >= 1024, every
// in-wave stage runs (known at compile time, so no stage is a branch).
// RD: the format every stage's results are rounded to (DT_F32: none).
template <bool FULL, int RD = DT_F32>
__device__ __forceinline__ void fwht_rows(float (&y)[16], int log2h, const LaneCx& cx) {
#pragma unroll
  for (int h = 1; h < 16; h *= 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    round16<RD>(y);
  }
  const int lb = FULL ? 6 : log2h - 4;  // chunk bits inside a block
  if (lb > 0) { TQ_DPP_FMAC16("quad_perm:[1,0,3,2]", cx.c[0], y); round16<RD>(y); }
  if (lb > 1) { TQ_DPP_FMAC16("quad_perm:[2,3,0,1]", cx.c[1], y); round16<RD>(y); }
  if (lb > 2) { TQ_DPP_FMAC16("row_half_mirror", cx.c[2], y); round16<RD>(y); }
  if (lb > 3) { TQ_DPP_FMAC16("row_mirror", cx.c[3], y); round16<RD>(y); }
  if (lb > 4) swap_stage<4, RD>(y);
  if (lb > 5) swap_stage<5, RD>(y);
}

// FWHT stages on the wave bits of a block longer than 1024 (index bits 10 ..
// log2h - 1, up to 4 of them), through LDS. Two bits at a time where two
// remain: each wave writes its values once, and after one barrier reads the
// three waves that differ from it in those bits and forms the two stages
// itself, in their order (bit 10 + b first), with the roundings of the staged
// form: with x0, x1 this wave's two bits and v[x1', x0'] the four waves'
// values, s[x1'] = v[x1', 0] +- v[x1', 1] (- where x0 = 1), then
// s[0] +- s[1] (- where x1 = 1). A lone last bit takes one partner. Every
// sum and difference is an fma with an exact +-1 factor, so it rounds as the
// plain add or subtract does (the operands commute). The lazy lane sign is
// the same in every wave at a given lane, so it passes through unchanged.
// The first exchange uses xa, which nobody reads outside these stages; a
// second one (5 or more wave bits in all: 8192 and 16384) uses xb, the
// staged row, which the first exchange's barrier has made free. The caller
// keeps the barrier that orders its next use of xb after these reads.
// The buffers hold quarter k of chunk c (4 values) at float (k nch + c) 4,
// nch = d / 16 chunks in the row: a wave's 64 lanes write and read 1 KB
// runs without bank conflicts (chunk-major, each lane's 64 bytes in a row,
// put lanes 4 apart on the same banks).
// NT: the block's wave count (0: 5..16), which bounds the wave bits.
template <int NT, int RD = DT_F32>
__device__ __forceinline__ void span_stages(float (&y)[16], float* xa, float* xb, int c, int wave,
                                            int log2h, int nch_rt) {
  constexpr int kMaxBits = NT == 0 ? 4 : NT == 4 ? 2 : 1;
  // a row with blocks over 1024 fills its waves: 64 NT chunks (constant
  // offsets for the exact wave counts)
  const int nch = NT > 0 ? 64 * NT : nch_rt;
  const int nb = log2h - 10;
  float* buf = xa;
  for (int b = 0; b < nb; buf = xb) {
    f32x4_t* q4 = reinterpret_cast<f32x4_t*>(buf);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      q4[k * nch + c] = f32x4_t{y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]};
    __syncthreads();
    const int h0 = 64 << b;  // chunk distance of wave bit b
    const float c0 = ((wave >> b) & 1) ? -1.0f : 1.0f;
    const f32x4_t* p1 = q4 + (c ^ h0);
    if (kMaxBits >= 2 && nb - b >= 2) {
      const float c1 = ((wave >> (b + 1)) & 1) ? -1.0f : 1.0f;
      const f32x4_t* p2 = q4 + (c ^ (2 * h0));
      const f32x4_t* p3 = q4 + (c ^ (3 * h0));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4_t o1 = p1[k * nch], o2 = p2[k * nch], o3 = p3[k * nch];
        float so[4], sx[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          so[e] = __builtin_fmaf(y[4 * k + e], c0, o1[e]);  // s[x1]
          sx[e] = __builtin_fmaf(o2[e], c0, o3[e]);         // s[1 - x1]
        }
        round_pair<RD>(so[0], so[1]);
        round_pair<RD>(so[2], so[3]);
        round_pair<RD>(sx[0], sx[1]);
        round_pair<RD>(sx[2], sx[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[4 * k + e] = __builtin_fmaf(so[e], c1, sx[e]);
        // one group's three partner reads in flight at a time: hoisting all
        // twelve costs 40 VGPRs (a lost wave per SIMD, or spills)
        __builtin_amdgcn_sched_barrier(0);
      }
      b += 2;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4_t o1 = p1[k * nch];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[4 * k + e] = __builtin_fmaf(y[4 * k + e], c0, o1[e]);
      }
      b += 1;
    }
    round16<RD>(y);
  }
}

// --------------------------------------------------------------- packing ---

// Code of u = number of codebook edges strictly below u, as BITS wave masks,
// most significant bit first.
//
// Any codebook: T_k = (e_k < u) for the 2^BITS - 1 ascending edges is a
// thermometer code, so bit j of the count is the XOR of T_k over the k that
// are multiples of 2^j (k = 1, 2, ...).
// Symmetric codebook (edges -e_H .. -e_1, 0, e_1 .. e_H, H = 2^(BITS-1) - 1):
// as for the TQ3 index, R = bits(u) rotated left by one compares with
// 2 * bits(e_i) as "|u| > e_i" for u >= 0 and "|u| >= e_i" for u < 0; with
// c = #{R > 2 bits(e_i)} the code is c ^ (u > 0 ? H + 1 : H): the top bit is
// (u > 0) and bit j below it is c_j xor (u <= 0).
template <int BITS, bool SYM>
__device__ __forceinline__ void code_masks(float u, const OrbitCodebook& cb,
                                           uint64_t (&m)[BITS]) {
  constexpr int L = 1 << BITS;
  if constexpr (SYM) {
    constexpr int H = L / 2 - 1;
    const uint32_t ub = as_u(u);
    const uint32_t r = __builtin_amdgcn_alignbit(ub, ub, 31);
    uint64_t T[H + 1];
#pragma unroll
    for (int i = 1; i <= H; ++i) T[i] = __builtin_amdgcn_ballot_w64(r > cb.th[i - 1]);
    const uint64_t pos = __builtin_amdgcn_ballot_w64(u > 0.0f);
    m[0] = pos;
#pragma unroll
    for (int j = 0; j < BITS - 1; ++j) {
      uint64_t x = ~pos;
#pragma unroll
      for (int i = 1 << j; i <= H; i += 1 << j) x ^= T[i];
      m[BITS - 1 - j] = x;
    }
  } else {
    uint64_t T[L];
#pragma unroll
    for (int k = 1; k < L; ++k) T[k] = __builtin_amdgcn_ballot_w64(cb.edge[k - 1] < u);
#pragma unroll
    for (int j = 0; j < BITS; ++j) {
      uint64_t x = 0;
#pragma unroll
      for (int k = 1 << j; k < L; k += 1 << j) x ^= T[k];
      m[BITS - 1 - j] = x;
    }
  }
}

__device__ __forceinline__ uint32_t bswap24(uint32_t w) {
  return (w >> 16) | (w & 0xff00u) | ((w & 0xffu) << 16);
}

// Codes of 16 consecutive elements -> their 2*BITS bytes of the packed row,
// as a little-endian 64-bit value (byte k of the result = stream byte k of
// this chunk). Bits enter 32-bit words through add-with-carry in stream order
// for MSB-first words and in reverse for LSB-first ones.
template <int BITS, bool LSB, bool SYM>
__device__ __forceinline__ uint64_t pack16(const float (&u)[16], const OrbitCodebook& cb) {
  constexpr int NW = BITS == 2 ? 1 : 2;  // 32-bit words (3 bits: 24-bit words)
  constexpr int PER = 16 / NW;           // codes per word
  uint32_t word[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t acc = 0;
#pragma unroll
    for (int s = 0; s < PER; ++s) {
      const int i = LSB ? w * PER + (PER - 1 - s) : w * PER + s;
      uint64_t m[BITS];
      code_masks<BITS, SYM>(u[i], cb, m);
#pragma unroll
      for (int b = 0; b < BITS; ++b) acc = shift_in(acc, m[b]);
    }
    word[w] = acc;
  }
  if constexpr (LSB) {
    // code i's bit t is stream bit BITS*i + t: the words are already in order
    if constexpr (BITS == 2) return word[0];
    else if constexpr (BITS == 3) return (uint64_t)word[0] | ((uint64_t)word[1] << 24);
    else return (uint64_t)word[0] | ((uint64_t)word[1] << 32);
  } else {
    // each word is big-endian: code 0 in its most significant bits
    if constexpr (BITS == 2) return __builtin_bswap32(word[0]);
    else if constexpr (BITS == 3)
      return (uint64_t)bswap24(word[0]) | ((uint64_t)bswap24(word[1]) << 24);
    else
      return (uint64_t)__builtin_bswap32(word[0]) | ((uint64_t)__builtin_bswap32(word[1]) << 32);
  }
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, uint64_t acc) {
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)acc;
  } else if constexpr (BITS == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2((uint32_t)acc, (uint32_t)(acc >> 32));
  } else {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
    q[0] = (uint16_t)acc;
    q[1] = (uint16_t)(acc >> 16);
    q[2] = (uint16_t)(acc >> 32);
  }
}

// Sign bit (bit 31) of the int8 +-1 value k of a little-endian word.
__device__ __forceinline__ uint32_t sign_of(uint32_t w, int k) {
  return (w << (24 - 8 * k)) & 0x80000000u;
}

// ------------------------------------------------------------- quantize ---

// One block of NT waves per row (NT = ceil(d / 1024)): wave w holds the row's
// elements [1024 w, 1024 w + 1024), lane l the 16 consecutive ones from
// 16 (l + 64 w). The row is staged in LDS once per block and gathered through
// the permutation, whose byte offsets (and the signs) each lane keeps in
// registers for the whole kernel; the next row's loads are in flight while
// the current one is processed.
//
// ROT: stop after the rotation and store it (rpbh_forward of activation rows,
// the forward's first step) to xrot instead of quantizing. DT: the format of
// the rows read and, with ROT, of xrot; for bf16 / fp16 every stage rounds
// to that format as the page's forward does on such activations.
// TOUT (ROT, bf16 / fp16): xrot in the MFMA fragment layout of the tiled
// linear layer: rows padded to a multiple of 16 (the pad rows zero); the
// 16 x 32 block of row tile t and column chunk kc is 1 KB at
// (t * d / 32 + kc) * 1024, lane l's 16 bytes at l * 16 holding row
// 16 t + l % 16, columns 32 kc + 8 (l / 16) .. + 7.
// SB: rebuild the sign masks from their packed bits on every row (two
// operations per element) instead of keeping 16 mask registers across rows:
// 15 VGPRs fewer, which gives blocks of 5 and 6 waves a third block per CU
// and keeps the kernels with blocks over 1024 free of spills.
template <int BITS, bool LSB, int NT, int HC, bool ROT = false, int DT = DT_F32,
          bool SYM = true, bool TOUT = false, bool MR = false, bool SB = false>
__global__ __launch_bounds__(NT == 0 ? 1024 : 256) void orbit_quantize_kernel(
    const void* __restrict__ W, int64_t rows, int d, int log2h, float kh,
    const int32_t* __restrict__ perm, const int8_t* __restrict__ signs, OrbitCodebook cb,
    uint8_t* __restrict__ packed, float* __restrict__ norms, void* __restrict__ xrot) {
  static_assert(ROT || DT == DT_F32, "the weight codec reads fp32 rows");
  static_assert(!TOUT || (ROT && DT != DT_F32), "the tiled form holds bf16 / fp16 rotations");
  extern __shared__ float lds[];
  // MR (one-wave blocks, rows of up to 512 elements): the wave takes
  // R = 64 / (d / 16) rows at a time, side by side (lane chunk lc -> row
  // lc / C, chunk lc % C, C = d / 16). A row's chunk count is a multiple of
  // its h-block's, so every butterfly and block sum stays inside its row.
  static_assert(!MR || (NT == 1 && HC == 0), "several rows per wave only for short rows");
  const int C = d >> 4;
  const int R = MR ? 64 / C : 1;
  float* rowbuf = lds;              // the staged rows; later the cross-wave exchange
  float* bsum = lds + R * d;        // block (or, for h > 1024, tile) sums of squares
  float* xbuf = lds + d + kMaxBlocks;  // h > 1024 (R = 1): the wave-bit stages' exchange
  const int nwaves = block_waves<NT>();
  const int NTHR = 64 * nwaves;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = lane_chunk(lane);
  const int grow = MR ? lc / C : 0;                 // row within the block's group
  const int c = MR ? lc - grow * C : lc + 64 * wave;  // chunk of 16 elements in the row
  const bool lane_ok = grow < R && c < C;
  const int cw = MR ? lc : c;                       // chunk within the staged rows
  const int nblk = d >> log2h;
  constexpr bool FULL = HC > 0, SPAN = HC == 2;
  static_assert(!SPAN || NT == 0 || NT % 2 == 0, "h > 1024 needs an even wave count");
  const int lb = FULL ? 6 : (log2h - 4 < 6 ? log2h - 4 : 6);
  const LaneCx cx = lane_cx(lc, log2h);
  const float ksig = kh * cx.sigma;
  const int64_t row_bytes = (int64_t)d * BITS / 8;
  const float eps = (float)1e-10;
  constexpr int ES = DT == DT_F32 ? 4 : 2;  // bytes per element of a row
  constexpr int KL = ES;                     // 16-byte loads per thread (d <= 1024 NT)
  const int nl = d * ES / 16;               // 16-byte pieces per row
  const int nlg = R * nl;                   // ... per group of rows

  // Byte offsets into the staged row and sign masks of this lane's elements.
  uint32_t poff[16], sbits = 0;  // sbits: bit i set when signs_j = -1 for element i
  {
    // lanes past the rows read row 0's chunk 0 and never use it
    const int cc = lane_ok ? c : 0;
    const uint32_t roff = lane_ok ? 4u * (uint32_t)(grow * d) : 0u;
    const u32x4* pp = reinterpret_cast<const u32x4*>(perm + 16 * cc);
    const u32x4 sv = *reinterpret_cast<const u32x4*>(signs + 16 * cc);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 p = pp[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        poff[4 * k + e] = roff + 4u * p[e];
        sbits |= (sign_of(sv[k], e) >> 31) << (4 * k + e);
      }
    }
  }

  // The next row, <= KL x 16 bytes per thread (d <= 1024 NT). Loads past the
  // row's end re-read its last 16 bytes (kept unconditional so the values
  // stay in registers); only those below the end reach LDS, widened to fp32.
  const char* Wb = static_cast<const char*>(W);
  const int64_t row_in = (int64_t)d * ES;
  u32x4 pre[KL];
  int frow[KL], fcol[KL];  // piece k of this thread: row of the group, piece in the row
#pragma unroll
  for (int k = 0; k < KL; ++k) {
    const int f = tid + NTHR * k < nlg ? tid + NTHR * k : nlg - 1;
    frow[k] = MR ? f / nl : 0;
    fcol[k] = MR ? f - frow[k] * nl : f;
  }
  // TOUT also covers the pad rows (their loads re-read valid rows)
  const int64_t rows_loop = TOUT ? (rows + 15) / 16 * 16 : rows;
  const int64_t ngroups = (rows_loop + R - 1) / R;
  auto load_group = [&](int64_t gg) {
    if constexpr (MR) {
#pragma unroll
      for (int k = 0; k < KL; ++k) {
        int64_t rr = gg * R + frow[k];
        rr = rr < rows ? rr : rows - 1;
        pre[k] = reinterpret_cast<const u32x4*>(Wb + rr * row_in)[fcol[k]];
      }
    } else {  // gg < rows: one row, pieces past its end re-read its last one
      const u32x4* src = reinterpret_cast<const u32x4*>(Wb + (gg < rows ? gg : rows - 1) * row_in);
#pragma unroll
      for (int k = 0; k < KL; ++k) pre[k] = src[fcol[k]];
    }
  };
  int64_t g = blockIdx.x;
  load_group(g < ngroups ? g : 0);
  for (; g < ngroups; g += gridDim.x) {
    const int64_t r = g * R + grow;  // this lane's row
    // (one row per block: every iteration's row is in range)
    const bool act = MR ? lane_ok && r < rows_loop : lane_ok;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int f = tid + NTHR * k;
      if (f < nlg) {
        if constexpr (DT == DT_F32) {
          reinterpret_cast<u32x4*>(rowbuf)[f] = pre[k];
        } else {
          u32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x4& src = pre[k];
            const uint32_t w = src[e];
            float f0, f1;
            if constexpr (DT == DT_BF16) {
              f0 = as_f(w << 16);
              f1 = as_f(w & 0xffff0000u);
            } else {
              f0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
              f1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
            }
            if (e < 2) { lo[2 * e] = as_u(f0); lo[2 * e + 1] = as_u(f1); }
            else { hi[2 * e - 4] = as_u(f0); hi[2 * e - 3] = as_u(f1); }
          }
          reinterpret_cast<u32x4*>(rowbuf)[2 * f] = lo;
          reinterpret_cast<u32x4*>(rowbuf)[2 * f + 1] = hi;
        }
      }
    }
    __syncthreads();
    load_group(g + gridDim.x < ngroups ? g + gridDim.x : 0);

    // y_j = W[perm_j] * signs_j. Lanes past the row (d not a multiple of
    // 1024) gather chunk 0 too: their chunks form whole h-blocks of their
    // own, so no butterfly or block sum mixes them with the row, and nothing
    // of theirs is stored. Unconditional reads are all in flight at once.
    float y[16];
    const char* rb = reinterpret_cast<const char*>(rowbuf);
    uint32_t sb = sbits;
    // SB: the empty asm makes sb new on every row, so the masks are built
    // here (a shift and one three-input bit operation with the scalar mask)
    if constexpr (SB) asm volatile("" : "+v"(sb));
    const uint32_t sgn = SB ? __builtin_amdgcn_readfirstlane(0x80000000u) : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      y[i] = as_f(*reinterpret_cast<const uint32_t*>(rb + poff[i]) ^ ((sb << (31 - i)) & sgn));

    // Butterflies inside the wave (index bits 0..9), then across waves
    // through LDS for blocks longer than 1024 (bits 10, 11): the lower tile
    // takes a + b, the upper b' - a' = a - b with the same lazy lane sign.
    constexpr int RD = ROT ? DT : DT_F32;
    fwht_rows<FULL, RD>(y, log2h, cx);
    if (SPAN) span_stages<NT, RD>(y, xbuf, rowbuf, c, wave, log2h, C);
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = y[i] * ksig;
    round16<RD>(y);
    if constexpr (ROT) {
      // An exact zero here stands for a cancellation a - a or a + (-a), which
      // IEEE arithmetic returns as +0; the lazy lane sign can leave -0 in its
      // place. Adding +0 restores +0 (and changes nothing else), so rows
      // without zero entries match the page's rotation bit for bit.
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = y[i] + 0.0f;
      if (act) {
        if constexpr (DT == DT_F32) {
          f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(xrot) + r * d + 16 * c);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            dst[k] = f32x4_t{y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]};
        } else {
          // the values are already in the format: the narrowing is exact
          uint32_t w[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if constexpr (DT == DT_BF16) {
              w[k] = (as_u(y[2 * k]) >> 16) | (as_u(y[2 * k + 1]) & 0xffff0000u);
            } else {
              w[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[2 * k]) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[2 * k + 1]) << 16);
            }
          }
          if constexpr (TOUT) {
            // columns 16 c .. 16 c + 15: chunk c / 2, lane groups 2 (c % 2) and + 1
            const bool pad = r >= rows;
            char* frag = static_cast<char*>(xrot) + ((r >> 4) * (d >> 5) + (c >> 1)) * 1024;
            const int l0 = (int)(r & 15) + 32 * (c & 1);
            *reinterpret_cast<u32x4*>(frag + 16 * l0) =
                pad ? u32x4{0u, 0u, 0u, 0u} : u32x4{w[0], w[1], w[2], w[3]};
            *reinterpret_cast<u32x4*>(frag + 16 * (l0 + 16)) =
                pad ? u32x4{0u, 0u, 0u, 0u} : u32x4{w[4], w[5], w[6], w[7]};
          } else {
            u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(xrot) + r * d + 16 * c);
            dst[0] = u32x4{w[0], w[1], w[2], w[3]};
            dst[1] = u32x4{w[4], w[5], w[6], w[7]};
          }
        }
      }
      __syncthreads();  // the row buffer is free for the next row
      continue;
    }

    // Sum of squares: bits 0-3 in registers, then the lane bits inside the
    // block; block (h <= 1024) or tile (h > 1024) sums meet in LDS.
    float s[16];
    float amin = __builtin_fabsf(y[0]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = y[i] * y[i];
      if (i > 0) amin = __builtin_fminf(amin, __builtin_fabsf(y[i]));
    }
#pragma unroll
    for (int w = 1; w < 16; w *= 2)
#pragma unroll
      for (int i = 0; i < 16; i += 2 * w) s[i] = s[i] + s[i + w];
    float part = s[0];
    if (lb > 0) part = lane_sum<0>(part);
    if (lb > 1) part = lane_sum<1>(part);
    if (lb > 2) part = lane_sum<2>(part);
    if (lb > 3) part = lane_sum<3>(part);
    if (lb > 4) part = lane_sum<4>(part);
    if (lb > 5) part = lane_sum<5>(part);
    if (act && (cw & ((1 << lb) - 1)) == 0) bsum[cw >> lb] = part;  // one writer per block/tile
    __syncthreads();
    const float norm =
        __builtin_sqrtf(row_sumsq<SPAN>(MR ? bsum + (lane_ok ? grow : 0) * nblk : bsum, log2h, nblk));
    const float denom = norm + eps;

    // u = y / denom, correctly rounded: shared reciprocal while every nonzero
    // |y| >= denom * 2^-60 (denom >= 1e-10 always), plain division otherwise.
    if (amin >= denom * 0x1p-60f && denom <= 0x1p100f) {
      const Recip rd = make_recip(denom);
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = div_rn(y[i], rd);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = y[i] / denom;
    }

    // Codes and packing (SYM: the codebook is mirror-symmetric).
    const uint64_t bytes = pack16<BITS, LSB, SYM>(y, cb);
    if (act) store_codes<BITS>(packed + r * row_bytes + 2 * BITS * c, bytes);
    if (MR ? act && c == 0 : tid == 0) norms[r] = norm;
  }
}

// ----------------------------------------------------------- dequantize ---

// 16 bytes of outputs (EPS = 4 fp32 or 8 bf16/fp16 values) at element j0.
template <int DT>
__device__ __forceinline__ void store_group(void* out, int64_t j0, const float* v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (DT == DT_F32) {
    *reinterpret_cast<u32x4*>(static_cast<float*>(out) + j0) =
        u32x4{as_u(v[0]), as_u(v[1]), as_u(v[2]), as_u(v[3])};
  } else {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      typedef float f2 __attribute__((ext_vector_type(2)));
      const f2 pr = {v[2 * k], v[2 * k + 1]};
      if constexpr (DT == DT_BF16) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, b2));
      } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, h2));
      }
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + j0) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// One block of NT waves per row, wave w owning the row's elements
// [1024 w, 1024 w + 1024). Codes are read in stream order (lane l: the 16
// from 16 (l + 64 w)); outputs leave in coalesced 16-byte groups (lane l:
// elements 1024 w + EPS l + 64 EPS k .. + EPS - 1, EPS values per 16 bytes),
// re-read from LDS in that order -- through the inverse permutation when
// the rotation is undone. The next row's codes and norm are loaded while the
// current row is processed.
template <int BITS, bool LSB, int DT, int NT, int HC, bool MR = false>
__global__ __launch_bounds__(NT == 0 ? 1024 : 256) void orbit_dequantize_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ norms, int64_t rows, int d,
    int log2h, float kh, const int32_t* __restrict__ inv_perm,
    const int8_t* __restrict__ signs, OrbitCodebook cb, int rotated_only,
    void* __restrict__ out) {
  extern __shared__ float lds[];
  // MR: as in the quantize kernel, a one-wave block takes R = 64 / (d / 16)
  // short rows side by side (lane chunk lc -> row lc / C, chunk lc % C). The
  // R rows are consecutive in memory, so the staged tile is stored as one
  // flat run of R d elements; each row has its own norm, so the lanes
  // multiply the codebook value by it (the same single rounding as a table
  // of products).
  static_assert(!MR || (NT == 1 && HC == 0), "several rows per wave only for short rows");
  const int C = d >> 4;
  const int R = MR ? 64 / C : 1;
  float* rowbuf = lds;  // R d floats
  constexpr int EPS = DT == DT_F32 ? 4 : 8;
  constexpr int NG = 16 / EPS;  // 16-byte output groups per lane per tile
  constexpr int L = 1 << BITS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // PT: the wave's table holds pairs -- entry e = the stream bits of two
  // consecutive codes a, b (pairs16) holds (cb[a] * norm, cb[b] * norm), the
  // same products as single entries -- so one 8-byte read decodes two
  // elements. For 2-bit codes, and 3-bit ones in blocks of up to 4 waves
  // (64 pairs: 128 floats a wave, inside the block-sum area).
  constexpr bool PT = !MR && (BITS == 2 || (BITS == 3 && NT >= 1 && NT <= 4));
  constexpr int TABF = PT ? 2 << (2 * BITS) : 16;  // floats of one wave's table
  static_assert(TABF * (NT == 0 ? 16 : NT) <= kMaxBlocks, "tables inside the block-sum area");
  float* tab = lds + R * d + TABF * wave;  // this wave's codebook x row norm (MR: codebook)
  const int lc = lane_chunk(lane);
  const int grow = MR ? lc / C : 0;
  const int c = MR ? lc - grow * C : lc + 64 * wave;
  const bool lane_ok = grow < R && c < C;
  const int cw = MR ? lc : c;  // chunk within the staged rows
  const LaneCx cx = lane_cx(lc, log2h);
  const float ksig = kh * cx.sigma;
  const int64_t row_bytes = (int64_t)d * BITS / 8;

  // Output groups of this lane and, when the rotation is undone, the byte
  // offsets of their sources in the staged row(s) and the signs of its chunk.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  int j0[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) j0[k] = 1024 * wave + EPS * lane + 64 * EPS * k;
  // The full path stages the transformed tile quarter-major: quarter q of
  // chunk cw (elements 16 cw + 4 q .. + 3) at float (q nch + cw) 4, nch =
  // R C chunks, so that a wave's 16-byte writes are contiguous (chunk-major,
  // lanes 4 apart would share banks); the gather offsets point there.
  const int nch = R * C;
  auto staged = [&](uint32_t pos) {  // float index of staged element pos
    return ((((pos >> 2) & 3u) * (uint32_t)nch + (pos >> 4)) << 2) + (pos & 3u);
  };
  uint32_t ioff[16], smask[16];
  if (!rotated_only) {
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      // flat position j0 -> row j0 / d, column j0 % d (a group never straddles rows)
      const int jr = MR ? j0[k] / d : 0;
      const int jc = j0[k] - jr * d;
      const bool ok = MR ? jr < R : jc < d;
      const u32x4* ip = reinterpret_cast<const u32x4*>(inv_perm + (ok ? jc : 0));
#pragma unroll
      for (int e4 = 0; e4 < EPS / 4; ++e4) {
        const u32x4 p = ip[e4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ioff[EPS * k + 4 * e4 + e] = 4u * staged((uint32_t)((ok ? jr * d : 0) + p[e]));
      }
    }
    const u32x4 sv = *reinterpret_cast<const u32x4*>(signs + 16 * (lane_ok ? c : 0));
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) smask[4 * k + e] = sign_of(sv[k], e);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) ioff[i] = smask[i] = 0;
  }

  const int64_t ngroups = (rows + R - 1) / R;
  int64_t g = blockIdx.x;
  const int cc = lane_ok ? c : 0;
  auto row_of = [&](int64_t gg) {
    const int64_t rr = gg * R + (lane_ok ? grow : 0);
    return rr < rows ? rr : rows - 1;
  };
  uint64_t ncodes = load_codes<BITS>(packed + row_of(g < ngroups ? g : 0) * row_bytes + 2 * BITS * cc);
  float nnorm = norms[row_of(g < ngroups ? g : 0)];
  if (MR && lane < L) tab[lane] = cb.cb[lane];
  for (; g < ngroups; g += gridDim.x) {
    const int64_t r = g * R;  // the group's first row
    const int64_t nflat = (rows - r < R ? rows - r : R) * d;  // its elements
    const bool act = lane_ok && r + grow < rows;
    const uint64_t codes = ncodes;
    const float norm = nnorm;
    {
      const int64_t gn = g + gridDim.x < ngroups ? g + gridDim.x : g;
      ncodes = load_codes<BITS>(packed + row_of(gn) * row_bytes + 2 * BITS * cc);
      nnorm = norms[row_of(gn)];
    }
    float w[16];
    if constexpr (PT) {
      for (int e = lane; e < L * L; e += 64) {
        const int a = LSB ? e % L : e / L, b = LSB ? e / L : e % L;
        reinterpret_cast<float2*>(tab)[e] = make_float2(cb.cb[a] * norm, cb.cb[b] * norm);
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t pi[8];
      pairs16<BITS, LSB>(codes, pi);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float2 v = reinterpret_cast<const float2*>(tab)[pi[p]];
        w[2 * p] = v.x;
        w[2 * p + 1] = v.y;
      }
    } else {
      if (!MR && lane < L) tab[lane] = cb.cb[lane] * norm;
      __builtin_amdgcn_wave_barrier();
      uint32_t code[16];
      unpack16<BITS, LSB>(codes, code);
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = MR ? tab[code[i]] * norm : tab[code[i]];
    }

    if (rotated_only) {
      // Stage this wave's tile in element order, re-read it in store order.
      if (act) {
        f32x4_t* mine = reinterpret_cast<f32x4_t*>(rowbuf + 16 * cw);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mine[k] = f32x4_t{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < NG; ++k)
        if (j0[k] < nflat) store_group<DT>(out, r * d + j0[k], rowbuf + j0[k]);
      __builtin_amdgcn_wave_barrier();
      continue;
    }

    // Inverse rotation: FWHT per block (across waves through LDS beyond
    // 1024), times h^-1/2 and the lazy lane sign, times signs_j.
    fwht_rows<(HC > 0)>(w, log2h, cx);
    if (HC == 2) span_stages<NT>(w, lds + d + kMaxBlocks, rowbuf, c, wave, log2h, d >> 4);
    __syncthreads();  // the row buffer is free
    if (act) {
      f32x4_t* q4 = reinterpret_cast<f32x4_t*>(rowbuf);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = as_f(as_u(w[4 * k + e] * ksig) ^ smask[4 * k + e]);
        q4[k * nch + cw] = f32x4_t{z[0], z[1], z[2], z[3]};
      }
    }
    __syncthreads();
    // out[j] = z[inv_perm_j], gathered from the staged row.
    const char* rb = reinterpret_cast<const char*>(rowbuf);
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      if (j0[k] >= nflat) continue;
      float o[EPS];
#pragma unroll
      for (int e = 0; e < EPS; ++e) o[e] = *reinterpret_cast<const float*>(rb + ioff[EPS * k + e]);
      store_group<DT>(out, r * d + j0[k], o);
    }
  }
}

// LDS of a block: the row (d <= 1024 NT floats), the block sums (or the
// dequantizer's per-wave tables) and, for h > 1024, a second row-sized buffer
// for the wave-bit stages. The resident-block count is taken once per block
// size at the largest LDS that size can need (35 KB for 4 waves: it then
// matches the register limit of four blocks per CU).
constexpr size_t orbit_lds(int d, bool span) {
  return (size_t)(d + kMaxBlocks + (span ? d : 0)) * sizeof(float);
}
inline int block_threads(int nt_tmpl, int nt) { return 64 * (nt_tmpl == 0 ? nt : nt_tmpl); }
// Rows a one-wave block of the rotation / quantize kernel takes at a time
// when rows are short (up to 512 elements): as many as fit the 64 lanes.
inline int rows_per_group(int d) { return 64 / (d >> 4); }

// Resident blocks per CU of one kernel instantiation, queried once per block
// size (one size for NT = 1..4; one per wave count 5..16 for NT = 0) at the
// largest LDS it takes (d = 1024 x waves). Racing first calls store the same
// value.
template <int NT, typename K>
int resident_cached(std::atomic<int> (&cache)[17], K kernel, int nt, bool span) {
  const int slot = NT == 0 ? nt : 0;
  int v = cache[slot].load(std::memory_order_relaxed);
  if (v == 0) {
    v = resident_blocks_per_cu(kernel, block_threads(NT, nt), orbit_lds(1024 * nt, span));
    cache[slot].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int BITS, bool LSB, int NT, int HC, bool SYM, bool MR = false, bool SB = false>
hipError_t launch_q_sym(const float* W, int64_t rows, int d, int log2h, float kh,
                        const int32_t* perm, const int8_t* signs, const OrbitCodebook& cb,
                        uint8_t* packed, float* norms, int cus, hipStream_t s) {
  if constexpr (NT == 1 && HC == 0 && !MR) {
    if (d <= 512)
      return launch_q_sym<BITS, LSB, NT, HC, SYM, true>(W, rows, d, log2h, kh, perm, signs, cb,
                                                        packed, norms, cus, s);
  }
  const int nt = (d + 1023) >> 10;
  if constexpr (NT == 0 && !SB) {
    // 5- and 6-wave blocks (a third block per CU) and blocks over 1024 (no
    // spills): 3 bits, 37.7 M elements: 65 -> 53 us at d = 5120, 75 -> 62
    // at 5632, 63 -> 59 at 8192, 74 -> 69 at 16384; blocks of 7-16 waves up
    // to 1024 lose 2-6%
    if constexpr (HC == 2)
      return launch_q_sym<BITS, LSB, NT, HC, SYM, MR, true>(W, rows, d, log2h, kh, perm, signs,
                                                            cb, packed, norms, cus, s);
    else if (nt == 5 || nt == 6)
      return launch_q_sym<BITS, LSB, NT, HC, SYM, MR, true>(W, rows, d, log2h, kh, perm, signs,
                                                            cb, packed, norms, cus, s);
  }
  auto kernel = orbit_quantize_kernel<BITS, LSB, NT, HC, false, DT_F32, SYM, false, MR, SB>;
  const int R = MR ? rows_per_group(d) : 1;
  const size_t shm = orbit_lds(R * d, HC == 2);
  static std::atomic<int> cache[17];
  const int per_cu = resident_cached<NT>(cache, kernel, nt, HC == 2);
  // Twice the resident blocks: blocks that start later fall out of step with
  // the first ones, so loads and arithmetic of different blocks overlap
  // (2-4% on the 12288 x 3072 weight against a resident-sized grid).
  const int grid = grid_size((rows + R - 1) / R, cus, per_cu * 2);
  kernel<<<grid, block_threads(NT, nt), shm, s>>>(W, rows, d, log2h, kh, perm, signs, cb, packed,
                                                  norms, nullptr);
  return hipGetLastError();
}

// One packing path per instantiation: with both in one kernel the loop ran
// out of scalar registers and spilled them to VGPR lanes.
template <int BITS, bool LSB, int NT, int HC>
hipError_t launch_q(const float* W, int64_t rows, int d, int log2h, float kh,
                    const int32_t* perm, const int8_t* signs, const OrbitCodebook& cb,
                    uint8_t* packed, float* norms, int cus, hipStream_t s) {
  if (cb.sym)
    return launch_q_sym<BITS, LSB, NT, HC, true>(W, rows, d, log2h, kh, perm, signs, cb, packed,
                                                   norms, cus, s);
  return launch_q_sym<BITS, LSB, NT, HC, false>(W, rows, d, log2h, kh, perm, signs, cb, packed,
                                                  norms, cus, s);
}

// Launch M(NT, HC) for the wave count nt and stage class hc (class 2 only
// for the even and run-time wave counts).
#define TQ_BY_NT_HC(M)                                               \
  switch (nt) {                                                      \
    case 1: return hc == 0 ? M(1, 0) : M(1, 1);                      \
    case 2: return hc == 0 ? M(2, 0) : hc == 1 ? M(2, 1) : M(2, 2);  \
    case 3: return hc == 0 ? M(3, 0) : M(3, 1);                      \
    case 4: return hc == 0 ? M(4, 0) : hc == 1 ? M(4, 1) : M(4, 2);  \
    default: return hc == 0 ? M(0, 0) : hc == 1 ? M(0, 1) : M(0, 2); \
  }

template <int BITS, bool LSB>
hipError_t launch_q_nt(int nt, const float* W, int64_t rows, int d, int log2h, float kh,
                       const int32_t* perm, const int8_t* signs, const OrbitCodebook& cb,
                       uint8_t* packed, float* norms, int cus, hipStream_t s) {
#define TQ_QN(N, C) \
  launch_q<BITS, LSB, N, C>(W, rows, d, log2h, kh, perm, signs, cb, packed, norms, cus, s)
  const int hc = stage_class(log2h);
  TQ_BY_NT_HC(TQ_QN)
#undef TQ_QN
}

template <int BITS, bool LSB, int DT, int NT, int HC, bool MR = false>
hipError_t launch_dq(const uint8_t* packed, const float* norms, int64_t rows, int d, int log2h,
                     float kh, const int32_t* inv_perm, const int8_t* signs,
                     const OrbitCodebook& cb, int rotated_only, void* out, int cus,
                     hipStream_t s) {
  if constexpr (NT == 1 && HC == 0 && !MR) {
    if (d <= 512)
      return launch_dq<BITS, LSB, DT, NT, HC, true>(packed, norms, rows, d, log2h, kh, inv_perm,
                                                    signs, cb, rotated_only, out, cus, s);
  }
  auto kernel = orbit_dequantize_kernel<BITS, LSB, DT, NT, HC, MR>;
  const int R = MR ? rows_per_group(d) : 1;
  const size_t shm = orbit_lds(R * d, HC == 2);
  const int nt = (d + 1023) >> 10;
  static std::atomic<int> cache[17];
  const int per_cu = resident_cached<NT>(cache, kernel, nt, HC == 2);
  const int grid = grid_size((rows + R - 1) / R, cus, per_cu);
  kernel<<<grid, block_threads(NT, nt), shm, s>>>(packed, norms, rows, d, log2h, kh, inv_perm,
                                                  signs, cb, rotated_only, out);
  return hipGetLastError();
}

template <int BITS, bool LSB, int DT>
hipError_t launch_dq_nt(int nt, const uint8_t* packed, const float* norms, int64_t rows, int d,
                        int log2h, float kh, const int32_t* inv_perm, const int8_t* signs,
                        const OrbitCodebook& cb, int rotated_only, void* out, int cus,
                        hipStream_t s) {
#define TQ_DQN(N, C) launch_dq<BITS, LSB, DT, N, C>(packed, norms, rows, d, log2h, kh, inv_perm, \
                                                 signs, cb, rotated_only, out, cus, s)
  const int hc = stage_class(log2h);
  TQ_BY_NT_HC(TQ_DQN)
#undef TQ_DQN
}

template <int BITS, bool LSB>
hipError_t launch_dq_dt(int dt, int nt, const uint8_t* packed, const float* norms, int64_t rows,
                        int d, int log2h, float kh, const int32_t* inv_perm, const int8_t* signs,
                        const OrbitCodebook& cb, int rotated_only, void* out, int cus,
                        hipStream_t s) {
  switch (dt) {
    case DT_F32:
      return launch_dq_nt<BITS, LSB, DT_F32>(nt, packed, norms, rows, d, log2h, kh, inv_perm,
                                             signs, cb, rotated_only, out, cus, s);
    case DT_BF16:
      return launch_dq_nt<BITS, LSB, DT_BF16>(nt, packed, norms, rows, d, log2h, kh, inv_perm,
                                              signs, cb, rotated_only, out, cus, s);
    default:
      return launch_dq_nt<BITS, LSB, DT_F16>(nt, packed, norms, rows, d, log2h, kh, inv_perm,
                                             signs, cb, rotated_only, out, cus, s);
  }
}

template <int NT, int HC, int DT, bool TOUT, bool MR = false>
hipError_t launch_rot(const void* x, int64_t rows, int d, int log2h, float kh,
                      const int32_t* perm, const int8_t* signs, void* xrot, int cus, hipStream_t s) {
  if constexpr (NT == 1 && HC == 0 && !MR) {
    if (d <= 512)
      return launch_rot<NT, HC, DT, TOUT, true>(x, rows, d, log2h, kh, perm, signs, xrot, cus, s);
  }
  auto kernel = orbit_quantize_kernel<2, false, NT, HC, true, DT, true, TOUT, MR>;
  const int nt = (d + 1023) >> 10;
  const int R = MR ? rows_per_group(d) : 1;
  const size_t shm = orbit_lds(R * d, HC == 2);
  static std::atomic<int> cache[17];
  const int per_cu = resident_cached<NT>(cache, kernel, nt, HC == 2);
  const int64_t rows_loop = TOUT ? (rows + 15) / 16 * 16 : rows;
  const int grid = grid_size((rows_loop + R - 1) / R, cus, per_cu);
  OrbitCodebook cb{};
  kernel<<<grid, block_threads(NT, nt), shm, s>>>(x, rows, d, log2h, kh, perm, signs, cb, nullptr,
                                                  nullptr, xrot);
  return hipGetLastError();
}

int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << (l + 1)) <= v) ++l;
  return l;
}

}  // namespace

hipError_t launch_orbit_quantize(const float* W, int64_t rows, int64_t d, int bits,
                                 const int32_t* perm, const int8_t* signs,
                                 const OrbitCodebook& cb, int lsb_first, uint8_t* packed,
                                 float* norms, int cus, hipStream_t s) {
  const int64_t h = d & -d;
  const int log2h = ilog2(h);
  const float kh = (float)pow((double)h, -0.5);
  const int di = (int)d;
  const int nt = (di + 1023) >> 10;  // tiles of 64 lanes x 16 elements
#define TQ_Q(B, O) launch_q_nt<B, O>(nt, W, rows, di, log2h, kh, perm, signs, cb, packed, norms, cus, s)
  if (lsb_first) {
    if (bits == 2) return TQ_Q(2, true);
    if (bits == 3) return TQ_Q(3, true);
    return TQ_Q(4, true);
  }
  if (bits == 2) return TQ_Q(2, false);
  if (bits == 3) return TQ_Q(3, false);
  return TQ_Q(4, false);
#undef TQ_Q
}

template <int DT, bool TOUT>
hipError_t launch_rot_dt(const void* x, int64_t rows, int di, int log2h, float kh,
                         const int32_t* perm, const int8_t* signs, void* xrot, int cus,
                         hipStream_t s) {
  const int nt = (di + 1023) >> 10;
  const int hc = stage_class(log2h);
#define TQ_R(N, C) launch_rot<N, C, DT, TOUT>(x, rows, di, log2h, kh, perm, signs, xrot, cus, s)
  TQ_BY_NT_HC(TQ_R)
#undef TQ_R
}

#undef TQ_BY_NT_HC

hipError_t launch_orbit_rotate(const void* x, int dt, int64_t rows, int64_t d,
                               const int32_t* perm, const int8_t* signs, void* xrot, int tiled,
                               int cus, hipStream_t s) {
  const int64_t h = d & -d;
  const int log2h = ilog2(h);
  const float kh = (float)pow((double)h, -0.5);
  const int di = (int)d;
#define TQ_RD(T, O) launch_rot_dt<T, O>(x, rows, di, log2h, kh, perm, signs, xrot, cus, s)
  switch (dt) {
    case DT_F32: return TQ_RD(DT_F32, false);
    case DT_BF16: return tiled ? TQ_RD(DT_BF16, true) : TQ_RD(DT_BF16, false);
    default: return tiled ? TQ_RD(DT_F16, true) : TQ_RD(DT_F16, false);
  }
#undef TQ_RD
}

hipError_t launch_orbit_dequantize(const uint8_t* packed, const float* norms, int64_t rows,
                                   int64_t d, int bits, const int32_t* inv_perm,
                                   const int8_t* signs, const OrbitCodebook& cb, int lsb_first,
                                   int rotated_only, void* out, int dt, int cus,
                                   hipStream_t s) {
  const int64_t h = d & -d;
  const int log2h = ilog2(h);
  const float kh = (float)pow((double)h, -0.5);
  const int di = (int)d;
  const int nt = (di + 1023) >> 10;
#define TQ_DQ(B, O) \
  launch_dq_dt<B, O>(dt, nt, packed, norms, rows, di, log2h, kh, inv_perm, signs, cb, rotated_only, out, cus, s)
  if (lsb_first) {
    if (bits == 2) return TQ_DQ(2, true);
    if (bits == 3) return TQ_DQ(3, true);
    return TQ_DQ(4, true);
  }
  if (bits == 2) return TQ_DQ(2, false);
  if (bits == 3) return TQ_DQ(3, false);
  return TQ_DQ(4, false);
#undef TQ_DQ
}

}  // namespace tq
