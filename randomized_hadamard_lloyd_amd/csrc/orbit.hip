// OrbitQuant weight-codec kernels for gfx950 -- "zerogpu-sdxlTrainer:
// toolkit/util/orbit_quant.py": rpbh_forward, _quantize_rows,
// _dequantize_rotated, dequantize.
//
// Work mapping. One block of NT = ceil(d / 1024) waves owns one weight row
// at a time; wave w holds the row's elements [1024 w, 1024 w + 1024) as 64
// chunks of 16, one chunk per lane (see lane_chunk for which lane holds
// which). Element j = 16 c + i of chunk c: index bits 0-3 are register bits,
// bits 4-9 chunk bits inside the wave, bits 10-11 the wave. FWHT stages run
// in the order 1, 2, 4, ..., h/2: in registers for bits 0-3; across lanes
// without LDS for bits 4-9 (DPP fmac with the lazy lane sign described in
// tq3.hip for bits 4-7, permlane16/32 swaps for bits 8 and 9); across waves
// through LDS for bits 10-11. The row norm's sum of squares follows the same
// bit order inside each h-block; block sums are then added left to right.
#include "orbit_codes.h"
#include "tq_common.h"
#include "tq_kernels.h"

namespace tq {

namespace {

constexpr int kMaxBlocks = 128; // d / h <= 4096 / 32
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
template <int BITS, bool LSB, int NT, bool FULL, bool ROT = false, int DT = DT_F32>
__global__ __launch_bounds__(256) void orbit_quantize_kernel(
    const void* __restrict__ W, int64_t rows, int d, int log2h, float kh,
    const int32_t* __restrict__ perm, const int8_t* __restrict__ signs, OrbitCodebook cb,
    uint8_t* __restrict__ packed, float* __restrict__ norms, void* __restrict__ xrot) {
  static_assert(ROT || DT == DT_F32, "the weight codec reads fp32 rows");
  extern __shared__ float lds[];
  float* rowbuf = lds;     // the row; later the cross-wave butterfly exchange
  float* bsum = lds + d;   // block (or, for h > 1024, tile) sums of squares
  constexpr int NTHR = 64 * NT;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = lane_chunk(lane);
  const int c = lc + 64 * wave;  // this lane's chunk of 16 elements
  const bool act = c < (d >> 4);
  const int nblk = d >> log2h;
  const int lb = FULL ? 6 : (log2h - 4 < 6 ? log2h - 4 : 6);
  const LaneCx cx = lane_cx(lc, log2h);
  const float ksig = kh * cx.sigma;
  const int64_t row_bytes = (int64_t)d * BITS / 8;
  const float eps = (float)1e-10;
  constexpr int ES = DT == DT_F32 ? 4 : 2;  // bytes per element of a row
  constexpr int KL = ES;                     // 16-byte loads per thread (d <= 1024 NT)
  const int nl = d * ES / 16;               // 16-byte pieces per row

  // Byte offsets into the staged row and sign masks of this lane's elements.
  uint32_t poff[16], sbits = 0;  // sbits: bit i set when signs_j = -1 for element i
  {
    const int cc = act ? c : 0;  // inactive lanes read chunk 0 and never use it
    const u32x4* pp = reinterpret_cast<const u32x4*>(perm + 16 * cc);
    const u32x4 sv = *reinterpret_cast<const u32x4*>(signs + 16 * cc);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 p = pp[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        poff[4 * k + e] = 4u * p[e];
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
  int fidx[KL];
#pragma unroll
  for (int k = 0; k < KL; ++k) {
    const int f = tid + NTHR * k;
    fidx[k] = f < nl ? f : nl - 1;
  }
  int64_t r = blockIdx.x;
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(Wb + (r < rows ? r : 0) * row_in);
#pragma unroll
    for (int k = 0; k < KL; ++k) pre[k] = src[fidx[k]];
  }
  for (; r < rows; r += gridDim.x) {
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int f = tid + NTHR * k;
      if (f < nl) {
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
    {
      const int64_t rn = r + gridDim.x < rows ? r + gridDim.x : r;
      const u32x4* src = reinterpret_cast<const u32x4*>(Wb + rn * row_in);
#pragma unroll
      for (int k = 0; k < KL; ++k) pre[k] = src[fidx[k]];
    }

    // y_j = W[perm_j] * signs_j.
    float y[16];
    const char* rb = reinterpret_cast<const char*>(rowbuf);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      y[i] = act ? as_f(*reinterpret_cast<const uint32_t*>(rb + poff[i]) ^
                        ((sbits << (31 - i)) & 0x80000000u))
                 : 0.0f;

    // Butterflies inside the wave (index bits 0..9), then across waves
    // through LDS for blocks longer than 1024 (bits 10, 11): the lower tile
    // takes a + b, the upper b' - a' = a - b with the same lazy lane sign.
    constexpr int RD = ROT ? DT : DT_F32;
    fwht_rows<FULL, RD>(y, log2h, cx);
    if (log2h > 10) {
      float4* mine = reinterpret_cast<float4*>(rowbuf + 16 * c);
#pragma unroll
      for (int ht = 1; ht < NT; ht *= 2) {
        if (log2h <= 9 + ht) break;
        __syncthreads();  // everyone is done reading the row buffer
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mine[k] = make_float4(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]);
        __syncthreads();
        const float4* other = reinterpret_cast<const float4*>(rowbuf + 16 * (c ^ (64 * ht)));
        const bool upper = (wave & ht) != 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 o = other[k];
          const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = y[4 * k + e];
            y[4 * k + e] = upper ? ov[e] - a : a + ov[e];
          }
        }
        round16<RD>(y);
      }
    }
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
          u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(xrot) + r * d + 16 * c);
          dst[0] = u32x4{w[0], w[1], w[2], w[3]};
          dst[1] = u32x4{w[4], w[5], w[6], w[7]};
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
    if (act && (c & ((1 << lb) - 1)) == 0) bsum[c >> lb] = part;  // one writer per block/tile
    __syncthreads();
    float total;
    if (log2h <= 10) {
      total = bsum[0];
      for (int bi = 1; bi < nblk; ++bi) total = total + bsum[bi];
    } else if (log2h == 11) {
      total = bsum[0] + bsum[1];
    } else {
      total = (bsum[0] + bsum[1]) + (bsum[2] + bsum[3]);
    }
    const float norm = __builtin_sqrtf(total);
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

    // Codes and packing (the codebook test is uniform).
    const uint64_t bytes =
        cb.sym ? pack16<BITS, LSB, true>(y, cb) : pack16<BITS, LSB, false>(y, cb);
    if (act) store_codes<BITS>(packed + r * row_bytes + 2 * BITS * c, bytes);
    if (tid == 0) norms[r] = norm;
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
template <int BITS, bool LSB, int DT, int NT, bool FULL>
__global__ __launch_bounds__(256) void orbit_dequantize_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ norms, int64_t rows, int d,
    int log2h, float kh, const int32_t* __restrict__ inv_perm,
    const int8_t* __restrict__ signs, OrbitCodebook cb, int rotated_only,
    void* __restrict__ out) {
  extern __shared__ float lds[];
  float* rowbuf = lds;  // d floats
  constexpr int EPS = DT == DT_F32 ? 4 : 8;
  constexpr int NG = 16 / EPS;  // 16-byte output groups per lane per tile
  constexpr int L = 1 << BITS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float* tab = lds + d + 16 * wave;  // this wave's codebook x row norm
  const int lc = lane_chunk(lane);
  const int c = lc + 64 * wave;
  const bool act = c < (d >> 4);
  const LaneCx cx = lane_cx(lc, log2h);
  const float ksig = kh * cx.sigma;
  const int64_t row_bytes = (int64_t)d * BITS / 8;

  // Output groups of this lane and, when the rotation is undone, the byte
  // offsets of their sources in the staged row and the signs of its chunk.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  int j0[NG];
  bool gact[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    j0[k] = 1024 * wave + EPS * lane + 64 * EPS * k;
    gact[k] = j0[k] < d;
  }
  uint32_t ioff[16], smask[16];
  if (!rotated_only) {
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const u32x4* ip = reinterpret_cast<const u32x4*>(inv_perm + (gact[k] ? j0[k] : 0));
#pragma unroll
      for (int e4 = 0; e4 < EPS / 4; ++e4) {
        const u32x4 p = ip[e4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ioff[EPS * k + 4 * e4 + e] = 4u * p[e];
      }
    }
    const u32x4 sv = *reinterpret_cast<const u32x4*>(signs + 16 * (act ? c : 0));
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) smask[4 * k + e] = sign_of(sv[k], e);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) ioff[i] = smask[i] = 0;
  }

  int64_t r = blockIdx.x;
  const int cc = act ? c : 0;
  uint64_t ncodes = load_codes<BITS>(packed + (r < rows ? r : 0) * row_bytes + 2 * BITS * cc);
  float nnorm = norms[r < rows ? r : 0];
  for (; r < rows; r += gridDim.x) {
    const uint64_t codes = ncodes;
    const float norm = nnorm;
    {
      const int64_t rn = r + gridDim.x < rows ? r + gridDim.x : r;
      ncodes = load_codes<BITS>(packed + rn * row_bytes + 2 * BITS * cc);
      nnorm = norms[rn];
    }
    if (lane < L) tab[lane] = cb.cb[lane] * norm;
    __builtin_amdgcn_wave_barrier();
    uint32_t code[16];
    unpack16<BITS, LSB>(codes, code);
    float w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = tab[code[i]];

    if (rotated_only) {
      // Stage this wave's tile in element order, re-read it in store order.
      if (act) {
        f32x4_t* mine = reinterpret_cast<f32x4_t*>(rowbuf + 16 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mine[k] = f32x4_t{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < NG; ++k)
        if (gact[k]) store_group<DT>(out, r * d + j0[k], rowbuf + j0[k]);
      __builtin_amdgcn_wave_barrier();
      continue;
    }

    // Inverse rotation: FWHT per block (across waves through LDS beyond
    // 1024), times h^-1/2 and the lazy lane sign, times signs_j.
    fwht_rows<FULL>(w, log2h, cx);
    if (log2h > 10) {
      f32x4_t* mine = reinterpret_cast<f32x4_t*>(rowbuf + 16 * c);
#pragma unroll
      for (int ht = 1; ht < NT; ht *= 2) {
        if (log2h <= 9 + ht) break;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mine[k] = f32x4_t{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
        __syncthreads();
        const f32x4_t* other = reinterpret_cast<const f32x4_t*>(rowbuf + 16 * (c ^ (64 * ht)));
        const bool upper = (wave & ht) != 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4_t o = other[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = w[4 * k + e];
            w[4 * k + e] = upper ? o[e] - a : a + o[e];
          }
        }
      }
    }
    __syncthreads();  // the row buffer is free
    if (act) {
      f32x4_t* mine = reinterpret_cast<f32x4_t*>(rowbuf + 16 * c);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = as_f(as_u(w[4 * k + e] * ksig) ^ smask[4 * k + e]);
        mine[k] = f32x4_t{z[0], z[1], z[2], z[3]};
      }
    }
    __syncthreads();
    // out[j] = z[inv_perm_j], gathered from the staged row.
    const char* rb = reinterpret_cast<const char*>(rowbuf);
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      if (!gact[k]) continue;
      float o[EPS];
#pragma unroll
      for (int e = 0; e < EPS; ++e) o[e] = *reinterpret_cast<const float*>(rb + ioff[EPS * k + e]);
      store_group<DT>(out, r * d + j0[k], o);
    }
  }
}

// LDS of a block: the row (d <= 1024 NT floats) and the block sums. The
// resident-block count is taken once per kernel instantiation at its largest
// LDS size (at most 17 KB: it never limits below the other resources).
constexpr size_t orbit_lds(int d) { return (size_t)(d + kMaxBlocks) * sizeof(float); }

template <int BITS, bool LSB, int NT, bool FULL>
hipError_t launch_q(const float* W, int64_t rows, int d, int log2h, float kh,
                    const int32_t* perm, const int8_t* signs, const OrbitCodebook& cb,
                    uint8_t* packed, float* norms, int cus, hipStream_t s) {
  const size_t shm = orbit_lds(d);
  static const int per_cu = resident_blocks_per_cu(orbit_quantize_kernel<BITS, LSB, NT, FULL>,
                                                   64 * NT, orbit_lds(1024 * NT));
  const int grid = grid_size(rows, cus, per_cu);
  orbit_quantize_kernel<BITS, LSB, NT, FULL><<<grid, 64 * NT, shm, s>>>(W, rows, d, log2h, kh, perm,
                                                                 signs, cb, packed, norms, nullptr);
  return hipGetLastError();
}

template <int BITS, bool LSB>
hipError_t launch_q_nt(int nt, const float* W, int64_t rows, int d, int log2h, float kh,
                       const int32_t* perm, const int8_t* signs, const OrbitCodebook& cb,
                       uint8_t* packed, float* norms, int cus, hipStream_t s) {
#define TQ_QN(N, F) \
  launch_q<BITS, LSB, N, F>(W, rows, d, log2h, kh, perm, signs, cb, packed, norms, cus, s)
  const bool full = log2h >= 10;
  switch (nt) {
    case 1: return full ? TQ_QN(1, true) : TQ_QN(1, false);
    case 2: return full ? TQ_QN(2, true) : TQ_QN(2, false);
    case 3: return full ? TQ_QN(3, true) : TQ_QN(3, false);
    default: return full ? TQ_QN(4, true) : TQ_QN(4, false);
  }
#undef TQ_QN
}

template <int BITS, bool LSB, int DT, int NT, bool FULL>
hipError_t launch_dq(const uint8_t* packed, const float* norms, int64_t rows, int d, int log2h,
                     float kh, const int32_t* inv_perm, const int8_t* signs,
                     const OrbitCodebook& cb, int rotated_only, void* out, int cus,
                     hipStream_t s) {
  const size_t shm = orbit_lds(d);
  static const int per_cu = resident_blocks_per_cu(
      orbit_dequantize_kernel<BITS, LSB, DT, NT, FULL>, 64 * NT, orbit_lds(1024 * NT));
  const int grid = grid_size(rows, cus, per_cu);
  orbit_dequantize_kernel<BITS, LSB, DT, NT, FULL><<<grid, 64 * NT, shm, s>>>(
      packed, norms, rows, d, log2h, kh, inv_perm, signs, cb, rotated_only, out);
  return hipGetLastError();
}

template <int BITS, bool LSB, int DT>
hipError_t launch_dq_nt(int nt, const uint8_t* packed, const float* norms, int64_t rows, int d,
                        int log2h, float kh, const int32_t* inv_perm, const int8_t* signs,
                        const OrbitCodebook& cb, int rotated_only, void* out, int cus,
                        hipStream_t s) {
#define TQ_DQN(N, F) launch_dq<BITS, LSB, DT, N, F>(packed, norms, rows, d, log2h, kh, inv_perm, \
                                                 signs, cb, rotated_only, out, cus, s)
  const bool full = log2h >= 10;
  switch (nt) {
    case 1: return full ? TQ_DQN(1, true) : TQ_DQN(1, false);
    case 2: return full ? TQ_DQN(2, true) : TQ_DQN(2, false);
    case 3: return full ? TQ_DQN(3, true) : TQ_DQN(3, false);
    default: return full ? TQ_DQN(4, true) : TQ_DQN(4, false);
  }
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

template <int NT, bool FULL, int DT>
hipError_t launch_rot(const void* x, int64_t rows, int d, int log2h, float kh,
                      const int32_t* perm, const int8_t* signs, void* xrot, int cus, hipStream_t s) {
  const size_t shm = orbit_lds(d);
  static const int per_cu = resident_blocks_per_cu(
      orbit_quantize_kernel<2, false, NT, FULL, true, DT>, 64 * NT, orbit_lds(1024 * NT));
  const int grid = grid_size(rows, cus, per_cu);
  OrbitCodebook cb{};
  orbit_quantize_kernel<2, false, NT, FULL, true, DT><<<grid, 64 * NT, shm, s>>>(
      x, rows, d, log2h, kh, perm, signs, cb, nullptr, nullptr, xrot);
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

template <int DT>
hipError_t launch_rot_dt(const void* x, int64_t rows, int di, int log2h, float kh,
                         const int32_t* perm, const int8_t* signs, void* xrot, int cus,
                         hipStream_t s) {
  const int nt = (di + 1023) >> 10;
  const bool full = log2h >= 10;
#define TQ_R(N, F) launch_rot<N, F, DT>(x, rows, di, log2h, kh, perm, signs, xrot, cus, s)
  switch (nt) {
    case 1: return full ? TQ_R(1, true) : TQ_R(1, false);
    case 2: return full ? TQ_R(2, true) : TQ_R(2, false);
    case 3: return full ? TQ_R(3, true) : TQ_R(3, false);
    default: return full ? TQ_R(4, true) : TQ_R(4, false);
  }
#undef TQ_R
}

hipError_t launch_orbit_rotate(const void* x, int dt, int64_t rows, int64_t d,
                               const int32_t* perm, const int8_t* signs, void* xrot, int cus,
                               hipStream_t s) {
  const int64_t h = d & -d;
  const int log2h = ilog2(h);
  const float kh = (float)pow((double)h, -0.5);
  const int di = (int)d;
  switch (dt) {
    case DT_F32: return launch_rot_dt<DT_F32>(x, rows, di, log2h, kh, perm, signs, xrot, cus, s);
    case DT_BF16: return launch_rot_dt<DT_BF16>(x, rows, di, log2h, kh, perm, signs, xrot, cus, s);
    default: return launch_rot_dt<DT_F16>(x, rows, di, log2h, kh, perm, signs, xrot, cus, s);
  }
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
