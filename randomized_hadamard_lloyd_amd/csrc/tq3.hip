// TQ3 codec kernels for gfx950 -- "ComfyUI-TurboQuant: tq3_core.py",
// tq3_quantize / tq3_dequantize.
//
// Work mapping. A 128-vector lives in one 4-lane quad: quad lane q holds the
// 32 elements j = i + 8q + 32g (i = 0..7, g = 0..3) in registers x[g][i], so a
// wave of 64 lanes carries 16 vectors and a 256-thread block 64 vectors.
// Index bits 0-2 (i) and 5-6 (g) are register bits; bits 3-4 are quad-lane
// bits. The FWHT stages with half-width 1, 2, 4 and 32, 64 are in-register
// butterflies; the stages with half-width 8 and 16 combine a lane's value with
// its quad partner's in one fmac that reads the partner through a DPP quad
// permute. Stages always run in the order 1, 2, 4, ..., 64, and the
// sum of squares follows the same bit order, so every fp32 operation matches
// the declared reference order exactly.
//
// Lazy lane sign. In a cross-lane stage the lower lane needs a + b and the
// upper lane a - b. Both lanes evaluate fma(partner, c, own) with c = +-1;
// the upper lane then holds -(a - b). The sign is tracked per lane (it only
// depends on the quad lane) and folded into the final multiply by
// 1/sqrt(128), which is exact because a sign change commutes with rounding.
#include "tq_common.h"
#include "tq_kernels.h"

namespace tq {

namespace {

static_assert(kTq3VecPerBlock == 64, "a 256-thread block carries 64 vectors, one per quad");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 of the page's printed centroid table (doubles rounded to float32).
__device__ __forceinline__ float tq3_centroid(int k) {
  constexpr float c[8] = {(float)-0.9816, (float)-0.6168, (float)-0.3479, (float)-0.1129,
                          (float)0.1129,  (float)0.3479,  (float)0.6168,  (float)0.9816};
  return c[k];
}
// Twice the bit patterns of the positive boundaries (see the index comment).
constexpr uint32_t kB1x2 = 2u * __builtin_bit_cast(uint32_t, (float)0.2304);
constexpr uint32_t kB2x2 = 2u * __builtin_bit_cast(uint32_t, (float)0.4824);
constexpr uint32_t kB3x2 = 2u * __builtin_bit_cast(uint32_t, (float)0.7992);
constexpr float kInvSqrt128 = (float)0.08838834764831845;  // fp32(1/sqrt(128))
constexpr float kFloor = (float)1e-8;                      // clamp of norm and scale

// Sign bit of element (q, g, i) from the 128-bit mask (bit j = element j).
__device__ __forceinline__ uint32_t sign_bit(const SignMask& m, int q, int g, int i) {
  return (m.w[g] >> (8 * q + i)) & 1u;
}

// ------------------------------------------------------------- loading ---

template <int DT>
struct Loader;

template <>
struct Loader<DT_F32> {
  // 32 masks, one per element, each 0 or 0x80000000
  uint32_t sm[4][8];
  __device__ __forceinline__ void init(const SignMask& m, int q) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) sm[g][i] = sign_bit(m, q, g, i) << 31;
  }
  // Raw 16-byte chunks of this lane's 32 elements of one row.
  struct Raw {
    u32x4 c[8];
  };
  __device__ __forceinline__ Raw fetch(const void* base, int64_t row, int64_t stride,
                                       int q) const {
    const float* r = static_cast<const float*>(base) + row * stride + 8 * q;
    Raw raw;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      raw.c[2 * g] = *reinterpret_cast<const u32x4*>(r + 32 * g);
      raw.c[2 * g + 1] = *reinterpret_cast<const u32x4*>(r + 32 * g + 4);
    }
    return raw;
  }
  // x: signed input (sign flips applied), used for both the norm and u
  __device__ __forceinline__ void convert(const Raw& raw, float (&x)[4][8]) const {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[g][i] = as_f(raw.c[2 * g + (i >> 2)][i & 3] ^ sm[g][i]);
  }
};

// bf16 and f16: eight 16-bit values per 16-byte load; sign flips are applied
// to the packed pairs (bit 15 low element, bit 31 high element).
template <int DT>
struct Loader16 {
  uint32_t sm[4][4];
  __device__ __forceinline__ void init(const SignMask& m, int q) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        sm[g][p] = (sign_bit(m, q, g, 2 * p) << 15) | (sign_bit(m, q, g, 2 * p + 1) << 31);
  }
  struct Raw {
    u32x4 c[4];
  };
  __device__ __forceinline__ Raw fetch(const void* base, int64_t row, int64_t stride,
                                       int q) const {
    const uint16_t* r = static_cast<const uint16_t*>(base) + row * stride + 8 * q;
    Raw raw;
#pragma unroll
    for (int g = 0; g < 4; ++g) raw.c[g] = *reinterpret_cast<const u32x4*>(r + 32 * g);
    return raw;
  }
  __device__ __forceinline__ void convert(const Raw& raw, float (&x)[4][8]) const {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4 a = raw.c[g];
      const uint32_t w[4] = {a.x ^ sm[g][0], a.y ^ sm[g][1], a.z ^ sm[g][2], a.w ^ sm[g][3]};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (DT == DT_BF16) {
          x[g][2 * p] = as_f(w[p] << 16);
          x[g][2 * p + 1] = as_f(w[p] & 0xffff0000u);
        } else {
          x[g][2 * p] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[p] & 0xffffu));
          x[g][2 * p + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[p] >> 16));
        }
      }
    }
  }
};
template <>
struct Loader<DT_BF16> : Loader16<DT_BF16> {};
template <>
struct Loader<DT_F16> : Loader16<DT_F16> {};

// ---------------------------------------------------------------- FWHT ---

// In-register stages over index bits 0..2 of each 8-element chunk.
__device__ __forceinline__ void fwht_low3(float (&x)[4][8]) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i & h) == 0) {
          const float a = x[g][i], b = x[g][i + h];
          x[g][i] = a + b;
          x[g][i + h] = a - b;
        }
}

// Stages over index bits 3, 4 (quad lanes) with the lazy lane sign, then bits
// 5, 6 (chunk index g) in registers.
__device__ __forceinline__ void fwht_high4(float (&x)[4][8], float c1, float c2) {
  float (&lo)[16] = *reinterpret_cast<float (*)[16]>(&x[0][0]);
  float (&hi)[16] = *reinterpret_cast<float (*)[16]>(&x[2][0]);
  TQ_DPP_FMAC16("quad_perm:[1,0,3,2]", c1, lo);
  TQ_DPP_FMAC16("quad_perm:[1,0,3,2]", c1, hi);
  TQ_DPP_FMAC16("quad_perm:[2,3,0,1]", c2, lo);
  TQ_DPP_FMAC16("quad_perm:[2,3,0,1]", c2, hi);
#pragma unroll
  for (int hg = 1; hg < 4; hg *= 2)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if ((g & hg) == 0)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float a = x[g][i], b = x[g + hg][i];
          x[g][i] = a + b;
          x[g + hg][i] = a - b;
        }
}

// Lane constants of the lazy-sign scheme (see the file comment).
struct LaneSigns {
  float c1, c2, sigma;
};
__device__ __forceinline__ LaneSigns lane_signs(int q) {
  LaneSigns s;
  s.c1 = (q & 1) ? -1.0f : 1.0f;
  s.c2 = (q & 2) ? -1.0f : 1.0f;
  s.sigma = (__builtin_popcount(q) & 1) ? -1.0f : 1.0f;
  return s;
}

// ------------------------------------------------------------ quantize ---

// SPLIT: the three fields go to separate arrays (indices [n, 48], norms [n],
// scales [n]) instead of 56-byte records; `rec` is then the index array.
template <int DT, bool SPLIT>
__global__ __launch_bounds__(256) void tq3_quantize_kernel(const void* __restrict__ x,
                                                           int64_t n_vec, int64_t stride,
                                                           SignMask mask,
                                                           uint8_t* __restrict__ rec,
                                                           float* __restrict__ norms_out,
                                                           float* __restrict__ scales_out) {
  const int q = threadIdx.x & 3;
  Loader<DT> ld;
  ld.init(mask, q);
  const LaneSigns ls = lane_signs(q);
  const float kq = ls.sigma * kInvSqrt128;

  const int64_t step = (int64_t)gridDim.x * kTq3VecPerBlock;
  for (int64_t v = (int64_t)blockIdx.x * kTq3VecPerBlock + (threadIdx.x >> 2); v < n_vec;
       v += step) {
    float x_[4][8];
    ld.convert(ld.fetch(x, v, stride, q), x_);

    // Smallest |x| of the vector (it decides the division path below).
    float amin = __builtin_inff();
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) amin = __builtin_fminf(amin, __builtin_fabsf(x_[g][i]));
    amin = __builtin_fminf(amin, swz<QP_XOR1>(amin));
    amin = __builtin_fminf(amin, swz<QP_XOR2>(amin));

    // Sum of squares: bits 0..2 in registers, 3..4 across the quad, 5..6 in
    // registers -- the reference tree's bit order. The square of an fp16
    // value (11 significant bits, at least 2^-24) is exact in fp32, and so is
    // the square of a bf16 value with |x| >= 2^-63 (a zero's too); then the
    // first level RN(RN(x0^2) + RN(x1^2)) equals the single fma
    // RN(x1^2 + RN(x0^2)). A bf16 vector holding a magnitude below 2^-63
    // (whose square loses bits) takes the separately rounded squares.
    float part[4];
    if (DT == DT_F16 || (DT == DT_BF16 && amin >= 0x1p-63f)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float a[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          a[k] = __builtin_fmaf(x_[g][2 * k + 1], x_[g][2 * k + 1], x_[g][2 * k] * x_[g][2 * k]);
        part[g] = (a[0] + a[1]) + (a[2] + a[3]);
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float a[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          a[k] = x_[g][2 * k] * x_[g][2 * k] + x_[g][2 * k + 1] * x_[g][2 * k + 1];
        part[g] = (a[0] + a[1]) + (a[2] + a[3]);
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) part[g] = part[g] + swz<QP_XOR1>(part[g]);
#pragma unroll
    for (int g = 0; g < 4; ++g) part[g] = part[g] + swz<QP_XOR2>(part[g]);
    const float ss = (part[0] + part[1]) + (part[2] + part[3]);

    const float norm = __builtin_fmaxf(sqrt_rn_large(ss), kFloor);

    // u = x / norm, correctly rounded. The shared-reciprocal path is exact
    // while every nonzero |x_j| >= norm * 2^-60 and norm <= 2^100; otherwise
    // the vector takes plain IEEE division.
    float u[4][8];
    if (amin >= norm * 0x1p-60f && norm <= 0x1p100f) {
      const Recip rn = make_recip(norm);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) u[g][i] = div_rn(x_[g][i], rn);
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) u[g][i] = x_[g][i] / norm;
    }

    fwht_low3(u);
    fwht_high4(u, ls.c1, ls.c2);

    // y = w * fp32(1/sqrt(128)); kq also undoes the lazy lane sign.
    float amax = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u[g][i] = u[g][i] * kq;
        amax = __builtin_fmaxf(amax, __builtin_fabsf(u[g][i]));
      }
    amax = __builtin_fmaxf(amax, swz<QP_XOR1>(amax));
    amax = __builtin_fmaxf(amax, swz<QP_XOR2>(amax));
    const float scale = __builtin_fmaxf(amax, kFloor);
    // |y_j| <= scale, so y_j / scale stays in [-1, 1]; its sign and its
    // comparisons with the boundaries are all the index needs, and the
    // shared-reciprocal quotient is exact wherever it can reach a boundary.
    const Recip rs = make_recip(scale);

    // Index = number of boundaries strictly below t. The table is symmetric,
    // so with a = |t| and P = {0.2304, 0.4824, 0.7992}:
    //   t > 0:  idx = 4 + #{b in P : b < a}
    //   t <= 0: idx = 3 - #{b in P : b <= a}
    // Rotating t's bits left by one puts the sign in bit 0: R = 2*bits(a) + sign.
    // Then R > 2*bits(b) means bits(a) > bits(b) for t >= 0 and bits(a) >= bits(b)
    // for t < 0 -- exactly the strict/non-strict split of the tie rule -- and
    // with c = #{R > 2*bits(b)} (a thermometer code m1 >= m2 >= m3),
    // idx = c ^ (t > 0 ? 4 : 3): bit 2 = (t > 0), bit 1 = m2 xnor (t > 0),
    // bit 0 = (m1 ^ m2 ^ m3) xnor (t > 0). The compares leave wave-wide lane
    // masks; the bit logic runs on the scalar unit and each bit enters the
    // lane's chunk through one add-with-carry.
    uint32_t chunk[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t c = 0;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        const float t = div_rn(u[g][i], rs);
        const uint32_t tb = as_u(t);
        const uint32_t r = __builtin_amdgcn_alignbit(tb, tb, 31);
        const uint64_t m1 = __builtin_amdgcn_ballot_w64(r > kB1x2);
        const uint64_t m2 = __builtin_amdgcn_ballot_w64(r > kB2x2);
        const uint64_t m3 = __builtin_amdgcn_ballot_w64(r > kB3x2);
        const uint64_t pos = __builtin_amdgcn_ballot_w64(t > 0.0f);
        c = shift_in(c, pos);
        c = shift_in(c, ~(m2 ^ pos));
        c = shift_in(c, ~(m1 ^ m2 ^ m3 ^ pos));
      }
      chunk[g] = c;
    }

    // Record: 48 bytes of indices = 4 groups of 3 dwords; in group g quad lane
    // k < 3 writes dword k, which takes its own 24-bit chunk and the next
    // lane's: (c_k >> 8k) | (c_{k+1} << (24 - 8k)). Lane 3 writes norm, scale.
    uint8_t* out = rec + v * (SPLIT ? 48 : 56);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t nb = swz<QP_NEXT>(chunk[g]);
      const uint32_t dw = (chunk[g] >> (8 * q)) | (nb << (24 - 8 * q));
      if (q < 3) *reinterpret_cast<uint32_t*>(out + 12 * g + 4 * q) = dw;
    }
    if constexpr (SPLIT) {
      if (q == 3) {
        norms_out[v] = norm;
        scales_out[v] = scale;
      }
    } else {
      if (q == 3) *reinterpret_cast<uint2*>(out + 48) = make_uint2(as_u(norm), as_u(scale));
    }
  }
}

// ---------------------------------------------------------- dequantize ---

constexpr int kStageRow = 320;     // padded bytes per staged 16-bit output row
constexpr int kStageRowF32 = 512;  // bytes per staged fp32 output row (XOR-swizzled)

// Byte offset of byte o of staged fp32 row v: the 16-byte slot index is XORed
// with the row's low two bits placed at slot bits 0 and 3, so that the 16
// lanes of a quarter-wave hit 16 distinct 4-bank groups both when quads write
// their 32-byte pieces and when lanes read consecutive 16-byte slots.
__device__ __forceinline__ int f32_stage_off(int v, int o) {
  const int sw = ((v & 1) | ((v & 2) << 2)) << 4;
  return v * kStageRowF32 + (o ^ sw);
}

// Two output values -> one dword of bf16 / fp16 (round to nearest even).
template <int DT>
__device__ __forceinline__ uint32_t narrow2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  if constexpr (DT == DT_BF16) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  }
}

// Quad lane q's 32 narrowed values of one row into its padded staging row.
template <int DT>
__device__ __forceinline__ void stage_row16(uint8_t* row, int q, const float (&y)[4][8]) {
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<u32x4*>(row + g * 64 + q * 16) =
        u32x4{narrow2<DT>(y[g][0], y[g][1]), narrow2<DT>(y[g][2], y[g][3]),
              narrow2<DT>(y[g][4], y[g][5]), narrow2<DT>(y[g][6], y[g][7])};
}

template <int DT>
__device__ __forceinline__ void store_row(void* base, int64_t row, int64_t stride, int q,
                                          const float (&y)[4][8]) {
  if constexpr (DT == DT_F32) {
    float* r = static_cast<float*>(base) + row * stride + 8 * q;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *reinterpret_cast<float4*>(r + 32 * g) = make_float4(y[g][0], y[g][1], y[g][2], y[g][3]);
      *reinterpret_cast<float4*>(r + 32 * g + 4) =
          make_float4(y[g][4], y[g][5], y[g][6], y[g][7]);
    }
  } else {
    uint16_t* r = static_cast<uint16_t*>(base) + row * stride + 8 * q;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (DT == DT_BF16) {
          typedef float f2 __attribute__((ext_vector_type(2)));
          typedef __bf16 b2 __attribute__((ext_vector_type(2)));
          const f2 v = {y[g][2 * p], y[g][2 * p + 1]};
          w[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
        } else {
          typedef float f2 __attribute__((ext_vector_type(2)));
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          const f2 v = {y[g][2 * p], y[g][2 * p + 1]};
          w[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
        }
      }
      *reinterpret_cast<uint4*>(r + 32 * g) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// SPLIT: the fields come from separate arrays (indices [n, 48], norms [n],
// scales [n]); `rec` is then the index array.
template <int DT, bool PF, bool SPLIT>
__global__ __launch_bounds__(256) void tq3_dequantize_kernel(const uint8_t* __restrict__ rec,
                                                             const float* __restrict__ norms_in,
                                                             const float* __restrict__ scales_in,
                                                             int64_t n_vec, SignMask mask,
                                                             void* __restrict__ y,
                                                             int64_t stride) {
  // The 64 centroid pairs, shared by the block: entry a | (b << 3) holds
  // (C[a], C[b]), the centroids of two consecutive elements with indices a
  // then b, which is the pair's 6-bit field of the record as it stands. One
  // 8-byte read serves two elements. Each element's value is the centroid
  // times its record's scale, the same fp32 product a per-record table of
  // scaled centroids would hold.
  __shared__ __attribute__((aligned(8))) float2 ptab[64];
  if (threadIdx.x < 64)
    ptab[threadIdx.x] = make_float2(tq3_centroid(threadIdx.x & 7), tq3_centroid(threadIdx.x >> 3));
  __syncthreads();
  // Per-wave staging of 16-bit outputs: 16 rows, each padded from 256 to 320
  // bytes so that both the quad-ordered writes and the row-ordered reads are
  // free of bank conflicts.
  __shared__ __attribute__((aligned(16)))
  uint8_t ostage[4][16 * (DT == DT_F32 ? kStageRowF32 : kStageRow)];
  uint8_t* ost = ostage[threadIdx.x >> 6];
  const int olane = threadIdx.x & 63;
  const int oqv = (threadIdx.x >> 2) & 15;
  const int q = threadIdx.x & 3;
  const int quad = threadIdx.x >> 2;
  const LaneSigns ls = lane_signs(q);
  // Final per-element factor: lazy lane sign * fp32(1/sqrt(128)) * s_j.
  float kf[4][8];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      kf[g][i] = (sign_bit(mask, q, g, i) ? -ls.sigma : ls.sigma) * kInvSqrt128;
  // The 24-bit chunk of (q, g) starts at byte 3q + 12g: dword 3g + (3q >> 2),
  // bit offset 24q mod 32. Only lanes 1 and 2 need the following dword. In a
  // record lane 3's spare read of group 3 lands on the norm; with split arrays
  // lanes 0 and 3 read their own dword twice, so no read leaves the 48 bytes.
  const int dsel = (3 * q) >> 2;
  const int dsel_hi = (!SPLIT || q == 1 || q == 2) ? dsel + 1 : dsel;
  const uint32_t shift = (24u * q) & 31u;

  const int64_t step = (int64_t)gridDim.x * kTq3VecPerBlock;
  // This lane's words of a record: two dwords per 24-bit group, norm/scale.
  struct RecRaw {
    uint32_t lo[4], hi[4];
    uint2 ns;
  };
  auto fetch = [&](int64_t vv) {
    RecRaw rr;
    const uint32_t* r32 = reinterpret_cast<const uint32_t*>(rec + vv * (SPLIT ? 48 : 56));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      rr.lo[g] = r32[3 * g + dsel];
      rr.hi[g] = r32[3 * g + dsel_hi];
    }
    if constexpr (SPLIT)
      rr.ns = make_uint2(as_u(norms_in[vv]), as_u(scales_in[vv]));
    else
      rr.ns = *reinterpret_cast<const uint2*>(rec + vv * 56 + 48);
    return rr;
  };
  int64_t v = (int64_t)blockIdx.x * kTq3VecPerBlock + quad;
  RecRaw nxt;
  if (PF && v < n_vec) nxt = fetch(v);
  for (; v < n_vec; v += step) {
    RecRaw cur;
    if constexpr (PF) {
      cur = nxt;
      nxt = fetch(v + step < n_vec ? v + step : v);
    } else {
      cur = fetch(v);
    }
    uint32_t chunk[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      chunk[g] = (uint32_t)((((uint64_t)cur.hi[g] << 32) | cur.lo[g]) >> shift) & 0xffffffu;
    const uint2 ns = cur.ns;
    const float norm = as_f(ns.x), scale = as_f(ns.y);

    // Byte offset of the pair entry of elements 2p, 2p + 1: 8 * (bits 6p ..
    // 6p + 5 of the chunk).
    float w[4][8];
    const char* tb = reinterpret_cast<const char*>(&ptab[0]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t c8 = chunk[g] << 3;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t off = (c8 >> (6 * p)) & 0x1f8u;
        const float2 c = *reinterpret_cast<const float2*>(tb + off);
        w[g][2 * p] = c.x * scale;
        w[g][2 * p + 1] = c.y * scale;
      }
    }

    fwht_low3(w);
    fwht_high4(w, ls.c1, ls.c2);

#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) w[g][i] = (w[g][i] * kf[g][i]) * norm;

    if (DT == DT_F32 && stride == 128 && (v - oqv) + 16 <= n_vec) {
      // fp32 rows: the wave's 8 KB leave as eight coalesced 1 KB stores.
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<u32x4*>(ost + f32_stage_off(oqv, g * 128 + q * 32 + h * 16)) =
              u32x4{as_u(w[g][4 * h]), as_u(w[g][4 * h + 1]), as_u(w[g][4 * h + 2]),
                    as_u(w[g][4 * h + 3])};
      __builtin_amdgcn_wave_barrier();
      uint8_t* dst = static_cast<uint8_t*>(y) + (v - oqv) * 512;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int o = olane * 16 + k * 1024;
        *reinterpret_cast<u32x4*>(dst + o) =
            *reinterpret_cast<const u32x4*>(ost + f32_stage_off(o >> 9, o & 511));
      }
      __builtin_amdgcn_wave_barrier();
    } else if (DT != DT_F32 && stride == 128 && (v - oqv) + 16 <= n_vec) {
      // The wave's 16 consecutive contiguous rows (4 KB) leave as four fully
      // coalesced 1 KB stores instead of sixteen 64-byte pieces per store.
      stage_row16<DT>(ost + oqv * kStageRow, q, w);
      __builtin_amdgcn_wave_barrier();
      uint8_t* dst = static_cast<uint8_t*>(y) + (v - oqv) * 256;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int o = olane * 16 + k * 1024;
        *reinterpret_cast<u32x4*>(dst + o) =
            *reinterpret_cast<const u32x4*>(ost + (o >> 8) * kStageRow + (o & 255));
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      store_row<DT>(y, v, stride, q, w);
    }
  }
}

}  // namespace

// ------------------------------------------------------------- launchers ---

// Iterations per wave from which the software-pipelined dequantize kernel
// pays off.
constexpr int kTq3PipelineMinIters = 16;
// Cap on the blocks per CU of a grid with one block per 64 vectors (so the
// grid stays far inside the 2^31 limit; beyond it the blocks loop).
constexpr int kTq3MaxBlocksPerCu = 1 << 16;

// Quantize grids hold four times the blocks the CUs keep resident (when there
// is that much work): the hardware then dispatches the remaining blocks as
// earlier ones finish, so the waves on a CU drift out of step and one wave's
// loads overlap another's arithmetic. With a resident-sized grid the waves
// start together and load, compute and store in lock-step. Measured on the
// KV layer (524288 bf16 vectors) 48.9 against 52.7 us, and on 2^20 vectors
// it also beat a software-pipelined loop (the next vector's loads issued
// before the current one is processed) by 6-8%.
constexpr int kTq3QuantizeOversubscribe = 4;
// fp32 rows (512 bytes a vector, 4 waves a SIMD): six times, 1.5% faster than
// four times on 2^20 vectors (four interleaved rounds).
constexpr int kTq3QuantizeOversubscribeF32 = 6;

template <int DT, bool SPLIT>
hipError_t tq3_q(const void* x, int64_t n_vec, int64_t stride, const SignMask& m, uint8_t* rec,
                 float* norms, float* scales, int cus, hipStream_t s) {
  static const int per_cu = resident_blocks_per_cu(tq3_quantize_kernel<DT, SPLIT>, 256, 0);
  const int64_t need = (n_vec + kTq3VecPerBlock - 1) / kTq3VecPerBlock;
  constexpr int over = DT == DT_F32 ? kTq3QuantizeOversubscribeF32 : kTq3QuantizeOversubscribe;
  tq3_quantize_kernel<DT, SPLIT><<<grid_size(need, cus, per_cu * over), 256, 0, s>>>(
      x, n_vec, stride, m, rec, norms, scales);
  return hipGetLastError();
}

template <int DT, bool SPLIT>
hipError_t tq3_dq(const uint8_t* rec, const float* norms, const float* scales, int64_t n_vec,
                  const SignMask& m, void* y, int64_t stride, int cus, hipStream_t s) {
  static const int per_cu =
      resident_blocks_per_cu(tq3_dequantize_kernel<DT, false, SPLIT>, 256, 0);
  static const int per_cu_pf =
      DT == DT_F32 ? 0 : resident_blocks_per_cu(tq3_dequantize_kernel<DT, true, SPLIT>, 256, 0);
  const int64_t need = (n_vec + kTq3VecPerBlock - 1) / kTq3VecPerBlock;
  const int grid_pf = grid_size(need, cus, per_cu_pf);
  if constexpr (DT == DT_F32) {
    // fp32 rows (512 bytes a vector): one block per 64 vectors, no
    // grid-stride loop. Measured on 2^20 vectors against the pipelined loop:
    // 117.5-118.3 against 121.8-122.5 us (for 16-bit rows the same grid is
    // 10-16% slower than the loops below).
    tq3_dequantize_kernel<DT, false, SPLIT>
        <<<grid_size(need, cus, kTq3MaxBlocksPerCu), 256, 0, s>>>(rec, norms, scales, n_vec, m,
                                                                  y, stride);
  } else {
    if (need >= (int64_t)grid_pf * kTq3PipelineMinIters)
      tq3_dequantize_kernel<DT, true, SPLIT>
          <<<grid_pf, 256, 0, s>>>(rec, norms, scales, n_vec, m, y, stride);
    else
      tq3_dequantize_kernel<DT, false, SPLIT>
          <<<grid_size(need, cus, per_cu), 256, 0, s>>>(rec, norms, scales, n_vec, m, y, stride);
  }
  return hipGetLastError();
}

template <bool SPLIT>
hipError_t tq3_q_dt(const void* x, int dt, int64_t n_vec, int64_t stride, const SignMask& m,
                    uint8_t* rec, float* norms, float* scales, int cus, hipStream_t s) {
  switch (dt) {
    case DT_F32: return tq3_q<DT_F32, SPLIT>(x, n_vec, stride, m, rec, norms, scales, cus, s);
    case DT_BF16: return tq3_q<DT_BF16, SPLIT>(x, n_vec, stride, m, rec, norms, scales, cus, s);
    default: return tq3_q<DT_F16, SPLIT>(x, n_vec, stride, m, rec, norms, scales, cus, s);
  }
}

template <bool SPLIT>
hipError_t tq3_dq_dt(const uint8_t* rec, const float* norms, const float* scales, int64_t n_vec,
                     const SignMask& m, void* y, int dt, int64_t stride, int cus,
                     hipStream_t s) {
  switch (dt) {
    case DT_F32: return tq3_dq<DT_F32, SPLIT>(rec, norms, scales, n_vec, m, y, stride, cus, s);
    case DT_BF16: return tq3_dq<DT_BF16, SPLIT>(rec, norms, scales, n_vec, m, y, stride, cus, s);
    default: return tq3_dq<DT_F16, SPLIT>(rec, norms, scales, n_vec, m, y, stride, cus, s);
  }
}

hipError_t launch_tq3_quantize(const void* x, int dt, int64_t n_vec, int64_t stride,
                               const SignMask& m, uint8_t* rec, int cus, hipStream_t s) {
  return tq3_q_dt<false>(x, dt, n_vec, stride, m, rec, nullptr, nullptr, cus, s);
}

hipError_t launch_tq3_dequantize(const uint8_t* rec, int64_t n_vec, const SignMask& m, void* y,
                                 int dt, int64_t stride, int cus, hipStream_t s) {
  return tq3_dq_dt<false>(rec, nullptr, nullptr, n_vec, m, y, dt, stride, cus, s);
}

hipError_t launch_tq3_quantize_split(const void* x, int dt, int64_t n_vec, int64_t stride,
                                     const SignMask& m, uint8_t* packed, float* norms,
                                     float* scales, int cus, hipStream_t s) {
  return tq3_q_dt<true>(x, dt, n_vec, stride, m, packed, norms, scales, cus, s);
}

hipError_t launch_tq3_dequantize_split(const uint8_t* packed, const float* norms,
                                       const float* scales, int64_t n_vec, const SignMask& m,
                                       void* y, int dt, int64_t stride, int cus, hipStream_t s) {
  return tq3_dq_dt<true>(packed, norms, scales, n_vec, m, y, dt, stride, cus, s);
}

}  // namespace tq
