// Shared device helpers for the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// ds_swizzle in quad-permute mode: lane i of every 4-lane quad receives the
// value of quad lane (PERM >> 2i) & 3. It runs on the LDS crossbar and costs
// no VALU issue slot.
constexpr int qperm(int a, int b, int c, int d) {
  return 0x8000 | a | (b << 2) | (c << 4) | (d << 6);
}
constexpr int QP_XOR1 = qperm(1, 0, 3, 2);
constexpr int QP_XOR2 = qperm(2, 3, 0, 1);
constexpr int QP_NEXT = qperm(1, 2, 3, 3);

template <int P>
__device__ __forceinline__ float swz(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), P));
}
template <int P>
__device__ __forceinline__ uint32_t swz(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), P));
}

// 16 butterflies across lanes, one VALU instruction each: v[k] += c *
// v[k](partner), the partner's value read through DPP (CTRL: a quad_perm,
// row_mirror or row_half_mirror control; no LDS crossbar trip). gfx9 needs
// two wait states between a VALU write of a register and a DPP read of it,
// and five after a VALU write of EXEC; the leading s_nop 4 covers both for
// whatever the compiler placed before the block, and no instruction inside
// it reads another one's result.
#define TQ_DPP_FMAC16(CTRL, c, v)                                                \
  asm volatile("s_nop 4\n"                                                       \
               "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"   \
               "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n" \
               "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n" \
               "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n" \
               "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n" \
               "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n" \
               "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n" \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), \
                 "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), \
                 "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                     \
               : "v"(c))

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Quotient a / d rounded to nearest, for a divisor shared by many numerators.
// rh = RN(1/d) (recip_rn); q0 = RN(a*rh) is within 1.5 ulp of a/d; the
// remainder a - d*q0 is exact (one fma), and one correction step
// q = RN(q0 + rem*rh) gives the correctly rounded quotient. (Markstein's
// theorem covers this step for a faithful q0 -- P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 1990; Muller et al., Handbook of Floating-Point Arithmetic -- which
// RN(a*rh) need not be.) Checked exhaustively on the device instead: every
// numerator mantissa against every divisor mantissa, the quotient on both
// sides of 1, 1.4e14 quotients, no mismatch (div_rn_check in
// stream_probe.hip, run by tests/test_gpu_arith_checks.py). Exponent shifts
// scale every step exactly while no step leaves the normal range: the callers
// only use it where |a/d| >= 2^-60 (or a = 0) and 1e-10 <= d <= 2^100.
//
// rh itself: the hardware reciprocal (within an ulp) and one correction with
// the exact residual 1 - d*r0, the same bits as the IEEE quotient 1.0f/d in
// three instructions instead of the division's ten; checked on the device
// for every normal d below 2^126 (recip_rn_check).
__device__ __forceinline__ float recip_rn(float d) {
  const float r0 = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, r0, 1.0f), r0, r0);
}
struct Recip {
  float d, rh;
};
__device__ __forceinline__ Recip make_recip(float d) {
  Recip r;
  r.d = d;
  r.rh = recip_rn(d);
  return r;
}
__device__ __forceinline__ float div_rn(float a, const Recip& r) {
  const float q0 = a * r.rh;
  const float rem = __builtin_fmaf(-q0, r.d, a);
  return __builtin_fmaf(rem, r.rh, q0);
}

// Square root rounded to nearest for x >= 2^-96 (and +inf): the hardware
// square root s (within an ulp) moved to a neighbour when the exact residual
// x - s'*s of that neighbour s' says so -- the correction of the IEEE
// sequence without its rescaling of tiny inputs. A caller that clamps the
// result to at least 1e-8 may pass any x >= 0: below 2^-96 every candidate is
// below the clamp. Checked on the device against the IEEE square root for
// every x in [2^-96, 2^128) (sqrt_rn_check in stream_probe.hip).
__device__ __forceinline__ float sqrt_rn_large(float x) {
  const float s = __builtin_amdgcn_sqrtf(x);
  const float sm = as_f(as_u(s) - 1u), sp = as_f(as_u(s) + 1u);
  float r = __builtin_fmaf(-sm, s, x) <= 0.0f ? sm : s;
  r = __builtin_fmaf(-sp, s, x) > 0.0f ? sp : r;
  return r;
}

// Tile (tx, ty) of an nx x ny tiling for block blockIdx.x of a 1-D grid of
// 8 * ceil(nx * ny / 8) blocks. Blocks go to the 8 XCDs round-robin, so block
// b runs on XCD b % 8; the tiles are dealt so that each XCD works through a
// contiguous run of them in row-major order, and the blocks that share a
// row of tiles (the same rows of the left operand) share that XCD's L2.
// Returns false for the blocks past the last tile.
__device__ __forceinline__ bool xcd_tile(int nx, int ny, int& tx, int& ty) {
  const int tiles = nx * ny;
  const int per = (tiles + 7) / 8;
  const int b = (int)blockIdx.x;
  const int t = (b % 8) * per + b / 8;
  if (t >= tiles) return false;
  ty = t / nx;
  tx = t - ty * nx;
  return true;
}
inline unsigned xcd_grid(int64_t nx, int64_t ny) { return (unsigned)(8 * ((nx * ny + 7) / 8)); }

// acc * 2 + (this lane's bit of the wave mask `bits`): one add with carry-in,
// so a wave-wide compare result enters a lane's bit field at one VALU op.
__device__ __forceinline__ uint32_t shift_in(uint32_t acc, uint64_t bits) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(acc), "s"(bits));
  return r;
}

}  // namespace tq
