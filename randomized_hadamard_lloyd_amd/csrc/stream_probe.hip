// Measurement probes (not part of the codec library): the memory traffic of
// the TQ3 kernels with no arithmetic, to measure what HBM gives each access
// pattern on this part, built into libtqprobe.so and timed by bench.py; and
// exhaustive device checks of the reciprocal, division and square root the
// codec kernels use.
//
//   kind 0 (quantize pattern): each 4-lane quad reads one 256-byte bf16 row
//     with four 16-byte loads per lane and writes one 56-byte record (lanes
//     0-2: one dword per 12-byte group; lane 3: 8 bytes), as
//     tq3_quantize_kernel does.
//   kind 1 (dequantize pattern): each quad reads one record with the
//     dequantize kernel's loads (two 8-byte words per lane, plus the 8-byte
//     norm and scale) and each wave writes its 16 consecutive 256-byte rows
//     as four 1 KB stores.
// The values written are a cheap function of the values read, so no load can
// be dropped. Every access stays inside n_vec rows / records.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_common.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_quantize_pattern(const uint16_t* __restrict__ x,
                                                              uint8_t* __restrict__ rec,
                                                              int64_t n) {
  const int q = threadIdx.x & 3;
  const int64_t step = (int64_t)gridDim.x * 64;
  for (int64_t v = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2); v < n; v += step) {
    const uint16_t* r = x + v * 128 + 8 * q;
    uint32_t s = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(r + 32 * g);
      s ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    uint8_t* out = rec + v * 56;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (q < 3) *reinterpret_cast<uint32_t*>(out + 12 * g + 4 * q) = s + g;
    if (q == 3) *reinterpret_cast<uint2*>(out + 48) = make_uint2(s, s + 1);
  }
}

__global__ __launch_bounds__(256) void probe_dequantize_pattern(const uint8_t* __restrict__ rec,
                                                                u32x4* __restrict__ y,
                                                                int64_t n) {
  const int q = threadIdx.x & 3;
  const int l = threadIdx.x & 63;
  const int64_t step = (int64_t)gridDim.x * 64;
  for (int64_t v = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2); v < n; v += step) {
    const uint2* r = reinterpret_cast<const uint2*>(rec + v * 56);
    const uint2 a = r[q], b = r[q + 3], c = r[6];
    const uint32_t s = a.x ^ a.y ^ b.x ^ b.y ^ c.x ^ c.y;
    const int64_t v0 = v - ((threadIdx.x >> 2) & 15);  // the wave's first row
    if (v0 + 16 <= n) {
      u32x4* dst = y + v0 * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[l + 64 * k] = u32x4{s, s + 1, s + 2, s + 3};
    }
  }
}

// Arithmetic check (not a stream probe): recip_rn against the IEEE quotient
// 1.0f / d for every fp32 d with exponent field 1 .. 252 (every normal d
// below 2^126, where 1/d stays normal) and every mantissa. One thread per
// mantissa, one grid row per exponent; cnt[0] counts the cases, cnt[1] the
// mismatches, cnt[2] the mismatches of the raw hardware reciprocal (which
// shows that the check can see a wrong result).
__global__ __launch_bounds__(256) void recip_rn_check(unsigned long long* __restrict__ cnt) {
  const uint32_t m = blockIdx.x * 256u + threadIdx.x;  // < 2^23
  const uint32_t e = 1u + blockIdx.y;                  // 1 .. 252
  const float d = __builtin_bit_cast(float, (e << 23) | m);
  const float r = tq::recip_rn(d);
  const float r0 = __builtin_amdgcn_rcpf(d);
  const float ref = 1.0f / d;
  unsigned long long bad = __builtin_bit_cast(uint32_t, r) != __builtin_bit_cast(uint32_t, ref);
  unsigned long long raw = __builtin_bit_cast(uint32_t, r0) != __builtin_bit_cast(uint32_t, ref);
  for (int o = 32; o > 0; o >>= 1) {
    bad += __shfl_xor(bad, o);
    raw += __shfl_xor(raw, o);
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&cnt[0], 64ull);
    atomicAdd(&cnt[1], bad);
    atomicAdd(&cnt[2], raw);
  }
}

// Arithmetic check: div_rn against the IEEE quotient a / d. One thread per
// divisor mantissa (d in [1, 2), 2^23 threads); each runs over the numerator
// bit patterns base .. base + span - 1 (inside [1, 4): exponent fields 127
// and 128, so the quotient lies on both sides of 1). cnt[0] counts the
// mismatches. With corrected = 0 the uncorrected product RN(a * rh) is
// checked instead (which shows that the check can see a wrong quotient).
__global__ __launch_bounds__(256) void div_rn_check(unsigned long long* __restrict__ cnt,
                                                    uint32_t base, uint32_t span, int corrected) {
  const uint32_t mn = blockIdx.x * 256u + threadIdx.x;  // < 2^23
  const tq::Recip r = tq::make_recip(__builtin_bit_cast(float, (127u << 23) | mn));
  unsigned long long bad = 0;
  for (uint32_t j = 0; j < span; ++j) {
    const float a = __builtin_bit_cast(float, base + j);
    const float q = corrected ? tq::div_rn(a, r) : a * r.rh;
    bad += __builtin_bit_cast(uint32_t, q) != __builtin_bit_cast(uint32_t, a / r.d);
  }
  for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(&cnt[0], bad);
}

// Arithmetic check: sqrt_rn_large against the IEEE square root for every x
// with exponent field 31 .. 254 (x in [2^-96, 2^128)) and every mantissa,
// plus +inf. cnt[0] counts the cases, cnt[1] the mismatches, cnt[2] the
// mismatches of the raw hardware square root.
__global__ __launch_bounds__(256) void sqrt_rn_check(unsigned long long* __restrict__ cnt) {
  const uint32_t m = blockIdx.x * 256u + threadIdx.x;  // < 2^23
  const uint32_t e = 31u + blockIdx.y;                 // 31 .. 254
  const bool inf = blockIdx.y == 224;                  // one extra row: +inf
  const float x = __builtin_bit_cast(float, inf ? 0x7f800000u : (e << 23) | m);
  const float r = tq::sqrt_rn_large(x), ref = __builtin_sqrtf(x);
  const float raw = __builtin_amdgcn_sqrtf(x);
  const bool one = !inf || m == 0;  // the inf row counts one case
  unsigned long long c = one;
  unsigned long long bad = one && __builtin_bit_cast(uint32_t, r) != __builtin_bit_cast(uint32_t, ref);
  unsigned long long rb = one && __builtin_bit_cast(uint32_t, raw) != __builtin_bit_cast(uint32_t, ref);
  for (int o = 32; o > 0; o >>= 1) {
    c += __shfl_xor(c, o);
    bad += __shfl_xor(bad, o);
    rb += __shfl_xor(rb, o);
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&cnt[0], c);
    atomicAdd(&cnt[1], bad);
    atomicAdd(&cnt[2], rb);
  }
}

}  // namespace

extern "C" {

// Runs sqrt_rn_check on `stream`: cnt = 3 zeroed 64-bit device counters.
int tqprobe_sqrt_check(unsigned long long* cnt, void* stream) {
  if (!cnt) return 1;
  sqrt_rn_check<<<dim3((1u << 23) / 256, 225), 256, 0, static_cast<hipStream_t>(stream)>>>(cnt);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Runs div_rn_check over numerators base .. base + span - 1 (bit patterns in
// [1, 4)) for every divisor mantissa; cnt = one zeroed 64-bit device counter.
// Returns 0, 1 for bad arguments, 2 if the launch failed.
int tqprobe_div_check(unsigned long long* cnt, uint32_t base, uint32_t span, int corrected,
                      void* stream) {
  if (!cnt || span == 0 || base < (127u << 23) || span > (129u << 23) - base) return 1;
  div_rn_check<<<(1u << 23) / 256, 256, 0, static_cast<hipStream_t>(stream)>>>(cnt, base, span,
                                                                              corrected);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Runs recip_rn_check on `stream`: cnt = 3 zeroed 64-bit device counters.
// Returns 0, 1 for a null pointer, 2 if the launch failed.
int tqprobe_recip_check(unsigned long long* cnt, void* stream) {
  if (!cnt) return 1;
  recip_rn_check<<<dim3((1u << 23) / 256, 252), 256, 0, static_cast<hipStream_t>(stream)>>>(cnt);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Enqueue one probe launch of `grid` 256-thread blocks on `stream`.
// kind 0: `in` = n_vec bf16 rows of 128 (16-byte aligned), `out` = n_vec
// records of 56 bytes (8-byte aligned). kind 1: `in` = n_vec records, `out`
// = n_vec rows of 128 bf16 (16-byte aligned); n_vec a multiple of 16.
// Returns 0, or 1 for bad arguments, 2 if the launch failed.
int tqprobe_stream(int kind, const void* in, void* out, int64_t n_vec, int grid,
                   void* stream) {
  if (!in || !out || n_vec <= 0 || grid <= 0 || (kind != 0 && kind != 1)) return 1;
  if (kind == 1 && n_vec % 16 != 0) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    probe_quantize_pattern<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(in),
                                                static_cast<uint8_t*>(out), n_vec);
  else
    probe_dequantize_pattern<<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(in),
                                                  static_cast<u32x4*>(out), n_vec);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
