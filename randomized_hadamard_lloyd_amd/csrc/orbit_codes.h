// Reading OrbitQuant code streams ("zerogpu-sdxlTrainer:
// toolkit/util/orbit_quant.py", pack_codes / unpack_codes): 16 consecutive
// codes of a row occupy 2*BITS bytes of its stream (rows are byte-aligned).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {
namespace {

template <int BITS>
__device__ __forceinline__ uint64_t load_codes(const uint8_t* p) {
  if constexpr (BITS == 2) {
    return *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (BITS == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return (uint64_t)v.x | ((uint64_t)v.y << 32);
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return (uint64_t)q[0] | ((uint64_t)q[1] << 16) | ((uint64_t)q[2] << 32);
  }
}

// The 16 codes of such a 64-bit little-endian chunk, in stream order, for
// MSB-first (the page's layout) or LSB-first bit order.
template <int BITS, bool LSB>
__device__ __forceinline__ void unpack16(uint64_t acc, uint32_t (&code)[16]) {
  constexpr uint32_t mask = (1u << BITS) - 1;
  if constexpr (LSB) {
#pragma unroll
    for (int i = 0; i < 16; ++i) code[i] = (uint32_t)(acc >> (BITS * i)) & mask;
  } else if constexpr (BITS == 3) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t le = (uint32_t)(acc >> (24 * g)) & 0xffffffu;
      const uint32_t w = (le >> 16) | (le & 0xff00u) | ((le & 0xffu) << 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) code[8 * g + i] = (w >> (21 - 3 * i)) & 7u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = BITS * i;
      const int shift = 8 * (q >> 3) + 8 - (q & 7) - BITS;
      code[i] = (uint32_t)(acc >> shift) & mask;
    }
  }
}

// Code pairs of a 64-bit chunk of 16 codes (stream order), as table indices:
// the pair's bits as they sit in the stream, (a << BITS) | b for MSB-first
// and a | (b << BITS) for LSB-first (a = the earlier code).
template <int BITS, bool LSB>
__device__ __forceinline__ void pairs16(uint64_t acc, uint32_t (&pi)[8]) {
  constexpr uint32_t mask = (1u << (2 * BITS)) - 1;
  if constexpr (LSB) {
#pragma unroll
    for (int p = 0; p < 8; ++p) pi[p] = (uint32_t)(acc >> (2 * BITS * p)) & mask;
  } else if constexpr (BITS == 3) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t le = (uint32_t)(acc >> (24 * g)) & 0xffffffu;
      const uint32_t w = (le >> 16) | (le & 0xff00u) | ((le & 0xffu) << 16);
#pragma unroll
      for (int p = 0; p < 4; ++p) pi[4 * g + p] = (w >> (18 - 6 * p)) & mask;
    }
  } else {
    // BITS = 2: each byte holds two pairs, the earlier in its high half
#pragma unroll
    for (int p = 0; p < 8; ++p) pi[p] = (uint32_t)(acc >> (8 * (p >> 1) + 4 - 4 * (p & 1))) & mask;
  }
}

}  // namespace
}  // namespace tq
