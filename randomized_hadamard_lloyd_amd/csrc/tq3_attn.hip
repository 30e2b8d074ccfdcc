// Decode attention over a TQ3-compressed KV cache for gfx950: the consumer of
// the "ComfyUI-TurboQuant: tq3_core.py" codec (module docstring: TQ3 holds
// the K and V vectors of a KV cache). One query token per head attends to T
// cached tokens whose K and V vectors are 56-byte records.
//
// Rotated-domain evaluation. tq3_dequantize reconstructs a vector as
//   v = norm * S (K H (scale * c)),   c_j = C[idx_j],
// with S the sign flips, H the unnormalised 128-point Hadamard matrix and
// K = fp32(1/sqrt(128)). S and H are symmetric, so
//   <q, v> = norm * scale * <K H S q, c>   and
//   sum_t p_t v_t = S K H (sum_t p_t norm_t scale_t c_t).
// Each query is rotated once (qr = K H S q, times softmax_scale and log2(e)
// so that exp2 gives the softmax weights); a score reads only a K record's
// indices and its two scalars; values are accumulated in the rotated domain;
// one inverse rotation per head finishes the output. No per-token transform.
//
// Work mapping. A group of 16 lanes owns one token at a time: lane r holds
// elements 8r .. 8r+7, i.e. its 24 bits of each record's indices. A
// 256-thread block (16 groups) handles one KV head over one chunk of tokens
// for the G query heads that share that KV head, each group keeping a running
// (max, sum, accumulator) per head (the online softmax). A group's partial
// scores are reduce-scattered over its lanes, so that each lane finishes one
// score and its softmax step. The block merges its groups and writes one
// partial per head; a second kernel merges the chunks, normalises, rotates
// back and stores.
#include "tq_common.h"
#include "tq_kernels.h"

#include <mutex>
#include <utility>

// Library-held partial results for tq3_decode_attention_noalloc: one copy per
// GPU, alive until the process ends. Host code never passes this name to a
// kernel (on the host it is a stand-in, not a device address); it uses the
// per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[tq::kAttnScratchBytes / sizeof(float)];

namespace tq {

namespace {

constexpr float kInvSqrt128A = (float)0.08838834764831845;  // fp32(1/sqrt(128))

__device__ __forceinline__ float tq3_centroid_a(int k) {
  constexpr float c[8] = {(float)-0.9816, (float)-0.6168, (float)-0.3479, (float)-0.1129,
                          (float)0.1129,  (float)0.3479,  (float)0.6168,  (float)0.9816};
  return c[k];
}

// Butterfly with the partner lane r ^ (1 << S): lower lane a + b, upper lane
// a - b (exact signs: fma(own, -1, partner) = partner - own).
template <int S>
__device__ __forceinline__ float lane_butterfly(float own, float c) {
  const int iv = __builtin_bit_cast(int, own);
  int o;
  if constexpr (S == 0) o = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, false);
  else if constexpr (S == 1) o = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, false);
  else if constexpr (S == 2) o = __builtin_amdgcn_ds_swizzle(iv, (4 << 10) | 0x1F);
  else o = __builtin_amdgcn_ds_swizzle(iv, (8 << 10) | 0x1F);
  return __builtin_fmaf(own, c, __builtin_bit_cast(float, o));
}

// Lane r's 8 elements of a 128-vector, in a 16-lane group: the unnormalised
// Hadamard transform (in registers for index bits 0-2, across the group's
// lanes for bits 3-6).
__device__ __forceinline__ void group_fwht(float (&x)[8], int r) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  const float c0 = (r & 1) ? -1.0f : 1.0f, c1 = (r & 2) ? -1.0f : 1.0f;
  const float c2 = (r & 4) ? -1.0f : 1.0f, c3 = (r & 8) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = lane_butterfly<0>(x[i], c0);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = lane_butterfly<1>(x[i], c1);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = lane_butterfly<2>(x[i], c2);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = lane_butterfly<3>(x[i], c3);
}

// Cross-lane reads inside a 16-lane group. The reduction partners of lane r
// are r ^ 1, r ^ 2 (quad_perm), r ^ 7 (row_half_mirror) and r ^ 15
// (row_mirror). In the basis (1, 2, 7, 15) of the lane index, step k's
// partner flips coordinate k alone; that coordinate vector is the lane's
// label: c3 = r3, c2 = r2 ^ r3, c1 = r1 ^ r2, c0 = r0 ^ r2.
template <int K>
__device__ __forceinline__ float group_partner(float v) {
  constexpr int ctrl = K == 0 ? 0xB1 : K == 1 ? 0x4E : K == 2 ? 0x141 : 0x140;
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               ctrl, 0xF, 0xF, true));
}

__device__ __forceinline__ int group_label(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  return (r0 ^ r2) | ((r1 ^ r2) << 1) | ((r2 ^ r3) << 2) | (r3 << 3);
}

// The lane whose label is l: l0 * 1 ^ l1 * 2 ^ l2 * 7 ^ l3 * 15.
constexpr int group_lane_of_label(int l) {
  return ((l & 1) ? 1 : 0) ^ ((l & 2) ? 2 : 0) ^ ((l & 4) ? 7 : 0) ^ ((l & 8) ? 15 : 0);
}

// Value v of lane LANE of this lane's 16-lane group (row_newbcast).
template <int LANE>
__device__ __forceinline__ float group_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x150 + LANE, 0xF, 0xF, true));
}

// Group sums of S partial values (S = 4, 8, 16), scattered by label: a lane
// with label c enters value f at position f ^ (c % S) and returns the group
// sum of value c % S. Step k (k < log2 S) pairs positions 2i and 2i + 1: the
// even one holds a value whose index bit k is the lane's own label bit k,
// and the partner (label bit k flipped) holds that same value at the odd
// position, so one DPP add per pair keeps it and halves the array, which
// then again holds value f at position (f >> (k + 1)) ^ (c % S >> (k + 1)).
// For S < 16 the remaining steps are plain sums with partners that hold the
// same value, so the 16 / S copies of each sum are identical.
template <int S>
__device__ __forceinline__ float group_reduce_scatter(float (&v)[S]) {
  static_assert(S == 4 || S == 8 || S == 16, "4, 8 or 16 values");
#pragma unroll
  for (int j = 0; j < S / 2; ++j) v[j] = v[2 * j] + group_partner<0>(v[2 * j + 1]);
#pragma unroll
  for (int j = 0; j < S / 4; ++j) v[j] = v[2 * j] + group_partner<1>(v[2 * j + 1]);
  if constexpr (S >= 8) {
#pragma unroll
    for (int j = 0; j < S / 8; ++j) v[j] = v[2 * j] + group_partner<2>(v[2 * j + 1]);
  } else {
    v[0] = v[0] + group_partner<2>(v[0]);
  }
  if constexpr (S == 16) v[0] = v[0] + group_partner<3>(v[1]);
  else v[0] = v[0] + group_partner<3>(v[0]);
  return v[0];
}

// f(integral_constant<0>), ..., f(integral_constant<N-1>): unrolled with the
// index usable as a template argument.
template <class F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// Sign of element j = 8r + i from the 128-bit mask (the word is selected
// from the scalar kernel arguments, not loaded per lane).
__device__ __forceinline__ bool mask_bit(const SignMask& m, int r, int i) {
  // readfirstlane keeps the four words in scalar registers (a select on
  // them is otherwise turned back into a per-lane load)
  const uint32_t w0 = __builtin_amdgcn_readfirstlane(m.w[0]);
  const uint32_t w1 = __builtin_amdgcn_readfirstlane(m.w[1]);
  const uint32_t w2 = __builtin_amdgcn_readfirstlane(m.w[2]);
  const uint32_t w3 = __builtin_amdgcn_readfirstlane(m.w[3]);
  const uint32_t w = (r & 8) ? ((r & 4) ? w3 : w2) : ((r & 4) ? w1 : w0);
  return (w >> (8 * (r & 3) + i)) & 1u;
}

// This lane's 24 index bits and the (norm, scale) pair of one record.
struct RecPart {
  uint32_t lo, hi;
  uint2 ns;
};

// From a record staged in LDS (16 dwords per record).
__device__ __forceinline__ RecPart lds_part(const uint32_t* rec, int dsel) {
  RecPart p;
  p.lo = rec[dsel];
  p.hi = rec[dsel + 1];
  p.ns = *reinterpret_cast<const uint2*>(rec + 12);
  return p;
}

// Centroid values of this lane's 8 elements: each 6-bit field (two indices)
// selects one 8-byte entry of the pair table.
__device__ __forceinline__ void decode8(const RecPart& p, uint32_t shift, const char* tb,
                                        float (&c)[8]) {
  const uint32_t c8 = (uint32_t)((((uint64_t)p.hi << 32) | p.lo) >> shift) << 3;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float2 v = *reinterpret_cast<const float2*>(tb + ((c8 >> (6 * k)) & 504u));
    c[2 * k] = v.x;
    c[2 * k + 1] = v.y;
  }
}

// Floats per (head, chunk) partial: max, sum, 2 pad, 128 accumulators.
constexpr int kPartFloats = 132;
constexpr int kAttnGroups = 16;        // 16-lane groups per 256-thread block
constexpr int kAttnTokPerGroup = 16;   // token slots per group: pieces of up to 256 tokens
#ifndef ATTN_TB
// tokens per iteration sharing one max update: G TB = 4, 8 or 16 scores,
// reduce-scattered over a group's 16 lanes
#define ATTN_TB(G) ((G) <= 4 ? 4 : 2)
#endif
#ifndef ATTN_WIN
// token slots whose record loads are in flight: fewer for many heads, whose
// scores and accumulators take the registers
#define ATTN_WIN(G) ((G) <= 2 ? 8 : 4)
#endif

// MULTI: chunks of more than one piece (256 tokens); the single-piece
// instantiation keeps fewer registers live.
template <int QDT, int G, bool MULTI>
__global__ __launch_bounds__(256) void tq3_attn_partial_kernel(
    const void* __restrict__ q, const uint8_t* __restrict__ krec,
    const uint8_t* __restrict__ vrec, int64_t n_tok, int hkv, SignMask mask, float qscale,
    int chunk, int nchunk, float* __restrict__ ws) {
  __shared__ float2 ctab[64];  // (C[p & 7], C[p >> 3]): two consecutive elements' values
  __shared__ __attribute__((aligned(16))) float red_m[G][16];
  __shared__ __attribute__((aligned(16))) float red_l[G][16];
  // Per wave, its groups' records: [token k][K, V][group in wave][16 dwords]
  // (14 used). Also holds the rotated queries before the loop and the
  // groups' weighted accumulators in the final merge.
  __shared__ __attribute__((aligned(16))) uint32_t stage[4][kAttnTokPerGroup][2][4][16];
  // (chunk, KV head) pairs in row-major runs per XCD: the blocks that read
  // the same cache lines of the token-major records (the KV heads of one
  // token) share an L2.
  int kv, ch;
  if (!xcd_tile(hkv, nchunk, kv, ch)) return;
  const int grp = threadIdx.x >> 4, r = threadIdx.x & 15;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x < 64)
    ctab[threadIdx.x] = make_float2(tq3_centroid_a(threadIdx.x & 7), tq3_centroid_a(threadIdx.x >> 3));
  __syncthreads();  // ctab

  // Group g < G rotates query head g: lane r loads its elements 8r .. 8r+7
  // before the records, so that waiting for them never waits for the record
  // copies.
  uint4 qraw[2] = {};
  if (grp < G) {
    const int64_t off = (int64_t)(kv * G + grp) * 128 + 8 * r;
    if constexpr (QDT == DT_F32) {
      qraw[0] = *reinterpret_cast<const uint4*>(static_cast<const float*>(q) + off);
      qraw[1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(q) + off + 4);
    } else {
      qraw[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + off);
    }
  }

  // The block's chunk [c0, c1) goes by in pieces [t0, t1) of up to 256
  // tokens (16 slots per group). This wave's records, one dword per lane and
  // record (lane 16a + d holds dword min(d, 13) of group a's record), K and
  // V, through a window of kAttnWin token slots in registers: slots past the
  // piece's end re-read a record of the piece (below), never used. Each slot
  // goes to LDS just before the loop reads it, and its registers then load
  // the slot kAttnWin later, so the loop waits only for the loads of the
  // slots it reaches while the next ones stay in flight. (Copies straight
  // into LDS would not overlap: the compiler waits for every such copy
  // before any later LDS read.)
  const int64_t c0 = (int64_t)ch * chunk;
  const int64_t c1 = c0 + chunk < n_tok ? c0 + chunk : n_tok;
  constexpr int kPiece = kAttnGroups * kAttnTokPerGroup;
  int64_t t0 = c0, t1 = c0 + kPiece < c1 ? c0 + kPiece : c1;
  constexpr int kAttnWin = ATTN_WIN(G);
  uint32_t kraw[kAttnWin], vraw[kAttnWin];
  const int rd = (lane & 15) < 14 ? (lane & 15) : 13;
  // Record addresses: a base at the piece's first token (uniform) plus a
  // 32-bit byte offset per lane (at most 255 tokens x 65535 KV heads x 56
  // bytes). Slots past the lane's last token of the piece re-read that
  // token's record (token t0's, if it has none); such slots are never used.
  const uint32_t rstride = (uint32_t)hkv * 56u;  // bytes from a token's record to the next
  const uint32_t lane_tok = 4 * wave + (lane >> 4);  // this lane's token within a slot
  const uint8_t* kb;
  const uint8_t* vb;
  uint32_t soff0, omax;
  auto set_piece = [&]() {
    kb = krec + (t0 * hkv + kv) * 56;
    vb = vrec + (t0 * hkv + kv) * 56;
    const uint32_t ntk = (uint32_t)(t1 - t0);  // 1 .. 256
    const uint32_t nval = lane_tok < ntk ? (ntk - lane_tok + 15) / 16 : 0;
    soff0 = lane_tok * rstride + 4 * rd;
    omax = nval > 0 ? soff0 + (nval - 1) * 16u * rstride : 4u * rd;
  };
  auto load_slot = [&](int k) {
    uint32_t o = soff0 + (uint32_t)k * 16u * rstride;
    o = o < omax ? o : omax;
    kraw[k % kAttnWin] = *reinterpret_cast<const uint32_t*>(kb + o);
    vraw[k % kAttnWin] = *reinterpret_cast<const uint32_t*>(vb + o);
    // keeps the loads in slot order, as the loop's waits assume
    asm volatile("" ::: "memory");
  };
  set_piece();
#pragma unroll
  for (int k = 0; k < kAttnWin; ++k) load_slot(k);

  // Rotated query head grp (groups below G): lane r's elements 8r .. 8r+7.
  float* qs = reinterpret_cast<float*>(&stage[0][0][0][0][0]);  // [G][128] rotated queries
  if (grp < G) {
    float x[8];
    if constexpr (QDT == DT_F32) {
      const uint4 a = qraw[0], b = qraw[1];
      x[0] = as_f(a.x); x[1] = as_f(a.y); x[2] = as_f(a.z); x[3] = as_f(a.w);
      x[4] = as_f(b.x); x[5] = as_f(b.y); x[6] = as_f(b.z); x[7] = as_f(b.w);
    } else {
      const uint4 a = qraw[0];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (QDT == DT_BF16) {
          x[2 * p] = as_f(w[p] << 16);
          x[2 * p + 1] = as_f(w[p] & 0xffff0000u);
        } else {
          x[2 * p] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[p] & 0xffffu));
          x[2 * p + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[p] >> 16));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (mask_bit(mask, r, i)) x[i] = -x[i];
    group_fwht(x, r);
#pragma unroll
    for (int i = 0; i < 8; i += 4)
      *reinterpret_cast<float4*>(qs + grp * 128 + 8 * r + i) =
          make_float4(x[i] * qscale, x[i + 1] * qscale, x[i + 2] * qscale, x[i + 3] * qscale);
  }

  // Token slots k = 0, 1, ... of this group (token t0 + grp + 16 k), TB per
  // iteration. The S = G TB scores of an iteration (index h TB + u) are
  // reduce-scattered over the group by lane label c: the lane finishes score
  // c % S (head hl, token ul) and scales, masks and exponentiates it alone;
  // a head's maximum and sum are over the TB lanes whose labels differ in
  // the low bits, and each weight reaches the value FMAs of every lane by a
  // broadcast from the lane that holds it. For S < 16 the merge reads the
  // lanes with labels below S (the other copies are identical).
  constexpr int TB = ATTN_TB(G);
  constexpr int S = G * TB;
  static_assert(TB == 2 || TB == 4, "a head's tokens are neighbours in the label");
  const int lab = group_label(r) & (S - 1);
  const int hl = lab / TB, ul = lab % TB;
  const bool first_copy = group_label(r) < S;

  // The rotated queries in this lane's order: position h' holds head
  // h' ^ hl, so that partial score h' TB + u' is value (h' TB + u') ^ lab
  // (the tokens are permuted the same way when read from LDS).
  float qr[G][8];
  __syncthreads();  // qs
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(qs + (h ^ hl) * 128 + 8 * r + i);
      qr[h][i] = a.x; qr[h][i + 1] = a.y; qr[h][i + 2] = a.z; qr[h][i + 3] = a.w;
    }
  __syncthreads();  // before the loop's first slot writes

  const int dsel = (3 * r) >> 2;
  const uint32_t shift = (24u * r) & 31u;
  float m_own = -__builtin_inff(), l_own = 0.0f, acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.0f;
  const char* tb = reinterpret_cast<const char*>(ctab);
  const uint32_t* my = &stage[wave][0][0][grp & 3][0];
  for (;;) {
    const int nk = (int)((t1 - t0 + kAttnGroups - 1) / kAttnGroups);  // token slots per group
    // this group's tokens: the first nkg slots (groups differ by at most one)
    const int nkg = (int)((t1 - t0 - grp + kAttnGroups - 1) / kAttnGroups);
#pragma unroll
    for (int it = 0; it < kAttnTokPerGroup / TB; ++it) {
      const int k0 = it * TB;
      if (k0 >= nkg) break;
      // this iteration's slots -> LDS (only this wave reads them); their
      // registers then fetch the slots kAttnWin later
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        (&stage[wave][k0 + u][0][0][0])[lane] = kraw[(k0 + u) % kAttnWin];
        (&stage[wave][k0 + u][1][0][0])[lane] = vraw[(k0 + u) % kAttnWin];
        if (k0 + u + kAttnWin < kAttnTokPerGroup) load_slot(k0 + u + kAttnWin);
      }
      const int64_t tb0 = t0 + grp + (int64_t)kAttnGroups * k0;
      // a loaded slot for token u of the iteration (finite values)
      auto slot = [&](int u) { return k0 + u < nk ? k0 + u : nk - 1; };
      // partial scores of this lane's 8 elements, in its order, then its
      // own score in base-2 logits (-inf past the end)
      float s;
      {
        float sc[S];
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          float ck[8];
          decode8(lds_part(my + slot(u ^ ul) * 128, dsel), shift, tb, ck);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float dot = qr[h][0] * ck[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) dot = __builtin_fmaf(qr[h][i], ck[i], dot);
            sc[h * TB + u] = dot;
          }
        }
        s = group_reduce_scatter<S>(sc);
        const uint2 kns = *reinterpret_cast<const uint2*>(my + slot(ul) * 128 + 12);
        const bool valid = tb0 + kAttnGroups * ul < t1;
        s = valid ? s * (as_f(kns.x) * as_f(kns.y)) : -__builtin_inff();
      }
      // online softmax: the head's maximum over its TB tokens; one update
      float bm = __builtin_amdgcn_fmed3f(s, group_partner<0>(s), __builtin_inff());
      if constexpr (TB == 4) bm = __builtin_amdgcn_fmed3f(bm, group_partner<1>(bm), __builtin_inff());
      if (__builtin_amdgcn_ballot_w64(bm > m_own)) {
        // some group of the wave has a new maximum: rescale (corr = 1 elsewhere)
        const float mn = __builtin_amdgcn_fmed3f(m_own, bm, __builtin_inff());
        const float corr = __builtin_amdgcn_exp2f(m_own - mn);
        l_own = l_own * corr;
        m_own = mn;
        unroll<G>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const float c = group_bcast<group_lane_of_label(h * TB)>(corr);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = acc[h][i] * c;
        });
      }
      const float p = __builtin_amdgcn_exp2f(s - m_own);  // 0 past the end
      l_own = l_own + p;
      const uint2 vns = *reinterpret_cast<const uint2*>(my + slot(ul) * 128 + 64 + 12);
      const float pw = p * (as_f(vns.x) * as_f(vns.y));
      // values: every lane's 8 elements of each token, weights from their lanes
      unroll<TB>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        float cv[8];
        decode8(lds_part(my + slot(u) * 128 + 64, dsel), shift, tb, cv);
        unroll<G>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const float w = group_bcast<group_lane_of_label(h * TB + u)>(pw);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = __builtin_fmaf(w, cv[i], acc[h][i]);
        });
      });
      // keeps the next iteration's slot writes (and so the waits for their
      // loads) from moving up into this one
      asm volatile("" ::: "memory");
    }
    // the next piece of the chunk (its slots reuse this wave's LDS rows, which
    // its own reads above have finished with)
    if constexpr (!MULTI) break;
    t0 = t1;
    if (t0 >= c1) break;
    t1 = t0 + kPiece < c1 ? t0 + kPiece : c1;
    set_piece();
#pragma unroll
    for (int k = 0; k < kAttnWin; ++k) load_slot(k);
  }

  // Merge the 16 groups: weights 2^(m_g - M), zero for groups that saw no
  // token (m = -inf). Up to four heads per pass: the pass's weighted
  // accumulators fill the staging area, then thread t sums outputs
  // t, t + 256, ... over the groups in group order, and the 16 lanes of row
  // hh sum head hh's softmax terms.
  float lh = l_own + group_partner<0>(l_own);  // each head's softmax sum over its TB lanes
  if constexpr (TB == 4) lh = lh + group_partner<1>(lh);
  if (first_copy && ul == 0) {
    red_m[hl][grp] = m_own;
    red_l[hl][grp] = lh;
  }
  __syncthreads();
  constexpr int HP = G < 4 ? G : 4;  // heads per pass
  float* red = reinterpret_cast<float*>(&stage[0][0][0][0][0]);  // [HP][16 groups][128]
  static_assert(sizeof(stage) >= HP * 16 * 128 * sizeof(float), "a pass fits the staging area");
#pragma unroll
  for (int h0 = 0; h0 < G; h0 += HP) {
    if (h0 > 0) __syncthreads();  // the previous pass's reads of red
    float mx[HP];
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
      const int h = h0 + hh;
      float mg[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v = reinterpret_cast<const float4*>(red_m[h])[k];
        mg[4 * k] = v.x; mg[4 * k + 1] = v.y; mg[4 * k + 2] = v.z; mg[4 * k + 3] = v.w;
      }
      mx[hh] = mg[0];
#pragma unroll
      for (int g = 1; g < 16; ++g) mx[hh] = __builtin_fmaxf(mx[hh], mg[g]);
      const float mh = red_m[h][grp];  // this group's maximum for head h
      const float f = mh == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mh - mx[hh]);
      float* dst = red + (hh * 16 + grp) * 128 + 8 * r;
      *reinterpret_cast<float4*>(dst) =
          make_float4(acc[h][0] * f, acc[h][1] * f, acc[h][2] * f, acc[h][3] * f);
      *reinterpret_cast<float4*>(dst + 4) =
          make_float4(acc[h][4] * f, acc[h][5] * f, acc[h][6] * f, acc[h][7] * f);
    }
    __syncthreads();
#pragma unroll
    for (int o = threadIdx.x; o < HP * 128; o += 256) {
      const int hh = o >> 7, e = o & 127;
      const float* src = red + hh * 16 * 128 + e;
      float a = src[0];
#pragma unroll
      for (int g = 1; g < 16; ++g) a = a + src[g * 128];
      ws[((int64_t)(kv * G + h0 + hh) * nchunk + ch) * kPartFloats + 4 + e] = a;
    }
    if (threadIdx.x < 16 * HP) {
      const int hh = threadIdx.x >> 4;  // one 16-lane row per head; lane r: group r
      float mxh = mx[0];
#pragma unroll
      for (int k = 1; k < HP; ++k)
        if (hh == k) mxh = mx[k];
      const float m = red_m[h0 + hh][r];
      float t = m == -__builtin_inff() ? 0.0f : red_l[h0 + hh][r] * __builtin_amdgcn_exp2f(m - mxh);
      t = t + group_partner<0>(t);
      t = t + group_partner<1>(t);
      t = t + group_partner<2>(t);
      t = t + group_partner<3>(t);
      if (r == 0) {
        float* part = ws + ((int64_t)(kv * G + h0 + hh) * nchunk + ch) * kPartFloats;
        part[0] = mxh;
        part[1] = t;
      }
    }
  }
}

// One 1024-thread block per query head. Slice sl (1024 / S threads, 128 S /
// 1024 elements each, for S slices) merges chunks sl, sl + S, ... with the
// online rule (running maximum, sum and accumulators, rescaled when the
// maximum grows); after one barrier the first wave merges the S slices,
// divides by the softmax sum, runs the inverse rotation (S K H) on its
// 2 x 64 elements -- the stage on element bit 6 in registers, bits 0..5
// across lanes -- and stores.
#ifndef ATTN_SLICES
// 32 slices of 32 threads, four elements each: each slice's chain of merges
// is a quarter as long as with 8 slices of one element per thread (-1 to
// -2 us a call), and the first wave's merge of the slices stays short
#define ATTN_SLICES 32
#endif
constexpr int kCombineSlices = ATTN_SLICES;
constexpr int kSliceElems = 128 * kCombineSlices / 1024;  // elements per thread
template <int ODT>
__global__ __launch_bounds__(1024) void tq3_attn_combine_kernel(const float* __restrict__ ws,
                                                               int nchunk, SignMask mask,
                                                               void* __restrict__ out) {
  __shared__ float sacc[kCombineSlices][128];
  __shared__ float smax[kCombineSlices], ssum[kCombineSlices];
  const int h = blockIdx.x;
  constexpr int kSliceThreads = 128 / kSliceElems;
  const int j = threadIdx.x % kSliceThreads, sl = threadIdx.x / kSliceThreads;
  const float* part = ws + (int64_t)h * nchunk * kPartFloats;
  float m = -__builtin_inff(), l = 0.0f, a[kSliceElems];
#pragma unroll
  for (int e = 0; e < kSliceElems; ++e) a[e] = 0.0f;
#pragma unroll 8
  for (int c = sl; c < nchunk; c += kCombineSlices) {
    const float* pc = part + (int64_t)c * kPartFloats;
    const float mc = pc[0], lc = pc[1];
    float ac[kSliceElems];
#pragma unroll
    for (int e = 0; e < kSliceElems; ++e) ac[e] = pc[4 + j + kSliceThreads * e];
    const float mn = __builtin_fmaxf(m, mc);
    // a chunk never has m = -inf (it holds at least one token), so mn is finite
    const float fo = __builtin_amdgcn_exp2f(m - mn), fc = __builtin_amdgcn_exp2f(mc - mn);
    l = __builtin_fmaf(l, fo, lc * fc);
#pragma unroll
    for (int e = 0; e < kSliceElems; ++e) a[e] = __builtin_fmaf(a[e], fo, ac[e] * fc);
    m = mn;
  }
#pragma unroll
  for (int e = 0; e < kSliceElems; ++e) sacc[sl][j + kSliceThreads * e] = a[e];
  if (j == 0) {
    smax[sl] = m;
    ssum[sl] = l;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  float mx = smax[0];
#pragma unroll
  for (int k = 1; k < kCombineSlices; ++k) mx = __builtin_fmaxf(mx, smax[k]);
  float lt = 0.0f, x0 = 0.0f, x1 = 0.0f;  // elements lane and lane + 64
#pragma unroll
  for (int k = 0; k < kCombineSlices; ++k) {
    // a slice without chunks has m = -inf and weighs 0
    const float f = smax[k] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(smax[k] - mx);
    lt = __builtin_fmaf(ssum[k], f, lt);
    x0 = __builtin_fmaf(sacc[k][lane], f, x0);
    x1 = __builtin_fmaf(sacc[k][lane + 64], f, x1);
  }
  x0 = x0 / lt;
  x1 = x1 / lt;
  // Unnormalised Hadamard transform: element j pairs with j ^ hh, the lower
  // taking the sum and the upper the lower minus itself.
  {
    const float s0 = x0 + x1, d0 = x0 - x1;
    x0 = s0;
    x1 = d0;
  }
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const float p0 = __shfl_xor(x0, 1 << b, 64), p1 = __shfl_xor(x1, 1 << b, 64);
    const bool upper = (lane >> b) & 1;
    x0 = upper ? p0 - x0 : x0 + p0;
    x1 = upper ? p1 - x1 : x1 + p1;
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int jj = lane + 64 * e;
    float o = (e ? x1 : x0) * kInvSqrt128A;
    if ((mask.w[jj >> 5] >> (jj & 31)) & 1u) o = -o;
    if constexpr (ODT == DT_F32) {
      static_cast<float*>(out)[(int64_t)h * 128 + jj] = o;
    } else if constexpr (ODT == DT_BF16) {
      static_cast<__bf16*>(out)[(int64_t)h * 128 + jj] = (__bf16)o;
    } else {
      static_cast<_Float16*>(out)[(int64_t)h * 128 + jj] = (_Float16)o;
    }
  }
}

template <int QDT, int G>
hipError_t launch_partial(const void* q, const uint8_t* k, const uint8_t* v, int64_t n_tok,
                          int hkv, const SignMask& m, float qscale, int chunk, int nchunk,
                          float* ws, hipStream_t s) {
  if (chunk <= kAttnGroups * kAttnTokPerGroup)
    tq3_attn_partial_kernel<QDT, G, false><<<xcd_grid(hkv, nchunk), 256, 0, s>>>(
        q, k, v, n_tok, hkv, m, qscale, chunk, nchunk, ws);
  else
    tq3_attn_partial_kernel<QDT, G, true><<<xcd_grid(hkv, nchunk), 256, 0, s>>>(
        q, k, v, n_tok, hkv, m, qscale, chunk, nchunk, ws);
  return hipGetLastError();
}

template <int QDT>
hipError_t launch_partial_g(int g, const void* q, const uint8_t* k, const uint8_t* v,
                            int64_t n_tok, int hkv, const SignMask& m, float qscale, int chunk,
                            int nchunk, float* ws, hipStream_t s) {
  switch (g) {
    case 1: return launch_partial<QDT, 1>(q, k, v, n_tok, hkv, m, qscale, chunk, nchunk, ws, s);
    case 2: return launch_partial<QDT, 2>(q, k, v, n_tok, hkv, m, qscale, chunk, nchunk, ws, s);
    case 4: return launch_partial<QDT, 4>(q, k, v, n_tok, hkv, m, qscale, chunk, nchunk, ws, s);
    default: return launch_partial<QDT, 8>(q, k, v, n_tok, hkv, m, qscale, chunk, nchunk, ws, s);
  }
}

}  // namespace

AttnPlan tq3_attention_plan(int64_t n_tok, int hkv, int g) {
  // One round of blocks over a 256-CU part: about 1024 (four per CU, as LDS
  // allows) up to 4 heads per KV head, when that gives chunks of at most one
  // piece (256 tokens); longer caches take 768 (three per CU) with chunks of
  // several pieces, so fewer blocks pay the query rotation and the merge.
  // Two per CU (512) at 8 heads, where the registers allow two. At least one
  // token per group (16 per chunk); chunks are multiples of 16 tokens.
  const int64_t max_ch = (n_tok + 15) / 16;
  auto chunk_for = [&](int64_t target) {
    int64_t nch = target / hkv;
    if (nch > max_ch) nch = max_ch;
    if (nch < 1) nch = 1;
    const int64_t c = (n_tok + nch - 1) / nch;
    return (c + 15) / 16 * 16;
  };
  int64_t chunk = chunk_for(g <= 4 ? 1024 : 512);
  if (g <= 4 && chunk > kAttnGroups * kAttnTokPerGroup) chunk = chunk_for(768);
  AttnPlan p;
  p.chunk = chunk;
  p.nchunk = (n_tok + chunk - 1) / chunk;
  return p;
}

size_t tq3_attention_ws_floats(int64_t n_tok, int hq, int hkv) {
  const AttnPlan p = tq3_attention_plan(n_tok, hkv, hkv > 0 ? hq / hkv : 1);
  return (size_t)hq * (size_t)p.nchunk * kPartFloats;
}

hipError_t launch_tq3_attention(const void* q, int qdt, int hq, const uint8_t* k,
                                const uint8_t* v, int64_t n_tok, int hkv, const SignMask& m,
                                float softmax_scale, float* ws, void* out, int odt,
                                hipStream_t s) {
  const int g = hq / hkv;
  const AttnPlan p = tq3_attention_plan(n_tok, hkv, g);
  // log2(e) turns the scores into base-2 logits for exp2; K = fp32(1/sqrt(128))
  // is the forward transform's factor.
  const float qscale = (float)((double)softmax_scale * 1.4426950408889634) * kInvSqrt128A;
  hipError_t e;
  if (qdt == DT_F32)
    e = launch_partial_g<DT_F32>(g, q, k, v, n_tok, hkv, m, qscale, (int)p.chunk, (int)p.nchunk, ws, s);
  else if (qdt == DT_BF16)
    e = launch_partial_g<DT_BF16>(g, q, k, v, n_tok, hkv, m, qscale, (int)p.chunk, (int)p.nchunk, ws, s);
  else
    e = launch_partial_g<DT_F16>(g, q, k, v, n_tok, hkv, m, qscale, (int)p.chunk, (int)p.nchunk, ws, s);
  if (e != hipSuccess) return e;
  if (odt == DT_F32)
    tq3_attn_combine_kernel<DT_F32><<<hq, 1024, 0, s>>>(ws, (int)p.nchunk, m, out);
  else if (odt == DT_BF16)
    tq3_attn_combine_kernel<DT_BF16><<<hq, 1024, 0, s>>>(ws, (int)p.nchunk, m, out);
  else
    tq3_attn_combine_kernel<DT_F16><<<hq, 1024, 0, s>>>(ws, (int)p.nchunk, m, out);
  return hipGetLastError();
}

namespace {
constexpr int kMaxScratchDevices = 64;
float* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
std::once_flag g_scratch_once[kMaxScratchDevices];
}  // namespace

hipError_t attention_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  // Once per device, with that device current (the caller's current device).
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<float*>(p) : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
