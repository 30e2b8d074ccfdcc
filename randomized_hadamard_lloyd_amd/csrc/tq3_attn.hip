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
// (max, sum, accumulator) per head (the online softmax). The block merges its
// groups and writes one partial per head; a second kernel merges the chunks,
// normalises, rotates back and stores.
#include "tq_common.h"
#include "tq_kernels.h"

#include <mutex>

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

// Sums over the 16-lane group, all in registers: DPP partners r ^ 1, r ^ 2
// (quad sums), then r ^ 7 (row_half_mirror: the other quad of the 8-lane
// half) and r ^ 15 (row_mirror: the other half). Every lane ends with the
// same bits, because each pairwise sum is commutative. Four values at once,
// one v_add_f32_dpp per step and value.
// gfx9 needs two wait states between a VALU write of a register and a DPP
// read of it (five after a VALU write of EXEC): the leading s_nop 4 covers
// whatever precedes the block, and inside it each value is read again only
// three instructions after its last write.
#define TQ_DPP_STEP4(CTRL)                                                          \
  "v_add_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n"                 \
  "v_add_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n"                 \
  "v_add_f32_dpp %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n"                 \
  "v_add_f32_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n"
__device__ __forceinline__ void group_allreduce4(float& a, float& b, float& c, float& d) {
  asm volatile("s_nop 4\n" TQ_DPP_STEP4("quad_perm:[1,0,3,2]") TQ_DPP_STEP4("quad_perm:[2,3,0,1]")
                   TQ_DPP_STEP4("row_half_mirror") TQ_DPP_STEP4("row_mirror")
               : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
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
// tokens per iteration sharing one max update (4 heads: 34.6 -> 32.1 us over
// 2 tokens on the 32768-token layer, at 168 VGPRs, still three waves a SIMD)
#define ATTN_TB(G) ((G) <= 4 ? 4 : 2)
#endif
#ifndef ATTN_WIN
// token slots whose record loads are in flight: fewer for many heads, whose
// scores and accumulators take the registers
#define ATTN_WIN(G) ((G) <= 2 ? 8 : 4)
#endif

template <int QDT, int G>
__global__ __launch_bounds__(256) void tq3_attn_partial_kernel(
    const void* __restrict__ q, const uint8_t* __restrict__ krec,
    const uint8_t* __restrict__ vrec, int64_t n_tok, int hkv, SignMask mask, float qscale,
    int chunk, float* __restrict__ ws) {
  __shared__ float2 ctab[64];  // (C[p & 7], C[p >> 3]): two consecutive elements' values
  __shared__ __attribute__((aligned(16))) float red_m[G][16];
  __shared__ __attribute__((aligned(16))) float red_l[G][16];
  // Per wave, its groups' records: [token k][K, V][group in wave][16 dwords]
  // (14 used). Reused by the final merge of the groups' accumulators.
  __shared__ __attribute__((aligned(16))) uint32_t stage[4][kAttnTokPerGroup][2][4][16];
  static_assert(sizeof(stage) >= 16 * 132 * sizeof(float), "merge buffer fits the staging area");
  float (*red_acc)[132] = reinterpret_cast<float (*)[132]>(&stage[0][0][0][0][0]);
  const int kv = blockIdx.y;
  const int nchunk = gridDim.x;
  const int grp = threadIdx.x >> 4, r = threadIdx.x & 15;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x < 64)
    ctab[threadIdx.x] = make_float2(tq3_centroid_a(threadIdx.x & 7), tq3_centroid_a(threadIdx.x >> 3));
  __syncthreads();  // ctab

  // The G heads' query elements 8r .. 8r+7 of lane r, loaded before the
  // records so that waiting for them never waits for the record copies.
  uint4 qraw[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t off = (int64_t)(kv * G + h) * 128 + 8 * r;
    if constexpr (QDT == DT_F32) {
      qraw[h][0] = *reinterpret_cast<const uint4*>(static_cast<const float*>(q) + off);
      qraw[h][1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(q) + off + 4);
    } else {
      qraw[h][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + off);
      qraw[h][1] = qraw[h][0];
    }
  }

  // The block's chunk [c0, c1) goes by in pieces [t0, t1) of up to 256
  // tokens (16 slots per group). This wave's records, one dword per lane and
  // record (lane 16a + d holds dword min(d, 13) of group a's record), K and
  // V, through a window of kAttnWin token slots in registers: slots past the
  // piece's end re-read token t0's record, which is never used. Each slot
  // goes to LDS just before the loop reads it, and its registers then load
  // the slot kAttnWin later, so the loop waits only for the loads of the
  // slots it reaches while the next ones stay in flight. (Copies straight
  // into LDS would not overlap: the compiler waits for every such copy
  // before any later LDS read.)
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = c0 + chunk < n_tok ? c0 + chunk : n_tok;
  constexpr int kPiece = kAttnGroups * kAttnTokPerGroup;
  int64_t t0 = c0, t1 = c0 + kPiece < c1 ? c0 + kPiece : c1;
  constexpr int kAttnWin = ATTN_WIN(G);
  uint32_t kraw[kAttnWin], vraw[kAttnWin];
  const int rd = (lane & 15) < 14 ? (lane & 15) : 13;
  auto load_slot = [&](int k) {
    const int64_t t = t0 + 4 * wave + (lane >> 4) + (int64_t)kAttnGroups * k;
    const int64_t rec = (t < t1 ? t : t0) * hkv + kv;
    kraw[k % kAttnWin] = *reinterpret_cast<const uint32_t*>(krec + rec * 56 + 4 * rd);
    vraw[k % kAttnWin] = *reinterpret_cast<const uint32_t*>(vrec + rec * 56 + 4 * rd);
    // keeps the loads in slot order, as the loop's waits assume
    asm volatile("" ::: "memory");
  };
#pragma unroll
  for (int k = 0; k < kAttnWin; ++k) load_slot(k);

  // Rotated queries: lane r keeps elements 8r .. 8r+7.
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if constexpr (QDT == DT_F32) {
      const uint4 a = qraw[h][0], b = qraw[h][1];
      qr[h][0] = as_f(a.x); qr[h][1] = as_f(a.y); qr[h][2] = as_f(a.z); qr[h][3] = as_f(a.w);
      qr[h][4] = as_f(b.x); qr[h][5] = as_f(b.y); qr[h][6] = as_f(b.z); qr[h][7] = as_f(b.w);
    } else {
      const uint4 a = qraw[h][0];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (QDT == DT_BF16) {
          qr[h][2 * p] = as_f(w[p] << 16);
          qr[h][2 * p + 1] = as_f(w[p] & 0xffff0000u);
        } else {
          qr[h][2 * p] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[p] & 0xffffu));
          qr[h][2 * p + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[p] >> 16));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (mask_bit(mask, r, i)) qr[h][i] = -qr[h][i];
    group_fwht(qr[h], r);
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[h][i] = qr[h][i] * qscale;
  }

  const int dsel = (3 * r) >> 2;
  const uint32_t shift = (24u * r) & 31u;
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -__builtin_inff();
    l[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.0f;
  }
  const char* tb = reinterpret_cast<const char*>(ctab);
  const uint32_t* my = &stage[wave][0][0][grp & 3][0];
  // Token slots k = 0, 1, ... of this group (token t0 + grp + 16 k), TB per
  // iteration; the TB scores of each head share one max update. TB shrinks
  // with G to keep the registers of G heads in budget.
  constexpr int TB = ATTN_TB(G);
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
      RecPart kp[TB], vp[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int ku = k0 + u < nk ? k0 + u : nk - 1;  // a loaded slot (finite values)
        kp[u] = lds_part(my + ku * 128, dsel);
        vp[u] = lds_part(my + ku * 128 + 64, dsel);
      }
      // scores (base-2 logits); -inf for the tokens past the end
      float sc[G][TB];
      {
        float ck[TB][8];
#pragma unroll
        for (int u = 0; u < TB; ++u) decode8(kp[u], shift, tb, ck[u]);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int u = 0; u < TB; ++u) {
            float dot = qr[h][0] * ck[u][0];
#pragma unroll
            for (int i = 1; i < 8; ++i) dot = __builtin_fmaf(qr[h][i], ck[u][i], dot);
            sc[h][u] = dot;
          }
        static_assert((G * TB) % 4 == 0, "scores reduce four at a time");
        float* flat = &sc[0][0];
#pragma unroll
        for (int k = 0; k < G * TB; k += 4) group_allreduce4(flat[k], flat[k + 1], flat[k + 2], flat[k + 3]);
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          const bool valid = tb0 + kAttnGroups * u < t1;
          const float wk = as_f(kp[u].ns.x) * as_f(kp[u].ns.y);
#pragma unroll
          for (int h = 0; h < G; ++h) sc[h][u] = valid ? sc[h][u] * wk : -__builtin_inff();
        }
      }
      // online softmax: one max update per head for the four tokens
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float bm = sc[h][0];
#pragma unroll
        for (int u = 1; u < TB; ++u) bm = __builtin_fmaxf(bm, sc[h][u]);
        if (__builtin_amdgcn_ballot_w64(bm > m[h])) {
          // some group of the wave has a new maximum: rescale (corr = 1 elsewhere)
          const float mn = __builtin_fmaxf(m[h], bm);
          const float corr = __builtin_amdgcn_exp2f(m[h] - mn);
          l[h] = l[h] * corr;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = acc[h][i] * corr;
          m[h] = mn;
        }
#pragma unroll
        for (int u = 0; u < TB; ++u) sc[h][u] = __builtin_amdgcn_exp2f(sc[h][u] - m[h]);  // p (0 past the end)
      }
      // values
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        float cv[8];
        decode8(vp[u], shift, tb, cv);
        const float wv = as_f(vp[u].ns.x) * as_f(vp[u].ns.y);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          l[h] = l[h] + sc[h][u];
          const float pw = sc[h][u] * wv;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = __builtin_fmaf(pw, cv[i], acc[h][i]);
        }
      }
      // keeps the next iteration's slot writes (and so the waits for their
      // loads) from moving up into this one
      asm volatile("" ::: "memory");
    }
    // the next piece of the chunk (its slots reuse this wave's LDS rows, which
    // its own reads above have finished with); chunks of up to 4 heads per KV
    // head are a single piece
    if constexpr (G <= 4) break;
    t0 = t1;
    if (t0 >= c1) break;
    t1 = t0 + kPiece < c1 ? t0 + kPiece : c1;
#pragma unroll
    for (int k = 0; k < kAttnWin; ++k) load_slot(k);
  }

  // Merge the 16 groups: weights 2^(m_g - M); groups that saw no token have
  // m = -inf and weigh 0.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (r == 0) {
      red_m[h][grp] = m[h];
      red_l[h][grp] = l[h];
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mg[16], lg[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a = reinterpret_cast<const float4*>(red_m[h])[k];
      const float4 b = reinterpret_cast<const float4*>(red_l[h])[k];
      mg[4 * k] = a.x; mg[4 * k + 1] = a.y; mg[4 * k + 2] = a.z; mg[4 * k + 3] = a.w;
      lg[4 * k] = b.x; lg[4 * k + 1] = b.y; lg[4 * k + 2] = b.z; lg[4 * k + 3] = b.w;
    }
    float mx = mg[0];
#pragma unroll
    for (int g = 1; g < 16; ++g) mx = __builtin_fmaxf(mx, mg[g]);
    const float f = m[h] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m[h] - mx);
#pragma unroll
    for (int i = 0; i < 8; ++i) red_acc[grp][8 * r + i] = acc[h][i] * f;
    __syncthreads();
    float* part = ws + ((int64_t)(kv * G + h) * nchunk + blockIdx.x) * kPartFloats;
    if (threadIdx.x < 128) {
      float a = red_acc[0][threadIdx.x];
#pragma unroll
      for (int g = 1; g < 16; ++g) a = a + red_acc[g][threadIdx.x];
      part[4 + threadIdx.x] = a;
    } else if (threadIdx.x == 128) {
      float sl = 0.0f;
#pragma unroll
      for (int g = 0; g < 16; ++g)
        sl = sl + (mg[g] == -__builtin_inff() ? 0.0f : lg[g] * __builtin_amdgcn_exp2f(mg[g] - mx));
      part[0] = mx;
      part[1] = sl;
    }
    __syncthreads();
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
  tq3_attn_partial_kernel<QDT, G><<<dim3(nchunk, hkv), 256, 0, s>>>(q, k, v, n_tok, hkv, m,
                                                                     qscale, chunk, ws);
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
  // About four blocks per CU of a 256-CU part up to 4 heads per KV head
  // (with 2 or 4 heads only three fit at once, but chunks sized for three
  // measured no faster), chunks of at most 256 tokens (one piece); two
  // blocks per CU at 8 heads, where the registers allow two and one round of
  // longer chunks beats two rounds; at least one token per group (16 per
  // chunk); chunks are multiples of 16 tokens.
  AttnPlan p;
  const int64_t target = 256 * (g <= 4 ? 4 : 2);
  int64_t nch = target / hkv;
  const int64_t max_ch = (n_tok + 15) / 16;
  if (nch > max_ch) nch = max_ch;
  if (nch < 1) nch = 1;
  int64_t chunk = (n_tok + nch - 1) / nch;
  chunk = (chunk + 15) / 16 * 16;
  if (g <= 4 && chunk > kAttnGroups * kAttnTokPerGroup) chunk = kAttnGroups * kAttnTokPerGroup;
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
