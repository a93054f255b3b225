// Key-range kernel for one query row per (batch, head): the decode step of
// fa_fwd_split (Nq = 1), for CDNA4 (gfx950), 16-bit inputs.
//
// With one query the score matrix is a matrix-vector product and the work is
// bound by reading K and V once.  The 128-row MFMA kernel would spend 31/32 of
// its matrix work and three of its four waves on absent rows, and its 64 KB of
// LDS tiles keeps at most two workgroups, so few bytes, in flight per CU.
// This kernel uses neither LDS tiles nor MFMA: each wave streams chunks of 16
// keys of K and V straight into registers, several chunks ahead, and computes
// on the vector units:
//   score of key j  = sum over 8-element slices of dot2(q, k_j), then a
//                     reduction over the D/8 lanes holding row j;
//   online softmax  = running max m, sum l and output o (fp32, 8 columns per
//                     lane) per wave, exact max per chunk;
//   merge           = the four waves' (m, l, o) combined through LDS into the
//                     range's normalised output and log-sum-exp, the same
//                     partial results fa_combine_kernel merges over ranges.
// The pages do not describe decode kernels; the arithmetic is the forward's
// definition and the online-softmax recurrence ("Flash Attention",
// wiki.ai-engineering.at, section "Lösung: Online Softmax").
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeChunk = 16;  // keys per chunk

namespace dec {
// dot product of two words of two 16-bit values each, added to acc (fp32)
__device__ __forceinline__ float dot2(BF16, uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}
__device__ __forceinline__ float dot2(F16, uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}
// the two 16-bit values of a word as fp32 (exact)
__device__ __forceinline__ void widen(BF16, uint32_t w, float& lo, float& hi) {
  lo = __builtin_bit_cast(float, w << 16);
  hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
}
__device__ __forceinline__ void widen(F16, uint32_t w, float& lo, float& hi) {
  const f16x2 v = __builtin_bit_cast(f16x2, w);
  lo = (float)v[0];
  hi = (float)v[1];
}
}  // namespace dec

// One workgroup per ((b, h), key range): range split of the key chunks
// [0, ceil(NK / 16)) into n_split contiguous runs; wave w of the workgroup
// takes the run's chunks w, w + 4, ...  Lane layout for a chunk: lane holds 16
// bytes (8 columns) of row r = lane / (D/8) of each 64/(D/8)-row slice, so a
// wave-wide load covers 1 KB; LD loads per tensor cover the 16 keys.
template <typename E, int D>
__global__ __launch_bounds__(kDecodeThreads) void fa_decode_kernel(FwdArgs a) {
  constexpr int LPR = D / 8;             // lanes per row
  constexpr int RPL = 64 / LPR;          // rows per wave-wide load
  constexpr int LD = kDecodeChunk / RPL; // loads per chunk and tensor
  constexpr int PF = D == 256 ? 2 : 3;   // chunks in flight per wave
  constexpr int NW = kDecodeThreads / 64;
  static_assert(LD >= 1 && RPL * LPR == 64, "lane layout");

  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ float sm_o[NW][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane / LPR, cl = lane % LPR;
  const int t = blockIdx.x;
  const int bh = t / a.n_split;
  const int split = t - bh * a.n_split;
  const int NK = a.nk;
  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * D;  // Nq = 1
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * NK * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * NK * D;

  const int n_ch = (NK + kDecodeChunk - 1) / kDecodeChunk;
  const int c_lo = (int)((long long)n_ch * split / a.n_split);
  const int c_hi = (int)((long long)n_ch * (split + 1) / a.n_split);

  // this lane's 8 query columns (signs flipped for a negative scale)
  u32x4 qw = *(const u32x4*)(Qg + cl * 8);
  {
    const u32x4 fl = {a.qflip, a.qflip, a.qflip, a.qflip};
    qw ^= fl;
  }
  const float c = a.c;

  // chunk registers: K and V words of the LD rows this lane holds
  struct Chunk {
    u32x4 k[LD], v[LD];
  };
  auto load = [&](Chunk& ch, int ci) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int key = ci * kDecodeChunk + i * RPL + r;
      const u32x4 z = {0u, 0u, 0u, 0u};
      ch.k[i] = z;
      ch.v[i] = z;
      if (ci < c_hi && key < NK) {
        ch.k[i] = *(const u32x4*)(Kg + (size_t)key * D + cl * 8);
        ch.v[i] = *(const u32x4*)(Vg + (size_t)key * D + cl * 8);
      }
    }
  };

  float m = neg_inf(), l = 0.0f;
  float o[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const Chunk& ch, int ci) __attribute__((always_inline)) {
    float s[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = dec::dot2(E(), qw[e], ch.k[i][e], acc);
      // sum over the LPR lanes of the row
#pragma unroll
      for (int x = 1; x < LPR; x <<= 1) acc += __shfl_xor(acc, x, 64);
      const int key = ci * kDecodeChunk + i * RPL + r;
      s[i] = key < NK ? acc * c : neg_inf();  // log2 units
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < LD; ++i) mx = fmaxf(mx, s[i]);
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) mx = fmaxf(mx, __shfl_xor(mx, x, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = m_new == neg_inf() ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
    m = m_new;
    const float mu = m == neg_inf() ? 0.0f : m;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[i] - mu);
      l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v0, v1;
        dec::widen(E(), ch.v[i][e], v0, v1);
        o[2 * e] = __builtin_fmaf(p, v0, o[2 * e]);
        o[2 * e + 1] = __builtin_fmaf(p, v1, o[2 * e + 1]);
      }
    }
  };

  // chunks c_lo + wave + 4 k, k = 0, 1, ...: PF of them in flight, ring
  // unrolled by PF so every slot is a separate set of registers
  Chunk ring[PF];
#pragma unroll
  for (int s = 0; s < PF; ++s) load(ring[s], c_lo + wave + NW * s);
  for (int ci = c_lo + wave; ci < c_hi; ci += NW * PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int cs = ci + NW * s;
      if (cs < c_hi) {
        compute(ring[s], cs);
        load(ring[s], cs + NW * PF);
      }
    }
  }

  // the wave's totals: l and o summed over the rows of the lanes (m is the same
  // in every lane of the wave)
#pragma unroll
  for (int x = LPR; x < 64; x <<= 1) {
    l += __shfl_xor(l, x, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], x, 64);
  }
  if (lane == 0) {
    sm_m[wave] = m;
    sm_l[wave] = l;
  }
  if (r == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[wave][cl * 8 + e] = o[e];
  }
  __syncthreads();

  // merge of the waves: lse_w = m_w + log2 l_w; one thread per output column
  if (tid < D) {
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (sm_m[w] == neg_inf()) continue;
      const float f = __builtin_amdgcn_exp2f(sm_m[w] - M);
      L += f * sm_l[w];
      O += f * sm_o[w][tid];
    }
    const float lse = L > 0.0f ? (M + __log2f(L)) * kLn2 : neg_inf();
    if (a.n_split == 1) {
      // the only range: O (rounded once) and LSE directly
      ((uint16_t*)a.o)[(size_t)bh * D + tid] = (uint16_t)(E::pack(L > 0.0f ? O / L : 0.0f, 0.0f) & 0xFFFFu);
      if (tid == 0) a.lse[bh] = lse;
    } else {
      const size_t prow = (size_t)split * a.n_bh + bh;  // Nq = 1
      a.o_part[prow * D + tid] = L > 0.0f ? O / L : 0.0f;
      if (tid == 0) a.lse_part[prow] = lse;
    }
  }
}

}  // namespace fa
