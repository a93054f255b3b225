// Attention forward on FP8 inputs with MX block scales, for CDNA4 (gfx950).
//
// Inputs: Q, K, V as OCP FP8 E4M3 codes [B*H][N][D], each row with one OCP MX
// E8M0 scale per 32 consecutive elements ([B*H][N][D/32] bytes).  The pages
// name FP8 support and block-scaled attention among the later FlashAttention
// versions ("Flash Attention: ускорить attention в 6 раз без потери
// точности", sections "Flash Attention 3" and "Flash Attention 4"); the result
// computed is the exact attention of the values the codes and scales denote,
// O = softmax(scale Q K^T [+ causal mask]) V and its LSE.
//
// S = Q K^T runs on v_mfma_scale_f32_32x32x64_f8f6f4: the matrix core applies
// the Q and K block scales itself (one scale byte per lane and operand), and
// products of E4M3 values are exact in its fp32 accumulation.  P V runs on the
// bf16 MFMA, as in the bf16 kernel: each V tile is converted once per
// workgroup from E4M3 to bf16 with its block scales (exact: E4M3 values fit
// bf16 and the scales are powers of two) into an LDS tile the value MFMA
// reads.  P is rounded to bf16, not to E4M3, whose 3-bit mantissa would put up
// to 6 % on every weight.  The online softmax is the bf16 kernel's.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Fp8Args {
  const uint8_t* q;
  const uint8_t* qs;  // [B*H][N][D/32] E8M0 scale codes
  const uint8_t* k;
  const uint8_t* ks;
  const uint8_t* v;
  const uint8_t* vs;
  void* o;            // bf16 [B*H][N][D]
  float* lse;         // [B*H][N]
  int n;
  int n_qblk;
  int n_blocks;
  float c;            // |scale| * log2(e), at least FLT_MIN
  uint32_t qflip;     // 0x80808080 for a negative scale: flips the sign bit of every Q code
};

constexpr int kFp8Threads = 256;
constexpr int kFp8Rows = 128;

namespace fp8 {
// XOR applied to the 16-byte chunk index of row `row` of an E4M3 tile (D
// bytes a row), a linear function of the row's bits 0-3 (so rows 32 apart
// share it).  Two read patterns use the tile: the score operand (lanes 0-31
// read rows swap23(lane) at one chunk, lanes 32-63 the next chunk) and the V
// conversion (16 consecutive rows at one chunk per 16 lanes).  Whether the
// LDS serves a 16-byte read 8 lanes a cycle over 32 banks or 16 lanes over 64
// banks, both patterns then hit distinct banks in every pass (checked over all
// lanes by a bank model; the row shift swizzle of half rows, (row >> 1) & 7,
// left the score reads 2-way conflicted in the 8-lane case, which the
// conflict counter showed).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row >> 1) & 1) | (((row ^ (row >> 2)) & 1) << 1) | (((row >> 3) & 1) << 2);
  else return (((row >> 1) ^ (row >> 2)) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1);
}
// Quarter of the row (D/4 values, at most one MX block) that lane (r, k)
// converts: row r of the wave's 16, k = lane / 16.  The XOR with bits of r
// makes the 16-byte bf16 writes of the conversion 2-way conflicted at most
// (the least possible for writes of one chunk position per instruction, given
// the bf16 tile's swizzle) and keeps the E4M3 reads conflict-free.
template <int D>
__device__ __forceinline__ int cv_part(int r, int k) {
  if constexpr (D == 128) return k ^ (((r >> 2) & 1) << 1);
  else return k ^ ((r >> 1) & 3);
}
// Order of a converting lane's two 8-byte halves of each E4M3 chunk (1:
// second half first), and so of its two bf16 chunk writes.  Lanes of one
// write instruction then alternate between the two chunk positions, which
// leaves the 16-byte writes conflict-free when the LDS serves 8 lanes a cycle
// (the conflict counter matched that case; 16 lanes a cycle would leave D = 128
// 2-way), and the 8-byte reads conflict-free.
template <int D>
__device__ __forceinline__ int cv_swap(int r) {
  if constexpr (D == 128) return (r >> 2) & 1;
  else return (r ^ (r >> 3)) & 1;
}
// A row's D/32 scale bytes as one word (read as 4-byte words: the scale
// arrays are 4-byte aligned); rows past N read as scale 1 (code 127).
template <int D>
__device__ __forceinline__ uint32_t scale_word(const uint8_t* p, bool valid) {
  if constexpr (D == 128) {
    return valid ? *(const uint32_t*)p : 0x7F7F7F7Fu;
  } else {
    return valid ? (uint32_t) * (const uint16_t*)p : 0x7F7F7F7Fu;
  }
}
template <int D>
__device__ __forceinline__ uint32_t addr(int row, int chunk) {
  return (uint32_t)(row * D + ((chunk ^ swz<D>(row)) * 16));
}
}  // namespace fp8

// Work split as in the bf16 kernel: 4 waves x 32 query rows, one workgroup per
// (b, h, 128-row query block), two workgroups per CU, and the same two-phase
// software pipeline inside each wave:
//
//   iteration j:  barrier ; DMA K_{j+2}, V_{j+2} (E4M3) and their scales
//                 phase A: S_{j+1} = K_{j+1} Q^T (scaled FP8 MFMA) || p = exp2(c s_j - m), P_j, sums
//                 phase B: O^T += V_j^T P_j^T   (bf16 MFMA)       || reference of S_{j+1};
//                          V_{j+1} converted to the bf16 tile it will be read from
//
// Every wave converts 16 rows of V_{j+1} in phase B of iteration j, into the
// bf16 buffer that V_{j-1} occupied (read in iteration j-1, before the barrier
// of iteration j); the barrier of iteration j+1 publishes it to the value MFMAs
// of iteration j+1.  So each tile costs one barrier, as in the bf16 kernel.
//
// D = 64 and 128; D = 256 runs on fa_fwd_fp8_rows16_kernel, whose 16-row
// waves fit two to a SIMD where 32-row ones need a SIMD each.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFp8Threads, 2) void fa_fwd_fp8_kernel(Fp8Args a) {
  constexpr int BN = 64;
  constexpr int CPR = D / 16;          // 16-byte chunks per E4M3 row
  constexpr int TILE16 = BN * CPR;     // 16-byte chunks per E4M3 tile
  constexpr int RPB = 64 / CPR;        // rows per wave-wide load
  constexpr int NLD = TILE16 / 256;    // wave-wide loads per wave per tile
  constexpr int NSC = D / 32;          // scale bytes per row
  constexpr int NKS = D / 64;          // 64-deep steps of the score contraction
  constexpr int NKB = BN / 32;         // 32-key blocks per tile
  constexpr int NDB = D / 32;          // 32-wide d blocks of O
  constexpr int NCC = BN / 16;         // 16-key steps of the value contraction
  constexpr int NSA = NKS * NKB;       // score MFMAs per tile
  constexpr int NSB = NDB * NCC;       // value MFMAs per tile (phase B slots)
  constexpr int NP = 2 * NCC;          // p slices (4 scores each): phase A slots
  constexpr int MST = NP / NSA;        // phase A slots per score MFMA
  constexpr int RBH = 2 * D;           // bytes per bf16 row
  constexpr int CPRH = D / 8;          // 16-byte chunks per bf16 row
  constexpr int VPL = D / 4;           // V values one lane converts per tile
  constexpr int NCH = VPL / 16;        // E4M3 chunks one lane converts per tile
  constexpr int G0 = NSB / 4;          // phase B slot of the first conversion group
  static_assert(D == 64 || D == 128, "head dimensions");
  static_assert(NLD >= 1 && RPB * CPR == 64 && NKB == 2 && NP % NSA == 0, "tile shape");
  static_assert(G0 >= 2 && G0 + 4 * NCH < NSB, "conversion slots");

  __shared__ u32x4 kA[TILE16], kB[TILE16], vA[TILE16], vB[TILE16];  // E4M3 tiles
  __shared__ u32x4 wA[BN * CPRH], wB[BN * CPRH];                     // bf16 V tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c32 = lane & 31;
  const int N = a.n;
  const HeadItem wi = head_item(xcd_remap(blockIdx.x, a.n_blocks), a.n_blocks / a.n_qblk, a.n_qblk, CAUSAL, true);
  const int bh = wi.bh;
  const int qb = CAUSAL ? a.n_qblk - 1 - wi.idx : wi.idx;  // causal: longest query blocks first
  const int q0 = qb * kFp8Rows;
  const uint8_t* Qg = a.q + (size_t)bh * N * D;
  const uint8_t* Kg = a.k + (size_t)bh * N * D;
  const uint8_t* Vg = a.v + (size_t)bh * N * D;
  const uint8_t* QSg = a.qs + (size_t)bh * N * NSC;
  const uint8_t* KSg = a.ks + (size_t)bh * N * NSC;
  const uint8_t* VSg = a.vs + (size_t)bh * N * NSC;

  const int kv_end = CAUSAL ? min(N, q0 + kFp8Rows) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int qrow = q0 + wave * 32 + c32;
  const int wave_q0 = q0 + wave * 32;
  const int n_vis = wave_q0 >= N ? 0 : CAUSAL ? min(n_tiles, (wave_q0 + 31) / BN + 1) : n_tiles;

  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < TILE16; i += kFp8Threads) kA[i] = kB[i] = vA[i] = vB[i] = z;
  }

  // Q as the B operand of the score MFMA: for step ks, bytes 0..15 are
  // Q[qrow][64ks + 16h .. +15] and bytes 16..31 Q[qrow][64ks + 32 + 16h .. +15]
  // (the instruction's first and second 32-wide block of the step); the lane
  // supplies the scale of block 2ks + h of its row.
  i32x8 qf[NKS];
  int qsc[NKS];
  {
    const u32x4 fl = {a.qflip, a.qflip, a.qflip, a.qflip};
    const uint32_t sdw = fp8::scale_word<D>(QSg + (size_t)qrow * NSC, qrow < N);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (qrow < N) {
        const u32x4* r = (const u32x4*)(Qg + (size_t)qrow * D);
        lo = r[4 * ks + h] ^ fl;
        hi = r[4 * ks + 2 + h] ^ fl;
      }
      const i32x8 f = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      qf[ks] = f;
      qsc[ks] = (int)((sdw >> (8 * (2 * ks + h))) & 0xFFu);
    }
  }

  // tile loads: E4M3 rows by buffer-to-LDS loads into the swizzled layout
  uint32_t toff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPB + lane / CPR;
    toff[i] = row * D + (((lane % CPR) ^ fp8::swz<D>(row)) * 16);
  }
  auto issue = [&](u32x4* dst, const uint8_t* src, int kv0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (size_t)kv0 * D), (short)0, (int)((uint32_t)(N - kv0) * D), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_load16(r, dst + (wave * NLD + i) * 64, toff[i]);
  };

  // V conversion: row 16 wave + lane % 16 of the tile, values d0 .. d0 + VPL - 1
  // (within one MX block), written as bf16 in the bf16 kernel's V layout
  const int cv_row = wave * 16 + (lane & 15);
  const int cv_d0 = fp8::cv_part<D>(lane & 15, lane >> 4) * VPL;
  const int cv_s = fp8::cv_swap<D>(lane & 15);

  // block scales of a tile, loaded into registers two tiles ahead (a row's
  // D/32 bytes need not fill whole dwords, so they do not go through the
  // 4-byte tile loads): the K scale bytes of this lane's two score rows, and
  // the V scale byte of the block this lane converts; rows past N read as 1
  struct TileScales {
    uint32_t k[2];
    uint32_t v;
  };
  auto load_scales = [&](TileScales& ts, int kv0) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = kv0 + 32 * kb + swap23(c32);
      ts.k[kb] = fp8::scale_word<D>(KSg + (size_t)row * NSC, row < N);
    }
    const int vrow = kv0 + cv_row;
    ts.v = vrow < N ? (uint32_t)VSg[(size_t)vrow * NSC + cv_d0 / 32] : 127u;
  };
  // the K scale words of this lane's two score rows, and the V scale byte of
  // the block it converts
  auto k_scales = [&](const TileScales& ts, uint32_t (&kw)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kw[kb] = ts.k[kb];
  };
  auto v_scales = [&](const TileScales& ts) __attribute__((always_inline)) { return ts.v; };

  // K operand of score MFMA (kb, ks): rows 32kb + swap23(c32), E4M3 chunks
  // 4ks + h (bytes 0..15) and 4ks + 2 + h (bytes 16..31).  With the row's
  // swizzle x on bits 1.. of the row only, chunk (h + 2m) ^ x = (h ^ x) ^ 2m, so
  // every address is one per-lane base XOR (m << 5), plus 32kb rows.
  const uint32_t kaddr0 = [&] {
    const int row = swap23(c32);
    return (uint32_t)(row * D + ((h ^ fp8::swz<D>(row)) * 16));
  }();
  auto kfrag = [&](const u32x4* Kt, int m) __attribute__((always_inline)) {
    const int kb = m / NKS, ks = m % NKS;
    const char* base = (const char*)Kt + kb * 32 * D;
    const u32x4 lo = *(const u32x4*)(base + (kaddr0 ^ ((2 * ks) << 5)));
    const u32x4 hi = *(const u32x4*)(base + (kaddr0 ^ ((2 * ks + 1) << 5)));
    const i32x8 f = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return f;
  };
  // V^T operand reads of the value MFMA (the bf16 kernel's lane layout)
  const uint32_t vaddr0 = [&] {
    const int g = lane >> 4, i16 = lane & 15;
    const int hh = g >> 1, gg = g & 1, r = i16 >> 2, q = i16 & 3;
    const int chunk = 2 * gg + (q >> 1);
    return (uint32_t)((8 * hh + r) * RBH + ((chunk ^ vswz<D>(r)) * 16) + (q & 1) * 8);
  }();
  auto vfrag = [&](const u32x4* Wt, int s) __attribute__((always_inline)) {
    const int db = s % NDB, cc = s / NDB;
    const char* p = (const char*)Wt + (vaddr0 ^ (db << 6)) + 16 * cc * RBH;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * RBH));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // state as in the bf16 kernel: o (unnormalised output), m_ref (running
  // reference, log2 units), lsacc (sum of the bf16-rounded p on the matrix
  // core: lane n < 16 holds queries n and n + 16), lx (fp32 sum of p: LSE),
  // pf (bf16 P^T of the tile whose values are next), a pending output rescale
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  f32x16 sA[NKB], sB[NKB];
  bf16x8 pf[NCC];
  float m_ref = neg_inf(), lx = 0.0f, mu = 0.0f;
  f32x4 lsacc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t one2 = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? BF16::kOnes2 : 0u;
  const bf16x8 ones_op = __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2});
  float thr = neg_inf();
  bool pend = false;
  float pend_alpha = 1.0f;
  const float c = a.c;

  // scores of one tile: NSA scaled FP8 MFMAs (the scale byte of K row
  // 32kb + swap23(c32), block 2ks + h, from the tile's scale dwords)
  auto score_mfma = [&](f32x16 (&s)[NKB], const i32x8& kf, const uint32_t (&kw)[2], int m)
      __attribute__((always_inline)) {
    const int kb = m / NKS, ks = m % NKS;
    const int ksc = (int)((kw[kb] >> (8 * (2 * ks + h))) & 0xFFu);
    const f32x16 z = {};
    s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[ks], ks == 0 ? z : s[kb], 0, 0, 0, ksc, 0,
                                                            qsc[ks]);
  };
  // element (kb, i) of tile j holds key j*BN + 32kb + 8h + kofs(i) of query qrow
  auto mask = [&](f32x16 (&s)[NKB], int j) __attribute__((always_inline)) {
    const int kv0 = j * BN;
    if (kv0 + BN > N || (CAUSAL && kv0 + BN - 1 > wave_q0)) {
      const int lim = (CAUSAL ? min(N - 1, qrow) : N - 1) - kv0 - 8 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = 32 * kb + 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
          if (kofs > lim) s[kb][i] = neg_inf();
        }
    }
  };
  // row max and the lazy reference update of the bf16 kernel, in slices
  // 0..NKB-1 (partial maxima) and NKB (the update)
  float mpart[NKB];
  auto ref_slice = [&](const f32x16 (&s)[NKB], int k) __attribute__((always_inline)) {
    if (k < NKB) {
      float mx = s[k][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = vmax(mx, s[k][i]);
      pin(mx);
      mpart[k] = mx;
    } else {
      float mx = mpart[0];
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) mx = vmax(mx, mpart[kb]);
      mx = pair_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
        const float m_new = vmax(m_ref, mx * c);
        const float alpha = m_new == neg_inf() ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        lx *= alpha;
        m_ref = m_new;
        pend = true;
        pend_alpha = alpha;
        mu = m_new == neg_inf() ? 0.0f : m_new;
        thr = (m_new + BF16::kTau) / c;  // P is bf16, as in the bf16 kernel
      }
      pin(mu);
      pin(pend_alpha);
      pin(lx);
      pin(thr);
    }
  };
  // p = exp2(c s - mu) for 4 scores of value step cc, their fp32 sum, and
  // their bf16 words
  float xsum[2] = {0.0f, 0.0f};
  auto p_slice = [&](f32x16 (&s)[NKB], int cc, int half) __attribute__((always_inline)) {
    const int kb = cc >> 1, base = (cc & 1) * 8 + 4 * half;
#pragma unroll
    for (int e = 0; e < 4; ++e) s[kb][base + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][base + e], c, -mu));
    const uint32_t w0 = pack_bf16(s[kb][base + 0], s[kb][base + 1]);
    const uint32_t w1 = pack_bf16(s[kb][base + 2], s[kb][base + 3]);
    const float part = (s[kb][base + 0] + s[kb][base + 1]) + (s[kb][base + 2] + s[kb][base + 3]);
    xsum[half] = cc == 0 ? part : xsum[half] + part;
    uint32_t r0 = w0, r1 = w1;
    pin(r0);
    pin(r1);
    pin(xsum[half]);
    return u32x2{r0, r1};
  };
  // conversion of this lane's VPL values of V tile (E4M3 in Vt) into the bf16
  // tile Wt, chunk by chunk: two 8-byte reads (in the order cv_s), 4 groups
  // of 2 conversions, two 16-byte writes (in phase B: the read 2 slots before the chunk's groups, the
  // writes in the slot after them)
  u32x4 cin[NCH];
  uint32_t cout[NCH][8];
  auto conv_read = [&](const u32x4* Vt, int cch) __attribute__((always_inline)) {
    const uint32_t ad = fp8::addr<D>(cv_row, cv_d0 / 16 + cch) + 8 * cv_s;
    const u32x2 lo = *(const u32x2*)((const char*)Vt + ad);
    const u32x2 hi = *(const u32x2*)((const char*)Vt + (ad ^ 8));
    cin[cch] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  auto conv_group = [&](uint32_t vsw, int g) __attribute__((always_inline)) {
    const int cch = g >> 2, e = g & 3;
    const uint32_t vb = vsw;  // the lane's values lie in one MX block
    const float sc = __builtin_bit_cast(float, vb << 23);
    const int w = (int)cin[cch][e];
    uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, false));
    uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, true));
    pin(lo);
    pin(hi);
    cout[cch][2 * e] = lo;
    cout[cch][2 * e + 1] = hi;
  };
  auto conv_write = [&](u32x4* Wt, int cch) __attribute__((always_inline)) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int cidx = cv_d0 / 8 + 2 * cch + (half ^ cv_s);  // bf16 chunk (8 values)
      const u32x4 o4 = {cout[cch][4 * half], cout[cch][4 * half + 1], cout[cch][4 * half + 2], cout[cch][4 * half + 3]};
      *(u32x4*)((char*)Wt + cv_row * RBH + ((cidx ^ vswz<D>(cv_row)) * 16)) = o4;
    }
  };
  auto convert_all = [&](const u32x4* Vt, u32x4* Wt, const TileScales& ts) __attribute__((always_inline)) {
    const uint32_t vsw = v_scales(ts);
    // chunk by chunk, one read ahead: few registers live at once
    conv_read(Vt, 0);
#pragma unroll
    for (int cch = 0; cch < NCH; ++cch) {
      if (cch + 1 < NCH) conv_read(Vt, cch + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) conv_group(vsw, 4 * cch + e);
      conv_write(Wt, cch);
    }
  };

  // ---- phases --------------------------------------------------------------
  // phase A: score MFMAs of tile j+1 (K in Kt, scales ts) into sn, one every
  // MST slots, beside the exponentials of tile j in sc (one p slice a slot);
  // K fragments are read one MFMA ahead
  auto phase_a = [&](f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], const u32x4* Kt, const TileScales& ts)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    uint32_t kw[2];
    k_scales(ts, kw);
    i32x8 kf[NSA];
    kf[0] = kfrag(Kt, 0);
    u32x2 pw[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      pw[k] = p_slice(sc, k >> 1, k & 1);
      if (k % MST == 0) {
        const int m = k / MST;
        if (m + 1 < NSA) kf[m + 1] = kfrag(Kt, m + 1);
        score_mfma(sn, kf[m], kw, m);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      const u32x4 x = {pw[2 * cc][0], pw[2 * cc][1], pw[2 * cc + 1][0], pw[2 * cc + 1][1]};
      pf[cc] = __builtin_bit_cast(bf16x8, x);
    }
    lx += xsum[0] + xsum[1];
    // the scores are pinned here: otherwise the score MFMAs, whose results are
    // first read after the rescale branch, are sunk past it and run back to
    // back there, beside nothing
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) pin(sn[kb]);
    __builtin_amdgcn_s_setprio(0);
  };
  // phase B: value MFMAs of tile j (bf16 V^T from Wc) and the rounded-P sum,
  // beside the reference update of tile j+1 (sn) and the conversion of the
  // next V tile (E4M3 in Vn, scales tsn) into Wn
  constexpr int PFB = 4;
  auto phase_b = [&](const f32x16 (&sn)[NKB], const u32x4* Wc, const u32x4* Vn, u32x4* Wn, const TileScales& tsn)
      __attribute__((always_inline)) {
    const uint32_t vsw = v_scales(tsn);
    u32x4 vf[NSB];
#pragma unroll
    for (int k = 0; k < PFB && k < NSB; ++k) vf[k] = vfrag(Wc, k);
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      if (k + PFB < NSB) vf[k + PFB] = vfrag(Wc, k + PFB);
      if (k <= NKB) ref_slice(sn, k);
#pragma unroll
      for (int cch = 0; cch < NCH; ++cch) {
        if (k == G0 - 2 + 4 * cch) conv_read(Vn, cch);
        if (k == G0 + 4 * cch + 4) conv_write(Wn, cch);
      }
      if (k >= G0 && k < G0 + 4 * NCH) conv_group(vsw, k - G0);
      const int db = k % NDB, cc = k / NDB;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[k]), pf[cc], o[db], 0, 0, 0);
      if (db == NDB - 1)
        lsacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_op, pf[cc], lsacc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (pend) {
      // lsacc[1] of lane n < 16 belongs to query n + 16 (lane n + 16)
      const float a_hi = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(((lane + 16) & 63) << 2, __builtin_bit_cast(int, pend_alpha)));
      lsacc[0] *= pend_alpha;
      lsacc[1] *= a_hi;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= pend_alpha;
      pend = false;
    }
  };

  // ---- prologue --------------------------------------------------------------
  TileScales tsA, tsB;  // scales of the tiles whose K / V codes are in kA, vA and kB, vB
  __syncthreads();  // zeroed tiles visible before any load lands
  if (n_tiles > 0) {
    issue(kA, Kg, 0);
    issue(vA, Vg, 0);
    load_scales(tsA, 0);
  }
  if (n_tiles > 1) {
    issue(kB, Kg, BN);
    issue(vB, Vg, BN);
    load_scales(tsB, BN);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // tiles 0 and 1 in LDS
  if (n_tiles > 0) convert_all(vA, wA, tsA);
  if (n_vis > 0) {
    uint32_t kw[2];
    k_scales(tsA, kw);
    i32x8 kf[NSA];
    kf[0] = kfrag(kA, 0);
#pragma unroll
    for (int m = 0; m < NSA; ++m) {
      if (m + 1 < NSA) kf[m + 1] = kfrag(kA, m + 1);  // one fragment ahead
      score_mfma(sA, kf[m], kw, m);
    }
    mask(sA, 0);
#pragma unroll
    for (int k = 0; k <= NKB; ++k) ref_slice(sA, k);
    pend = false;
  }

  // ---- main loop: iteration j consumes S_j (in sc) and V_j (bf16 in Wc) ------
  // Buffers: K_{j+1}, V_{j+1} codes in Kn, Vn with scales tsn; K_{j+2}, V_{j+2}
  // go to Kd, Vd (which held K_j, V_j) with scales into tsd; V_{j+1} is
  // converted into Wn (which held V_{j-1}).
  auto iteration = [&](int j, f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], const u32x4* Kn, u32x4* Kd,
                       const u32x4* Vn, u32x4* Vd, const TileScales& tsn, TileScales& tsd, const u32x4* Wc,
                       u32x4* Wn) __attribute__((always_inline)) {
    // the explicit wait: at a barrier that heads a loop this compiler can drop
    // the wait for the tile loads issued in the previous iteration
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < n_tiles) {
      issue(Kd, Kg, (j + 2) * BN);
      issue(Vd, Vg, (j + 2) * BN);
      load_scales(tsd, (j + 2) * BN);
    }
    if (j >= n_vis) {
      // no key of this tile or later is visible to this wave; its share of the
      // next V tile is still converted for the other waves
      if (j + 1 < n_tiles) convert_all(Vn, Wn, tsn);
      return;
    }
    // after the last visible tile the "next" scores come from whatever K
    // buffer is there and are fully masked; the next V conversion likewise
    // converts codes no wave reads
    phase_a(sc, sn, Kn, tsn);
    apply_rescale();
    mask(sn, j + 1);
    phase_b(sn, Wc, Vn, Wn, tsn);
  };
  for (int j = 0; j < n_tiles; j += 2) {
    iteration(j, sA, sB, kB, kA, vB, vA, tsB, tsA, wA, wB);
    if (j + 1 < n_tiles) iteration(j + 1, sB, sA, kA, kB, vA, vB, tsA, tsB, wB, wA);
  }

  // epilogue: O = o / l, LSE = (m + log2 lx) ln 2.  Query c32's rounded-P sum
  // sits in lane c32 % 16, element c32 / 16 (elements copied to scalars before
  // their bit casts).
  float e0 = lsacc[0], e1 = lsacc[1];
  pin(e0);
  pin(e1);
  const int src = (c32 & 15) << 2;
  const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, e0)));
  const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, e1)));
  const float l_tot = c32 < 16 ? s0 : s1;
  const float lx_tot = pair_sum(lx);
  if (qrow < N) {
    const float inv = 1.0f / l_tot;
    uint16_t* Og = (uint16_t*)a.o + ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * h;
        const u32x2 w = {pack_bf16(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                         pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        *(u32x2*)(Og + d) = w;
      }
    if (h == 0) a.lse[(size_t)bh * N + qrow] = (m_ref + __log2f(lx_tot)) * kLn2;
  }
}

}  // namespace fa
