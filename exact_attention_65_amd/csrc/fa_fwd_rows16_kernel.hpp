// Exact attention forward with 16 query rows per wave on the 16x16x32 MFMA
// (bf16 or fp16 inputs, one key range): for small grids at D = 64, 96, 128 and
// 256 (D = 96 in LDS rows of 128 columns, as in the 128-row kernel), and for
// every larger grid at D = 256.
//
// The method is the 128-row kernel's: the tiled loop of "Flash Attention"
// (wiki.ai-engineering.at, section "Tiling Algorithm") with the online
// softmax of its section "Lösung: Online Softmax", fused into one kernel that
// reads Q, K, V once and writes O and LSE.  Only the work split differs.
//
// When a launch holds about one 128-row workgroup per compute unit or fewer,
// its time is the longest query block's walk over the key tiles, one tile
// after another, each wave alone on its SIMD, so one wave's time per tile
// sets the pace.  Here a workgroup holds 64 query rows in 4 slices of 16: each
// wave does half the MFMA work per tile, and the grid has twice as many
// workgroups to spread over the chip.  With KS = 2 two waves share a slice,
// each taking half of every tile's keys, and merge their partial results at
// the end (the exact merge of two softmax partial results over disjoint key
// sets); the per-wave work halves again, until the K and V bytes each
// workgroup must fetch per tile (32 KB) bound the tile time instead.  On large
// grids the 128-row kernel stays faster (its 32x32 tiles use each K and V
// byte fetched into a CU for twice as many queries), except at D = 256.
//
// At D = 256 the 128-row kernel's 128 KB of tiles and 32-row waves leave one
// workgroup of 4 waves per CU, one wave alone on each SIMD.  With SL = 8
// slices of 16 rows a workgroup holds the same 128 rows and tiles in 8 waves
// (252 VGPRs each), two per SIMD, which fill each other's gaps; each K and V
// byte fetched into the CU still serves 128 queries.  The 16x16 tiles read
// each LDS operand byte for 16 queries instead of 32, which at D = 128 costs
// more than the second wave per SIMD gains there.  The arithmetic is the
// 128-row kernel's: scores, the lazy reference with the same headroom, P
// rounded to the input type, the sum of the rounded P on the matrix core and
// the fp32 sum for the LSE.
//
// Layouts (16x16x32: A lane l -> row l % 16, k block l / 16; B lane l -> column
// l % 16, k block l / 16; result lane l -> rows 4 (l / 16) + i, column l % 16):
//   * scores S^T = K Q^T per 16-key block b: the A operand's row t of block b
//     is key 32 (b >> 1) + 8 (t >> 2) + 4 (b & 1) + (t & 3), so that lane l's
//     four results of blocks 2s and 2s + 1 are keys 32s + 8 (l/16) + 0..7 of
//     its query l % 16, which is exactly the P^T fragment (k block l / 16) of
//     the value MFMA of key step s;
//   * O^T += V^T P^T per 16-wide d block and 32-key step: V^T by two
//     transposed reads (4 keys x 16 d per 16-lane group each);
//   * a row's 64 keys of a tile spread over the 4 lanes l % 16 + 16 g, so its
//     max and fp32 sum reduce across lanes l ^ 16 and l ^ 32.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

constexpr int kRows16Rows = 64;  // query rows per workgroup of the small-grid form: 4 slices of 16

namespace rows16 {
// Key of row t of score block b of a 64-key tile.
__device__ __forceinline__ int key_of(int b, int t) { return 32 * (b >> 1) + 8 * (t >> 2) + 4 * (b & 1) + (t & 3); }
// XOR applied to the 16-byte chunk index of a K row.  The 16 lanes of a score
// read take rows key_of(b, 0..15) at one chunk.  The swizzle reads only row
// bits 0, 1, 3 and 4, which are the lane's t and not the block b, so a lane's
// read addresses differ by constants.  At D = 128, (row & 3) | ((row >> 3) & 3) << 2
// equals t: 16 different chunk positions (the same at D = 256, whose 512-byte
// rows put every row on the same banks).  At D = 64 (8 chunks, 128-byte rows)
// the 3-bit (r1, r3, r0 ^ r4) keeps the 8 lanes of one pass over 32 banks, and
// the 16 of one pass over 64 banks, on distinct banks (checked by a bank model).
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D >= 128) return (row & 3) | (((row >> 3) & 3) << 2);
  else return ((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row ^ (row >> 4)) & 1) << 2);
}
// XOR applied to a V row's chunk index: a transposed read takes 4 rows
// 8g + 4x + r (r < 4) x 2 chunks per 16-lane group g.  At D = 128 and 256,
// 2 ((row & 3) | (row >> 3 & 1) << 2) sends the 8 rows of groups g, g + 1 to 8
// different even chunk offsets; at D = 64, 2 (r1 | (r0 ^ r3) << 1) does the
// same for the 4 offsets a 128-byte row has, with the row's parity telling the
// 64-bank passes apart.  Both leave bit 2 of the row out (rows r and r + 4
// share the swizzle), and the offset is even.
template <int D>
__device__ __forceinline__ int vswz(int row) {
  if constexpr (D >= 128) return 2 * ((row & 3) | (((row >> 3) & 1) << 2));
  else return 2 * (((row >> 1) & 1) | (((row ^ (row >> 3)) & 1) << 1));
}

// Exchanges the odd 16-lane rows of a with the even rows of b; on two copies
// of x, a then holds x of rows 0, 0, 2, 2 and b x of rows 1, 1, 3, 3, so their
// max / sum is that over lanes l and l ^ 16.  Inline asm, as the 32-lane swap.
__device__ __forceinline__ void swap_rows(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// Max and sum over the 4 lanes l % 16 + 16 g of one query row.
__device__ __forceinline__ float quad_max(float x) {
  x = pair_max(x);
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_rows(a, b);
  return vmax(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float quad_sum(float x) {
  x = pair_sum(x);
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_rows(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
}  // namespace rows16

// SL slices of 16 rows per workgroup (4: 64 rows, or 8: 128 rows) and KS
// waves per slice: with KS = 2, wave (slice, half) takes keys 32 half ..
// 32 half + 31 of every tile, so each tile's work per wave halves again, and
// the two halves' (reference, sums, O) are merged at the end.
template <typename E, int D, bool CAUSAL, int KS, int SL>
__device__ __forceinline__ void fwd_rows16_body(const FwdArgs& a) {
  constexpr int ROWS = 16 * SL;                // query rows per workgroup
  typedef typename E::vec8 vec8;
  constexpr int BN = 64;                       // keys per tile
  constexpr int DP = D == 96 ? 128 : D;        // LDS row width (columns)
  constexpr int RB = DP * 2;                   // bytes per K / V row in LDS
  constexpr int GRB = D * 2;                   // bytes per K / V row in memory
  constexpr int CPR = DP / 8;                  // 16-byte chunks per LDS row
  constexpr int RPB = 64 / CPR;                // rows per wave-wide load
  constexpr int TILE16 = BN * CPR;             // chunks per tile
  constexpr int NT = 64 * SL * KS;             // threads
  constexpr int NLD = TILE16 / 64 / (SL * KS);  // wave-wide loads per wave per tile
  constexpr int NKS = DP / 32;                 // 32-deep steps of the score contraction
  constexpr int NKB = BN / 16 / KS;            // 16-key score blocks per wave and tile
  constexpr int NSA = NKS * NKB;               // score MFMAs per wave and tile (phase A slots)
  constexpr int NDB = D / 16;                  // 16-wide d blocks of O
  constexpr int NST = BN / 32 / KS;            // 32-key steps of the value contraction per wave
  constexpr int NSB = NDB * NST;               // value MFMAs per wave and tile (phase B slots)
  constexpr int PFA = 3, PFB = 4;              // fragment reads in flight
  static_assert(KS == 1 || KS == 2, "one or two waves per slice");
  static_assert(SL == 4 || (SL == 8 && KS == 1), "slices");
  static_assert(NLD >= 1, "tile loads");
  static_assert(D == 64 || D == 96 || D == 128 || D == 256, "head dimensions");
  static_assert(NKS >= 2 && NKB >= 2 && NSB > NKB, "slot layout");

  __shared__ u32x4 kA[TILE16], kB[TILE16], vA[TILE16], vB[TILE16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = wave % SL, half = wave / SL;  // half = 0 when KS = 1
  const int kb0 = half * NKB, st0 = half * NST;  // this wave's first score block and key step
  const int g = lane >> 4, t16 = lane & 15;
  const int NQ = a.nq, NK = a.nk;
  const int OFF = CAUSAL ? NK - NQ : 0;
  // (the causal pairing of long and short blocks on a CU is for two
  // workgroups per CU, which the 128 KB of tiles at D = 256 do not allow)
  const HeadItem wi = head_item(xcd_remap(blockIdx.x, a.n_blocks), a.n_bh, a.n_qblk, CAUSAL, D != 256);
  const int bh = wi.bh;
  const int qb = CAUSAL ? a.n_qblk - 1 - wi.idx : wi.idx;  // causal: longest query blocks first
  const int q0 = qb * ROWS;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + (size_t)bh * NQ * D;
  const uint16_t* __restrict__ Kg = (const uint16_t*)a.k + (size_t)bh * NK * D;
  const uint16_t* __restrict__ Vg = (const uint16_t*)a.v + (size_t)bh * NK * D;

  const int kv_end = CAUSAL ? min(NK, q0 + ROWS + OFF) : NK;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int qrow = q0 + slice * 16 + t16;  // this lane's query row
  const int wave_q0 = q0 + slice * 16;
  const int wave_end = CAUSAL ? min(n_tiles, (wave_q0 + 15 + OFF) / BN + 1) : n_tiles;
  const int n_vis = wave_q0 < NQ ? wave_end : 0;

  // Tile rows past the last key are never loaded: their K rows give scores
  // that the mask overwrites with -inf, their V rows meet weight 0, and 0
  // times a non-finite value is NaN.  So a V buffer is zeroed when a partial
  // tile can land in it before any full one: when one of the first two tiles
  // is partial.  At D = 96 the columns past D are never loaded either, and K's
  // meet Q's zeros: then every tile is zeroed.
  const bool zero_tiles = D != DP || (NK % BN != 0 && NK < 2 * BN);
  if (zero_tiles) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = tid; i < TILE16; i += NT) {
      if constexpr (D != DP) {
        kA[i] = z;
        kB[i] = z;
      }
      vA[i] = z;
      vB[i] = z;
    }
  }

  // Q as the B operand of the score MFMA: query qrow, d = 32 ks + 8 g .. +7
  vec8 qf[NKS];
  {
    const u32x4 flip = {a.qflip, a.qflip, a.qflip, a.qflip};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      const bool col_ok = D == DP || 32 * ks + 8 * g < D;  // columns past D stay zero
      if (qrow < NQ && col_ok) x = *(const u32x4*)(Qg + (size_t)qrow * D + 32 * ks + 8 * g) ^ flip;
      qf[ks] = __builtin_bit_cast(vec8, x);
    }
  }

  // tile DMA: LDS position cl of a row holds global chunk cl ^ swizzle(row)
  // (at D = 96 the lanes whose chunk is past the row load nothing)
  uint32_t koff[NLD], voff[NLD];
  bool kon[NLD], von[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPB + lane / CPR;
    const int cl = lane % CPR;
    const int kg = cl ^ rows16::kswz<DP>(row), vg = cl ^ rows16::vswz<DP>(row);
    koff[i] = row * GRB + kg * 16;
    voff[i] = row * GRB + vg * 16;
    kon[i] = kg < D / 8;
    von[i] = vg < D / 8;
  }
  auto issue = [&](u32x4* dst, const uint16_t* src, const uint32_t (&off)[NLD], const bool (&on)[NLD], int kv0)
      __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (size_t)kv0 * D), (short)0, (int)((uint32_t)(NK - kv0) * GRB), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if constexpr (D == DP) lds_load16(r, dst + (wave * NLD + i) * 64, off[i]);
      else if (on[i]) lds_load16(r, dst + (wave * NLD + i) * 64, off[i]);
    }
  };

  // K operand of score MFMA (kb, ks) (kb counts the tile's blocks): row
  // key_of(kb, t16), whose swizzle x is that of key_of(0, t16), global chunk
  // 4 ks + g.  Since (4 ks + g) ^ x = (g ^ x) ^ 4 ks, the address is one
  // per-lane base XOR (ks << 6) plus the block's row offset.
  const uint32_t kaddr0 = [&] {
    const int row = rows16::key_of(0, t16);
    return (uint32_t)(row * RB + ((g ^ rows16::kswz<DP>(row)) * 16));
  }();
  auto kfrag = [&](const u32x4* Kt, int m) __attribute__((always_inline)) {
    const int ks = m / NKB, kb = kb0 + m % NKB;
    return *(const u32x4*)((const char*)Kt + ((kaddr0 ^ (ks << 6)) + (32 * (kb >> 1) + 4 * (kb & 1)) * RB));
  };
  // V^T operand of value MFMA (db, st) by two transposed reads: in 16-lane
  // group g, lane 4r + q addresses row 32 st + 8 g + r (and + 4), columns
  // 16 db + 4q .. +3; with the row's swizzle even, d block db XORs (db << 5).
  const uint32_t vaddr0 = [&] {
    const int r = t16 >> 2, q = t16 & 3;
    const int row = 8 * g + r;
    return (uint32_t)(row * RB + ((rows16::vswz<DP>(row) + (q >> 1)) * 16) + (q & 1) * 8);
  }();
  auto vfrag = [&](const u32x4* Vt, int s) __attribute__((always_inline)) {
    const int db = s % NDB, st = st0 + s / NDB;
    const char* p = (const char*)Vt + (vaddr0 ^ (db << 5)) + 32 * st * RB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * RB));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // state: o (unnormalised O^T blocks), the score blocks of two tiles, pf (P^T
  // of the tile whose values are next), m_ref / mu / thr (lazy reference),
  // lsacc (rounded-P sum: lane n < 16 holds query n in element 0), lx (fp32
  // sum for LSE, per lane over its keys), a pending output rescale
  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[db][i] = 0.0f;
  f32x4 sA[NKB], sB[NKB];
  vec8 pf[NST];
  float m_ref = neg_inf(), lx = 0.0f, mu = 0.0f;
  f32x4 lsacc = {0.0f, 0.0f, 0.0f, 0.0f};
  // row 0 of the constant operand is all ones (lanes 16 g of k block g)
  const uint32_t one2 = t16 == 0 ? E::kOnes2 : 0u;
  const vec8 ones_op = __builtin_bit_cast(vec8, u32x4{one2, one2, one2, one2});
  float thr = neg_inf();
  bool pend = false;
  float pend_alpha = 1.0f;
  const float c = a.c;

  // element i of the wave's block kb of tile j: key j BN + key_of(kb0 + kb, 4 g + i)
  auto mask = [&](f32x4 (&s)[NKB], int j) __attribute__((always_inline)) {
    const int kv0 = j * BN;
    if (kv0 + BN > NK || (CAUSAL && kv0 + BN - 1 > wave_q0 + OFF)) {
      const int lim = (CAUSAL ? min(NK - 1, qrow + OFF) : NK - 1) - kv0;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rows16::key_of(kb0 + kb, 4 * g + i) > lim) s[kb][i] = neg_inf();
    }
  };
  // row max and the reference update, in slices: 0..NKB-1 block maxima, NKB
  // the row's max across its 4 lanes and the wave-uniform update
  float mpart[NKB];
  auto ref_slice = [&](const f32x4 (&s)[NKB], int k) __attribute__((always_inline)) {
    if (k < NKB) {
      float mx = vmax(vmax(s[k][0], s[k][1]), vmax(s[k][2], s[k][3]));
      pin(mx);
      mpart[k] = mx;
    } else {
      float mx = mpart[0];
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) mx = vmax(mx, mpart[kb]);
      mx = rows16::quad_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
        const float m_new = vmax(m_ref, mx * c);
        const float alpha = m_new == neg_inf() ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        lx *= alpha;
        m_ref = m_new;
        pend = true;
        pend_alpha = alpha;
        mu = m_new == neg_inf() ? 0.0f : m_new;
        thr = (m_new + E::kTau) / c;
      }
      pin(mu);
      pin(pend_alpha);
      pin(lx);
      pin(thr);
    }
  };
  // p = exp2(c s - mu) for block kb, its fp32 sum, its two 16-bit words
  float xsum = 0.0f;
  auto p_slice = [&](f32x4 (&s)[NKB], int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[kb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], c, -mu));
    const uint32_t w0 = E::pack(s[kb][0], s[kb][1]);
    const uint32_t w1 = E::pack(s[kb][2], s[kb][3]);
    const float part = (s[kb][0] + s[kb][1]) + (s[kb][2] + s[kb][3]);
    xsum = kb == 0 ? part : xsum + part;
    uint32_t r0 = w0, r1 = w1;
    pin(r0);
    pin(r1);
    pin(xsum);
    return u32x2{r0, r1};
  };

  // phase A of iteration j: score MFMAs of tile j+1 into sn beside the
  // exponentials of tile j in sc (one block of 4 scores every NKS slots); K
  // fragments PFA slots ahead, the first value fragments in the last PFB slots
  auto phase_a = [&](f32x4 (&sc)[NKB], f32x4 (&sn)[NKB], const u32x4* Kt, const u32x4* Vc, u32x4 (&vf)[NSB])
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    u32x4 kf[NSA];
#pragma unroll
    for (int k = 0; k < PFA; ++k) kf[k] = kfrag(Kt, k);
    u32x2 pw[NKB];
#pragma unroll
    for (int k = 0; k < NSA; ++k) {
      if (k + PFA < NSA) kf[k + PFA] = kfrag(Kt, k + PFA);
      if (k >= NSA - PFB) vf[k - (NSA - PFB)] = vfrag(Vc, k - (NSA - PFB));
      if (k % NKS == 1) pw[k / NKS] = p_slice(sc, k / NKS);
      const int ks = k / NKB, kb = k % NKB;
      const f32x4 z = {};
      sn[kb] = E::mfma16(__builtin_bit_cast(vec8, kf[k]), qf[ks], ks == 0 ? z : sn[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const u32x4 x = {pw[2 * st][0], pw[2 * st][1], pw[2 * st + 1][0], pw[2 * st + 1][1]};
      pf[st] = __builtin_bit_cast(vec8, x);
    }
    lx += xsum;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) pin(sn[kb]);
    __builtin_amdgcn_s_setprio(0);
  };
  // phase B of iteration j: value MFMAs of tile j and the rounded-P sum
  // beside the reference update of tile j+1
  auto phase_b = [&](const f32x4 (&sn)[NKB], const u32x4* Vt, u32x4 (&vf)[NSB]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      if (k + PFB < NSB) vf[k + PFB] = vfrag(Vt, k + PFB);
      if (k <= NKB) ref_slice(sn, k);
      const int db = k % NDB, st = k / NDB;
      o[db] = E::mfma16(__builtin_bit_cast(vec8, vf[k]), pf[st], o[db]);
      if (db == NDB - 1) lsacc = E::mfma16(ones_op, pf[st], lsacc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (pend) {
      lsacc[0] *= pend_alpha;  // lane n < 16 holds query n, whose factor it has
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] *= pend_alpha;
      pend = false;
    }
  };

  // ---- prologue ------------------------------------------------------------
  // zeroed tiles in place before any load lands; without them the first tile
  // loads go out at once, in flight together with the Q loads
  if (zero_tiles) __syncthreads();
  if (n_tiles > 0) {
    issue(kA, Kg, koff, kon, 0);
    issue(vA, Vg, voff, von, 0);
  }
  if (n_tiles > 1) issue(kB, Kg, koff, kon, BN);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // the first two K tiles and the first V tile in LDS
  if (n_vis > 0) {
#pragma unroll
    for (int k = 0; k < NSA; ++k) {
      const int ks = k / NKB, kb = k % NKB;
      const f32x4 z = {};
      sA[kb] = E::mfma16(__builtin_bit_cast(vec8, kfrag(kA, k)), qf[ks], ks == 0 ? z : sA[kb]);
    }
    mask(sA, 0);
#pragma unroll
    for (int k = 0; k <= NKB; ++k) ref_slice(sA, k);
    pend = false;
  }

  // ---- main loop: iteration j consumes S_j (in sc) and V_j ------------------
  // It reads K_{j+1} and V_j and loads V_{j+1} and K_{j+2} into the buffers
  // that V_{j-1} and K_j leave.
  auto iteration = [&](int j, f32x4 (&sc)[NKB], f32x4 (&sn)[NKB], const u32x4* Kn, u32x4* Kd, const u32x4* Vc,
                       u32x4* Vd) __attribute__((always_inline)) {
    // the explicit wait: at a barrier that heads a loop this compiler can drop
    // the wait for the tile loads issued in the previous iteration
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < n_tiles) issue(Vd, Vg, voff, von, (j + 1) * BN);
    if (j + 2 < n_tiles) issue(Kd, Kg, koff, kon, (j + 2) * BN);
    if (j >= n_vis) return;
    // after the wave's last visible tile the "next" scores come from whatever
    // K buffer is there and are fully masked
    u32x4 vf[NSB];
    phase_a(sc, sn, Kn, Vc, vf);
    apply_rescale();
    mask(sn, j + 1);
    phase_b(sn, Vc, vf);
  };
  for (int j = 0; j < n_tiles; j += 2) {
    iteration(j, sA, sB, kB, kA, vA, vB);
    if (j + 1 < n_tiles) iteration(j + 1, sB, sA, kA, kB, vB, vA);
  }

  // ---- epilogue: O = o / l, LSE = (m + log2 lx) ln 2 ----------------------
  // query t16's rounded-P sum is in lane t16, element 0 (copied to a scalar
  // before its bit cast: this compiler has folded a bit cast of a vector
  // element into a wrong value)
  float e0 = lsacc[0];
  pin(e0);
  float l_tot = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(t16 << 2, __builtin_bit_cast(int, e0)));
  float lx_tot = rows16::quad_sum(lx);
  float m_out = m_ref;
  if constexpr (KS == 2) {
    // The two halves of a slice hold o, l and lx against their own references
    // mu_0, mu_1 (lane for lane the same query and columns).  With M the
    // larger reference of the halves that saw a key, each half's terms take
    // the factor 2^(mu_h - M) (0 for a half that saw none): the sums over all
    // keys against M.  The tiles are free once every wave is past its last
    // iteration; half 1 leaves its values there for half 0.  (No tile load is
    // in flight after the last iteration; the wait states it for the barrier.)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x4* const ob = (f32x4*)(slice < 2 ? kA : kB) + (slice & 1) * (NDB * 64);
    float* const sb = (float*)vA + slice * 3 * 64;
    if (half == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) ob[db * 64 + lane] = o[db];
      sb[lane] = mu;
      sb[64 + lane] = l_tot;
      sb[128 + lane] = lx_tot;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (half == 0) {
      const float mu1 = sb[lane], l1 = sb[64 + lane], lx1 = sb[128 + lane];
      const bool live0 = l_tot > 0.0f, live1 = l1 > 0.0f;
      const float M = live0 && live1 ? vmax(mu, mu1) : live0 ? mu : mu1;
      const float a0 = live0 ? __builtin_amdgcn_exp2f(mu - M) : 0.0f;
      const float a1 = live1 ? __builtin_amdgcn_exp2f(mu1 - M) : 0.0f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const f32x4 o1 = ob[db * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] = __builtin_fmaf(o[db][i], a0, o1[i] * a1);
      }
      l_tot = __builtin_fmaf(l_tot, a0, l1 * a1);
      lx_tot = __builtin_fmaf(lx_tot, a0, lx1 * a1);
      m_out = M;
    }
  }
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < NQ && half == 0) {
    uint16_t* __restrict__ Og = (uint16_t*)a.o + ((size_t)bh * NQ + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 w = {E::pack(o[db][0] * inv, o[db][1] * inv), E::pack(o[db][2] * inv, o[db][3] * inv)};
      *(u32x2*)(Og + 16 * db + 4 * g) = w;
    }
    if (g == 0) a.lse[(size_t)bh * NQ + qrow] = l_tot > 0.0f ? (m_out + __log2f(lx_tot)) * kLn2 : neg_inf();
  }
}

// 64-row workgroups of 256 KS threads; two workgroups per CU with one wave
// per slice, one with two
template <int D, bool CAUSAL, int KS>
__global__ __launch_bounds__(256 * KS, KS == 1 ? 2 : 1) void fa_fwd_bf16_rows16_kernel(FwdArgs a) {
  fwd_rows16_body<BF16, D, CAUSAL, KS, 4>(a);
}
template <int D, bool CAUSAL, int KS>
__global__ __launch_bounds__(256 * KS, KS == 1 ? 2 : 1) void fa_fwd_f16_rows16_kernel(FwdArgs a) {
  fwd_rows16_body<F16, D, CAUSAL, KS, 4>(a);
}
// 128-row workgroups of 8 waves (D = 256), one per CU
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_fwd_bf16_rows16x8_kernel(FwdArgs a) {
  fwd_rows16_body<BF16, D, CAUSAL, 1, 8>(a);
}
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_fwd_f16_rows16x8_kernel(FwdArgs a) {
  fwd_rows16_body<F16, D, CAUSAL, 1, 8>(a);
}

}  // namespace fa
