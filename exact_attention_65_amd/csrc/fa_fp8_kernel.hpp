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
// bytes a row).  The score operand reads 2 x 16 bytes from 32 rows per lane
// group; 16 lanes of one read hit 16 different rows, which share bank lines in
// pairs (D = 128) or fours (D = 64), so the XOR spreads rows of one line over
// distinct chunks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ uint32_t addr(int row, int chunk) {
  return (uint32_t)(row * D + ((chunk ^ swz<D>(row)) * 16));
}
}  // namespace fp8

// Work split as in the bf16 kernel: 4 waves x 32 query rows, one workgroup per
// (b, h, 128-row query block).  Per 64-key tile j:
//   barrier; loads of tile j+1 (K, V codes into the other LDS buffers, their
//   scales into registers);
//   every wave converts 16 rows of V_j to the bf16 tile;
//   scores S^T = K Q^T (2 x D/64 scaled MFMAs), mask, online softmax, bf16 P;
//   barrier (the bf16 V tile complete);
//   O^T += V^T P^T (16 bf16 MFMAs at D = 128).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFp8Threads, 2) void fa_fwd_fp8_kernel(Fp8Args a) {
  constexpr int BN = 64;
  constexpr int CPR = D / 16;          // 16-byte chunks per E4M3 row
  constexpr int TILE16 = BN * CPR;     // 16-byte chunks per E4M3 tile
  constexpr int RPB = 64 / CPR;        // rows per wave-wide load
  constexpr int NLD = TILE16 / 256;    // wave-wide loads per wave per tile
  constexpr int NSC = D / 32;          // scale bytes per row
  constexpr int NKS = D / 64;          // 64-deep steps of the score contraction
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NCC = BN / 16;
  constexpr int RBH = 2 * D;           // bytes per bf16 row
  constexpr int CPRH = D / 8;          // 16-byte chunks per bf16 row
  constexpr int VPL = D / 4;           // V values one lane converts per tile
  static_assert(NLD >= 1 && RPB * CPR == 64 && NKB == 2, "tile shape");

  __shared__ u32x4 kA[TILE16], kB[TILE16], vA[TILE16], vB[TILE16];
  __shared__ u32x4 vb[BN * CPRH];

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
    uint32_t sdw = 0x7F7F7F7Fu;
    if (qrow < N) sdw = NSC == 4 ? *(const uint32_t*)(QSg + (size_t)qrow * 4)
                                 : (uint32_t) * (const uint16_t*)(QSg + (size_t)qrow * 2);
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

  // V conversion: rows 16 wave + lane/4, values d0 .. d0 + VPL - 1 of one MX
  // block, written as bf16 into vb in the bf16 kernel's V layout
  const int cv_row = wave * 16 + (lane >> 2);
  const int cv_d0 = (lane & 3) * VPL;

  // block scales of a tile, loaded into registers one tile ahead (a row's
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
      ts.k[kb] = 0x7F7F7F7Fu;
      if (row < N) ts.k[kb] = NSC == 4 ? *(const uint32_t*)(KSg + (size_t)row * 4)
                                       : (uint32_t) * (const uint16_t*)(KSg + (size_t)row * 2);
    }
    const int vrow = kv0 + cv_row;
    ts.v = vrow < N ? (uint32_t)VSg[(size_t)vrow * NSC + cv_d0 / 32] : 127u;
  };

  auto convert = [&](const u32x4* Vt, const TileScales& ts) __attribute__((always_inline)) {
    const float s = __builtin_bit_cast(float, ts.v << 23);
    constexpr int NCH = VPL / 16;  // E4M3 chunks read
#pragma unroll
    for (int cch = 0; cch < NCH; ++cch) {
      const u32x4 w = *(const u32x4*)((const char*)Vt + fp8::addr<D>(cv_row, cv_d0 / 16 + cch));
      uint32_t outw[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        outw[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[e], s, false));
        outw[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[e], s, true));
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = cv_d0 / 8 + 2 * cch + half;  // bf16 chunk (8 values)
        const u32x4 o4 = {outw[4 * half], outw[4 * half + 1], outw[4 * half + 2], outw[4 * half + 3]};
        *(u32x4*)((char*)vb + cv_row * RBH + ((c ^ vswz<D>(cv_row)) * 16)) = o4;
      }
    }
  };

  // V^T operand reads of the value MFMA (the bf16 kernel's lane layout)
  const uint32_t vaddr0 = [&] {
    const int g = lane >> 4, i16 = lane & 15;
    const int hh = g >> 1, gg = g & 1, r = i16 >> 2, q = i16 & 3;
    const int chunk = 2 * gg + (q >> 1);
    return (uint32_t)((8 * hh + r) * RBH + ((chunk ^ vswz<D>(r)) * 16) + (q & 1) * 8);
  }();
  auto vfrag = [&](int db, int cc) __attribute__((always_inline)) {
    const char* p = (const char*)vb + (vaddr0 ^ (db << 6)) + 16 * cc * RBH;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * RBH));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m_ref = neg_inf(), l = 0.0f, lx = 0.0f;
  const float c = a.c;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pf[NCC];

  // scores, mask, online softmax and bf16 P of tile j
  auto softmax_tile = [&](const u32x4* Kt, const TileScales& ts, int j) __attribute__((always_inline)) {
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int row = 32 * kb + swap23(c32);
      const uint32_t sdw = ts.k[kb];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 lo = *(const u32x4*)((const char*)Kt + fp8::addr<D>(row, 4 * ks + h));
        const u32x4 hi = *(const u32x4*)((const char*)Kt + fp8::addr<D>(row, 4 * ks + 2 + h));
        const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const int ksc = (int)((sdw >> (8 * (2 * ks + h))) & 0xFFu);
        const f32x16 z = {};
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[ks], ks == 0 ? z : s[kb], 0, 0, 0, ksc, 0,
                                                                qsc[ks]);
      }
    }
    // element (kb, i) holds key j*BN + 32kb + 8h + kofs(i) of query qrow
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
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = vmax(mx, s[kb][i]);
    mx = pair_max(mx);
    const float mt = mx * c;
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0) {
      const float m_new = vmax(m_ref, mt);
      const float alpha = m_new == neg_inf() ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      l *= alpha;
      lx *= alpha;
      m_ref = m_new;
    }
    const float mu = m_ref == neg_inf() ? 0.0f : m_ref;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      const int kb = cc >> 1, base = (cc & 1) * 8;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][base + 2 * e], c, -mu));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][base + 2 * e + 1], c, -mu));
        w[e] = pack_bf16(p0, p1);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, l, false);
        lx += p0 + p1;
      }
      const u32x4 x = {w[0], w[1], w[2], w[3]};
      pf[cc] = __builtin_bit_cast(bf16x8, x);
    }
  };

  __syncthreads();  // zeroed tiles visible before any load lands
  TileScales scA, scB;
  if (n_tiles > 0) {
    issue(kA, Kg, 0);
    issue(vA, Vg, 0);
    load_scales(scA, 0);
  }
  auto step = [&](int j, const u32x4* Kt, const u32x4* Vt, const TileScales& sc, u32x4* Kn, u32x4* Vn,
                  TileScales& scn) __attribute__((always_inline)) {
    // tile j has landed and every wave is done reading the bf16 V tile; the
    // explicit wait: this compiler can drop the wait for tile loads at a
    // barrier heading a loop
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < n_tiles) {
      issue(Kn, Kg, (j + 1) * BN);
      issue(Vn, Vg, (j + 1) * BN);
      load_scales(scn, (j + 1) * BN);
    }
    convert(Vt, sc);
    if (j < n_vis) softmax_tile(Kt, sc, j);
    __syncthreads();  // the bf16 V tile is complete
    if (j < n_vis) {
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(db, cc), pf[cc], o[db], 0, 0, 0);
    }
  };
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, kA, vA, scA, kB, vB, scB);
    if (j + 1 < n_tiles) step(j + 1, kB, vB, scB, kA, vA, scA);
  }

  // epilogue: O = o / l, LSE = (m + log2 lx) ln 2
  const float l_tot = pair_sum(l);
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
