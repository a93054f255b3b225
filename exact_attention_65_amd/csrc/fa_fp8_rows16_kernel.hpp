// FP8 attention forward at D = 256 with 16 query rows per wave (8 waves, 128
// rows per workgroup, one workgroup per CU): the inputs, scales and result of
// fa_fwd_fp8_kernel, the work split of the 16-row-wave bf16 kernel.
//
// At D = 256 a 32-row wave holds 128 output and 64 Q registers per lane, so
// fa_fwd_fp8_kernel runs one wave per SIMD.  Here a wave holds 16 rows (64
// output registers, 16 of Q) and two waves share each SIMD.  Per 64-key tile
// and wave:
//   * S^T = K Q^T on v_mfma_scale_f32_16x16x128_f8f6f4: 4 blocks of 16 keys x
//     2 steps of 128 d.  Operand layout (an in-bounds probe on the device,
//     random codes and scales against a host model): lane l holds row (or
//     column) l % 16, its bytes 0-15 are k = 16 (l / 16) .. +15 of the step and
//     bytes 16-31 are k = 64 + 16 (l / 16) .. +15; the scale of row r and
//     32-wide k block kb comes from lane r + 16 kb.  So lane l reads K chunks
//     8s + l/16 and 8s + 4 + l/16 of its row and supplies scale byte
//     4s + l/16 of that row, and the same for Q.  Key row t of block b is
//     key_of(b, t) of the 16-row-wave kernel, so the results are the P^T
//     fragments of the value MFMA directly.
//   * The online softmax of that kernel: lazy reference with the bf16
//     headroom, P rounded to bf16, the rounded-P sum on the matrix core, the
//     fp32 sum for the LSE.
//   * O^T += V^T P^T on the bf16 MFMA from a bf16 V tile, converted once per
//     workgroup from E4M3 with its block scales (exact, as in
//     fa_fwd_fp8_kernel) one tile ahead, into that kernel's V layout and
//     swizzle.
// One barrier per tile: iteration j reads K_j and the bf16 V_j, converts
// E4M3 V_{j+1} into the bf16 buffer V_{j-1} left, and loads K_{j+1} and E4M3
// V_{j+2} into the buffers K_{j-1} and V_j left; the barrier at the top of
// iteration j+1 publishes all of it.
#pragma once

#include "fa_fp8_kernel.hpp"
#include "fa_fwd_rows16_kernel.hpp"

namespace fa {

namespace fp8r16 {
// XOR on the 16-byte chunk index of an E4M3 K row (256 bytes, 16 chunks): the
// 16 lanes of a score read take rows key_of(b, 0..15) at one chunk, and the
// XOR, which reads only row bits 0, 1, 3 and 4 (the lanes' t), sends them to
// 16 different chunk positions: the bf16 kernel's K swizzle at D = 128, whose
// rows have the same 256 bytes.
__device__ __forceinline__ int ksw(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
// XOR on the chunk index of an E4M3 V row: the conversion's 16-lane passes
// take rows r and r + 1 at the same chunks, which the row's parity separates.
__device__ __forceinline__ int vsw(int row) { return row & 1; }
}  // namespace fp8r16

template <bool CAUSAL>
__device__ __forceinline__ void fp8_rows16_body(const Fp8Args& a) {
  typedef typename BF16::vec8 vec8;
  constexpr int D = 256, BN = 64, NSC = D / 32;  // NSC: scale bytes per row
  constexpr int NW = 8, NT = 64 * NW, ROWS = 16 * NW;
  constexpr int T8 = BN * D / 16;       // 16-byte chunks of an E4M3 tile
  constexpr int TB = BN * D * 2 / 16;   // 16-byte chunks of a bf16 tile
  constexpr int SCW = BN * NSC / 4;     // scale dwords of a tile
  constexpr int RB = D * 2;             // bytes per bf16 row
  constexpr int NLD = T8 / 64 / NW;     // wave-wide E4M3 loads per wave and tensor
  constexpr int NKB = BN / 16;          // 16-key score blocks
  constexpr int NKS = D / 128;          // 128-deep steps of the scaled MFMA
  constexpr int NDB = D / 16;           // 16-wide d blocks of O
  constexpr int NST = BN / 32;          // 32-key steps of the value MFMA
  constexpr int NSB = NDB * NST;        // value MFMAs per tile and wave
  constexpr int PFB = 4;                // value-fragment reads in flight
  static_assert(ROWS == kFp8Rows && NLD == 2 && SCW == 2 * 64 && NKS == 2, "layout");
  __shared__ u32x4 kA[T8], kB[T8], eA[T8], eB[T8];  // E4M3 K and V tiles
  __shared__ u32x4 wA[TB], wB[TB];                  // bf16 V tiles
  __shared__ uint32_t ksA[SCW], ksB[SCW], vsA[SCW], vsB[SCW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, t16 = lane & 15;
  const int N = a.n;
  const HeadItem wi = head_item(xcd_remap(blockIdx.x, a.n_blocks), a.n_blocks / a.n_qblk, a.n_qblk, CAUSAL, false);
  const int bh = wi.bh;
  const int qb = CAUSAL ? a.n_qblk - 1 - wi.idx : wi.idx;  // causal: longest query blocks first
  const int q0 = qb * ROWS;
  const uint8_t* Qg = a.q + (size_t)bh * N * D;
  const uint8_t* Kg = a.k + (size_t)bh * N * D;
  const uint8_t* Vg = a.v + (size_t)bh * N * D;
  const uint8_t* QSg = a.qs + (size_t)bh * N * NSC;
  const uint8_t* KSg = a.ks + (size_t)bh * N * NSC;
  const uint8_t* VSg = a.vs + (size_t)bh * N * NSC;

  const int kv_end = CAUSAL ? min(N, q0 + ROWS) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int qrow = q0 + wave * 16 + t16;  // this lane's query row
  const int wave_q0 = q0 + wave * 16;
  const int n_vis = wave_q0 >= N ? 0 : CAUSAL ? min(n_tiles, (wave_q0 + 15) / BN + 1) : n_tiles;

  // Rows past N are never loaded: every tile starts as zero codes (finite
  // values, which the mask or a zero weight then cancels) and zero scale codes.
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < T8; i += NT) kA[i] = kB[i] = eA[i] = eB[i] = z;
    for (int i = tid; i < TB; i += NT) wA[i] = wB[i] = z;
    for (int i = tid; i < SCW; i += NT) ksA[i] = ksB[i] = vsA[i] = vsB[i] = 0u;
  }

  // Q as the B operand: step s, bytes 0-15 Q[qrow][128 s + 16 g .. +15], bytes
  // 16-31 Q[qrow][128 s + 64 + 16 g .. +15] (signs flipped for a negative
  // scale); byte s of qsc is the scale of block 4 s + g of the row
  i32x8 qf[NKS];
  int qsc = 0;
  {
    const u32x4 fl = {a.qflip, a.qflip, a.qflip, a.qflip};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      int sb = 127;
      if (qrow < N) {
        const u32x4* r = (const u32x4*)(Qg + (size_t)qrow * D);
        lo = r[8 * s + g] ^ fl;
        hi = r[8 * s + 4 + g] ^ fl;
        sb = QSg[(size_t)qrow * NSC + 4 * s + g];
      }
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      qsc |= sb << (8 * s);
    }
  }

  // tile DMA: LDS position cl of a row holds global chunk cl ^ swizzle(row);
  // the scale rows of a tile (512 bytes) by 4-byte loads, K's by waves 0-1,
  // V's by waves 2-3
  uint32_t koff[NLD], voff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * 4 + lane / 16;
    const int cl = lane % 16;
    koff[i] = row * D + ((cl ^ fp8r16::ksw(row)) * 16);
    voff[i] = row * D + ((cl ^ fp8r16::vsw(row)) * 16);
  }
  auto issue = [&](u32x4* dst, const uint8_t* src, const uint32_t (&off)[NLD], uint32_t* sdst, const uint8_t* ssrc,
                   bool scale_wave, int kv0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (size_t)kv0 * D), (short)0, (int)((uint32_t)(N - kv0) * D), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i) lds_load16(r, dst + (wave * NLD + i) * 64, off[i]);
    if (scale_wave) {
      const int part = wave & 1;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ssrc + (size_t)kv0 * NSC), (short)0, (int)((uint32_t)(N - kv0) * NSC), kRsrcWord3);
      lds_load4(rs, (float*)(sdst + 64 * part), (uint32_t)(256 * part + 4 * lane));
    }
  };
  auto issue_k = [&](u32x4* kd, uint32_t* ksd, int kv0) __attribute__((always_inline)) {
    issue(kd, Kg, koff, ksd, KSg, wave < 2, kv0);
  };
  auto issue_v = [&](u32x4* ed, uint32_t* vsd, int kv0) __attribute__((always_inline)) {
    issue(ed, Vg, voff, vsd, VSg, wave >= 2 && wave < 4, kv0);
  };

  // E4M3 V tile -> bf16 V tile: thread (row cr, part cp) converts values
  // 32 cp .. 32 cp + 31 of its row with the row's scale of block cp into bf16
  // chunks 4 cp .. 4 cp + 3, placed with the 16-row-wave kernel's V swizzle
  // The conversion runs in steps beside the value MFMAs of the tile being
  // computed: cv_read brings the lane's 32 codes and scale into registers,
  // cv_group(e) converts and stores bf16 chunk e.
  const int cr = tid >> 3, cp = tid & 7;
  u32x4 cx0, cx1;
  float csc;
  auto cv_read = [&](const u32x4* ed, const uint32_t* vsd) __attribute__((always_inline)) {
    cx0 = ed[cr * 16 + ((2 * cp) ^ fp8r16::vsw(cr))];
    cx1 = ed[cr * 16 + ((2 * cp + 1) ^ fp8r16::vsw(cr))];
    const uint32_t code = ((const uint8_t*)vsd)[cr * NSC + cp];
    csc = __builtin_bit_cast(float, code << 23);
  };
  auto cv_group = [&](u32x4* wd, int e) __attribute__((always_inline)) {
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = 2 * e + h;
      const int x = (int)(m < 4 ? cx0[m] : cx1[m - 4]);
      w[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, csc, false));
      w[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, csc, true));
    }
    wd[cr * 32 + ((4 * cp + e) ^ rows16::vswz<D>(cr))] = u32x4{w[0], w[1], w[2], w[3]};
  };
  auto convert = [&](const u32x4* ed, const uint32_t* vsd, u32x4* wd) __attribute__((always_inline)) {
    cv_read(ed, vsd);
#pragma unroll
    for (int e = 0; e < 4; ++e) cv_group(wd, e);
  };

  // K operand of block b, step s: row key_of(b, t16), chunks 8 s + g and
  // 8 s + 4 + g; every block's row has the swizzle of key_of(0, t16)
  const int krow0 = rows16::key_of(0, t16);
  const int kx = fp8r16::ksw(krow0);
  auto kfrag = [&](const u32x4* Kt, int b, int s) __attribute__((always_inline)) {
    const int row = krow0 + 32 * (b >> 1) + 4 * (b & 1);
    const u32x4 lo = Kt[row * 16 + ((8 * s + g) ^ kx)];
    const u32x4 hi = Kt[row * 16 + ((8 * s + 4 + g) ^ kx)];
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto kscale = [&](const uint32_t* kst, int b, int s) __attribute__((always_inline)) {
    const int row = krow0 + 32 * (b >> 1) + 4 * (b & 1);
    return (int)((const uint8_t*)kst)[row * NSC + 4 * s + g];
  };
  // V^T operand of value MFMA (db, st): the 16-row-wave kernel's transposed reads
  const uint32_t vaddr0 = [&] {
    const int r = t16 >> 2, q = t16 & 3;
    const int row = 8 * g + r;
    return (uint32_t)(row * RB + ((rows16::vswz<D>(row) + (q >> 1)) * 16) + (q & 1) * 8);
  }();
  auto vfrag = [&](const u32x4* Wt, int k) __attribute__((always_inline)) {
    const int db = k % NDB, st = k / NDB;
    const char* p = (const char*)Wt + (vaddr0 ^ (db << 5)) + 32 * st * RB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * RB));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // state, as in the 16-row-wave kernel: o (unnormalised O^T blocks), m_ref /
  // mu / thr (lazy reference), lsacc (rounded-P sum: lane n < 16 holds query n
  // in element 0), lx (fp32 sum for the LSE, per lane over its keys)
  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[db][i] = 0.0f;
  float m_ref = neg_inf(), lx = 0.0f, mu = 0.0f, thr = neg_inf();
  f32x4 lsacc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t one2 = t16 == 0 ? BF16::kOnes2 : 0u;
  const vec8 ones_op = __builtin_bit_cast(vec8, u32x4{one2, one2, one2, one2});
  const float c = a.c;

  // cvt: whether this tile's iteration converts the next V tile (into Wn)
  auto compute = [&](const u32x4* Kt, const uint32_t* kst, const u32x4* Wt, int j, bool cvt, u32x4* Wn)
      __attribute__((always_inline)) {
    // scores: K fragments two MFMAs ahead
    f32x4 s[NKB];
    constexpr int NSA = NKB * NKS;
    i32x8 kf[NSA];
    int ksb[NSA];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      kf[m] = kfrag(Kt, m / NKS, m % NKS);
      ksb[m] = kscale(kst, m / NKS, m % NKS);
    }
#pragma unroll
    for (int m = 0; m < NSA; ++m) {
      if (m + 2 < NSA) {
        kf[m + 2] = kfrag(Kt, (m + 2) / NKS, (m + 2) % NKS);
        ksb[m + 2] = kscale(kst, (m + 2) / NKS, (m + 2) % NKS);
      }
      const int b = m / NKS, st = m % NKS;
      const f32x4 z = {};
      s[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[m], qf[st], st == 0 ? z : s[b], 0, 0, 0, ksb[m], 0,
                                                              (qsc >> (8 * st)) & 0xFF);
      __builtin_amdgcn_sched_barrier(0);
    }
    // mask: element i of block b is key j BN + key_of(b, 4 g + i) of query qrow
    const int kv0 = j * BN;
    if (kv0 + BN > N || (CAUSAL && kv0 + BN - 1 > wave_q0)) {
      const int lim = (CAUSAL ? min(N - 1, qrow) : N - 1) - kv0;
#pragma unroll
      for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rows16::key_of(b, 4 * g + i) > lim) s[b][i] = neg_inf();
    }
    // row max over the 4 lanes of the row, lazy reference update
    float mx = neg_inf();
#pragma unroll
    for (int b = 0; b < NKB; ++b) mx = vmax(mx, vmax(vmax(s[b][0], s[b][1]), vmax(s[b][2], s[b][3])));
    mx = rows16::quad_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
      const float m_new = vmax(m_ref, mx * c);
      const float alpha = m_new == neg_inf() ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      lx *= alpha;
      lsacc[0] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] *= alpha;
      m_ref = m_new;
      mu = m_new == neg_inf() ? 0.0f : m_new;
      thr = (m_new + BF16::kTau) / c;
    }
    // p = exp2(c s - mu), its fp32 sum, P^T of key step st from blocks 2 st, 2 st + 1
    vec8 pf[NST];
    float xsum = 0.0f;
    uint32_t pw[NKB][2];
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[b][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][e], c, -mu));
      pw[b][0] = BF16::pack(s[b][0], s[b][1]);
      pw[b][1] = BF16::pack(s[b][2], s[b][3]);
      xsum += (s[b][0] + s[b][1]) + (s[b][2] + s[b][3]);
    }
    lx += xsum;
#pragma unroll
    for (int st = 0; st < NST; ++st)
      pf[st] = __builtin_bit_cast(vec8, u32x4{pw[2 * st][0], pw[2 * st][1], pw[2 * st + 1][0], pw[2 * st + 1][1]});
    // O^T += V^T P^T and the rounded-P sum
    u32x4 vf[NSB];
#pragma unroll
    for (int k = 0; k < PFB; ++k) vf[k] = vfrag(Wt, k);
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      if (k + PFB < NSB) vf[k + PFB] = vfrag(Wt, k + PFB);
      const int db = k % NDB, st = k / NDB;
      o[db] = BF16::mfma16(__builtin_bit_cast(vec8, vf[k]), pf[st], o[db]);
      if (db == NDB - 1) lsacc = BF16::mfma16(ones_op, pf[st], lsacc);
      if (cvt && k >= 8 && k % 6 == 2) cv_group(Wn, (k - 8) / 6);  // slots 8, 14, 20, 26
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: K_0, E4M3 V_0 and V_1 in; V_0 converted -------------------
  __syncthreads();  // zeroed tiles in place before any load lands
  if (n_tiles > 0) {
    issue_k(kA, ksA, 0);
    issue_v(eA, vsA, 0);
  }
  if (n_tiles > 1) issue_v(eB, vsB, BN);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n_tiles > 0) convert(eA, vsA, wA);

  // ---- main loop ------------------------------------------------------------
  auto iteration = [&](int j, const u32x4* Kc, const uint32_t* ksc, u32x4* Kn, uint32_t* ksn, u32x4* Ec, uint32_t* vsc,
                       const u32x4* En, const uint32_t* vsn, const u32x4* Wc, u32x4* Wn) __attribute__((always_inline)) {
    // the explicit wait: at a barrier that heads a loop this compiler can drop
    // the wait for the tile loads issued in the previous iteration
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < n_tiles) issue_k(Kn, ksn, (j + 1) * BN);
    if (j + 2 < n_tiles) issue_v(Ec, vsc, (j + 2) * BN);
    // the next V tile's conversion: beside this tile's value MFMAs, or on its
    // own when this wave has no keys to compute here
    const bool cvt = j + 1 < n_tiles;
    if (cvt) cv_read(En, vsn);
    if (j < n_vis) {
      compute(Kc, ksc, Wc, j, cvt, Wn);
    } else if (cvt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) cv_group(Wn, e);
    }
  };
  for (int j = 0; j < n_tiles; j += 2) {
    iteration(j, kA, ksA, kB, ksB, eA, vsA, eB, vsB, wA, wB);
    if (j + 1 < n_tiles) iteration(j + 1, kB, ksB, kA, ksA, eB, vsB, eA, vsA, wB, wA);
  }

  // ---- epilogue: O = o / l, LSE = (m + log2 lx) ln 2 -------------------------
  float e0 = lsacc[0];
  pin(e0);
  const float l_tot = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(t16 << 2, __builtin_bit_cast(int, e0)));
  const float lx_tot = rows16::quad_sum(lx);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < N) {
    uint16_t* __restrict__ Og = (uint16_t*)a.o + ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 w = {BF16::pack(o[db][0] * inv, o[db][1] * inv), BF16::pack(o[db][2] * inv, o[db][3] * inv)};
      *(u32x2*)(Og + 16 * db + 4 * g) = w;
    }
    if (g == 0) a.lse[(size_t)bh * N + qrow] = l_tot > 0.0f ? (m_ref + __log2f(lx_tot)) * kLn2 : neg_inf();
  }
}

// 128-row workgroups of 8 waves, one per CU
template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_fwd_fp8_rows16_kernel(Fp8Args a) {
  fp8_rows16_body<CAUSAL>(a);
}

}  // namespace fa
