// Gradients of the exact attention forward for CDNA4 (gfx950), bf16 or fp16 inputs.
//
// The pages say only that a second pass computes the gradients over the same
// chunks without storing the score matrix ("Flash Attention: ускорить
// attention в 6 раз без потери точности", johe.ru, section "Стадии
// вычисления").  With the forward's log-sum-exp saved, every weight is
// recomputed exactly as P = exp(scale q.k - LSE), and for the upstream dO:
//   Delta_i = sum_d dO_id O_id,  dP = dO V^T,  dS = P (dP - Delta),
//   dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q.
// Two kernels, neither using atomics:
//   fa_bwd_dq_kernel    one workgroup per 128 query rows, K and V tiles streamed
//                       (the forward's loop): S^T = K Q^T, dP^T = V dO^T, then
//                       dQ^T += K^T dS^T; it also writes Delta for its rows;
//   fa_bwd_dkdv_kernel  one workgroup per 128 keys, Q and dO tiles streamed:
//                       S = Q K^T, dP = dO V^T, then dV^T += dO^T P and
//                       dK^T += Q^T dS (at D = 256 fa_bwd_dkdv16_kernel, one
//                       workgroup per 64 keys, the same products on the
//                       16x16x32 MFMA).
// Every other contraction runs on the 32x32x16 MFMA of the input type (bf16
// or fp16) with fp32 accumulators; P and dS are rounded to that type as MFMA operands,
// the outputs once.  The kernels are templates over the element type E (BF16 or
// F16, the forward's element-type structs).
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B*H*N], natural log, from the forward
  void* dq;
  void* dk;
  void* dv;
  float* delta;      // [B*H*Nq] workspace: sum_d dO O per query row
  float* nlse2;      // [B*H*Nq] workspace: -LSE log2(e) per query row
  int nq, nk;        // queries and keys per (b, h); causal: query i is position i + nk - nq
  int n_qblk;        // 128-row query blocks per (b, h)
  int n_kblk;        // dk/dv key blocks per (b, h): 128 keys, 64 at D = 256
  int n_qblocks;     // dq workgroups: B * H * n_qblk
  int n_kblocks;     // dk/dv workgroups: B * H * n_kblk
  float c;           // |scale| * log2(e), at least FLT_MIN
  float scale;       // the signed scale, applied to dQ and dK at the end
  uint32_t flip;     // XOR on the register-held Q (dq kernel) or K (dkdv kernel) bits: sign of scale
};

constexpr int kBwdThreads = 256;
constexpr int kBwdRows = 128;
constexpr float kLog2e = 1.44269504088896340736f;

namespace bwd {

// XOR applied to the 16-byte chunk index of tile row `row`.  Every tile here
// is read both ways: 16 bytes a lane from 32 rows x 1 chunk (row_frag), and
// transposed, 8 bytes a lane from 4 rows x 4 chunks (tr_frag).  With 64 banks
// of 4 bytes both are conflict-free when the XOR is a bijection on the rows
// that share a bank line and sends each aligned group of 4 rows to 4
// different groups of 4 chunks:
//   D = 128 (one row per line):  row = 4a + b  ->  4b + a  (a, b < 4);
//   D = 64  (two rows per line): the 3 bits of (row >> 1) & 7 reversed;
//   D = 256 (two lines per row): as D = 128, since every row starts on the
//   same bank and the XOR keeps a chunk within its 256-byte line.
template <int D>
__device__ __forceinline__ int bswz(int row) {
  if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else {
    const int u = (row >> 1) & 7;
    return ((u & 1) << 2) | (u & 2) | (u >> 2);
  }
}

// Byte offset of 16-byte chunk `chunk` of tile row `row` (rows of D 16-bit elements).
template <int D>
__device__ __forceinline__ uint32_t chunk_addr(int row, int chunk) {
  return (uint32_t)(row * D * 2 + ((chunk ^ bswz<D>(row)) * 16));
}

// Per-lane LDS addresses of the two operand reads.  bswz depends on the row
// only through bits 0..3, and a chunk index enters the byte address as
// 16 * (chunk ^ bswz(row)), so the row block (kb, cc) adds a constant and the
// column block (kk, db) XORs a constant into one per-lane base:
//   row read (A rows 32kb + swap23(c32), columns 16kk + 8h .. +7):
//       (rbase ^ (kk << 5)) + 32 kb RB
//   transposed read (A rows = tile columns 32db .. +31, A columns = tile rows
//   16cc + 8hh + r and +4; the lane layout of the forward's V^T read):
//       (tbase[x] ^ (db << 6)) + 16 cc RB,  x = 0, 1 for the rows r and r + 4
template <int D>
__device__ __forceinline__ uint32_t row_base(int c32, int h) {
  return chunk_addr<D>(swap23(c32), h);
}
template <int D>
__device__ __forceinline__ uint32_t tr_base(int lane, int x) {
  const int g = lane >> 4, i16 = lane & 15;
  const int hh = g >> 1, gg = g & 1, r = i16 >> 2, q = i16 & 3;
  return chunk_addr<D>(8 * hh + r + 4 * x, 2 * gg + (q >> 1)) + (q & 1) * 8;
}

template <int D>
__device__ __forceinline__ u32x4 row_frag(const u32x4* t, uint32_t rbase, int kb, int kk) {
  return *(const u32x4*)((const char*)t + ((rbase ^ (uint32_t)(kk << 5)) + kb * 32 * D * 2));
}

template <int D>
__device__ __forceinline__ u32x4 tr_frag(const u32x4* t, uint32_t tb0, uint32_t tb1, int db, int cc) {
  const char* base = (const char*)t + cc * 16 * D * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + (tb0 ^ (uint32_t)(db << 6))));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + (tb1 ^ (uint32_t)(db << 6))));
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row of the operand held in registers: [row][16kk + 8h .. +7] as MFMA B
// fragments, signs flipped by `flip`, zero for rows past N.
template <typename V, int NKK>
__device__ __forceinline__ void load_row(V (&f)[NKK], const uint16_t* g, int row, int N, int D, int h,
                                         uint32_t flip) {
  const u32x4 fl = {flip, flip, flip, flip};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < N) x = *(const u32x4*)(g + (size_t)row * D + 16 * kk + 8 * h) ^ fl;
    f[kk] = __builtin_bit_cast(V, x);
  }
}

// Pack 8 consecutive fp32 values of an accumulator into one 16-bit operand.
template <typename E>
__device__ __forceinline__ typename E::vec8 pack8(const f32x16& s, int base) {
  // scalars first: this compiler miscompiles __builtin_bit_cast of a vector element
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = E::pack(s[base + 2 * e], s[base + 2 * e + 1]);
  const u32x4 x = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(typename E::vec8, x);
}

// Store a [D x 32] MFMA accumulator (rows d, this lane's column = one row of
// the output) in the 16-bit type after multiplying by mul.
template <typename E, int NDB>
__device__ __forceinline__ void store_rows(uint16_t* out_row, const f32x16 (&acc)[NDB], int h, float mul) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * h;
      const u32x2 w = {E::pack(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul),
                       E::pack(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      *(u32x2*)(out_row + d) = w;
    }
}

// Delta = sum_d dO O of this lane's row (rows past N: 0): dot products of the
// 16-bit pairs of its half of the row (dO already in dof), then the two
// halves' sum.
template <typename E, int D>
__device__ __forceinline__ float row_delta(const typename E::vec8 (&dof)[D / 16], const uint16_t* Og, int row,
                                           int N, int h) {
  constexpr int NKK = D / 16;
  typename E::vec8 of[NKK];
  load_row(of, Og, row, N, D, h, 0u);
  float dsum = 0.0f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const u32x4 x = __builtin_bit_cast(u32x4, dof[kk]), y = __builtin_bit_cast(u32x4, of[kk]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t xe = x[e], ye = y[e];
      dsum = E::dot2(xe, ye, dsum);
    }
  }
  return pair_sum(dsum);
}

}  // namespace bwd

// ---------------------------------------------------------------------------
// Delta and -LSE log2(e) of every row into the workspace, by the dq kernel's
// prologue arithmetic (4 waves x 32 rows per workgroup): the first launch of a
// backward whose dq and dk/dv workgroups share the second.
template <typename E, int D>
__global__ __launch_bounds__(kBwdThreads) void fa_bwd_delta_kernel(BwdArgs a) {
  typedef typename E::vec8 vec8;
  constexpr int NKK = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int N = a.nq;
  const int bh = blockIdx.x / a.n_qblk, qb = blockIdx.x % a.n_qblk;
  const int qrow = qb * kBwdRows + wave * 32 + c32;
  const size_t head = (size_t)bh * N * D;
  vec8 dof[NKK];
  bwd::load_row(dof, (const uint16_t*)a.dout + head, qrow, N, D, h, 0u);
  const float delta = bwd::row_delta<E, D>(dof, (const uint16_t*)a.o + head, qrow, N, h);
  if (qrow < N && h == 0) {
    a.delta[(size_t)bh * N + qrow] = delta;
    a.nlse2[(size_t)bh * N + qrow] = -(a.lse[(size_t)bh * N + qrow] * kLog2e);
  }
}

// ---------------------------------------------------------------------------
// dQ (and Delta): 4 waves x 32 query rows; 64-key K and V tiles streamed
// through double-buffered LDS by buffer-to-LDS loads, one barrier per tile.
// Per tile and wave: 16 MFMAs S^T = K Q^T (keys on rows, this lane's query on
// the columns: the forward's orientation), 16 MFMAs dP^T = V dO^T, the
// elementwise dS^T = P^T (dP^T - Delta), and 16 MFMAs dQ^T += K^T dS^T with
// K^T read transposed from the same tile (for D = 128; half as many for 64).
//
// The body takes the workgroup index blk (blockIdx.x of its own launch, or its
// offset in a launch shared with the dk/dv workgroups).  DELTA: the prologue
// also writes Delta and -LSE log2(e) of the rows to the workspace (otherwise
// fa_bwd_delta_kernel has written them).
template <typename E, int D, bool CAUSAL, bool DELTA>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a, int blk) {
  typedef typename E::vec8 vec8;
  // D = 96 rows sit in LDS as 128-wide rows whose last 4 chunks stay zero (the
  // LDS addresses are the D = 128 ones); global rows keep their width
  constexpr int DP = D == 96 ? 128 : D;
  constexpr int BN = 64, RB = DP * 2, GRB = D * 2, CPR = DP / 8, RPB = 64 / CPR, TILE16 = BN * CPR;
  constexpr int NLD = TILE16 / 64 / 4, NKB = BN / 32, NDB = D / 32, NKK = D / 16, NCC = BN / 16;
  __shared__ u32x4 kA[TILE16], kB[TILE16], vA[TILE16], vB[TILE16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c32 = lane & 31;
  // N: queries, NK: keys; under the causal mask key j is visible to query i
  // iff j <= i + OFF
  const int N = a.nq, NK = a.nk, OFF = CAUSAL ? NK - N : 0;
  const HeadItem wi = head_item(xcd_remap(blk, a.n_qblocks), a.n_qblocks / a.n_qblk, a.n_qblk, CAUSAL, true);
  const int bh = wi.bh;
  const int qb = CAUSAL ? a.n_qblk - 1 - wi.idx : wi.idx;  // causal: longest query blocks first
  const int q0 = qb * kBwdRows;
  const size_t head = (size_t)bh * N * D, headk = (size_t)bh * NK * D;
  const uint16_t* Qg = (const uint16_t*)a.q + head;
  const uint16_t* Kg = (const uint16_t*)a.k + headk;
  const uint16_t* Vg = (const uint16_t*)a.v + headk;
  const uint16_t* Og = (const uint16_t*)a.o + head;
  const uint16_t* dOg = (const uint16_t*)a.dout + head;

  const int kv_end = CAUSAL ? min(NK, q0 + kBwdRows + OFF) : NK;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int qrow = q0 + wave * 32 + c32;
  const int wave_q0 = q0 + wave * 32;
  const int n_vis = wave_q0 >= N ? 0 : CAUSAL ? min(n_tiles, (wave_q0 + 31 + OFF) / BN + 1) : n_tiles;

  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < TILE16; i += kBwdThreads) kA[i] = kB[i] = vA[i] = vB[i] = z;
  }

  // this lane's query row: Q (signs flipped for a negative scale) and dO as MFMA
  // B fragments; Delta = sum_d dO O (each half-wave holds half the d's)
  vec8 qf[NKK], dof[NKK];
  bwd::load_row(qf, Qg, qrow, N, D, h, a.flip);
  bwd::load_row(dof, dOg, qrow, N, D, h, 0u);
  const float delta = bwd::row_delta<E, D>(dof, Og, qrow, N, h);
  const float lse2 = qrow < N ? a.lse[(size_t)bh * N + qrow] * kLog2e : 0.0f;
  if (DELTA && qrow < N && h == 0) {
    a.delta[(size_t)bh * N + qrow] = delta;
    a.nlse2[(size_t)bh * N + qrow] = -lse2;
  }

  // LDS position cl of a row holds global chunk cl ^ swizzle(row); at D = 96
  // the lanes whose chunk is past the row load nothing
  uint32_t koff[NLD];
  bool kon[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPB + lane / CPR;
    const int kg = (lane % CPR) ^ bwd::bswz<DP>(row);
    koff[i] = row * GRB + kg * 16;
    kon[i] = kg < D / 8;
  }
  auto issue = [&](u32x4* dst, const uint16_t* src, int kv0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (size_t)kv0 * D), (short)0, (int)((uint32_t)(NK - kv0) * GRB), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      if (D == DP || kon[i]) lds_load16(r, dst + (wave * NLD + i) * 64, koff[i]);
  };

  f32x16 dqa[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[db][i] = 0.0f;

  // operand of score slot f: rows of block f / (2 NKK), chunk (f / 2) % NKK of
  // K (even f: S^T) or V (odd f: dP^T); of dQ slot f: key step f / NDB, d
  // block f % NDB of K^T
  const uint32_t rbase = bwd::row_base<DP>(c32, h), tb0 = bwd::tr_base<DP>(lane, 0), tb1 = bwd::tr_base<DP>(lane, 1);
  auto sfrag = [&](const u32x4* Kt, const u32x4* Vt, int f) __attribute__((always_inline)) {
    return bwd::row_frag<DP>((f & 1) ? Vt : Kt, rbase, f / (2 * NKK), (f / 2) % NKK);
  };
  auto gfrag = [&](const u32x4* Kt, int f) __attribute__((always_inline)) {
    return bwd::tr_frag<DP>(Kt, tb0, tb1, f % NDB, f / NDB);
  };
  // per tile and wave, two phases of MFMA slots: the score phase (S^T and
  // dP^T, block kb = 0 then 1), then the dQ phase (key steps cc = 0 .. 3);
  // block 0's elementwise dS^T runs beside block 1's score MFMAs, block 1's
  // beside the dQ MFMAs of block 0's steps; LDS operands are read PF slots ahead
  auto compute = [&](const u32x4* Kt, const u32x4* Vt, int j) __attribute__((always_inline)) {
    constexpr int NSS = 2 * NKB * NKK, NSG = NDB * NCC, PF = 4;
    // a block's 16 elementwise steps spread over half a phase's slots: slot
    // k of that half takes steps [16k / H, 16(k+1) / H), H = slots / 2 (at
    // D = 256, 32 slots: one step every second slot)
    constexpr int HS = NSS / 2, HG = NSG / 2;
    static_assert(HS <= 32 && HG <= 16 && NKB == 2, "slot layout");
    const int kv0 = j * BN;
    const bool masked = kv0 + BN > NK || (CAUSAL && kv0 + BN - 1 > wave_q0 + OFF);
    f32x16 s[NKB], dp[NKB];
    vec8 dsf[NCC];
    // element (kb, i) holds key kv0 + 32kb + 8h + kofs(i) of query qrow
    auto mask_block = [&](int kb) __attribute__((always_inline)) {
      if (masked) {
        const int lim = (CAUSAL ? min(NK - 1, qrow + OFF) : NK - 1) - kv0 - 8 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = 32 * kb + 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
          if (kofs > lim) s[kb][i] = neg_inf();
        }
      }
    };
    auto ds_elem = [&](int kb, int i) __attribute__((always_inline)) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], a.c, -lse2));
      float ds = p * (dp[kb][i] - delta);
      pin(ds);
      s[kb][i] = ds;
      if ((i & 7) == 7) dsf[2 * kb + (i >> 3)] = bwd::pack8<E>(s[kb], i & 8);
    };
    u32x4 sf[NSS], gf[NSG];
#pragma unroll
    for (int k = 0; k < PF; ++k) sf[k] = sfrag(Kt, Vt, k);
#pragma unroll
    for (int k = 0; k < NSS; ++k) {
      if (k + PF < NSS) sf[k + PF] = sfrag(Kt, Vt, k + PF);
      else gf[k + PF - NSS] = gfrag(Kt, k + PF - NSS);
      const int kb = k / (2 * NKK), kk = (k / 2) % NKK;
      const f32x16 z = {};
      if (k & 1)
        dp[kb] = E::mfma(__builtin_bit_cast(vec8, sf[k]), dof[kk], kk == 0 ? z : dp[kb]);
      else
        s[kb] = E::mfma(__builtin_bit_cast(vec8, sf[k]), qf[kk], kk == 0 ? z : s[kb]);
      if (k == NSS / 2) mask_block(0);
      if (k >= NSS / 2)
#pragma unroll
        for (int e = (k - HS) * 16 / HS; e < (k - HS + 1) * 16 / HS; ++e) ds_elem(0, e);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k = 0; k < NSG; ++k) {
      if (k + PF < NSG) gf[k + PF] = gfrag(Kt, k + PF);
      const int cc = k / NDB, db = k % NDB;
      dqa[db] = E::mfma(__builtin_bit_cast(vec8, gf[k]), dsf[cc], dqa[db]);
      if (k == 0) mask_block(1);
      if (k < NSG / 2)
#pragma unroll
        for (int e = k * 16 / HG; e < (k + 1) * 16 / HG; ++e) ds_elem(1, e);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __syncthreads();  // zeroed tiles visible before any load lands
  if (n_tiles > 0) {
    issue(kA, Kg, 0);
    issue(vA, Vg, 0);
  }
  auto step = [&](int j, const u32x4* Kt, const u32x4* Vt, u32x4* Kn, u32x4* Vn) __attribute__((always_inline)) {
    // the explicit wait: this compiler can drop the wait for tile loads at a
    // barrier heading a loop
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < n_tiles) {
      issue(Kn, Kg, (j + 1) * BN);
      issue(Vn, Vg, (j + 1) * BN);
    }
    if (j < n_vis) compute(Kt, Vt, j);
  };
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, kA, vA, kB, vB);
    if (j + 1 < n_tiles) step(j + 1, kB, vB, kA, vA);
  }

  if (qrow < N) bwd::store_rows<E>((uint16_t*)a.dq + head + (size_t)qrow * D, dqa, h, a.scale);
}

// two workgroups per CU; at D = 256 (Q, dO and dQ of 32 rows take 256
// registers per lane) one, with 512 registers per lane over VGPRs and AGPRs
template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, D == 256 ? 1 : 2) void fa_bwd_dq_kernel(BwdArgs a) {
  bwd_dq_body<E, D, CAUSAL, true>(a, blockIdx.x);
}

// ---------------------------------------------------------------------------
// dK and dV: 4 waves x 32 keys; 64-query Q and dO tiles streamed through
// double-buffered LDS, with the rows' -LSE log2(e) and Delta.  Per tile and
// wave, two phases of MFMA slots (one MFMA each):
//   score phase     S = Q K^T and dP = dO V^T, block kb = 0 then 1 (32 query
//                   rows each, permuted by swap23 so that each lane's values
//                   of one key come in runs of 8 consecutive queries; this
//                   lane's key on the columns);
//   gradient phase  dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
//                   transposed, query steps cc = 0 .. 3.
// The elementwise P = exp2(c s - LSE log2 e), dS = P (dP - Delta) and the 16-bit
// packing of block 0 run beside block 1's score MFMAs, those of block 1 beside
// the gradient MFMAs of block 0's steps; LDS operands are read PF slots ahead.
// Queries past N (and, under the causal mask, before the key) get weight 0.
template <typename E, int D, bool CAUSAL>
__device__ __forceinline__ void bwd_dkdv_body(const BwdArgs& a, int blk) {
  typedef typename E::vec8 vec8;
  constexpr int DP = D == 96 ? 128 : D;  // LDS row width (as in the dq body)
  constexpr int BQ = 64, RB = DP * 2, GRB = D * 2, CPR = DP / 8, RPB = 64 / CPR, TILE16 = BQ * CPR;
  constexpr int NLD = TILE16 / 64 / 4, NKB = BQ / 32, NDB = D / 32, NKK = D / 16, NCC = BQ / 16;
  constexpr int NSS = 2 * NKB * NKK;  // score-phase slots
  constexpr int NSG = 2 * NDB * NCC;  // gradient-phase slots
  constexpr int PF = 4;               // operand reads in flight
  // softmax steps of a block per slot: slot k of the half phase beside which a
  // block's 16 steps run takes steps [16k / H, 16(k+1) / H) (block 0 beside
  // block 1's score MFMAs, block 1 beside the gradient MFMAs)
  constexpr int HS = NSS / 2, HG = NSG / 2;
  static_assert(HS <= 16 && HG <= 16 && NKB == 2, "slot layout");
  __shared__ u32x4 qA[TILE16], qB[TILE16], gA[TILE16], gB[TILE16];
  __shared__ f32x4 lA[BQ / 4], lB[BQ / 4], dA[BQ / 4], dB[BQ / 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c32 = lane & 31;
  // N: queries, NK: keys; under the causal mask key j is visible to query i
  // iff i + OFF >= j
  const int N = a.nq, NK = a.nk, OFF = CAUSAL ? NK - N : 0;
  const HeadItem wi = head_item(xcd_remap(blk, a.n_kblocks), a.n_kblocks / a.n_kblk, a.n_kblk, CAUSAL, false);
  const int bh = wi.bh;
  const int kblk = wi.idx;  // causal: the first key blocks see the most queries
  const int k0 = kblk * kBwdRows;
  const size_t head = (size_t)bh * N * D, headk = (size_t)bh * NK * D;
  const uint16_t* Qg = (const uint16_t*)a.q + head;
  const uint16_t* Kg = (const uint16_t*)a.k + headk;
  const uint16_t* Vg = (const uint16_t*)a.v + headk;
  const uint16_t* dOg = (const uint16_t*)a.dout + head;
  const float* Lg = a.nlse2 + (size_t)bh * N;
  const float* Dg = a.delta + (size_t)bh * N;

  const int key = k0 + wave * 32 + c32;  // this lane's key
  const int wave_k0 = k0 + wave * 32;
  const int n_qt = (N + BQ - 1) / BQ;
  const int t_first = CAUSAL ? max(0, k0 - OFF) / BQ : 0;      // first query tile seeing key k0
  const int t_wave = CAUSAL ? max(0, wave_k0 - OFF) / BQ : 0;  // first one seeing this wave's first key
  const bool active = wave_k0 < NK;

  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < TILE16; i += kBwdThreads) qA[i] = qB[i] = gA[i] = gB[i] = z;
  }

  // this lane's key: K (signs flipped for a negative scale) and V as MFMA B fragments
  vec8 kreg[NKK], vreg[NKK];
  bwd::load_row(kreg, Kg, key, NK, D, h, a.flip);
  bwd::load_row(vreg, Vg, key, NK, D, h, 0u);

  uint32_t toff[NLD];
  bool ton[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPB + lane / CPR;
    const int kg = (lane % CPR) ^ bwd::bswz<DP>(row);
    toff[i] = row * GRB + kg * 16;
    ton[i] = kg < D / 8;
  }
  // query tile t: Q and dO rows, and the rows' -LSE log2(e) and Delta (the
  // first wave, 4 bytes a lane), all by buffer-to-LDS loads
  auto issue = [&](u32x4* qd, u32x4* gd, f32x4* ld, f32x4* dd, int tq) __attribute__((always_inline)) {
    const int r0 = tq * BQ;
    const uint32_t bytes = (uint32_t)(N - r0) * GRB;
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Qg + (size_t)r0 * D), (short)0, (int)bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rg =
        __builtin_amdgcn_make_buffer_rsrc((void*)(dOg + (size_t)r0 * D), (short)0, (int)bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      if (D == DP || ton[i]) {
        lds_load16(rq, qd + (wave * NLD + i) * 64, toff[i]);
        lds_load16(rg, gd + (wave * NLD + i) * 64, toff[i]);
      }
    if (wave == 0) {
      const uint32_t fbytes = (uint32_t)(N - r0) * 4;
      const __amdgpu_buffer_rsrc_t rl =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Lg + r0), (short)0, (int)fbytes, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rd =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Dg + r0), (short)0, (int)fbytes, kRsrcWord3);
      lds_load4(rl, (float*)ld, (uint32_t)lane * 4);
      lds_load4(rd, (float*)dd, (uint32_t)lane * 4);
    }
  };

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[db][i] = dva[db][i] = 0.0f;

  // operand of score slot f: rows of block f / (2 NKK), chunk (f / 2) % NKK of
  // Q (even f: S) or dO (odd f: dP); of gradient slot f: step f / (2 NDB),
  // d block (f / 2) % NDB of dO^T (even f: dV) or Q^T (odd f: dK)
  const uint32_t rbase = bwd::row_base<DP>(c32, h), tb0 = bwd::tr_base<DP>(lane, 0), tb1 = bwd::tr_base<DP>(lane, 1);
  auto sfrag = [&](const u32x4* Qt, const u32x4* Gt, int f) __attribute__((always_inline)) {
    return bwd::row_frag<DP>((f & 1) ? Gt : Qt, rbase, f / (2 * NKK), (f / 2) % NKK);
  };
  auto gfrag = [&](const u32x4* Qt, const u32x4* Gt, int f) __attribute__((always_inline)) {
    return bwd::tr_frag<DP>((f & 1) ? Qt : Gt, tb0, tb1, (f / 2) % NDB, f / (2 * NDB));
  };

  auto compute = [&](const u32x4* Qt, const u32x4* Gt, const f32x4* Lt, const f32x4* Dt, int tq)
      __attribute__((always_inline)) {
    // tiles with a query past N or (causal) before one of the wave's keys
    const bool masked = (CAUSAL && tq * BQ + OFF < wave_k0 + 31) || tq * BQ + BQ > N;
    const float c = a.c;
    f32x16 s[NKB], dp[NKB];
    vec8 pf[NCC], dsf[NCC];
    // element (kb, i) holds query tq*BQ + 4 q4 + (i & 3) of this lane's key,
    // q4 = 8kb + 2h + 4(i >> 3) + ((i >> 2) & 1)
    auto q4_of = [&](int kb, int i) __attribute__((always_inline)) {
      return 8 * kb + 2 * h + 4 * (i >> 3) + ((i >> 2) & 1);
    };
    // the rows' -LSE log2(e) and Delta, read before the tile's first MFMA so
    // that no wait for them drains the operand reads in flight
    f32x4 nl[NKB][4], dl[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        nl[kb][g] = Lt[q4_of(kb, 4 * g)];
        dl[kb][g] = Dt[q4_of(kb, 4 * g)];
      }
    // a masked block's scores, once, before its first softmax element
    auto mask_block = [&](int kb) __attribute__((always_inline)) {
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qg = tq * BQ + 4 * q4_of(kb, i) + (i & 3);
          if (qg >= N || (CAUSAL && qg + OFF < key)) s[kb][i] = neg_inf();
        }
      }
    };
    auto softmax_elem = [&](int kb, int i) __attribute__((always_inline)) {
      const int g = i >> 2, e = i & 3;
      const float sv = s[kb][i];
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, nl[kb][g][e]));
      float ds = p * (dp[kb][i] - dl[kb][g][e]);
      float pp = p;
      pin(pp);
      pin(ds);
      s[kb][i] = pp;
      dp[kb][i] = ds;
      if ((i & 7) == 7) {
        const int cc = 2 * kb + (i >> 3);
        pf[cc] = bwd::pack8<E>(s[kb], i & 8);
        dsf[cc] = bwd::pack8<E>(dp[kb], i & 8);
      }
    };

    u32x4 sf[NSS], gf[NSG];
#pragma unroll
    for (int k = 0; k < PF; ++k) sf[k] = sfrag(Qt, Gt, k);
    // score phase
#pragma unroll
    for (int k = 0; k < NSS; ++k) {
      if (k + PF < NSS) sf[k + PF] = sfrag(Qt, Gt, k + PF);
      else gf[k + PF - NSS] = gfrag(Qt, Gt, k + PF - NSS);
      const int kb = k / (2 * NKK), kk = (k / 2) % NKK;
      const f32x16 z = {};
      if (k & 1)
        dp[kb] = E::mfma(__builtin_bit_cast(vec8, sf[k]), vreg[kk], kk == 0 ? z : dp[kb]);
      else
        s[kb] = E::mfma(__builtin_bit_cast(vec8, sf[k]), kreg[kk], kk == 0 ? z : s[kb]);
      if (k == NSS / 2) mask_block(0);
      if (k >= NSS / 2)
#pragma unroll
        for (int e = (k - HS) * 16 / HS; e < (k - HS + 1) * 16 / HS; ++e) softmax_elem(0, e);
      __builtin_amdgcn_sched_barrier(0);
    }
    // gradient phase
#pragma unroll
    for (int k = 0; k < NSG; ++k) {
      if (k + PF < NSG) gf[k + PF] = gfrag(Qt, Gt, k + PF);
      const int cc = k / (2 * NDB), db = (k / 2) % NDB;
      if (k & 1)
        dka[db] = E::mfma(__builtin_bit_cast(vec8, gf[k]), dsf[cc], dka[db]);
      else
        dva[db] = E::mfma(__builtin_bit_cast(vec8, gf[k]), pf[cc], dva[db]);
      if (k == 0) mask_block(1);
      if (k < NSG / 2)
#pragma unroll
        for (int e = k * 16 / HG; e < (k + 1) * 16 / HG; ++e) softmax_elem(1, e);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __syncthreads();  // zeroed tiles visible before any load lands
  if (t_first < n_qt) issue(qA, gA, lA, dA, t_first);
  auto step = [&](int tq, const u32x4* Qt, const u32x4* Gt, const f32x4* Lt, const f32x4* Dt, u32x4* Qn,
                  u32x4* Gn, f32x4* Ln, f32x4* Dn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);  // see the dQ kernel
    __syncthreads();
    if (tq + 1 < n_qt) issue(Qn, Gn, Ln, Dn, tq + 1);
    if (active && tq >= t_wave) compute(Qt, Gt, Lt, Dt, tq);
  };
  for (int tq = t_first; tq < n_qt; tq += 2) {
    step(tq, qA, gA, lA, dA, qB, gB, lB, dB);
    if (tq + 1 < n_qt) step(tq + 1, qB, gB, lB, dB, qA, gA, lA, dA);
  }

  if (key < NK) {
    bwd::store_rows<E>((uint16_t*)a.dk + headk + (size_t)key * D, dka, h, a.scale);
    bwd::store_rows<E>((uint16_t*)a.dv + headk + (size_t)key * D, dva, h, 1.0f);
  }
}

template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void fa_bwd_dkdv_kernel(BwdArgs a) {
  bwd_dkdv_body<E, D, CAUSAL>(a, blockIdx.x);
}

// ---------------------------------------------------------------------------
// dK and dV at D = 256: 16 keys per wave on the 16x16x32 MFMA, 4 waves (64
// keys) per workgroup.  With 32 keys per wave the body above would hold
// 256 registers of dK and dV accumulators and 128 of K and V per lane, more
// than a wave can have; with 16 keys it holds half of each (about 300 in all,
// one wave per SIMD).  Q and dO tiles of 64 queries and their -LSE log2(e)
// and Delta stream through double-buffered LDS as there.  Per tile and wave:
//   * S = Q K^T and dP = dO V^T: 4 blocks of 16 queries x D/32 steps of 32 d
//     (A = Q or dO rows from LDS, B = this lane's key from registers).  Row t
//     of block b is query 32 (b >> 1) + 8 (t >> 2) + 4 (b & 1) + (t & 3), so
//     lane l's results of blocks 2s and 2s + 1 are queries 32s + 8 (l / 16)
//     + 0..7 of its key l % 16: the B fragment (k block l / 16) of gradient
//     step s, with no data movement;
//   * P = exp2(c s - LSE log2 e) and dS = P (dP - Delta), rounded to the
//     16-bit type;
//   * dV^T += dO^T P and dK^T += Q^T dS: D/16 blocks of 16 d x 2 steps of 32
//     queries, dO^T and Q^T by transposed reads (two ds_read_b64_tr_b16 per
//     fragment, the forward's V^T pattern).
// Each tile is read both ways, so one chunk swizzle serves both patterns:
// the 64-row forward kernel's V swizzle, 2 (r0 | r1 << 1 | r3 << 2), whose
// transposed reads are known conflict-free.  Measured with the LDS conflict
// counter, the row reads are conflict-free with it too (512-byte rows all
// start on the same bank).  An odd swizzle that a bank model of 8-byte reads
// had passed, (r3 ^ r4) | r0 << 1 | r1 << 2 | r3 << 3, cost 256 conflict
// cycles per wave and tile in the transposed reads.  The swizzle reads only
// row bits 0, 1 and 3, which are constant over a lane's reads.
namespace bwd16 {
__device__ __forceinline__ int query_of(int b, int t) { return 32 * (b >> 1) + 8 * (t >> 2) + 4 * (b & 1) + (t & 3); }
__device__ __forceinline__ int swz(int row) { return 2 * ((row & 3) | (((row >> 3) & 1) << 2)); }
}  // namespace bwd16

template <typename E, int D, bool CAUSAL>
__device__ __forceinline__ void bwd_dkdv16_body(const BwdArgs& a, int blk) {
  typedef typename E::vec8 vec8;
  constexpr int NW = kBwdThreads / 64;    // waves, 16 keys each
  constexpr int KPB = 16 * NW;            // keys per workgroup
  constexpr int BQ = 64, RB = D * 2, CPR = D / 8, RPB = 64 / CPR, TILE16 = BQ * CPR;
  constexpr int NLD = TILE16 / 64 / NW;   // wave-wide loads per wave and tensor
  constexpr int NQB = BQ / 16;            // 16-query score blocks per tile
  constexpr int NKS = D / 32;             // 32-deep d steps of S and dP
  constexpr int NDB = D / 16;             // 16-wide d blocks of dK^T and dV^T
  constexpr int NST = BQ / 32;            // 32-query steps of the gradient products
  constexpr int NSS = 2 * NQB * NKS;      // score-phase slots (S, dP alternating)
  constexpr int NSG = 2 * NDB * NST;      // gradient-phase slots (dV, dK alternating)
  constexpr int HS = NSS / 2, HG = NSG / 2;
  constexpr int PF = 4;                   // operand reads in flight
  static_assert(D == 256 && NLD >= 1 && NQB == 4 && NST == 2, "tile layout");
  __shared__ u32x4 qA[TILE16], qB[TILE16], gA[TILE16], gB[TILE16];
  __shared__ f32x4 lA[BQ / 4], lB[BQ / 4], dA[BQ / 4], dB[BQ / 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, t16 = lane & 15;
  const int N = a.nq, NK = a.nk, OFF = CAUSAL ? NK - N : 0;
  const HeadItem wi = head_item(xcd_remap(blk, a.n_kblocks), a.n_kblocks / a.n_kblk, a.n_kblk, CAUSAL, false);
  const int bh = wi.bh;
  const int k0 = wi.idx * KPB;  // causal: the first key blocks see the most queries
  const size_t head = (size_t)bh * N * D, headk = (size_t)bh * NK * D;
  const uint16_t* Qg = (const uint16_t*)a.q + head;
  const uint16_t* Kg = (const uint16_t*)a.k + headk;
  const uint16_t* Vg = (const uint16_t*)a.v + headk;
  const uint16_t* dOg = (const uint16_t*)a.dout + head;
  const float* Lg = a.nlse2 + (size_t)bh * N;
  const float* Dg = a.delta + (size_t)bh * N;

  const int key = k0 + wave * 16 + t16;  // this lane's key
  const int wave_k0 = k0 + wave * 16;
  const int n_qt = (N + BQ - 1) / BQ;
  const int t_first = CAUSAL ? max(0, k0 - OFF) / BQ : 0;      // first query tile seeing key k0
  const int t_wave = CAUSAL ? max(0, wave_k0 - OFF) / BQ : 0;  // first one seeing this wave's first key
  const bool active = wave_k0 < NK;

  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < TILE16; i += kBwdThreads) qA[i] = qB[i] = gA[i] = gB[i] = z;
  }

  // this lane's key as B fragments of the score products: K[key][32 ks + 8 g
  // .. +7] (signs flipped for a negative scale) and V likewise; zero past NK
  vec8 kreg[NKS], vreg[NKS];
  {
    const u32x4 fl = {a.flip, a.flip, a.flip, a.flip};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (key < NK) {
        x = *(const u32x4*)(Kg + (size_t)key * D + 32 * ks + 8 * g) ^ fl;
        y = *(const u32x4*)(Vg + (size_t)key * D + 32 * ks + 8 * g);
      }
      kreg[ks] = __builtin_bit_cast(vec8, x);
      vreg[ks] = __builtin_bit_cast(vec8, y);
    }
  }

  // tile DMA: LDS position cl of a row holds global chunk cl ^ swz(row)
  uint32_t toff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPB + lane / CPR;
    toff[i] = row * RB + ((lane % CPR) ^ bwd16::swz(row)) * 16;
  }
  // query tile t: Q and dO rows, and the rows' -LSE log2(e) and Delta (the
  // first wave, 4 bytes a lane); rows past N are outside the descriptors and
  // arrive as zeros
  auto issue = [&](u32x4* qd, u32x4* gd, f32x4* ld, f32x4* dd, int tq) __attribute__((always_inline)) {
    const int r0 = tq * BQ;
    const uint32_t bytes = (uint32_t)(N - r0) * RB;
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Qg + (size_t)r0 * D), (short)0, (int)bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rg =
        __builtin_amdgcn_make_buffer_rsrc((void*)(dOg + (size_t)r0 * D), (short)0, (int)bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      lds_load16(rq, qd + (wave * NLD + i) * 64, toff[i]);
      lds_load16(rg, gd + (wave * NLD + i) * 64, toff[i]);
    }
    if (wave == 0) {
      const uint32_t fbytes = (uint32_t)(N - r0) * 4;
      const __amdgpu_buffer_rsrc_t rl =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Lg + r0), (short)0, (int)fbytes, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rd =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Dg + r0), (short)0, (int)fbytes, kRsrcWord3);
      lds_load4(rl, (float*)ld, (uint32_t)lane * 4);
      lds_load4(rd, (float*)dd, (uint32_t)lane * 4);
    }
  };

  f32x4 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) dka[db][i] = dva[db][i] = 0.0f;

  // row read of block b, step ks: row query_of(b, t16), chunk 4 ks + g; the
  // swizzle of query_of(b, t16) is that of query_of(0, t16), so the address is
  // one per-lane base XOR (ks << 6) plus the block's row offset
  const uint32_t raddr0 = [&] {
    const int row = bwd16::query_of(0, t16);
    return (uint32_t)(row * RB + ((g ^ bwd16::swz(row)) * 16));
  }();
  // transposed read of d block db, step st: in 16-lane group g, lane 4r + q
  // addresses row 32 st + 8 g + r (and + 4), columns 16 db + 4q .. +3; chunk
  // (2 db + q / 2) ^ swz(row) is the db = 0 one XOR 2 db
  const uint32_t taddr0 = [&] {
    const int r = t16 >> 2, q = t16 & 3;
    const int row = 8 * g + r;
    return (uint32_t)(row * RB + (((q >> 1) ^ bwd16::swz(row)) * 16) + (q & 1) * 8);
  }();
  // operand of score slot f: block f / (2 NKS), step (f / 2) % NKS of Q (even
  // f: S) or dO (odd f: dP); of gradient slot f: step f / (2 NDB), d block
  // (f / 2) % NDB of dO^T (even f: dV) or Q^T (odd f: dK)
  auto sfrag = [&](const u32x4* Qt, const u32x4* Gt, int f) __attribute__((always_inline)) {
    const int b = f / (2 * NKS), ks = (f / 2) % NKS;
    const char* t = (const char*)((f & 1) ? Gt : Qt);
    return *(const u32x4*)(t + ((raddr0 ^ (uint32_t)(ks << 6)) + (32 * (b >> 1) + 4 * (b & 1)) * RB));
  };
  auto gfrag = [&](const u32x4* Qt, const u32x4* Gt, int f) __attribute__((always_inline)) {
    const int st = f / (2 * NDB), db = (f / 2) % NDB;
    const char* p = (const char*)((f & 1) ? Qt : Gt) + (taddr0 ^ (uint32_t)(db << 5)) + 32 * st * RB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * RB));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  auto compute = [&](const u32x4* Qt, const u32x4* Gt, const f32x4* Lt, const f32x4* Dt, int tq)
      __attribute__((always_inline)) {
    // tiles with a query past N or (causal) before one of the wave's keys
    const bool masked = (CAUSAL && tq * BQ + OFF < wave_k0 + 15) || tq * BQ + BQ > N;
    const float c = a.c;
    f32x4 s[NQB], dp[NQB];
    vec8 pf[NST], dsf[NST];
    uint32_t pw[NQB][2], dw[NQB][2];
    // element i of block b is query tq BQ + 32 (b >> 1) + 8 g + 4 (b & 1) + i of
    // this lane's key; the rows' -LSE log2(e) and Delta, read before the tile's
    // first MFMA so that no wait for them drains the operand reads in flight
    f32x4 nl[NQB], dl[NQB];
#pragma unroll
    for (int b = 0; b < NQB; ++b) {
      const int q4 = 8 * (b >> 1) + 2 * g + (b & 1);
      nl[b] = Lt[q4];
      dl[b] = Dt[q4];
    }
    auto mask_block = [&](int b) __attribute__((always_inline)) {
      if (masked) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qg = tq * BQ + 32 * (b >> 1) + 8 * g + 4 * (b & 1) + i;
          if (qg >= N || (CAUSAL && qg + OFF < key)) s[b][i] = neg_inf();
        }
      }
    };
    // element e: block e / 4, entry e % 4; a block's four 16-bit P and dS
    // values once its last entry is done, and gradient step s's fragments
    // once blocks 2s and 2s + 1 are
    auto elem = [&](int e) __attribute__((always_inline)) {
      const int b = e >> 2, i = e & 3;
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][i], c, nl[b][i]));
      float ds = p * (dp[b][i] - dl[b][i]);
      float pp = p;
      pin(pp);
      pin(ds);
      s[b][i] = pp;
      dp[b][i] = ds;
      if (i == 3) {
        pw[b][0] = E::pack(s[b][0], s[b][1]);
        pw[b][1] = E::pack(s[b][2], s[b][3]);
        dw[b][0] = E::pack(dp[b][0], dp[b][1]);
        dw[b][1] = E::pack(dp[b][2], dp[b][3]);
        if (b & 1) {
          const int st = b >> 1;
          pf[st] = __builtin_bit_cast(vec8, u32x4{pw[b - 1][0], pw[b - 1][1], pw[b][0], pw[b][1]});
          dsf[st] = __builtin_bit_cast(vec8, u32x4{dw[b - 1][0], dw[b - 1][1], dw[b][0], dw[b][1]});
        }
      }
    };

    u32x4 sf[NSS], gf[NSG];
#pragma unroll
    for (int k = 0; k < PF; ++k) sf[k] = sfrag(Qt, Gt, k);
    // score phase; blocks 0 and 1's elements beside blocks 2 and 3's MFMAs
#pragma unroll
    for (int k = 0; k < NSS; ++k) {
      if (k + PF < NSS) sf[k + PF] = sfrag(Qt, Gt, k + PF);
      else gf[k + PF - NSS] = gfrag(Qt, Gt, k + PF - NSS);
      const int b = k / (2 * NKS), ks = (k / 2) % NKS;
      const f32x4 z = {};
      if (k & 1)
        dp[b] = E::mfma16(__builtin_bit_cast(vec8, sf[k]), vreg[ks], ks == 0 ? z : dp[b]);
      else
        s[b] = E::mfma16(__builtin_bit_cast(vec8, sf[k]), kreg[ks], ks == 0 ? z : s[b]);
      if (k == HS) {
        mask_block(0);
        mask_block(1);
      }
      if (k >= HS)
#pragma unroll
        for (int e = (k - HS) * 8 / HS; e < (k - HS + 1) * 8 / HS; ++e) elem(e);
      __builtin_amdgcn_sched_barrier(0);
    }
    // gradient phase; blocks 2 and 3's elements beside step 0's MFMAs
#pragma unroll
    for (int k = 0; k < NSG; ++k) {
      if (k + PF < NSG) gf[k + PF] = gfrag(Qt, Gt, k + PF);
      const int st = k / (2 * NDB), db = (k / 2) % NDB;
      if (k & 1)
        dka[db] = E::mfma16(__builtin_bit_cast(vec8, gf[k]), dsf[st], dka[db]);
      else
        dva[db] = E::mfma16(__builtin_bit_cast(vec8, gf[k]), pf[st], dva[db]);
      if (k == 0) {
        mask_block(2);
        mask_block(3);
      }
      if (k < HG)
#pragma unroll
        for (int e = k * 8 / HG; e < (k + 1) * 8 / HG; ++e) elem(8 + e);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __syncthreads();  // zeroed tiles visible before any load lands
  if (t_first < n_qt) issue(qA, gA, lA, dA, t_first);
  auto step = [&](int tq, const u32x4* Qt, const u32x4* Gt, const f32x4* Lt, const f32x4* Dt, u32x4* Qn,
                  u32x4* Gn, f32x4* Ln, f32x4* Dn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);  // see the dQ kernel
    __syncthreads();
    if (tq + 1 < n_qt) issue(Qn, Gn, Ln, Dn, tq + 1);
    if (active && tq >= t_wave) compute(Qt, Gt, Lt, Dt, tq);
  };
  for (int tq = t_first; tq < n_qt; tq += 2) {
    step(tq, qA, gA, lA, dA, qB, gB, lB, dB);
    if (tq + 1 < n_qt) step(tq + 1, qB, gB, lB, dB, qA, gA, lA, dA);
  }

  // dK^T and dV^T blocks: lane l holds d = 16 db + 4 (l / 16) + i of key l % 16
  if (key < NK) {
    uint16_t* dkr = (uint16_t*)a.dk + headk + (size_t)key * D;
    uint16_t* dvr = (uint16_t*)a.dv + headk + (size_t)key * D;
    const float mul = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 16 * db + 4 * g;
      *(u32x2*)(dkr + d) = u32x2{E::pack(dka[db][0] * mul, dka[db][1] * mul),
                                 E::pack(dka[db][2] * mul, dka[db][3] * mul)};
      *(u32x2*)(dvr + d) = u32x2{E::pack(dva[db][0], dva[db][1]), E::pack(dva[db][2], dva[db][3])};
    }
  }
}

template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void fa_bwd_dkdv16_kernel(BwdArgs a) {
  bwd_dkdv16_body<E, D, CAUSAL>(a, blockIdx.x);
}

// ---------------------------------------------------------------------------
// dk/dv and dq workgroups in one launch (the first n_kblocks workgroups are
// dk/dv ones, the next n_qblocks dq ones), after fa_bwd_delta_kernel: for grids
// that leave most compute units idle, where each kernel's time is the walk of
// its longest workgroup over the tiles and the two walks can run side by side
// instead of one after the other.  The two are independent given Delta and
// -LSE log2(e).  One workgroup per CU (the dk/dv body's registers, both
// bodies' LDS).
template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void fa_bwd_fused_kernel(BwdArgs a) {
  if ((int)blockIdx.x < a.n_kblocks) bwd_dkdv_body<E, D, CAUSAL>(a, blockIdx.x);
  else bwd_dq_body<E, D, CAUSAL, false>(a, (int)blockIdx.x - a.n_kblocks);
}

}  // namespace fa
