// Exact attention forward for CDNA4 (gfx950): one workgroup per (batch, head,
// 128-row query block), online softmax over 64-key (bf16) or 32-key (fp32)
// tiles held in LDS, both contractions on MFMA with fp32 accumulators.
//
// The method is the tiled loop of "Flash Attention" (wiki.ai-engineering.at),
// section "Tiling Algorithm" — an outer loop over query blocks, an inner loop
// over key/value blocks — with the running max / running sum / rescaled
// output of the section "Lösung: Online Softmax" on the same page, and the
// final division by the running sum that makes the result plain attention
// (johe.ru "Flash Attention: ускорить attention в 6 раз без потери точности",
// section "Почему это точно?").  Scores, scaling, masking, normalisation and
// the value aggregation all happen inside one kernel (ZimaSpace, "Wie
// reduziert Flash Attention den Speicherverkehr während der lokalen
// Inferenz?", section "Kernel-Fusion hält mehr Schritte der Attention-Kette in
// einem Ausführungspfad"); only Q, K, V are read and only O and LSE written.
//
// Layout of the work (bf16):
//   * 4 waves x 32 query rows.  Each wave computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16: keys on the MFMA rows, queries on the lanes.
//     A lane then holds 16 scores of ONE query per 32-key block, so the row
//     max is an in-register reduction plus one exchange with lane^32, and
//     the rescale factor of the output is a per-lane scalar.
//   * O^T = V^T P^T with the same MFMA: P^T is the B operand straight from the
//     score registers (converted to bf16); V^T comes from LDS.  To make the
//     eight keys a lane holds for one MFMA consecutive, the K rows of the
//     score MFMA are permuted (bits 2 and 3 of the row index swapped); V^T is
//     then read in natural key order.
//   * K tiles are stored row-major in LDS with the 16-byte chunk index XORed by
//     the row, V tiles transposed (V^T, [d][key]) with a chunk XOR by d, so the
//     MFMA operand reads of 32 different rows hit distinct banks.  Tiles are
//     double buffered: the global loads of tile j+1 are issued before tile j is
//     consumed and written to the other buffer afterwards (one barrier per tile).
//   * The running reference max moves only when a row's tile max exceeds it by
//     more than kTau (log2 units), so the output rescale is rare; the final
//     o / l and LSE = (m + log2 l) ln 2 are exact for any reference <= max.
//
// Scale: scores are multiplied by c = |scale| * log2(e) and exponentiated with
// exp2; a negative scale is applied by negating Q (exact) so c > 0 and the max
// of c*s is c times the max of s.  scale = 0 uses the smallest normal c, for
// which every finite c*s rounds to a value whose exp2 is exactly 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int n;          // sequence length N
  int n_qblk;     // query blocks per (b, h): ceil(N / 128)
  int n_blocks;   // workgroups in the grid: B * H * n_qblk
  float c;        // |scale| * log2(e), at least FLT_MIN
  uint32_t qflip; // XOR mask applied to Q's bits: flips every sign when scale < 0
};

constexpr int kThreads = 256;
constexpr int kBM = 128;        // query rows per workgroup
constexpr float kTau = 8.0f;    // log2 headroom before the running reference max moves
constexpr float kLn2 = 0.69314718055994530942f;

// Hardware dispatches consecutive workgroups round-robin over the 8 XCDs, each
// with its own L2.  Remap so that logical tiles t, t+1, ... (the query blocks
// of one head, which all stream that head's K and V) land on one XCD.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int X = 8;
  const int q = n / X, r = n % X;
  const int x = bid % X, j = bid / X;
  const int base = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return base + j;
}

// Row i of a 32-row MFMA block holds key swap23(i): swaps bits 2 and 3.
__device__ __forceinline__ int swap23(int i) {
  return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Lane i and lane i^32 hold the two halves of one query's keys.  v_permlane32_swap
// exchanges lanes 32-63 of its first operand with lanes 0-31 of its second;
// applied to two copies of x, one copy ends up holding x of lanes 0-31 in both
// halves and the other x of lanes 32-63, so their max / sum is the pair's.
// Written as inline asm: this compiler folds the builtin's two results into one
// when both operands start from the same value.  The s_nop gives the two wait
// states a VALU write needs before v_permlane32_swap reads it.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_halves(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float pair_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_halves(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// ---------------------------------------------------------------------------
// Online-softmax update for one tile.  s[] holds the raw scores of this lane's
// query (masked ones -inf); afterwards s[] holds p = exp2(c*s - m_ref).  The
// caller adds this tile's p to the running sums l and l2 (after any rescale of
// them here).
template <int NS>
__device__ __forceinline__ void online_softmax(float (&s)[NS], float c, float& m_ref, float& l,
                                               float& l2, float& alpha_out, bool& rescaled) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < NS; ++i) mx = fmaxf(mx, s[i]);
  mx = pair_max(mx);  // the other half-wave holds the other keys of this query
  const float mt = mx * c;         // -inf when every key of the tile is masked for this row
  const bool need = mt > m_ref + kTau;
  rescaled = false;
  alpha_out = 1.0f;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    const float m_new = fmaxf(m_ref, mt);
    const float alpha = m_new == neg_inf() ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    l *= alpha;
    l2 *= alpha;
    alpha_out = alpha;
    rescaled = true;
  }
  const float mu = m_ref == neg_inf() ? 0.0f : m_ref;
#pragma unroll
  for (int i = 0; i < NS; ++i) s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -mu));
}

// ---------------------------------------------------------------------------
// bf16 kernel
//
// LDS: four static 64-key tiles (K and V, double buffered), row-major.  The
// 16-byte chunk index of each row is XORed with a function of the row so that
// the MFMA operand reads hit distinct banks (checked for 32- and 64-bank LDS):
//   K (read 16 B per lane, 32 rows x 1 chunk):        kswz(row)
//   V (read transposed, 8 B per lane, 4 rows x 32 B):  vswz(key & 3)
// Tiles arrive by buffer loads straight into LDS (no registers, no VALU): each
// lane's byte offset inside a tile is fixed, the tile start lives in the buffer
// descriptor, and rows past N fall outside the descriptor's range.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return swap23(row & 15);
  else return ((row ^ (row >> 2)) & 1) | (row & 2) | ((row >> 1) & 4);
}
template <int D>
__device__ __forceinline__ int vswz(int key) {
  const int r = key & 3;
  if constexpr (D == 128) return 4 * r | (r & 2);
  else return 2 * r;
}

// Raw buffer descriptor word 3 for gfx9-family: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

// 16 bytes per lane from buffer r at byte offset voff into LDS: the wave's 64
// lanes fill the 1 KB at lds in lane order.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, u32x4* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_bf16_kernel(FwdArgs a) {
  constexpr int BN = 64;                // keys per tile
  constexpr int RB = D * 2;             // bytes per row
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPB = 64 / CPR;         // rows per 1 KB block (one wave-wide load)
  constexpr int TILE16 = BN * CPR;      // 16-byte chunks per tile
  constexpr int NLD = TILE16 / 64 / 4;  // 1 KB loads per wave per tile
  constexpr int NKB = BN / 32;          // 32-key MFMA blocks per tile
  constexpr int NDB = D / 32;           // 32-wide d blocks of O
  static_assert(NLD >= 1, "tile loads");

  __shared__ u32x4 kA[TILE16], kB[TILE16], vA[TILE16], vB[TILE16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int N = a.n;

  const int t = xcd_remap(blockIdx.x, a.n_blocks);
  const int bh = t / a.n_qblk;
  int qb = t - bh * a.n_qblk;
  if (CAUSAL) qb = a.n_qblk - 1 - qb;  // longest query blocks first
  const int q0 = qb * kBM;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + head;
  const uint16_t* __restrict__ Kg = (const uint16_t*)a.k + head;
  const uint16_t* __restrict__ Vg = (const uint16_t*)a.v + head;
  uint16_t* __restrict__ Og = (uint16_t*)a.o + head;

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int qrow = q0 + wave * 32 + c32;  // this lane's query row
  const int wave_q0 = q0 + wave * 32;

  // zero the tiles once: rows past N are never loaded, so they must hold finite values
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = tid; i < TILE16; i += kThreads) {
      kA[i] = z; kB[i] = z; vA[i] = z; vB[i] = z;
    }
  }

  // Q fragments: B operand of the score MFMA, Q[qrow][16kk + 8h .. +7]
  bf16x8 qf[D / 16];
  {
    const u32x4 flip = {a.qflip, a.qflip, a.qflip, a.qflip};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < N) x = *(const u32x4*)(Qg + (size_t)qrow * D + 16 * kk + 8 * h) ^ flip;
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // per-lane byte offsets of the tile loads (fixed for every tile)
  uint32_t koff[NLD], voff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPB + lane / CPR;
    const int cl = lane % CPR;
    koff[i] = row * RB + ((cl ^ kswz<D>(row)) * 16);
    voff[i] = row * RB + ((cl ^ vswz<D>(row)) * 16);
  }
  // per-lane LDS read addresses (bytes): K rows 32kb + swap23(c32), chunk 2kk + h
  uint32_t kaddr[D / 16];
  {
    const int row = swap23(c32);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kaddr[kk] = row * RB + (((2 * kk + h) ^ kswz<D>(row)) * 16);
  }
  // V^T operand by transposed reads: within each 16-lane group, lane 4r+q
  // addresses row r (key 16c + 8h + 4s + r), columns 32db + 16gg + 4q .. +3
  uint32_t vaddr[NDB];
  {
    const int g = lane >> 4, i16 = lane & 15;
    const int hh = g >> 1, gg = g & 1, r = i16 >> 2, q = i16 & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int chunk = 4 * db + 2 * gg + (q >> 1);
      vaddr[db] = (8 * hh + r) * RB + ((chunk ^ vswz<D>(r)) * 16) + (q & 1) * 8;
    }
  }

  auto issue = [&](u32x4* kd, u32x4* vd, int kv0) {
    const uint32_t bytes = (uint32_t)(N - kv0) * RB;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + (size_t)kv0 * D), (short)0, (int)bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + (size_t)kv0 * D), (short)0, (int)bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int blk = wave * NLD + i;
      lds_load16(kr, kd + blk * 64, koff[i]);
      lds_load16(vr, vd + blk * 64, voff[i]);
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  // l sums the bf16-rounded p the MFMA consumes, so the weights applied to V sum
  // to exactly l; lx sums the fp32 p for the log-sum-exp.
  float m_ref = neg_inf(), l = 0.0f, lx = 0.0f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto compute = [&](const u32x4* Kt, const u32x4* Vt, int kv0) {
    if (CAUSAL && kv0 > wave_q0 + 31) return;  // no key of this tile is visible to this wave
    const char* kt = (const char*)Kt;
    const char* vt = (const char*)Vt;

    // S^T = K Q^T for 64 keys x this wave's 32 queries
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 kx = *(const u32x4*)(kt + kaddr[kk] + kb * 32 * RB);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx), qf[kk],
                                                           sacc[kb], 0, 0, 0);
      }
    }

    float s[NKB * 16];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb * 16 + i] = sacc[kb][i];

    // mask: keys past N, and keys after the query under the causal mask.
    // Element (kb, i) of this lane holds key kv0 + 32kb + 8h + kofs(i).
    const bool tail = kv0 + BN > N;
    const bool diag = CAUSAL && (kv0 + BN - 1 > wave_q0);
    if (tail || diag) {
      const int lim = (CAUSAL ? min(N - 1, qrow) : N - 1) - kv0 - 8 * h;  // visible iff offset <= lim
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = 32 * kb + 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
          if (kofs > lim) s[kb * 16 + i] = neg_inf();
        }
    }

    float alpha;
    bool rescaled;
    online_softmax(s, a.c, m_ref, l, lx, alpha, rescaled);
    if (rescaled) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    {
      float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < NKB * 16; ++i) ps[i & 3] += s[i];
      lx += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }

    // P^T fragments: chunk c covers keys 16c .. 16c+15; this lane holds keys 16c + 8h + 0..7.
    bf16x8 pf[BN / 16];
    float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
      const int base = (c >> 1) * 16 + (c & 1) * 8;
      // each packed word is a scalar before it is bit-cast: this compiler
      // miscompiles __builtin_bit_cast applied to an element of a vector variable
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = pack_bf16(s[base + 2 * e], s[base + 2 * e + 1]);
        lsum[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, lsum[e], false);
      }
      const u32x4 x = {w[0], w[1], w[2], w[3]};
      pf[c] = __builtin_bit_cast(bf16x8, x);
    }
    l += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);

    // O^T += V^T P^T; V^T fragments by two transposed 8-byte reads
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
        const char* p = vt + vaddr[db] + 16 * c * RB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * RB));
        const i16x8 vx = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vx), pf[c], o[db], 0, 0, 0);
      }
    }
  };

  __syncthreads();  // zeroed tiles visible before any load lands
  if (n_tiles > 0) issue(kA, vA, 0);
  __syncthreads();

  for (int j = 0; j < n_tiles; j += 2) {
    if (j + 1 < n_tiles) issue(kB, vB, (j + 1) * BN);
    compute(kA, vA, j * BN);
    __syncthreads();
    if (j + 1 < n_tiles) {
      if (j + 2 < n_tiles) issue(kA, vA, (j + 2) * BN);
      compute(kB, vB, (j + 1) * BN);
      __syncthreads();
    }
  }

  // epilogue: O = o / l, LSE = (m + log2 lx) ln 2
  const float l_tot = pair_sum(l);
  const float lx_tot = pair_sum(lx);
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * h;
        const u32x2 w = {pack_bf16(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                         pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        *(u32x2*)(Og + (size_t)qrow * D + d) = w;
      }
    if (h == 0) a.lse[(size_t)bh * N + qrow] = (m_ref + __log2f(lx_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// float32 kernel: v_mfma_f32_32x32x2_f32, P kept in fp32.  With two keys per
// MFMA the value operand needs no transpose: V stays row-major in LDS.
// D = 128 needs more than 256 registers per lane (64 Q values + 64 accumulators
// + staging), so that variant runs one wave per SIMD.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void fa_fwd_f32_kernel(FwdArgs a) {
  constexpr int BN = 32;           // keys per tile
  constexpr int LD = D + 4;        // padded LDS row stride (floats), keeps 16-byte alignment
  constexpr int TILE = BN * LD;    // floats per K or V tile
  constexpr int BUF = 2 * TILE;
  constexpr int CPR = D / 4;       // 16-byte chunks per row
  constexpr int NLD = BN * CPR / kThreads;
  constexpr int NDB = D / 32;
  static_assert((BN * CPR) % kThreads == 0, "tile staging");

  __shared__ float smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int N = a.n;

  const int t = xcd_remap(blockIdx.x, a.n_blocks);
  const int bh = t / a.n_qblk;
  int qb = t - bh * a.n_qblk;
  if (CAUSAL) qb = a.n_qblk - 1 - qb;
  const int q0 = qb * kBM;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float* __restrict__ Qg = (const float*)a.q + head;
  const float* __restrict__ Kg = (const float*)a.k + head;
  const float* __restrict__ Vg = (const float*)a.v + head;
  float* __restrict__ Og = (float*)a.o + head;

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int qrow = q0 + wave * 32 + c32;
  const int wave_q0 = q0 + wave * 32;

  float qf[D / 2];  // Q[qrow][2kk + h]
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) {
    const uint32_t x = qrow < N ? __builtin_bit_cast(uint32_t, Qg[(size_t)qrow * D + 2 * kk + h]) : 0u;
    qf[kk] = __builtin_bit_cast(float, x ^ a.qflip);
  }

  f32x4 kst[NLD], vst[NLD];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
      const int id = tid + kThreads * r;
      const int row = id / CPR, cc = id % CPR;
      const int key = min(kv0 + row, N - 1);  // rows past N: masked scores, p = 0
      kst[r] = *(const f32x4*)(Kg + (size_t)key * D + cc * 4);
      vst[r] = *(const f32x4*)(Vg + (size_t)key * D + cc * 4);
    }
  };
  auto store_tile = [&](int buf) {
    float* Ks = smem + buf * BUF;
    float* Vs = Ks + TILE;
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
      const int id = tid + kThreads * r;
      const int row = id / CPR, cc = id % CPR;
      *(f32x4*)(Ks + row * LD + cc * 4) = kst[r];
      *(f32x4*)(Vs + row * LD + cc * 4) = vst[r];
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m_ref = neg_inf(), l = 0.0f;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = j * BN;
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(kv0 + BN);
    const float* Ks = smem + buf * BUF;
    const float* Vs = Ks + TILE;

    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[c32 * LD + 2 * kk + h], qf[kk], sacc, 0, 0, 0);

    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = sacc[i];
    const bool tail = kv0 + BN > N;
    const bool diag = CAUSAL && (kv0 + BN - 1 > wave_q0);
    if (tail || diag) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= N || (CAUSAL && key > qrow)) s[i] = neg_inf();
      }
    }

    float alpha;
    bool rescaled;
    float l_unused = 0.0f;  // P stays fp32 here: one sum serves both O and LSE
    online_softmax(s, a.c, m_ref, l, l_unused, alpha, rescaled);
    if (rescaled) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    {
      float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i & 3] += s[i];
      l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }

    // O^T += V^T P^T, two keys per MFMA: slot h holds key 8(i>>2) + 4h + (i&3)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * h + (i & 3);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * LD + 32 * db + c32], s[i], o[db], 0, 0, 0);
      }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(l);
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * h;
        const f32x4 w = {o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                         o[db][4 * g + 3] * inv};
        *(f32x4*)(Og + (size_t)qrow * D + d) = w;
      }
    if (h == 0) a.lse[(size_t)bh * N + qrow] = (m_ref + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace fa
