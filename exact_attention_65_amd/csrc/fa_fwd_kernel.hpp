// Exact attention forward for CDNA4 (gfx950): one workgroup per (batch, head,
// query block of 128 rows), online softmax over 64-key (16-bit inputs) or
// 32-key (fp32) tiles held in LDS, both contractions on MFMA with fp32
// accumulators.
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
// Layout of the work (16-bit inputs):
//   * 4 waves x 32 query rows.  Each wave computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16 (or _f16): keys on the MFMA rows, queries on
//     the lanes.  A lane then holds 16 scores of ONE query per 32-key block, so
//     the row max is an in-register reduction plus one exchange with lane^32,
//     and the rescale factor of the output is a per-lane scalar.
//   * O^T = V^T P^T with the same MFMA: P^T is the B operand straight from the
//     score registers (rounded to 16 bits); V^T is read from the row-major V
//     tile with the transposing LDS read.  To make the eight keys a lane holds
//     for one MFMA consecutive, the K rows of the score MFMA are permuted (bits
//     2 and 3 of the row index swapped); V^T is then read in natural key order.
//   * K and V tiles are stored row-major in LDS with the 16-byte chunk index
//     XORed by a function of the row, so the MFMA operand reads of 32 different
//     rows hit distinct banks.  Tiles are double buffered and loaded (global to
//     LDS, no registers) while the previous tile is consumed.
//   * The running reference max moves only when a row's tile max exceeds it by
//     more than a headroom (kTau log2 units: 8 for the fp32 kernel and fp16 P,
//     32 for bf16 P), so the output rescale is rare; the final
//     o / l and LSE = (m + log2 l) ln 2 are exact for any reference <= max.
//
// Scale: scores are multiplied by c = |scale| * log2(e) and exponentiated with
// exp2; a negative scale is applied by negating Q (exact) so c > 0 and the max
// of c*s is c times the max of s.  scale = 0 uses the smallest normal c, for
// which every finite c*s rounds to a value whose exp2 is exactly 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int nq;         // query rows per (b, h)
  int nk;         // key / value rows per (b, h); nq <= nk under the causal mask
  int n_bh;       // B * H
  int n_qblk;     // query blocks per (b, h): ceil(nq / rows per workgroup)
  int n_split;    // workgroups that share the keys of one query block (16-bit types only)
  int n_blocks;   // workgroups in the grid: n_bh * n_qblk * n_split
  float c;        // |scale| * log2(e), at least FLT_MIN
  uint32_t qflip; // XOR mask applied to Q's bits: flips every sign when scale < 0
  float* o_part;   // with n_split > 1: [n_split][n_bh][nq][D] fp32 outputs of each key range
  float* lse_part; //                   [n_split][n_bh][nq] their log-sum-exps (-inf: no key)
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

// Work item t (after xcd_remap) of a grid of n_bh heads x per_bh items: its
// head and its index within the head.  Plain order: a head's items one after
// another.  Interleaved order (for the causal mask, where item 0 of a head is
// its longest): when n_bh is a multiple of 8, each XCD holds n_bh/8 whole heads
// and takes them in groups of up to 4, the items of a group round-robin over
// its heads.  Each XCD then starts all its long items first; head by head, the
// long items of the last heads on an XCD would start after the short items of
// the others and end late.  Groups of at most 4 heads keep the K/V bytes in
// use on an XCD at a few heads' worth.
//
// For kernels that run two workgroups per CU (two_per_cu): when an XCD has
// more items than CUs but at most two per CU (32 < items <= 64 on MI355X's 32
// CUs per XCD), every item starts at once, and the dispatcher places item
// positions c and c + 32 on CU c.  An item that shares its CU runs slower than
// one alone, so the longest items get CUs of their own and the others share
// CUs longest with shortest.
constexpr int kCusPerXcd = 32;
__device__ __forceinline__ int pair_rank(int p, int n) {
  if (n <= kCusPerXcd || n > 2 * kCusPerXcd) return p;
  const int shared = n - kCusPerXcd;               // CUs 0 .. shared-1 hold two items
  if (p >= kCusPerXcd) return n - 1 - (p - kCusPerXcd);  // second item of CU p-32: the shortest
  return p >= shared ? p - shared : (kCusPerXcd - shared) + p;
}

struct HeadItem {
  int bh, idx;
};
__device__ __forceinline__ HeadItem head_item(int t, int n_bh, int per_bh, bool interleave, bool two_per_cu) {
  if (interleave && (n_bh & 7) == 0) {
    const int hp = n_bh >> 3;                                       // heads per XCD
    const int g = hp <= 4 ? hp : (hp & 3) == 0 ? 4 : (hp & 1) == 0 ? 2 : 1;  // heads per group
    const int per_x = hp * per_bh;  // = n_blocks / 8: xcd_remap gives XCD x the items [x per_x, (x+1) per_x)
    const int x = t / per_x, j = two_per_cu ? pair_rank(t - x * per_x, per_x) : t - x * per_x;
    const int grp = j / (g * per_bh), jj = j - grp * (g * per_bh);
    return {x * hp + grp * g + jj % g, jj / g};
  }
  const int bh = t / per_bh;
  return {bh, t - bh * per_bh};
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// The 16-bit element types of the MFMA kernels: the 8-element operand vector,
// two fp32 values rounded (to nearest even) into one word, the 32x32x16 MFMA
// with fp32 accumulation, the 16x16x32 MFMA and a word holding two ones (for
// row sums on the matrix core), the sum of the two elements of a word added to
// an fp32 accumulator (a dot product with (1, 1)), and the dot product of two
// words added to an fp32 accumulator.
struct BF16 {
  typedef bf16x8 vec8;
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) { return pack_bf16(lo, hi); }
  __device__ static __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr uint32_t kOnes2 = 0x3F803F80u;  // two bf16 ones
  // log2 headroom of the lazy reference: weights up to 2^kTau.  bf16 has fp32's
  // exponent range, so a wide headroom costs no precision and leaves the
  // rescale to rows whose max climbs by more than 2^32 (it fired on a few
  // percent of the tiles of 16x scores at 8); o stays finite while
  // N 2^32 max|v| does.
  static constexpr float kTau = 32.0f;
  __device__ static __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
  }
  __device__ static __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc, false);
  }
};
struct F16 {
  typedef f16x8 vec8;
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) { return pack_f16(lo, hi); }
  __device__ static __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static constexpr uint32_t kOnes2 = 0x3C003C00u;  // two fp16 ones
  static constexpr float kTau = 8.0f;  // fp16 weights stay far below fp16's maximum, 65504
  __device__ static __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) {
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, acc, false);
  }
  __device__ static __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), acc, false);
  }
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Maximum that propagates NaN (IEEE maximum).  It lowers to v_maximum3_f32,
// two new operands per instruction; fmaxf (maxNum) makes the compiler first
// quieten every operand that is not known to be canonical, such as MFMA
// results, with an extra v_max each.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Pins a value in place: the empty asm "reads and rewrites" it, so its
// computation cannot be moved past this point (the optimiser otherwise sinks
// arithmetic toward its first use, out of the slot it was placed in).
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

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
  return vmax(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
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
// the MFMA operand reads hit distinct banks:
//   K (read 16 B per lane, 32 rows x 1 chunk):        kswz(row)
//   V (read transposed, 8 B per lane, 4 rows x 32 B):  vswz(key & 3)
// Tiles arrive by buffer loads straight into LDS (no registers, no VALU): each
// lane's byte offset inside a tile is fixed, the tile start lives in the buffer
// descriptor, and rows past N fall outside the descriptor's range.  The V^T
// operand of the value MFMA is read with the transposing LDS read
// (ds_read_b64_tr_b16), which on this pattern runs near the plain read's rate.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D >= 128) return swap23(row & 15);
  else return ((row ^ (row >> 2)) & 1) | (row & 2) | ((row >> 1) & 4);
}
template <int D>
__device__ __forceinline__ int vswz(int key) {
  const int r = key & 3;
  if constexpr (D >= 128) return 4 * r | (r & 2);
  else return 2 * r;
}

// Raw buffer descriptor word 3 for gfx9-family: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

// 16 bytes per lane from buffer r at byte offset voff into LDS: the wave's 64
// lanes fill the 1 KB at lds in lane order.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, u32x4* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// 4 bytes per lane likewise: the wave's 64 lanes fill 256 bytes at lds.
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, float* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

// Work split: 4 waves x 32 query rows (128 rows per workgroup), two
// workgroups per CU (one wave of each per SIMD).  Each wave runs its own
// software pipeline over the key tiles so that its matrix-core work and its
// softmax arithmetic overlap inside the wave:
//
//   iteration j:  barrier ; DMA V_{j+1} and K_{j+2}
//                 phase A: S_{j+1} = K_{j+1} Q^T  (MFMA)   ||  p = exp2(c s_j - m), P_j, sums
//                 phase B: O^T += V_j^T P_j^T     (MFMA)   ||  mask / row max / reference of S_{j+1}
//
// The MFMAs of a phase do not depend on the arithmetic beside them, so the
// two are issued in alternation: one MFMA runs 32 cycles on the matrix core
// while the same wave issues the VALU work of its slot.  The output rescale
// decided in phase B of iteration j is applied before the value MFMAs of
// iteration j+1, after the ones it must not touch.  One barrier per tile: a
// buffer is refilled only after every wave has finished the iteration that
// read it, and everything issued at the top of iteration j is waited for by the
// barrier of iteration j+1, a full iteration later.
constexpr int kBF16Threads = 256;
constexpr int kBF16Rows = 128;

// SPLIT: the keys of each query block are divided into n_split contiguous
// ranges of whole tiles, one workgroup each; a workgroup writes its rows'
// normalised fp32 output and log-sum-exp over its range to o_part / lse_part,
// and fa_combine_kernel merges them.  Without SPLIT the one workgroup of a query
// block covers all its keys and writes O and LSE.
//
// The body serves both 16-bit input types (E = BF16 or F16): the kernels
// fa_fwd_bf16_kernel and fa_fwd_f16_kernel below instantiate it.
template <typename E, int D, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void fwd16_body(const FwdArgs& a) {
  typedef typename E::vec8 vec8;
  constexpr int BN = 64;                // keys per tile
  // D = 96 rows are stored in LDS as 128-wide rows whose last 4 chunks stay
  // zero: every LDS address is the D = 128 one (same swizzles); global rows
  // keep their real width
  constexpr int DP = D == 96 ? 128 : D; // head dimension of the LDS layout
  constexpr int GRB = D * 2;            // bytes per global K / V row
  constexpr int RB = DP * 2;            // bytes per LDS K / V row
  constexpr int CPR = DP / 8;           // 16-byte chunks per LDS row
  constexpr int RPB = 64 / CPR;         // rows per 1 KB block (one wave-wide load)
  constexpr int TILE16 = BN * CPR;      // 16-byte chunks per tile
  constexpr int NLD = TILE16 / 64 / 4;  // 1 KB K loads per wave per tile
  constexpr int NKB = BN / 32;          // 32-key MFMA blocks per tile
  // the MFMAs cover the D real columns only (at D = 96 the padded LDS columns
  // are never read)
  constexpr int NDB = D / 32;           // 32-wide d blocks of O
  constexpr int NKK = D / 16;           // 16-deep steps of the score contraction
  constexpr int NCC = BN / 16;          // 16-key steps of the value contraction
  constexpr int NSA = NKK * NKB;        // score MFMAs per tile (phase A slots)
  constexpr int NSB = NDB * NCC;        // value MFMAs per tile (phase B slots)
  constexpr int PFA = 3;                // score-fragment reads in flight in phase A
  constexpr int PFB = 4;                // value-fragment reads in flight in phase B
  static_assert(NLD >= 1, "tile loads");
  static_assert(NSA == 2 * D / 16 && NSB == D / 8, "slot counts");
  // fragment arrays: one entry per slot, or at D = 256 (32 slots a phase) a
  // ring of PF + 1 entries, which the compiler keeps in registers where it
  // puts a 32-entry array in scratch memory
  constexpr int RKA = D == 256 ? PFA + 1 : NSA;
  constexpr int RVB = D == 256 ? PFB + 1 : NSB;

  // four separate arrays, picked at compile time by the two-step unrolled loop:
  // the compiler then sees that a tile load into one buffer cannot alias reads
  // of another and does not wait for the load before those reads
  __shared__ u32x4 kA[TILE16], kB[TILE16], vA[TILE16], vB[TILE16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c32 = lane & 31;
  const int NQ = a.nq, NK = a.nk;
  // query i is position i + OFF of the sequence: key j is visible iff j <= i + OFF
  const int OFF = CAUSAL ? NK - NQ : 0;

  // workgroup -> (b, h), query block, key range; under the causal mask the
  // longest query blocks first
  const HeadItem wi = head_item(xcd_remap(blockIdx.x, a.n_blocks), a.n_bh, a.n_qblk * a.n_split, CAUSAL, D != 256);
  const int bh = wi.bh;
  int qb = SPLIT ? wi.idx / a.n_split : wi.idx;
  const int split = SPLIT ? wi.idx - qb * a.n_split : 0;
  if (CAUSAL) qb = a.n_qblk - 1 - qb;
  const int q0 = qb * kBF16Rows;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + (size_t)bh * NQ * D;
  const uint16_t* __restrict__ Kg = (const uint16_t*)a.k + (size_t)bh * NK * D;
  const uint16_t* __restrict__ Vg = (const uint16_t*)a.v + (size_t)bh * NK * D;

  // key tiles of the query block: 0 .. n_tiles-1; this workgroup's: t_lo .. t_hi-1
  const int kv_end = CAUSAL ? min(NK, q0 + kBF16Rows + OFF) : NK;
  const int n_tiles = (kv_end + BN - 1) / BN;
  const int t_lo = SPLIT ? (int)((long long)n_tiles * split / a.n_split) : 0;
  const int t_hi = SPLIT ? (int)((long long)n_tiles * (split + 1) / a.n_split) : n_tiles;
  const int n_loc = t_hi - t_lo;         // tiles this workgroup loads
  const int kv_lim = min(NK, t_hi * BN);  // keys past this one are outside the range
  const int qrow = q0 + wave * 32 + c32;  // this lane's query row
  const int wave_q0 = q0 + wave * 32;
  // tiles t_lo .. t_lo+n_vis-1 hold keys visible to some row of this wave (none
  // when all its rows are past the last query)
  const int wave_end = CAUSAL ? min(t_hi, (wave_q0 + 31 + OFF) / BN + 1) : t_hi;
  const int n_vis = wave_q0 < NQ ? max(0, wave_end - t_lo) : 0;

  // Tile rows past the last key are never loaded.  Their K rows give scores
  // that the mask overwrites with -inf, whatever the LDS held; their V rows
  // meet weight 0 in the value product, and 0 times a non-finite value is NaN,
  // so a V buffer must hold finite values before a partial tile lands in it.
  // One that held a full tile before does; a fresh one is zeroed, when one of
  // the workgroup's first two tiles is partial.  At D = 96 the columns past D
  // are never loaded either and meet zeros of Q and P: then every tile is
  // zeroed.
  const bool zero_tiles = D != DP || (NK % BN != 0 && NK < (t_lo + 2) * BN);
  if (zero_tiles) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = tid; i < TILE16; i += kBF16Threads) {
      if constexpr (D != DP) {
        kA[i] = z;
        kB[i] = z;
      }
      vA[i] = z;
      vB[i] = z;
    }
  }

  // Q fragments: B operand of the score MFMA, Q[qrow][16kk + 8h .. +7] (signs
  // flipped for a negative scale)
  vec8 qf[NKK];
  {
    const u32x4 flip = {a.qflip, a.qflip, a.qflip, a.qflip};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      const bool col_ok = D == DP || 16 * kk + 8 * h < D;  // columns past D stay zero
      if (qrow < NQ && col_ok) x = *(const u32x4*)(Qg + (size_t)qrow * D + 16 * kk + 8 * h) ^ flip;
      qf[kk] = __builtin_bit_cast(vec8, x);
    }
  }

  // tile DMA: per-lane byte offsets (fixed for every tile)
  // (LDS position cl of a row holds global chunk cl ^ swizzle(row); at D = 96
  // the lanes whose chunk is past the row load nothing)
  uint32_t koff[NLD], voff[NLD];
  bool kon[NLD], von[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = (wave * NLD + i) * RPB + lane / CPR;
    const int cl = lane % CPR;
    const int kg = cl ^ kswz<DP>(row), vg = cl ^ vswz<DP>(row);
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

  // per-lane LDS read addresses (bytes).  K operand of score slot (kk, kb): row
  // 32kb + swap23(c32), chunk 2kk + h -> (kaddr0 ^ (kk << 5)) + kb * 32 * RB.
  // V^T operand of value slot (db, cc) by two transposed reads: within each
  // 16-lane group, lane 4r+q addresses row r (key 16cc + 8h + 4s + r),
  // columns 32db + 16gg + 4q .. +3; d block db's address is the db = 0 address
  // XOR (db << 6), key step cc adds 16 rows.
  const uint32_t kaddr0 = [&] {
    const int row = swap23(c32);
    return (uint32_t)(row * RB + ((h ^ kswz<DP>(row)) * 16));
  }();
  const uint32_t vaddr0 = [&] {
    const int g = lane >> 4, i16 = lane & 15;
    const int hh = g >> 1, gg = g & 1, r = i16 >> 2, q = i16 & 3;
    const int chunk = 2 * gg + (q >> 1);
    return (uint32_t)((8 * hh + r) * RB + ((chunk ^ vswz<DP>(r)) * 16) + (q & 1) * 8);
  }();
  auto kfrag = [&](const u32x4* Kt, int s) __attribute__((always_inline)) {
    const int kk = s / NKB, kb = s % NKB;
    return *(const u32x4*)((const char*)Kt + (kaddr0 ^ (kk << 5)) + kb * 32 * RB);
  };
  auto vfrag = [&](const u32x4* Vt, int s) __attribute__((always_inline)) {
    const int db = s % NDB, cc = s / NDB;
    const char* p = (const char*)Vt + (vaddr0 ^ (db << 6)) + 16 * cc * RB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * RB));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // state: o (unnormalised output), m_ref (running reference max, log2 units),
  // l or lsacc (sum of the bf16-rounded p: normalises O), lx (sum of fp32 p:
  // LSE), pf (bf16 P^T of the tile whose values are next), a pending output
  // rescale
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  f32x16 sA[NKB], sB[NKB];
  vec8 pf[NCC];
  float m_ref = neg_inf(), l = 0.0f, lx = 0.0f, mu = 0.0f;
  // The sum of the rounded P is taken on the matrix core for D <= 128: one
  // 16x16x32 MFMA per value step multiplies a constant 0/1 operand with that
  // step's P^T fragment (the B operand of the value MFMAs, read again as the B
  // operand of the 16x16x32 form: lane L holds query L % 32, keys 8 (L / 32)
  // .. +7 of the step, and lands in column L % 16, k block L / 16).  Row 0 of
  // the constant picks k blocks 0 and 2 (lanes 0 and 32: both key halves of
  // query n), row 1 blocks 1 and 3 (lanes 17 and 49: query n + 16), so lane
  // n < 16 accumulates query n in lsacc[0] and query n + 16 in lsacc[1].  This
  // replaces 8 dot products per step on the vector unit.  D = 256 has no
  // registers left for it and keeps the dot products (into l).
  constexpr bool kMfmaSum = D <= 128;
  f32x4 lsacc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t one2 = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? E::kOnes2 : 0u;
  const vec8 ones_op = __builtin_bit_cast(vec8, u32x4{one2, one2, one2, one2});
  // raw tile maxima above thr move the reference: c thr = m_ref + E::kTau (-inf
  // until a key is seen; +inf when that overflows, at the smallest c, where
  // every c s is too small to move it)
  float thr = neg_inf();
  bool pend = false;
  float pend_alpha = 1.0f;
  const float c = a.c;

  // ---- pieces of the softmax -------------------------------------------
  // mask keys past the workgroup's key range (past NK, or in the next
  // workgroup's range) and, under the causal mask, after the query (only on
  // the tiles that have such keys).  Element (kb, i) of tile j holds key
  // j*BN + 32kb + 8h + kofs(i).
  auto mask = [&](f32x16 (&s)[NKB], int j) __attribute__((always_inline)) {
    const int kv0 = j * BN;
    if (kv0 + BN > kv_lim || (CAUSAL && kv0 + BN - 1 > wave_q0 + OFF)) {
      const int lim = (CAUSAL ? min(kv_lim - 1, qrow + OFF) : kv_lim - 1) - kv0 - 8 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = 32 * kb + 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
          if (kofs > lim) s[kb][i] = neg_inf();
        }
    }
  };
  // row max of the tile and the reference update: the wave moves its
  // references only when some row's tile max exceeds its reference by more
  // than kTau.  Split in slices so it can sit beside the value MFMAs:
  // slice 0..NKB-1: partial max of block kb; slice NKB: the update.
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
      // wave-uniform branch: the update runs only when a row's tile max
      // exceeds its reference by more than kTau (rare after the first tiles);
      // then every row takes the larger of its reference and its tile max
      if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
        const float m_new = vmax(m_ref, mx * c);
        const float alpha = m_new == neg_inf() ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        if constexpr (!kMfmaSum) l *= alpha;
        lx *= alpha;
        m_ref = m_new;
        pend = true;
        pend_alpha = alpha;
        mu = m_new == neg_inf() ? 0.0f : m_new;
        thr = (m_new + E::kTau) / c;  // a division in the rare path: no register for 1/c
      }
      pin(mu);
      pin(pend_alpha);
      if constexpr (!kMfmaSum) pin(l);
      pin(lx);
      pin(thr);
    }
  };
  // p = exp2(c s - mu) for the 8 scores of value step cc, their sums, and the
  // bf16 P^T fragment of step cc (keys 16cc + 8h .. +7 of this lane's query)
  float lsum[2] = {0.0f, 0.0f}, xsum[2] = {0.0f, 0.0f};
  auto p_slice = [&](f32x16 (&s)[NKB], int cc, int half) __attribute__((always_inline)) {
    const int kb = cc >> 1, base = (cc & 1) * 8 + 4 * half;
#pragma unroll
    for (int e = 0; e < 4; ++e) s[kb][base + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][base + e], c, -mu));
    // each packed word is a scalar before it is bit-cast: this compiler
    // miscompiles __builtin_bit_cast applied to an element of a vector variable
    const uint32_t w0 = E::pack(s[kb][base + 0], s[kb][base + 1]);
    const uint32_t w1 = E::pack(s[kb][base + 2], s[kb][base + 3]);
    if constexpr (!kMfmaSum) {
      lsum[half] = E::sum2(w0, lsum[half]);
      lsum[half] = E::sum2(w1, lsum[half]);
    }
    // the first slice of a phase starts the fp32 sum (adding it to a zero
    // would cost an instruction: x + 0 is not x for x = -0)
    const float part = (s[kb][base + 0] + s[kb][base + 1]) + (s[kb][base + 2] + s[kb][base + 3]);
    xsum[half] = cc == 0 ? part : xsum[half] + part;
    uint32_t r0 = w0, r1 = w1;
    pin(r0);
    pin(r1);
    if constexpr (!kMfmaSum) pin(lsum[half]);
    pin(xsum[half]);
    return u32x2{r0, r1};
  };

  // ---- phases --------------------------------------------------------------
  // phase A of iteration j: score MFMAs of tile j+1 into sn beside the
  // exponentials of tile j in sc: one slot per score MFMA (16 for D = 128, 8
  // for D = 64), the 8 four-score p slices spread evenly over the slots.  K
  // fragments are read PFA slots ahead; the last PFB slots also start the
  // reads of phase B's first value fragments (from Vc) so that phase B does
  // not begin by waiting on LDS.
  auto phase_a = [&](f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], const u32x4* Kt, const u32x4* Vc,
                     u32x4 (&vf)[RVB]) __attribute__((always_inline)) {
    constexpr int NP = 2 * NCC;  // p slices (4 scores each)
    constexpr int SLOTS = NSA > NP ? NSA : NP;
    static_assert(PFB <= SLOTS && PFA <= NSA, "prefetch depths");
    // the exponentials make this the VALU-heavy phase: it gets issue priority
    // over the other wave on the SIMD, which is then typically in its
    // MFMA-heavy phase B
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!kMfmaSum) lsum[0] = lsum[1] = 0.0f;
    u32x4 kf[RKA];
#pragma unroll
    for (int k = 0; k < PFA; ++k) kf[k % RKA] = kfrag(Kt, k);
    u32x2 pw[NP];
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      if (k + PFA < NSA) kf[(k + PFA) % RKA] = kfrag(Kt, k + PFA);
      if (k >= SLOTS - PFB) vf[(k - (SLOTS - PFB)) % RVB] = vfrag(Vc, k - (SLOTS - PFB));
#pragma unroll
      for (int q = k * NP / SLOTS; q < (k + 1) * NP / SLOTS; ++q) pw[q] = p_slice(sc, q >> 1, q & 1);
      if (k < NSA) {
        const int kk = k / NKB, kb = k % NKB;
        const f32x16 z = {};
        sn[kb] = E::mfma(__builtin_bit_cast(vec8, kf[k % RKA]), qf[kk], kk == 0 ? z : sn[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      const u32x4 x = {pw[2 * cc][0], pw[2 * cc][1], pw[2 * cc + 1][0], pw[2 * cc + 1][1]};
      pf[cc] = __builtin_bit_cast(vec8, x);
    }
    if constexpr (!kMfmaSum) l += lsum[0] + lsum[1];
    lx += xsum[0] + xsum[1];
    __builtin_amdgcn_s_setprio(0);
  };
  // phase B of iteration j: value MFMAs of tile j (V^T from Vt, P^T in pf;
  // fragments 0 .. PFB-1 already requested in phase A) beside the reference
  // update of tile j+1's scores in sn
  auto phase_b = [&](const f32x16 (&sn)[NKB], const u32x4* Vt, u32x4 (&vf)[RVB]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
      if (k + PFB < NSB) vf[(k + PFB) % RVB] = vfrag(Vt, k + PFB);
      // the reference slices go in the early slots so the update is known
      // well before the next phase needs mu
      if (k <= NKB) ref_slice(sn, k);
      const int db = k % NDB, cc = k / NDB;
      o[db] = E::mfma(__builtin_bit_cast(vec8, vf[k % RVB]), pf[cc], o[db]);
      if constexpr (kMfmaSum)
        if (db == NDB - 1) lsacc = E::mfma16(ones_op, pf[cc], lsacc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (pend) {
      if constexpr (kMfmaSum) {
        // lsacc[1] of lane n < 16 belongs to query n + 16 (lane n + 16)
        const float a_hi = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(((lane + 16) & 63) << 2, __builtin_bit_cast(int, pend_alpha)));
        lsacc[0] *= pend_alpha;
        lsacc[1] *= a_hi;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= pend_alpha;
      pend = false;
    }
  };

  // ---- prologue ------------------------------------------------------------
  // zeroed tiles in place before any load lands; without them the first tile
  // loads go out at once, in flight together with the Q loads
  if (zero_tiles) __syncthreads();
  if (n_loc > 0) {
    issue(kA, Kg, koff, kon, t_lo * BN);
    issue(vA, Vg, voff, von, t_lo * BN);
  }
  if (n_loc > 1) issue(kB, Kg, koff, kon, (t_lo + 1) * BN);
  __syncthreads();  // the first two K tiles and the first V tile in LDS
  if (n_vis > 0) {
    // scores of the first tile and their reference (the running sums are still zero)
#pragma unroll
    for (int k = 0; k < NSA; ++k) {
      const int kk = k / NKB, kb = k % NKB;
      const f32x16 z = {};
      sA[kb] = E::mfma(__builtin_bit_cast(vec8, kfrag(kA, k)), qf[kk], kk == 0 ? z : sA[kb]);
    }
    mask(sA, t_lo);
#pragma unroll
    for (int k = 0; k <= NKB; ++k) ref_slice(sA, k);
    pend = false;
  }

  // ---- main loop: iteration j consumes S_j (scores in sc) and V_j^T --------
  // j counts the workgroup's tiles from 0 (key tile t_lo + j).  Buffers:
  // K_{j+1} is in Kn, K_{j+2} goes to Kd (which held K_j), V_j is in Vc, V_{j+1}
  // goes to Vd (which held V_{j-1}).
  auto iteration = [&](int j, f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], const u32x4* Kn, u32x4* Kd,
                       const u32x4* Vc, u32x4* Vd) __attribute__((always_inline)) {
    // Everyone is done with iteration j-1 and its tile loads have landed.  The
    // explicit wait is required: at the barrier that heads the loop this
    // compiler drops the wait for the loads issued in the previous iteration
    // (it keeps it only at the barrier inside the loop body).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < n_loc) issue(Vd, Vg, voff, von, (t_lo + j + 1) * BN);
    if (j + 2 < n_loc) issue(Kd, Kg, koff, kon, (t_lo + j + 2) * BN);
    if (j >= n_vis) return;  // nothing of this tile or later is visible to this wave
    // One code path for every iteration (a second one for the last tile costs
    // more registers than the chip has): after the last visible tile the
    // "next" scores are computed from whatever K buffer is there and then fully
    // masked (they lie past the key range or after every query of the wave),
    // which leaves the reference and the sums unchanged, and are never used.
    u32x4 vf[RVB];
    phase_a(sc, sn, Kn, Vc, vf);
    apply_rescale();
    mask(sn, t_lo + j + 1);
    phase_b(sn, Vc, vf);
  };
  for (int j = 0; j < n_loc; j += 2) {
    iteration(j, sA, sB, kB, kA, vA, vB);
    if (j + 1 < n_loc) iteration(j + 1, sB, sA, kA, kB, vB, vA);
  }

  // epilogue: O = o / l, LSE = (m + log2 lx) ln 2.  A split row that sees no
  // key of its range (l = 0) records LSE = -inf and O = 0.
  float l_tot;
  if constexpr (kMfmaSum) {
    // query c32's sum sits in lane c32 % 16, element c32 / 16 (each element
    // is copied to a scalar before its bit cast: see the packed words above)
    float e0 = lsacc[0], e1 = lsacc[1];
    pin(e0);
    pin(e1);
    const int src = (c32 & 15) << 2;
    const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, e0)));
    const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, e1)));
    l_tot = c32 < 16 ? s0 : s1;
  } else {
    l_tot = pair_sum(l);
  }
  const float lx_tot = pair_sum(lx);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < NQ) {
    const float lse_row = l_tot > 0.0f ? (m_ref + __log2f(lx_tot)) * kLn2 : neg_inf();
    if constexpr (SPLIT) {
      const size_t prow = ((size_t)split * a.n_bh + bh) * NQ + qrow;
      float* __restrict__ Op = a.o_part + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * h;
          if (32 * db >= D) continue;
          const f32x4 w = {o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                           o[db][4 * g + 3] * inv};
          *(f32x4*)(Op + d) = w;
        }
      if (h == 0) a.lse_part[prow] = lse_row;
    } else {
      uint16_t* __restrict__ Og = (uint16_t*)a.o + ((size_t)bh * NQ + qrow) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * h;
          if (32 * db >= D) continue;
          const u32x2 w = {E::pack(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                           E::pack(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
          *(u32x2*)(Og + d) = w;
        }
      if (h == 0) a.lse[(size_t)bh * NQ + qrow] = lse_row;
    }
  }
}

// D = 256 holds 64 Q and 128 output registers per lane and 128 KB of tiles:
// one workgroup per CU, one wave per SIMD.
template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kBF16Threads, D == 256 ? 1 : 2) void fa_fwd_bf16_kernel(FwdArgs a) {
  fwd16_body<BF16, D, CAUSAL, SPLIT>(a);
}
template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kBF16Threads, D == 256 ? 1 : 2) void fa_fwd_f16_kernel(FwdArgs a) {
  fwd16_body<F16, D, CAUSAL, SPLIT>(a);
}

// ---------------------------------------------------------------------------
// Merge of the key ranges of a split launch: for every (b, h, query row),
//   lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s,
// the online-softmax update of "Flash Attention" (wiki.ai-engineering.at,
// section "Lösung: Online Softmax") applied to the summaries of whole key
// ranges, with the largest lse_s subtracted before exponentiating.  Ranges in
// which a row sees no key (lse_s = -inf) add nothing.  Each group of D/8 lanes
// handles one row, 8 output elements per lane; O is rounded to the output's
// 16-bit type once.
constexpr int kCombineThreads = 256;

template <typename E, int D>
__device__ __forceinline__ void combine_body(const FwdArgs& a) {
  constexpr int TPR = D / 8;                       // lanes per row
  constexpr int RPB = kCombineThreads / TPR;       // rows per workgroup
  const int tid = threadIdx.x;
  if (tid >= RPB * TPR) return;  // D = 96: 12 lanes a row leave 4 of 256 idle
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int d0 = (tid % TPR) * 8;
  if (row >= (long long)a.n_bh * a.nq) return;
  const size_t stride = (size_t)a.n_bh * a.nq;     // between key ranges, in rows
  float m = neg_inf();
  for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, a.lse_part[s * stride + row]);
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float tot = 0.0f;
  constexpr float kLog2e = 1.44269504088896340736f;
  for (int s = 0; s < a.n_split; ++s) {
    const float ls = a.lse_part[s * stride + row];
    if (ls == neg_inf()) continue;
    const float w = __builtin_amdgcn_exp2f((ls - m) * kLog2e);
    tot += w;
    const float* __restrict__ op = a.o_part + (s * stride + row) * D + d0;
    const f32x4 x0 = *(const f32x4*)op, x1 = *(const f32x4*)(op + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = __builtin_fmaf(w, x0[e], acc[e]);
      acc[4 + e] = __builtin_fmaf(w, x1[e], acc[4 + e]);
    }
  }
  const float inv = 1.0f / tot;
  const u32x4 w = {E::pack(acc[0] * inv, acc[1] * inv), E::pack(acc[2] * inv, acc[3] * inv),
                   E::pack(acc[4] * inv, acc[5] * inv), E::pack(acc[6] * inv, acc[7] * inv)};
  *(u32x4*)((uint16_t*)a.o + row * D + d0) = w;
  if (d0 == 0) a.lse[row] = m + __logf(tot);
}

template <int D>
__global__ __launch_bounds__(kCombineThreads) void fa_combine_kernel(FwdArgs a) {
  combine_body<BF16, D>(a);
}
template <int D>
__global__ __launch_bounds__(kCombineThreads) void fa_combine_f16_kernel(FwdArgs a) {
  combine_body<F16, D>(a);
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
  const int N = a.nq;  // the fp32 path has as many queries as keys

  const HeadItem wi = head_item(xcd_remap(blockIdx.x, a.n_blocks), a.n_bh, a.n_qblk, CAUSAL, D != 128);
  const int bh = wi.bh;
  const int qb = CAUSAL ? a.n_qblk - 1 - wi.idx : wi.idx;  // causal: longest query blocks first
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
