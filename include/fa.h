/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * The library computes, for every batch index b and head h,
 *
 *     O[b,h] = softmax_over_keys(scale * Q[b,h] K[b,h]^T  [+ causal mask]) V[b,h]
 *     LSE[b,h,i] = ln sum_{j visible to i} exp(scale * q_i . k_j)
 *
 * which is the attention of "Flash Attention" (wiki.ai-engineering.at),
 * section "Das Grundproblem", and of "Flash Attention: ускорить attention в 6
 * раз без потери точности" (johe.ru), section "Введение: проблема attention".
 * It is evaluated tile by tile with the online-softmax recurrence of the first
 * page (section "Lösung: Online Softmax"), so the N x N score matrix is never
 * written to device memory (ZimaSpace, "Wie reduziert Flash Attention den
 * Speicherverkehr während der lokalen Inferenz?", section "Online-Softmax
 * vermeidet das Speichern der vollständigen Score-Matrix").  The result equals
 * plain attention up to floating-point rounding (johe.ru, section "Почему это
 * точно?").
 *
 * Causal mask: key j is visible to query i iff j <= i (queries and keys share
 * one sequence of length N).  With fewer queries (Nq) than keys (Nk), in
 * fa_fwd_split, the queries are the last Nq positions of the sequence: key j
 * is visible to query i iff j <= i + Nk - Nq, as when new tokens attend to a
 * kept KV cache (ZimaSpace, section "Weniger IO bedeutet nicht, dass der
 * KV-Cache entfällt").  The pages name masking without defining it; these are
 * the readings the library implements.
 *
 * LSE is not on the pages: it is the per-row statistic a backward pass needs,
 * returned in natural-log units for every row.
 *
 * No entry point allocates or frees device memory, synchronises the device,
 * or falls back to another implementation.  This header includes no HIP
 * header so host-only code can use it.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 9

/* Identical to hipStream_t.  NULL means the device's null stream. */
typedef struct ihipStream_t* fa_stream_t;

/* Element type of q, k, v and o.  lse is always float32. */
typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,  /* IEEE binary32 in and out; float32 MFMA                     */
  FA_DTYPE_BF16 = 1, /* bfloat16 in and out; products exact, sums and softmax fp32 */
  FA_DTYPE_F16 = 2   /* IEEE binary16 in and out; as bfloat16, P rounded to fp16   */
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                              */
  FA_ERR_BAD_SHAPE = 2,    /* B, H, N or D <= 0, or a byte size overflows size_t      */
  FA_ERR_BAD_SCALE = 3,    /* scale is NaN or infinite                                */
  FA_ERR_BAD_DTYPE = 4,    /* dtype is not one of fa_dtype                            */
  FA_ERR_MISALIGNED = 5,   /* a pointer is not 16-byte aligned                        */
  FA_ERR_ALIASING = 6,     /* o or lse overlaps q, k, v or each other                 */
  FA_ERR_UNSUPPORTED = 7,  /* valid but not built: a head dimension or dtype the     */
                           /* entry point lacks, N*D >= 2^31, more than 2^31-1        */
                           /* workgroups, or the device is not gfx950                 */
  FA_ERR_HIP = 8,          /* a HIP runtime call failed (no device, launch failure)   */
  FA_ERR_WORKSPACE = 9     /* workspace_bytes below what the call needs               */
} fa_status;

/* Byte sizes of every buffer of one call. */
typedef struct fa_sizes {
  size_t q_bytes;         /* B*H*N*D*elt */
  size_t k_bytes;         /* B*H*N*D*elt */
  size_t v_bytes;         /* B*H*N*D*elt */
  size_t o_bytes;         /* B*H*N*D*elt */
  size_t lse_bytes;       /* B*H*N*4     */
  size_t workspace_bytes; /* device scratch the call needs beyond the above: always 0 */
} fa_sizes;

/*
 * fa_fwd_query - sizes of the buffers of an fa_fwd call with these arguments.
 *
 * Pure host function: needs no device and touches no HIP state.  Fills *out
 * whenever the shape and dtype are valid, then returns FA_OK when fa_fwd
 * supports the shape, FA_ERR_UNSUPPORTED when it does not (D not in {64, 128}
 * for float32 or {64, 96, 128, 256} for bfloat16 and float16, N*D >= 2^31, or
 * more than 2^31-1 workgroups), FA_ERR_BAD_SHAPE /
 * FA_ERR_BAD_DTYPE for invalid arguments and FA_ERR_NULL_POINTER if out is
 * NULL.  The device architecture is not checked here.
 */
fa_status fa_fwd_query(int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                       fa_dtype dtype, fa_sizes* out);

/*
 * fa_fwd - exact attention forward, enqueued on `stream`.
 *
 * q, k, v : device pointers, [B, H, N, D] contiguous (row-major, D fastest),
 *           element type `dtype`; read only.  They may alias one another.
 * o       : device pointer, [B, H, N, D] contiguous, element type `dtype`;
 *           every element is overwritten.
 * lse     : device pointer, float32 [B, H, N] contiguous; every element is
 *           overwritten with ln sum_j exp(scale * q_i . k_j) over the keys
 *           visible to row i.
 * causal  : 0 = every key is visible; nonzero = key j visible to query i iff j <= i.
 * scale   : any finite value (the pages use 1/sqrt(D)); negative and zero are
 *           valid.
 * stream  : HIP stream the single kernel launch is enqueued on.
 *
 * The kernel takes 128 query rows per workgroup; for bfloat16 and float16 a
 * grid of at most one such workgroup per compute unit
 * (B * H * ceil(N / 128) <= the device's CU count) runs instead on a kernel of
 * 64 rows per workgroup and 16 per wave, whose waves finish each key tile in
 * about half the time, and at D = 256 a larger grid runs on that kernel in
 * 128-row workgroups of 8 waves (two per SIMD instead of one).  All give the
 * same results up to the order of the fp32 additions (the sums that
 * normalise O and give the LSE).
 *
 * The caller owns every buffer; the call allocates nothing (workspace 0).
 * Arguments are validated on the host before anything is enqueued and an
 * error is returned synchronously, with nothing launched: NULL pointers,
 * non-positive sizes, non-finite scale, unknown dtype, pointers not 16-byte
 * aligned, o/lse overlapping an input or each other, unsupported shapes,
 * non-gfx950 devices.  FA_OK means the kernel was enqueued; execution is
 * asynchronous and a fault during execution surfaces at the caller's next
 * synchronisation.  Thread-safe; the only global state is a per-device cache
 * of the architecture and the compute-unit count.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale,
                 fa_dtype dtype, fa_stream_t stream);

/* fa_fwd_split: let the library choose the number of key ranges. */
#define FA_SPLIT_AUTO 0
/* Largest number of key ranges fa_fwd_split accepts. */
#define FA_SPLIT_MAX 256

/*
 * fa_fwd_split_query - buffer sizes of an fa_fwd_split call, and the number of
 * key ranges it will use.
 *
 * Pure host function (no device).  q and o are [B, H, Nq, D], k and v
 * [B, H, Nk, D], lse [B, H, Nq]; workspace_bytes is what the call needs beyond
 * them: 0 for one range, else n_splits * B * H * Nq * (D + 1) * 4 (a float32
 * output row and log-sum-exp per query row and range).  *splits_out (if not
 * NULL) receives the number of ranges: n_splits itself, or for FA_SPLIT_AUTO
 * the library's choice, which depends only on the arguments: enough ranges
 * for about 512 workgroups, but at least 8 key tiles of 64 per range, at most
 * Nk / (4 Nq) ranges (partial results within a quarter of the K/V bytes) and at
 * most 64; so one range unless the queries are few against many keys.
 * *out and *splits_out are written only on FA_OK.
 * Returns FA_OK, FA_ERR_BAD_SHAPE (a size <= 0, Nq > Nk with
 * causal, n_splits outside 0..FA_SPLIT_MAX, overflow), FA_ERR_BAD_DTYPE,
 * FA_ERR_NULL_POINTER (out NULL) or FA_ERR_UNSUPPORTED (float32, D not in
 * {64, 96, 128, 256}, Nq*D or Nk*D >= 2^31, more than 2^31-1 workgroups).
 */
fa_status fa_fwd_split_query(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
                             int n_splits, fa_dtype dtype, fa_sizes* out, int* splits_out);

/*
 * fa_fwd_split - exact attention forward with the keys of every query block
 * divided into contiguous ranges processed by separate workgroups, then merged.
 *
 * Fills the device when B*H*ceil(Nq/128) alone gives few workgroups (short
 * sequences, one or a few new tokens against a long KV cache).  Each range
 * yields, per query row, its normalised output and log-sum-exp; a second
 * kernel on the same stream merges them, lse = ln sum_s exp(lse_s),
 * o = sum_s exp(lse_s - lse) o_s: the online-softmax update of "Flash
 * Attention" (wiki.ai-engineering.at, section "Lösung: Online Softmax")
 * applied to whole ranges.  The pages name this use ("Flash-Decoding", same
 * page, section "Flash Attention v2: Noch besser (2023)") without giving its
 * steps.
 *
 * q, o      : [B, H, Nq, D] bfloat16 or float16 contiguous (o written).
 * k, v      : [B, H, Nk, D] of the same type, contiguous; q, k, v may alias.
 * lse       : float32 [B, H, Nq], written.
 * workspace : device scratch of workspace_bytes >= the size fa_fwd_split_query
 *             reports (may be NULL when that is 0), 16-byte aligned, not
 *             overlapping any other buffer; owned by the caller, contents on
 *             entry ignored, clobbered.  Calls that share a workspace must be
 *             ordered (same stream or synchronised).
 * causal    : as in fa_fwd, with the queries as the last Nq positions (Nq <= Nk).
 * n_splits  : FA_SPLIT_AUTO or 1 .. FA_SPLIT_MAX.  With one range no workspace
 *             is used and a single kernel writes o and lse (chosen as in
 *             fa_fwd, with B * H * ceil(Nq / 128) for the grid).
 *
 * Validation and asynchrony as in fa_fwd; FA_ERR_WORKSPACE when workspace_bytes
 * is too small.  bfloat16 or float16 (not float32).  Allocates nothing.
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                       int64_t Nk, int64_t D, int causal, float scale, int n_splits, fa_dtype dtype,
                       fa_stream_t stream);

/* Size of the library's own scratch used by fa_fwd_split_static (64 MiB). */
#define FA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fa_fwd_split_static - fa_fwd_split without a caller workspace: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, results, validation and asynchrony as fa_fwd_split with the same
 * q, k, v, o, lse, shapes, causal, scale, n_splits, dtype and stream.  The key
 * ranges' partial results go to a scratch array the library holds per device
 * (FA_STATIC_SCRATCH_BYTES, held from the first use on a device until the
 * process ends) instead of a workspace.  Returns FA_ERR_WORKSPACE when the
 * workspace fa_fwd_split_query reports for these arguments exceeds
 * FA_STATIC_SCRATCH_BYTES (checked on the host, before any device call).
 * Allocates nothing: no hipMalloc or hipFree, no allocating library call; the
 * first call on a device looks up the scratch's device address once.
 * Every call on one device shares that device's scratch, which keeps the
 * last call's contents: calls that overlap in time on one device (different
 * streams, or threads without ordering) race and must be serialised by the
 * caller.
 */
fa_status fa_fwd_split_static(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                              int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                              int n_splits, fa_dtype dtype, fa_stream_t stream);

/*
 * fa_bwd_query - buffer sizes of an fa_bwd call.
 *
 * Pure host function.  q_bytes .. o_bytes are the sizes of q, k, v, o (and of
 * dout, dq, dk, dv, which share them), lse_bytes that of lse, and
 * workspace_bytes = B*H*N*8 (two floats per query row: sum_d dO O and
 * -LSE log2(e)).  Returns as fa_fwd_query; FA_ERR_UNSUPPORTED also for float32
 * (the backward takes bfloat16 and float16) and for D not in {64, 96, 128, 256}
 * (D = 256 since ABI version 9).
 */
fa_status fa_bwd_query(int64_t B, int64_t H, int64_t N, int64_t D, int causal, fa_dtype dtype,
                       fa_sizes* out);

/*
 * fa_bwd - gradients of fa_fwd's O with respect to q, k and v, enqueued on `stream`.
 *
 * For the upstream gradient dout of O (LSE receives none), with the forward's
 * o and lse: P = exp(scale q k^T - lse) over the visible keys,
 * Delta = rowsum(dout * o), dS = P * (dout v^T - Delta), and
 *     dq = scale dS k,   dk = scale dS^T q,   dv = P^T dout.
 * The pages say the gradients are computed in a second pass over the same
 * chunks without storing the score matrix ("Flash Attention: ускорить
 * attention в 6 раз без потери точности", section "Стадии вычисления"); the
 * formulas are the derivatives of the forward.  Two kernels on `stream`: one
 * per 128 query rows (dq, and per row Delta and the LSE in base 2 into the
 * workspace), then one per 128 keys (dk, dv; 64 keys at D = 256); when those
 * two grids together hold at most one workgroup per compute unit (D < 256), a
 * small kernel writes Delta and the LSE in base 2 and one grid then runs both
 * kinds of workgroup.  No atomics: the result is deterministic.
 *
 * q, k, v, o, dout : [B, H, N, D] contiguous, element type `dtype` (bfloat16
 *                    or float16), read only (may alias).
 * lse              : float32 [B, H, N] from fa_fwd with the same q, k, v,
 *                    causal and scale.
 * dq, dk, dv       : [B, H, N, D] of the same type, written; not overlapping any other
 *                    buffer.
 * workspace        : >= fa_bwd_query's workspace_bytes, 16-byte aligned,
 *                    caller-owned, clobbered.
 *
 * Validation and asynchrony as in fa_fwd; FA_ERR_WORKSPACE when
 * workspace_bytes is too small.  bfloat16 or float16, D in {64, 96, 128, 256}.
 * Allocates nothing.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale, fa_dtype dtype,
                 fa_stream_t stream);

/*
 * fa_bwd_qk_query - buffer sizes of an fa_bwd_qk call.
 *
 * Pure host function.  q_bytes and o_bytes are the sizes of q, o (and of dout,
 * dq) with Nq rows, k_bytes and v_bytes those of k, v (and dk, dv) with Nk rows,
 * lse_bytes that of lse (Nq rows), workspace_bytes = B*H*Nq*8.  Returns as
 * fa_bwd_query, and FA_ERR_BAD_SHAPE also for causal with Nq > Nk.
 */
fa_status fa_bwd_qk_query(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, fa_dtype dtype,
                          fa_sizes* out);

/*
 * fa_bwd_qk - fa_bwd for Nq queries against Nk keys per (b, h): the gradients
 * of fa_fwd_split's O (any number of key ranges) for such a shape, e.g. a
 * chunk of new tokens attending to the keys and values kept from earlier ones
 * ("Wie reduziert Flash Attention den Speicherverkehr während der lokalen
 * Inferenz?", section "Weniger IO bedeutet nicht, dass der KV-Cache
 * entfällt").  Same formulas, kernels and determinism as fa_bwd, which is its
 * Nq = Nk case.
 *
 * q, o, dout, dq   : [B, H, Nq, D];  k, v, dk, dv : [B, H, Nk, D]; element type
 *                    `dtype` (bfloat16 or float16), contiguous; dq, dk, dv
 *                    written, not overlapping any other buffer.
 * lse              : float32 [B, H, Nq] from fa_fwd_split with the same inputs.
 * causal           : as in fa_fwd_split: query i is position i + Nk - Nq and
 *                    sees keys 0 .. i + Nk - Nq (Nq <= Nk).
 * workspace        : >= fa_bwd_qk_query's workspace_bytes, 16-byte aligned,
 *                    caller-owned, clobbered.
 *
 * Validation and asynchrony as in fa_bwd.  D in {64, 96, 128, 256}.  Allocates
 * nothing.
 */
fa_status fa_bwd_qk(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                    int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                    fa_dtype dtype, fa_stream_t stream);

/*
 * fa_fwd_fp8_query - buffer sizes of an fa_fwd_fp8 call.
 *
 * Pure host function.  q_bytes = k_bytes = v_bytes = B*H*N*D (one byte per
 * E4M3 code), o_bytes = B*H*N*D*2 (bf16), lse_bytes = B*H*N*4, no workspace.
 * Each scale array holds B*H*N*(D/32) bytes.  Returns as fa_fwd_query, with
 * FA_ERR_UNSUPPORTED for D not in {64, 128, 256}.
 */
fa_status fa_fwd_fp8_query(int64_t B, int64_t H, int64_t N, int64_t D, int causal, fa_sizes* out);

/*
 * fa_fwd_fp8 - attention forward on FP8 inputs with MX block scales, enqueued on `stream`.
 *
 * q, k, v         : [B, H, N, D] OCP FP8 E4M3 codes (uint8), contiguous.
 * q_scale, k_scale, v_scale
 *                 : [B, H, N, D/32] OCP MX E8M0 scale codes (uint8): element
 *                   (row, d) denotes e4m3(code) * 2^(scale[row][d/32] - 127).
 *                   V scale codes must lie in 1..254.
 * o               : [B, H, N, D] bfloat16, written.
 * lse             : [B, H, N] float32, written (natural log).
 *
 * Computes fa_fwd's O and LSE for the values the codes and scales denote.
 * The pages only name FP8 support and block-scaled attention among the later
 * FlashAttention versions ("Flash Attention: ускорить attention в 6 раз без
 * потери точности", sections "Flash Attention 3" and "Flash Attention 4");
 * the MX format with blocks of 32 along D is this library's reading.  Q K^T
 * runs on the scaled FP8 matrix instruction (block scales applied by the
 * hardware, products exact); V is widened to bf16 with its scales (exact) and
 * P V runs in bf16 with P rounded to bf16, as in fa_fwd.
 *
 * q, k, v, o, lse must be 16-byte aligned, the scale arrays 4-byte aligned;
 * o and lse must not overlap any input or each other (inputs may alias).
 * Validation and asynchrony as in fa_fwd.  D in {64, 128, 256} (D = 256 since
 * ABI version 8); no workspace, nothing allocated.
 */
fa_status fa_fwd_fp8(const void* q, const void* q_scale, const void* k, const void* k_scale, const void* v,
                     const void* v_scale, void* o, float* lse, int64_t B, int64_t H, int64_t N, int64_t D,
                     int causal, float scale, fa_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_str(fa_status s);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
