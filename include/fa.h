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
 * one sequence of length N).  The pages name masking without defining it; this
 * is the reading the library implements.
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

#define FA_ABI_VERSION 1

/* Identical to hipStream_t.  NULL means the device's null stream. */
typedef struct ihipStream_t* fa_stream_t;

/* Element type of q, k, v and o.  lse is always float32. */
typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,  /* IEEE binary32 in and out; float32 MFMA                     */
  FA_DTYPE_BF16 = 1  /* bfloat16 in and out; products exact, sums and softmax fp32 */
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                              */
  FA_ERR_BAD_SHAPE = 2,    /* B, H, N or D <= 0, or a byte size overflows size_t      */
  FA_ERR_BAD_SCALE = 3,    /* scale is NaN or infinite                                */
  FA_ERR_BAD_DTYPE = 4,    /* dtype is not one of fa_dtype                            */
  FA_ERR_MISALIGNED = 5,   /* a pointer is not 16-byte aligned                        */
  FA_ERR_ALIASING = 6,     /* o or lse overlaps q, k, v or each other                 */
  FA_ERR_UNSUPPORTED = 7,  /* valid but not built: D not 64/128, N*D >= 2^31, more   */
                           /* than 2^31-1 workgroups, or the device is not gfx950     */
  FA_ERR_HIP = 8           /* a HIP runtime call failed (no device, launch failure)   */
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
 * supports the shape, FA_ERR_UNSUPPORTED when it does not (D not in {64, 128},
 * N*D >= 2^31, or more than 2^31-1 workgroups), FA_ERR_BAD_SHAPE /
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
 * The caller owns every buffer; the call allocates nothing (workspace 0).
 * Arguments are validated on the host before anything is enqueued and an
 * error is returned synchronously, with nothing launched: NULL pointers,
 * non-positive sizes, non-finite scale, unknown dtype, pointers not 16-byte
 * aligned, o/lse overlapping an input or each other, unsupported shapes,
 * non-gfx950 devices.  FA_OK means the kernel was enqueued; execution is
 * asynchronous and a fault during execution surfaces at the caller's next
 * synchronisation.  Thread-safe; the only global state is a per-device
 * architecture cache.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale,
                 fa_dtype dtype, fa_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_str(fa_status s);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
