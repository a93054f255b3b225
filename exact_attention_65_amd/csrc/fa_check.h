// Host-side argument validation for fa_fwd / fa_fwd_query.  Pure C++: no HIP
// header, no device access, so it can be compiled and tested on any host.
#pragma once

#include "fa.h"

namespace fa {

// Largest number of workgroups one launch may use (grid x dimension).
constexpr int64_t kMaxGrid = 2147483647;
// Query rows per workgroup of the kernels the grid limit is checked for (the
// 64-row kernel for small grids runs only grids far below the limit).
constexpr int64_t kRowsPerBlock = 128;

// Element size of a dtype, 0 if the dtype is unknown.
size_t elem_size(int dtype);

// Shape/dtype validation shared by both entry points; fills sizes on success.
fa_status check_shape(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, fa_sizes* sizes);

// Whether a valid shape is one the kernels are built for.  D = 96 and 256
// exist only for the 16-bit forward kernels (wide = true).
fa_status check_supported(int64_t B, int64_t H, int64_t N, int64_t D, bool wide = false);

// Full validation of an fa_fwd call, without touching the device.
fa_status check_call(const void* q, const void* k, const void* v, const void* o, const void* lse,
                     int64_t B, int64_t H, int64_t N, int64_t D, float scale, int dtype);

// Keys per tile of the bf16 kernel (the unit a key range is made of).
constexpr int64_t kKeysPerTile = 64;

// Keys per dk/dv workgroup of the backward: 128 (4 waves of 32 keys), or at
// D = 256 64 (4 waves of 16 keys).
constexpr int64_t bwd_keys_per_block(int64_t D) { return D == 256 ? 64 : 128; }

// Whether fa_fwd_split runs the one-query-row kernel (Nq = 1, D in {64, 128, 256}).
inline bool uses_decode_kernel(int64_t Nq, int64_t D) { return Nq == 1 && (D == 64 || D == 128 || D == 256); }

// fa_fwd_split_query: sizes and the resolved number of key ranges.
fa_status check_split_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
                            int n_splits, int dtype, fa_sizes* sizes, int* splits);

// Full validation of an fa_fwd_split call, without touching the device.
fa_status check_split_call(const void* q, const void* k, const void* v, const void* o, const void* lse,
                           const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                           int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, int n_splits,
                           int dtype, int* splits);

// fa_bwd_qk_query: sizes (workspace: two floats per query row); fa_bwd_query
// is the Nq = Nk case.
fa_status check_bwd_qk_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, int dtype,
                             fa_sizes* sizes);
fa_status check_bwd_shape(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, fa_sizes* sizes);

// Full validation of an fa_bwd_qk call, without touching the device.
fa_status check_bwd_qk_call(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const void* lse, const void* dq, const void* dk, const void* dv, const void* workspace,
                            size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                            int causal, float scale, int dtype);

// Full validation of an fa_bwd call, without touching the device.
fa_status check_bwd_call(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const void* lse, const void* dq, const void* dk, const void* dv, const void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t D, float scale,
                         int dtype);

// fa_fwd_fp8_query: sizes of the E4M3 inputs (1 byte each), the bf16 output
// and the LSE; no workspace.  The scale arrays hold B*H*N*D/32 bytes each.
fa_status check_fp8_shape(int64_t B, int64_t H, int64_t N, int64_t D, fa_sizes* sizes);

// Full validation of an fa_fwd_fp8 call, without touching the device.
fa_status check_fp8_call(const void* q, const void* qs, const void* k, const void* ks, const void* v,
                         const void* vs, const void* o, const void* lse, int64_t B, int64_t H, int64_t N,
                         int64_t D, float scale);

}  // namespace fa
