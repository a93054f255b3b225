// Host-side argument validation of the attention forward.  See fa_check.h.
#include "fa_check.h"

#include <cmath>
#include <cstdint>

namespace fa {

size_t elem_size(int dtype) {
  switch (dtype) {
    case FA_DTYPE_F32: return 4;
    case FA_DTYPE_BF16: return 2;
    case FA_DTYPE_F16: return 2;
    default: return 0;
  }
}

static bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
  if (a != 0 && b > UINT64_MAX / a) return false;
  *out = a * b;
  return true;
}

fa_status check_shape(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, fa_sizes* sizes) {
  const size_t elt = elem_size(dtype);
  if (elt == 0) return FA_ERR_BAD_DTYPE;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return FA_ERR_BAD_SHAPE;
  uint64_t bh, rows, elems, bytes, lse_bytes;
  if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || !mul_ok(bh, (uint64_t)N, &rows) ||
      !mul_ok(rows, (uint64_t)D, &elems) || !mul_ok(elems, elt, &bytes) ||
      !mul_ok(rows, 4, &lse_bytes))
    return FA_ERR_BAD_SHAPE;
  if (bytes > (uint64_t)SIZE_MAX || lse_bytes > (uint64_t)SIZE_MAX) return FA_ERR_BAD_SHAPE;
  if (sizes) {
    sizes->q_bytes = sizes->k_bytes = sizes->v_bytes = sizes->o_bytes = (size_t)bytes;
    sizes->lse_bytes = (size_t)lse_bytes;
    sizes->workspace_bytes = 0;
  }
  return FA_OK;
}

fa_status check_supported(int64_t B, int64_t H, int64_t N, int64_t D, bool wide) {
  if (D != 64 && D != 128 && !(wide && (D == 96 || D == 256))) return FA_ERR_UNSUPPORTED;
  // offsets inside one (b, h) slice are 32-bit
  if (N * D > (int64_t)INT32_MAX) return FA_ERR_UNSUPPORTED;
  const int64_t qblocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  // B*H*qblocks may overflow int64 only if B*H alone is huge: compare by division
  if (B > kMaxGrid / H || B * H > kMaxGrid / qblocks) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

fa_status check_call(const void* q, const void* k, const void* v, const void* o, const void* lse,
                     int64_t B, int64_t H, int64_t N, int64_t D, float scale, int dtype) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  fa_sizes sz;
  fa_status st = check_shape(B, H, N, D, dtype, &sz);
  if (st != FA_OK) return st;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SCALE;
  const void* ptrs[5] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if ((uintptr_t)p % 16 != 0) return FA_ERR_MISALIGNED;
  // outputs may not overlap inputs or each other; inputs may alias each other
  if (overlaps(o, sz.o_bytes, lse, sz.lse_bytes)) return FA_ERR_ALIASING;
  const void* ins[3] = {q, k, v};
  for (const void* p : ins)
    if (overlaps(o, sz.o_bytes, p, sz.q_bytes) || overlaps(lse, sz.lse_bytes, p, sz.q_bytes))
      return FA_ERR_ALIASING;
  return check_supported(B, H, N, D, dtype != FA_DTYPE_F32);
}

// Number of key ranges: the requested count, or for FA_SPLIT_AUTO enough for
// about 512 workgroups in all (two per CU on 256 CUs: one round, so the merge
// reads few partials), but no more than leaves 8 key tiles of 64 per
// range, keeps the partial results (Nq rows of D+1 floats per range) within a
// quarter of the K/V bytes (S <= Nk / (4 Nq)), and at most 64.  Square shapes
// therefore stay on one range: their partial results would double the traffic.
// For one query row (the vector-unit kernel): enough ranges for about 512
// workgroups (two waves per SIMD; measured, more ranges only add merge work),
// each range at least 1024 keys, at most 64.
static int resolve_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int requested) {
  if (requested != FA_SPLIT_AUTO) return requested;
  if (uses_decode_kernel(Nq, D)) {
    int64_t s = (512 + B * H - 1) / (B * H);
    if (s > Nk / 1024) s = Nk / 1024;
    if (s > 64) s = 64;
    return s < 1 ? 1 : (int)s;
  }
  const int64_t blocks = B * H * ((Nq + kRowsPerBlock - 1) / kRowsPerBlock);
  const int64_t tiles = (Nk + kKeysPerTile - 1) / kKeysPerTile;
  int64_t s = (512 + blocks - 1) / blocks;
  if (s > tiles / 8) s = tiles / 8;
  if (s > Nk / (4 * Nq)) s = Nk / (4 * Nq);
  if (s > 64) s = 64;
  return s < 1 ? 1 : (int)s;
}

fa_status check_split_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
                            int n_splits, int dtype, fa_sizes* sizes, int* splits) {
  const size_t elt = elem_size(dtype);
  if (elt == 0) return FA_ERR_BAD_DTYPE;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || D <= 0) return FA_ERR_BAD_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_BAD_SHAPE;
  if (n_splits < 0 || n_splits > FA_SPLIT_MAX) return FA_ERR_BAD_SHAPE;
  uint64_t bh, qrows, krows, qel, kel, qbytes, kbytes, lbytes;
  if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || !mul_ok(bh, (uint64_t)Nq, &qrows) ||
      !mul_ok(bh, (uint64_t)Nk, &krows) || !mul_ok(qrows, (uint64_t)D, &qel) ||
      !mul_ok(krows, (uint64_t)D, &kel) || !mul_ok(qel, elt, &qbytes) || !mul_ok(kel, elt, &kbytes) ||
      !mul_ok(qrows, 4, &lbytes))
    return FA_ERR_BAD_SHAPE;
  if (qbytes > (uint64_t)SIZE_MAX || kbytes > (uint64_t)SIZE_MAX) return FA_ERR_BAD_SHAPE;
  // the arguments are valid; what follows decides whether the kernels support them
  if (D != 64 && D != 96 && D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  if (Nq * D > (int64_t)INT32_MAX || Nk * D > (int64_t)INT32_MAX) return FA_ERR_UNSUPPORTED;
  const int64_t qblocks = (Nq + kRowsPerBlock - 1) / kRowsPerBlock;
  if (B > kMaxGrid / H || B * H > kMaxGrid / qblocks) return FA_ERR_UNSUPPORTED;
  const int s = resolve_splits(B, H, Nq, Nk, D, n_splits);
  if (B * H * qblocks > kMaxGrid / s) return FA_ERR_UNSUPPORTED;
  uint64_t ws = 0;
  if (s > 1 && (!mul_ok(qrows, (uint64_t)(D + 1) * 4, &ws) || !mul_ok(ws, (uint64_t)s, &ws)))
    return FA_ERR_BAD_SHAPE;
  if (ws > (uint64_t)SIZE_MAX) return FA_ERR_BAD_SHAPE;
  if (sizes) {
    sizes->q_bytes = sizes->o_bytes = (size_t)qbytes;
    sizes->k_bytes = sizes->v_bytes = (size_t)kbytes;
    sizes->lse_bytes = (size_t)lbytes;
    sizes->workspace_bytes = (size_t)ws;
  }
  if (splits) *splits = s;
  return FA_OK;
}

fa_status check_split_call(const void* q, const void* k, const void* v, const void* o, const void* lse,
                           const void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                           int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, int n_splits,
                           int dtype, int* splits) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  fa_sizes sz;
  int s = 1;
  // invalid arguments first; a valid but unsupported shape is reported after them
  fa_status st = check_split_shape(B, H, Nq, Nk, D, causal, n_splits, dtype, &sz, &s);
  if (st != FA_OK && st != FA_ERR_UNSUPPORTED) return st;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (st == FA_ERR_UNSUPPORTED) return st;
  const bool ws = sz.workspace_bytes > 0;
  if (ws && !workspace) return FA_ERR_NULL_POINTER;
  const void* ptrs[6] = {q, k, v, o, lse, ws ? workspace : q};
  for (const void* p : ptrs)
    if ((uintptr_t)p % 16 != 0) return FA_ERR_MISALIGNED;
  if (workspace_bytes < sz.workspace_bytes) return FA_ERR_WORKSPACE;
  // outputs and workspace may not overlap inputs or each other
  struct Buf { const void* p; size_t n; };
  const Buf outs[3] = {{o, sz.o_bytes}, {lse, sz.lse_bytes}, {workspace, ws ? sz.workspace_bytes : 0}};
  const Buf ins[3] = {{q, sz.q_bytes}, {k, sz.k_bytes}, {v, sz.v_bytes}};
  for (int i = 0; i < 3; ++i) {
    if (outs[i].n == 0) continue;
    for (int j = i + 1; j < 3; ++j)
      if (outs[j].n && overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return FA_ERR_ALIASING;
    for (const Buf& b : ins)
      if (overlaps(outs[i].p, outs[i].n, b.p, b.n)) return FA_ERR_ALIASING;
  }
  if (splits) *splits = s;
  return FA_OK;
}

fa_status check_bwd_qk_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, int dtype,
                             fa_sizes* sizes) {
  const size_t elt = elem_size(dtype);
  if (elt == 0) return FA_ERR_BAD_DTYPE;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || D <= 0) return FA_ERR_BAD_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_BAD_SHAPE;
  uint64_t bh, qrows, krows, qel, kel, qbytes, kbytes, lbytes, wbytes;
  if (!mul_ok((uint64_t)B, (uint64_t)H, &bh) || !mul_ok(bh, (uint64_t)Nq, &qrows) ||
      !mul_ok(bh, (uint64_t)Nk, &krows) || !mul_ok(qrows, (uint64_t)D, &qel) ||
      !mul_ok(krows, (uint64_t)D, &kel) || !mul_ok(qel, elt, &qbytes) || !mul_ok(kel, elt, &kbytes) ||
      !mul_ok(qrows, 4, &lbytes) || !mul_ok(lbytes, 2, &wbytes))
    return FA_ERR_BAD_SHAPE;
  if (qbytes > (uint64_t)SIZE_MAX || kbytes > (uint64_t)SIZE_MAX || wbytes > (uint64_t)SIZE_MAX)
    return FA_ERR_BAD_SHAPE;
  if (sizes) {
    sizes->q_bytes = sizes->o_bytes = (size_t)qbytes;
    sizes->k_bytes = sizes->v_bytes = (size_t)kbytes;
    sizes->lse_bytes = (size_t)lbytes;
    sizes->workspace_bytes = (size_t)wbytes;  // Delta and -LSE log2(e) per query row
  }
  // the arguments are valid; what follows decides whether the kernels support them
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  if (D != 64 && D != 96 && D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
  if (Nq * D > (int64_t)INT32_MAX || Nk * D > (int64_t)INT32_MAX) return FA_ERR_UNSUPPORTED;
  // both grids, and their sum (the one-launch plan), within the grid limit
  const int64_t kpb = bwd_keys_per_block(D);
  const int64_t blocks = (Nq + kRowsPerBlock - 1) / kRowsPerBlock + (Nk + kpb - 1) / kpb;
  if (B > kMaxGrid / H || B * H > kMaxGrid / blocks) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa_status check_bwd_shape(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, fa_sizes* sizes) {
  return check_bwd_qk_shape(B, H, N, N, D, 0, dtype, sizes);
}

fa_status check_bwd_qk_call(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const void* lse, const void* dq, const void* dk, const void* dv, const void* workspace,
                            size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                            int causal, float scale, int dtype) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL_POINTER;
  fa_sizes sz;
  fa_status st = check_bwd_qk_shape(B, H, Nq, Nk, D, causal, dtype, &sz);
  if (st != FA_OK && st != FA_ERR_UNSUPPORTED) return st;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (st == FA_ERR_UNSUPPORTED) return st;
  const void* ptrs[10] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if ((uintptr_t)p % 16 != 0) return FA_ERR_MISALIGNED;
  if (workspace_bytes < sz.workspace_bytes) return FA_ERR_WORKSPACE;
  // outputs and workspace may not overlap any buffer or each other; inputs may alias
  struct Buf { const void* p; size_t n; };
  const Buf outs[4] = {{dq, sz.q_bytes}, {dk, sz.k_bytes}, {dv, sz.v_bytes}, {workspace, sz.workspace_bytes}};
  const Buf ins[6] = {{q, sz.q_bytes}, {k, sz.k_bytes}, {v, sz.v_bytes}, {o, sz.o_bytes}, {dout, sz.o_bytes},
                      {lse, sz.lse_bytes}};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return FA_ERR_ALIASING;
    for (const Buf& b : ins)
      if (overlaps(outs[i].p, outs[i].n, b.p, b.n)) return FA_ERR_ALIASING;
  }
  return FA_OK;
}

fa_status check_bwd_call(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const void* lse, const void* dq, const void* dk, const void* dv, const void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t D, float scale,
                         int dtype) {
  return check_bwd_qk_call(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, N, D, 0, scale,
                           dtype);
}

fa_status check_fp8_shape(int64_t B, int64_t H, int64_t N, int64_t D, fa_sizes* sizes) {
  fa_sizes sz;
  fa_status st = check_shape(B, H, N, D, FA_DTYPE_BF16, &sz);  // the bf16 output's limits
  if (st != FA_OK) return st;
  const size_t codes = sz.q_bytes / 2;
  sz.q_bytes = sz.k_bytes = sz.v_bytes = codes;
  if (sizes) *sizes = sz;
  if (D == 96) return FA_ERR_UNSUPPORTED;   // D in {64, 128, 256}
  return check_supported(B, H, N, D, true);
}

fa_status check_fp8_call(const void* q, const void* qs, const void* k, const void* ks, const void* v,
                         const void* vs, const void* o, const void* lse, int64_t B, int64_t H, int64_t N,
                         int64_t D, float scale) {
  if (!q || !qs || !k || !ks || !v || !vs || !o || !lse) return FA_ERR_NULL_POINTER;
  fa_sizes sz;
  fa_status st = check_fp8_shape(B, H, N, D, &sz);
  if (st != FA_OK && st != FA_ERR_UNSUPPORTED) return st;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (st == FA_ERR_UNSUPPORTED) return st;
  const void* a16[6] = {q, k, v, o, lse, nullptr};
  for (const void* p : a16)
    if (p && (uintptr_t)p % 16 != 0) return FA_ERR_MISALIGNED;
  const void* a4[3] = {qs, ks, vs};
  for (const void* p : a4)
    if ((uintptr_t)p % 4 != 0) return FA_ERR_MISALIGNED;
  const size_t sc_bytes = sz.q_bytes / 32;
  struct Buf { const void* p; size_t n; };
  const Buf ins[6] = {{q, sz.q_bytes}, {qs, sc_bytes}, {k, sz.q_bytes}, {ks, sc_bytes}, {v, sz.q_bytes}, {vs, sc_bytes}};
  const Buf outs[2] = {{o, sz.o_bytes}, {lse, sz.lse_bytes}};
  if (overlaps(outs[0].p, outs[0].n, outs[1].p, outs[1].n)) return FA_ERR_ALIASING;
  for (const Buf& ob : outs)
    for (const Buf& ib : ins)
      if (overlaps(ob.p, ob.n, ib.p, ib.n)) return FA_ERR_ALIASING;
  return FA_OK;
}

}  // namespace fa

extern "C" {

__attribute__((visibility("default"))) fa_status fa_bwd_query(int64_t B, int64_t H, int64_t N, int64_t D,
                                                               int causal, fa_dtype dtype, fa_sizes* out) {
  (void)causal;
  if (!out) return FA_ERR_NULL_POINTER;
  return fa::check_bwd_shape(B, H, N, D, (int)dtype, out);
}

__attribute__((visibility("default"))) fa_status fa_bwd_qk_query(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                                                  int64_t D, int causal, fa_dtype dtype,
                                                                  fa_sizes* out) {
  if (!out) return FA_ERR_NULL_POINTER;
  return fa::check_bwd_qk_shape(B, H, Nq, Nk, D, causal, (int)dtype, out);
}

__attribute__((visibility("default"))) fa_status fa_fwd_split_query(int64_t B, int64_t H, int64_t Nq,
                                                                     int64_t Nk, int64_t D, int causal,
                                                                     int n_splits, fa_dtype dtype,
                                                                     fa_sizes* out, int* splits_out) {
  if (!out) return FA_ERR_NULL_POINTER;
  return fa::check_split_shape(B, H, Nq, Nk, D, causal, n_splits, (int)dtype, out, splits_out);
}

__attribute__((visibility("default"))) fa_status fa_fwd_query(int64_t B, int64_t H, int64_t N,
                                                               int64_t D, int causal,
                                                               fa_dtype dtype, fa_sizes* out) {
  (void)causal;
  if (!out) return FA_ERR_NULL_POINTER;
  fa_status st = fa::check_shape(B, H, N, D, (int)dtype, out);
  if (st != FA_OK) return st;
  return fa::check_supported(B, H, N, D, dtype != FA_DTYPE_F32);
}

__attribute__((visibility("default"))) const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: B, H, N, D must be positive and sizes must fit size_t";
    case FA_ERR_BAD_SCALE: return "FA_ERR_BAD_SCALE: scale must be finite";
    case FA_ERR_BAD_DTYPE: return "FA_ERR_BAD_DTYPE: dtype must be FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: every pointer must be 16-byte aligned";
    case FA_ERR_ALIASING: return "FA_ERR_ALIASING: outputs and workspace must not overlap the inputs or each other";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: a head dimension or dtype the entry point lacks (D in {64,96,128,256} for 16-bit "
             "forward inputs and the backward, {64,128,256} for FP8, {64,128} for fp32), N*D >= 2^31, "
             "more than 2^31-1 workgroups, or not a gfx950 device";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP runtime call failed";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace_bytes is smaller than the call needs";
  }
  return "unknown fa_status";
}

__attribute__((visibility("default"))) int fa_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
