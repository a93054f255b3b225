// Host-side argument validation of the attention forward.  See fa_check.h.
#include "fa_check.h"

#include <cmath>
#include <cstdint>

namespace fa {

size_t elem_size(int dtype) {
  switch (dtype) {
    case FA_DTYPE_F32: return 4;
    case FA_DTYPE_BF16: return 2;
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

fa_status check_supported(int64_t B, int64_t H, int64_t N, int64_t D) {
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
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
  return check_supported(B, H, N, D);
}

}  // namespace fa

extern "C" {

__attribute__((visibility("default"))) fa_status fa_fwd_query(int64_t B, int64_t H, int64_t N,
                                                               int64_t D, int causal,
                                                               fa_dtype dtype, fa_sizes* out) {
  (void)causal;
  if (!out) return FA_ERR_NULL_POINTER;
  fa_status st = fa::check_shape(B, H, N, D, (int)dtype, out);
  if (st != FA_OK) return st;
  return fa::check_supported(B, H, N, D);
}

__attribute__((visibility("default"))) const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: B, H, N, D must be positive and sizes must fit size_t";
    case FA_ERR_BAD_SCALE: return "FA_ERR_BAD_SCALE: scale must be finite";
    case FA_ERR_BAD_DTYPE: return "FA_ERR_BAD_DTYPE: dtype must be FA_DTYPE_F32 or FA_DTYPE_BF16";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: every pointer must be 16-byte aligned";
    case FA_ERR_ALIASING: return "FA_ERR_ALIASING: o and lse must not overlap the inputs or each other";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: needs D in {64,128}, N*D < 2^31, at most 2^31-1 workgroups, a gfx950 device";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP runtime call failed";
  }
  return "unknown fa_status";
}

__attribute__((visibility("default"))) int fa_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
