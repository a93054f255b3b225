// Host launcher and C entry point of the attention backward (see include/fa.h).
//
// Two launches on the caller's stream: fa_bwd_dq_kernel (one workgroup per 128
// query rows: dq, and per row Delta = rowsum(dO O) and -LSE log2(e) into the
// workspace), then fa_bwd_dkdv_kernel (one workgroup per 128 keys: dk, dv),
// which reads both.  When the dq and dk/dv workgroups together fit one per
// compute unit, the two walks over the tiles can run side by side instead:
// fa_bwd_delta_kernel writes Delta and -LSE log2(e), then fa_bwd_fused_kernel
// runs the dk/dv and dq workgroups in one grid.  At D = 256 the dk/dv work
// runs on fa_bwd_dkdv16_kernel (16 keys per wave, 64 per workgroup), always
// after the dq kernel (the two bodies' tiles together exceed the LDS).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>

#include "fa.h"
#include "fa_bwd_kernel.hpp"
#include "fa_check.h"
#include "fa_device.h"

namespace fa {
namespace {

// the host's key blocks are the kernels' workgroups
static_assert(bwd_keys_per_block(128) == kBwdRows && bwd_keys_per_block(256) == 16 * (kBwdThreads / 64),
              "dk/dv keys per workgroup");

template <typename Kern>
hipError_t launch(Kern kern, const BwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBwdThreads), 0, s, a);
  return hipGetLastError();
}

// true when the dq and dk/dv grids together hold at most one workgroup per
// compute unit of the current device
bool fuse_bwd(const BwdArgs& a) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  return (int64_t)a.n_qblocks + a.n_kblocks <= cus;
}

template <typename E, int D>
hipError_t launch_fused(bool causal, const BwdArgs& a, hipStream_t s) {
  hipError_t e = launch(fa_bwd_delta_kernel<E, D>, a, a.n_qblocks, s);
  if (e != hipSuccess) return e;
  const int grid = a.n_kblocks + a.n_qblocks;
  return causal ? launch(fa_bwd_fused_kernel<E, D, true>, a, grid, s)
                : launch(fa_bwd_fused_kernel<E, D, false>, a, grid, s);
}

template <typename E, int D>
hipError_t launch_bwd_d(bool causal, const BwdArgs& a, hipStream_t s) {
  if constexpr (D != 256)
    if (fuse_bwd(a)) return launch_fused<E, D>(causal, a, s);
  const hipError_t e = causal ? launch(fa_bwd_dq_kernel<E, D, true>, a, a.n_qblocks, s)
                              : launch(fa_bwd_dq_kernel<E, D, false>, a, a.n_qblocks, s);
  if (e != hipSuccess) return e;
  if constexpr (D == 256)
    return causal ? launch(fa_bwd_dkdv16_kernel<E, D, true>, a, a.n_kblocks, s)
                  : launch(fa_bwd_dkdv16_kernel<E, D, false>, a, a.n_kblocks, s);
  else
    return causal ? launch(fa_bwd_dkdv_kernel<E, D, true>, a, a.n_kblocks, s)
                  : launch(fa_bwd_dkdv_kernel<E, D, false>, a, a.n_kblocks, s);
}

template <typename E>
hipError_t launch_bwd_typed(int D, bool causal, BwdArgs a, float scale, hipStream_t s) {
  // Q's signs (dq work) and K's (dk/dv work) carry the sign of scale (the sign
  // bit of both 16-bit types is bit 15)
  a.flip = std::signbit(scale) && scale != 0.0f ? 0x80008000u : 0u;
  if (D == 128) return launch_bwd_d<E, 128>(causal, a, s);
  if (D == 256) return launch_bwd_d<E, 256>(causal, a, s);
  if (D == 96) return launch_bwd_d<E, 96>(causal, a, s);
  return launch_bwd_d<E, 64>(causal, a, s);
}

hipError_t launch_bwd(int dtype, int D, bool causal, const BwdArgs& a, float scale, hipStream_t s) {
  return dtype == FA_DTYPE_F16 ? launch_bwd_typed<F16>(D, causal, a, scale, s)
                               : launch_bwd_typed<BF16>(D, causal, a, scale, s);
}

}  // namespace
}  // namespace fa

namespace fa {
namespace {

// The common call after validation: Nq queries and Nk keys per (b, h).
fa_status run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, void* workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                  int64_t D, int causal, float scale, fa_dtype dtype, fa_stream_t stream) {
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = (float*)workspace;
  a.nlse2 = a.delta + B * H * Nq;
  a.nq = (int)Nq;
  a.nk = (int)Nk;
  a.n_qblk = (int)((Nq + kBwdRows - 1) / kBwdRows);
  const int64_t kpb = bwd_keys_per_block(D);  // keys per dk/dv workgroup
  a.n_kblk = (int)((Nk + kpb - 1) / kpb);
  a.n_qblocks = (int)(B * H * a.n_qblk);
  a.n_kblocks = (int)(B * H * a.n_kblk);
  const float c = std::fabs(scale) * 1.44269504088896340736f;
  a.c = c < FLT_MIN ? FLT_MIN : c;
  a.scale = scale;
  a.flip = 0u;
  const hipError_t e = launch_bwd((int)dtype, (int)D, causal != 0, a, scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace
}  // namespace fa

extern "C" __attribute__((visibility("default"))) fa_status fa_bwd(
    const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
    void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t D,
    int causal, float scale, fa_dtype dtype, fa_stream_t stream) {
  fa_status st = fa::check_bwd_call(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, D,
                                    scale, (int)dtype);
  if (st != FA_OK) return st;
  if ((st = fa::device_check()) != FA_OK) return st;
  return fa::run_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, N, D, causal, scale, dtype, stream);
}

extern "C" __attribute__((visibility("default"))) fa_status fa_bwd_qk(
    const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
    void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
    int64_t D, int causal, float scale, fa_dtype dtype, fa_stream_t stream) {
  fa_status st = fa::check_bwd_qk_call(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Nq, Nk,
                                       D, causal, scale, (int)dtype);
  if (st != FA_OK) return st;
  if ((st = fa::device_check()) != FA_OK) return st;
  return fa::run_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, D, causal, scale, dtype, stream);
}
