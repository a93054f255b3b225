// Host launcher and C entry points of the FP8 attention forward (see include/fa.h).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>

#include "fa.h"
#include "fa_check.h"
#include "fa_device.h"
#include "fa_fp8_kernel.hpp"
#include "fa_fp8_rows16_kernel.hpp"

namespace fa {
namespace {

template <typename Kern>
hipError_t launch(Kern kern, const Fp8Args& a, hipStream_t s, int threads = kFp8Threads) {
  hipLaunchKernelGGL(kern, dim3(a.n_blocks), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace fa

extern "C" {

__attribute__((visibility("default"))) fa_status fa_fwd_fp8_query(int64_t B, int64_t H, int64_t N, int64_t D,
                                                                   int causal, fa_sizes* out) {
  (void)causal;
  if (!out) return FA_ERR_NULL_POINTER;
  return fa::check_fp8_shape(B, H, N, D, out);
}

__attribute__((visibility("default"))) fa_status fa_fwd_fp8(const void* q, const void* q_scale, const void* k,
                                                            const void* k_scale, const void* v, const void* v_scale,
                                                            void* o, float* lse, int64_t B, int64_t H, int64_t N,
                                                            int64_t D, int causal, float scale, fa_stream_t stream) {
  fa_status st = fa::check_fp8_call(q, q_scale, k, k_scale, v, v_scale, o, lse, B, H, N, D, scale);
  if (st != FA_OK) return st;
  if ((st = fa::device_check()) != FA_OK) return st;
  fa::Fp8Args a;
  a.q = (const uint8_t*)q;
  a.qs = (const uint8_t*)q_scale;
  a.k = (const uint8_t*)k;
  a.ks = (const uint8_t*)k_scale;
  a.v = (const uint8_t*)v;
  a.vs = (const uint8_t*)v_scale;
  a.o = o;
  a.lse = lse;
  a.n = (int)N;
  a.n_qblk = (int)((N + fa::kFp8Rows - 1) / fa::kFp8Rows);
  a.n_blocks = (int)(B * H * a.n_qblk);
  const float c = std::fabs(scale) * 1.44269504088896340736f;
  a.c = c < FLT_MIN ? FLT_MIN : c;
  a.qflip = std::signbit(scale) && scale != 0.0f ? 0x80808080u : 0u;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  // D = 256: 16 query rows per wave, two waves per SIMD (the same 128-row blocks)
  if (D == 256) e = causal ? fa::launch(fa::fa_fwd_fp8_rows16_kernel<true>, a, s, 512)
                           : fa::launch(fa::fa_fwd_fp8_rows16_kernel<false>, a, s, 512);
  else if (D == 128) e = causal ? fa::launch(fa::fa_fwd_fp8_kernel<128, true>, a, s) : fa::launch(fa::fa_fwd_fp8_kernel<128, false>, a, s);
  else e = causal ? fa::launch(fa::fa_fwd_fp8_kernel<64, true>, a, s) : fa::launch(fa::fa_fwd_fp8_kernel<64, false>, a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
