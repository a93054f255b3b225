// Host launcher and C entry point of the attention forward (see include/fa.h).
//
// One kernel launch per call: a 1-D grid of B*H*ceil(N/128) workgroups of 256
// threads, each computing one 128-row query block of one (batch, head) — the
// outer loop over query blocks of the tiled algorithm in "Flash Attention"
// (wiki.ai-engineering.at), section "Tiling Algorithm".  Under the causal mask
// a query block only visits key tiles up to its last row, so tiles above the
// diagonal are never loaded or computed.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstring>

#include "fa.h"
#include "fa_check.h"
#include "fa_fwd_kernel.hpp"

namespace fa {
namespace {

constexpr int kMaxDevices = 64;
// 0 = not yet checked, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch[kMaxDevices];

bool device_is_gfx950(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  int v = g_arch[dev].load(std::memory_order_acquire);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(v, std::memory_order_release);
  }
  return v == 1;
}

template <typename Kern>
hipError_t launch(Kern kern, const FwdArgs& a, int threads, hipStream_t stream) {
  hipLaunchKernelGGL(kern, dim3(a.n_blocks), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

// 256 threads and 128 query rows per workgroup for both element types
hipError_t dispatch(int dtype, int D, bool causal, const FwdArgs& a, hipStream_t s) {
  if (dtype == FA_DTYPE_BF16) {
    const int t = kBF16Threads;
    if (D == 128) return causal ? launch(fa_fwd_bf16_kernel<128, true>, a, t, s)
                                : launch(fa_fwd_bf16_kernel<128, false>, a, t, s);
    return causal ? launch(fa_fwd_bf16_kernel<64, true>, a, t, s)
                  : launch(fa_fwd_bf16_kernel<64, false>, a, t, s);
  }
  const int t = kThreads;
  if (D == 128) return causal ? launch(fa_fwd_f32_kernel<128, true>, a, t, s)
                              : launch(fa_fwd_f32_kernel<128, false>, a, t, s);
  return causal ? launch(fa_fwd_f32_kernel<64, true>, a, t, s)
                : launch(fa_fwd_f32_kernel<64, false>, a, t, s);
}

}  // namespace
}  // namespace fa

extern "C" __attribute__((visibility("default"))) fa_status fa_fwd(
    const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
    int64_t N, int64_t D, int causal, float scale, fa_dtype dtype, fa_stream_t stream) {
  fa_status st = fa::check_call(q, k, v, o, lse, B, H, N, D, scale, (int)dtype);
  if (st != FA_OK) return st;

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (!fa::device_is_gfx950(dev)) return FA_ERR_UNSUPPORTED;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.n = (int)N;
  const int rows = dtype == FA_DTYPE_BF16 ? fa::kBF16Rows : fa::kBM;
  a.n_qblk = (int)((N + rows - 1) / rows);
  a.n_blocks = (int)(B * H * a.n_qblk);
  const float c = std::fabs(scale) * 1.44269504088896340736f;
  a.c = c < FLT_MIN ? FLT_MIN : c;
  a.qflip = 0u;
  if (std::signbit(scale) && scale != 0.0f)
    a.qflip = dtype == FA_DTYPE_BF16 ? 0x80008000u : 0x80000000u;

  if (fa::dispatch((int)dtype, (int)D, causal != 0, a, (hipStream_t)stream) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}
