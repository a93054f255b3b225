// Host launchers and C entry points of the attention forward (see include/fa.h).
//
// fa_fwd: one kernel launch, a 1-D grid of B*H*ceil(N/128) workgroups of 256
// threads, each computing one 128-row query block of one (batch, head) — the
// outer loop over query blocks of the tiled algorithm in "Flash Attention"
// (wiki.ai-engineering.at), section "Tiling Algorithm".  Under the causal mask
// a query block only visits key tiles up to its last row, so tiles above the
// diagonal are never loaded or computed.
//
// fa_fwd_split: the same kernel with the key tiles of each query block divided
// into n_splits contiguous ranges (one workgroup each, writing fp32 partial
// results to the caller's workspace), then a merge kernel on the same stream;
// with one range, a single launch writing O and LSE.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_check.h"
#include "fa_device.h"
#include "fa_decode_kernel.hpp"
#include "fa_fwd_kernel.hpp"
#include "fa_fwd_rows16_kernel.hpp"

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
hipError_t launch(Kern kern, int blocks, const FwdArgs& a, int threads, hipStream_t stream) {
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

// 16-bit (bf16 or fp16) attention kernel for (D, causal, split); 256 threads,
// 128 query rows
template <bool SPLIT>
hipError_t launch_h16(int dtype, int D, bool causal, const FwdArgs& a, hipStream_t s) {
  const int t = kBF16Threads, n = a.n_blocks;
  if (dtype == FA_DTYPE_F16) {
    if (D == 256) return causal ? launch(fa_fwd_f16_kernel<256, true, SPLIT>, n, a, t, s)
                                : launch(fa_fwd_f16_kernel<256, false, SPLIT>, n, a, t, s);
    if (D == 96) return causal ? launch(fa_fwd_f16_kernel<96, true, SPLIT>, n, a, t, s)
                               : launch(fa_fwd_f16_kernel<96, false, SPLIT>, n, a, t, s);
    if (D == 128) return causal ? launch(fa_fwd_f16_kernel<128, true, SPLIT>, n, a, t, s)
                                : launch(fa_fwd_f16_kernel<128, false, SPLIT>, n, a, t, s);
    return causal ? launch(fa_fwd_f16_kernel<64, true, SPLIT>, n, a, t, s)
                  : launch(fa_fwd_f16_kernel<64, false, SPLIT>, n, a, t, s);
  }
  if (D == 256) return causal ? launch(fa_fwd_bf16_kernel<256, true, SPLIT>, n, a, t, s)
                              : launch(fa_fwd_bf16_kernel<256, false, SPLIT>, n, a, t, s);
  if (D == 96) return causal ? launch(fa_fwd_bf16_kernel<96, true, SPLIT>, n, a, t, s)
                             : launch(fa_fwd_bf16_kernel<96, false, SPLIT>, n, a, t, s);
  if (D == 128) return causal ? launch(fa_fwd_bf16_kernel<128, true, SPLIT>, n, a, t, s)
                              : launch(fa_fwd_bf16_kernel<128, false, SPLIT>, n, a, t, s);
  return causal ? launch(fa_fwd_bf16_kernel<64, true, SPLIT>, n, a, t, s)
                : launch(fa_fwd_bf16_kernel<64, false, SPLIT>, n, a, t, s);
}

// Compute units of the current device, looked up once per device (0 if the
// lookup fails).
std::atomic<int> g_cus[kMaxDevices];
int cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_cus[dev].load(std::memory_order_acquire);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cus[dev].store(n, std::memory_order_release);
  }
  return n;
}

// Whether a one-range 16-bit launch goes to the 16-row-wave kernel: when its
// 128-row grid (a, made for 128 rows) holds at most one workgroup per compute
// unit.  There a wave's time per tile sets the kernel's, and halving a wave's
// rows per tile wins; on larger grids the 128-row kernel's larger MFMA tiles
// read LDS half as often per query and win (except at D = 256, below).
bool use_rows16(int dtype, const FwdArgs& a) {
  return dtype != FA_DTYPE_F32 && a.n_split == 1 && a.n_blocks <= cu_count();
}

// The 16-row-wave kernel for arguments made for 128-row blocks: 64-row blocks
// of the same rows, KS waves per 16-row slice.
template <int D, int KS>
hipError_t launch_rows16(int dtype, bool causal, FwdArgs a, hipStream_t s) {
  a.n_qblk = (a.nq + kRows16Rows - 1) / kRows16Rows;
  a.n_blocks = a.n_bh * a.n_qblk;
  const int t = 256 * KS, n = a.n_blocks;
  if (dtype == FA_DTYPE_F16)
    return causal ? launch(fa_fwd_f16_rows16_kernel<D, true, KS>, n, a, t, s)
                  : launch(fa_fwd_f16_rows16_kernel<D, false, KS>, n, a, t, s);
  return causal ? launch(fa_fwd_bf16_rows16_kernel<D, true, KS>, n, a, t, s)
                : launch(fa_fwd_bf16_rows16_kernel<D, false, KS>, n, a, t, s);
}

// The 16-row-wave kernel in 128-row workgroups of 8 waves, for D = 256 on
// grids larger than the small-grid form's; the arguments are the 128-row
// kernel's (same blocks and order).
hipError_t launch_rows16x8(int dtype, bool causal, const FwdArgs& a, hipStream_t s) {
  const int t = 512, n = a.n_blocks;
  if (dtype == FA_DTYPE_F16)
    return causal ? launch(fa_fwd_f16_rows16x8_kernel<256, true>, n, a, t, s)
                  : launch(fa_fwd_f16_rows16x8_kernel<256, false>, n, a, t, s);
  return causal ? launch(fa_fwd_bf16_rows16x8_kernel<256, true>, n, a, t, s)
                : launch(fa_fwd_bf16_rows16x8_kernel<256, false>, n, a, t, s);
}

// One-range 16-bit launch: on small grids the 16-row-wave kernel in 64-row
// workgroups; on larger ones the 128-row kernel, or at D = 256 the 16-row-wave
// kernel in 128-row workgroups.  At D = 64, 96 and 128 the small-grid kernel
// runs two waves per slice when its 64-row grid fits one workgroup per CU
// (8 waves, one workgroup per CU) and one wave per slice when it needs two
// per CU.  At D = 256 its 128 KB of tiles allow one workgroup per CU either
// way, and two waves per slice (two per SIMD) are always the faster.
hipError_t launch_h16_one(int dtype, int D, bool causal, const FwdArgs& a, hipStream_t s) {
  if (use_rows16(dtype, a)) {
    if (D == 256) return launch_rows16<256, 2>(dtype, causal, a, s);
    const bool two = a.n_bh * ((a.nq + kRows16Rows - 1) / kRows16Rows) <= cu_count();
    if (D == 64) return two ? launch_rows16<64, 2>(dtype, causal, a, s) : launch_rows16<64, 1>(dtype, causal, a, s);
    if (D == 96) return two ? launch_rows16<96, 2>(dtype, causal, a, s) : launch_rows16<96, 1>(dtype, causal, a, s);
    return two ? launch_rows16<128, 2>(dtype, causal, a, s) : launch_rows16<128, 1>(dtype, causal, a, s);
  }
  if (D == 256) return launch_rows16x8(dtype, causal, a, s);
  return launch_h16<false>(dtype, D, causal, a, s);
}

// fp32 attention kernel; 256 threads and 128 query rows per workgroup
hipError_t launch_f32(int D, bool causal, const FwdArgs& a, hipStream_t s) {
  const int t = kThreads, n = a.n_blocks;
  if (D == 128) return causal ? launch(fa_fwd_f32_kernel<128, true>, n, a, t, s)
                              : launch(fa_fwd_f32_kernel<128, false>, n, a, t, s);
  return causal ? launch(fa_fwd_f32_kernel<64, true>, n, a, t, s)
                : launch(fa_fwd_f32_kernel<64, false>, n, a, t, s);
}

// merge of the key ranges: one lane group per output row
hipError_t launch_combine(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  const long long rows = (long long)a.n_bh * a.nq;
  const int per_block = kCombineThreads / (D / 8);
  const int blocks = (int)((rows + per_block - 1) / per_block);
  if (dtype == FA_DTYPE_F16)
    return D == 256   ? launch(fa_combine_f16_kernel<256>, blocks, a, kCombineThreads, s)
           : D == 128 ? launch(fa_combine_f16_kernel<128>, blocks, a, kCombineThreads, s)
           : D == 96  ? launch(fa_combine_f16_kernel<96>, blocks, a, kCombineThreads, s)
                      : launch(fa_combine_f16_kernel<64>, blocks, a, kCombineThreads, s);
  if (D == 256) return launch(fa_combine_kernel<256>, blocks, a, kCombineThreads, s);
  if (D == 96) return launch(fa_combine_kernel<96>, blocks, a, kCombineThreads, s);
  if (D == 128) return launch(fa_combine_kernel<128>, blocks, a, kCombineThreads, s);
  return launch(fa_combine_kernel<64>, blocks, a, kCombineThreads, s);
}

// one query row per (b, h): the vector-unit key-range kernel
hipError_t launch_decode(int dtype, int D, const FwdArgs& a, hipStream_t s) {
  const int n = a.n_bh * a.n_split, t = kDecodeThreads;
  if (dtype == FA_DTYPE_F16)
    return D == 256   ? launch(fa_decode_kernel<F16, 256>, n, a, t, s)
           : D == 128 ? launch(fa_decode_kernel<F16, 128>, n, a, t, s)
                      : launch(fa_decode_kernel<F16, 64>, n, a, t, s);
  return D == 256   ? launch(fa_decode_kernel<BF16, 256>, n, a, t, s)
         : D == 128 ? launch(fa_decode_kernel<BF16, 128>, n, a, t, s)
                    : launch(fa_decode_kernel<BF16, 64>, n, a, t, s);
}

// Arguments shared by both entry points.  scale: |scale| log2(e) for exp2, the
// sign applied to Q's bits.
FwdArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                  int64_t Nq, int64_t Nk, float scale, int dtype, int rows, int splits) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.nq = (int)Nq;
  a.nk = (int)Nk;
  a.n_bh = (int)(B * H);
  a.n_qblk = (int)((Nq + rows - 1) / rows);
  a.n_split = splits;
  a.n_blocks = (int)(B * H * a.n_qblk * splits);
  const float c = std::fabs(scale) * 1.44269504088896340736f;
  a.c = c < FLT_MIN ? FLT_MIN : c;
  a.qflip = 0u;
  if (std::signbit(scale) && scale != 0.0f) a.qflip = dtype == FA_DTYPE_F32 ? 0x80000000u : 0x80008000u;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  return a;
}

// Scratch of fa_fwd_split_static: the key ranges' partial rows live here
// instead of in a caller workspace.  Each device the library runs on holds its
// own copy for the life of the process.  In host code `scratch` names a host
// stand-in, not device memory: kernels get the address hipGetSymbolAddress
// returns for the current device (scratch_ptr), never the array's name.
static __device__ __align__(256) unsigned char scratch[FA_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
fa_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FA_OK;
}

}  // namespace

fa_status device_check() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (!device_is_gfx950(dev)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace fa

extern "C" __attribute__((visibility("default"))) fa_status fa_fwd(
    const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
    int64_t N, int64_t D, int causal, float scale, fa_dtype dtype, fa_stream_t stream) {
  fa_status st = fa::check_call(q, k, v, o, lse, B, H, N, D, scale, (int)dtype);
  if (st != FA_OK) return st;
  if ((st = fa::device_check()) != FA_OK) return st;

  const bool h16 = dtype != FA_DTYPE_F32;
  const fa::FwdArgs a =
      fa::make_args(q, k, v, o, lse, B, H, N, N, scale, (int)dtype, h16 ? fa::kBF16Rows : fa::kBM, 1);
  const hipStream_t s = (hipStream_t)stream;
  const hipError_t e = h16 ? fa::launch_h16_one((int)dtype, (int)D, causal != 0, a, s)
                           : fa::launch_f32((int)D, causal != 0, a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" __attribute__((visibility("default"))) fa_status fa_fwd_split(
    const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
    size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
    float scale, int n_splits, fa_dtype dtype, fa_stream_t stream) {
  int splits = 1;
  fa_status st = fa::check_split_call(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, D,
                                      causal, scale, n_splits, (int)dtype, &splits);
  if (st != FA_OK) return st;
  if ((st = fa::device_check()) != FA_OK) return st;

  fa::FwdArgs a = fa::make_args(q, k, v, o, lse, B, H, Nq, Nk, scale, (int)dtype, fa::kBF16Rows, splits);
  const hipStream_t s = (hipStream_t)stream;
  if (fa::uses_decode_kernel(Nq, D)) {
    // one query row: every key is visible to it, with or without the causal mask
    if (splits > 1) {
      a.o_part = (float*)workspace;
      a.lse_part = a.o_part + (size_t)splits * a.n_bh * a.nq * D;
    }
    if (fa::launch_decode((int)dtype, (int)D, a, s) != hipSuccess) return FA_ERR_HIP;
    if (splits == 1) return FA_OK;
    return fa::launch_combine((int)dtype, (int)D, a, s) == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  if (splits == 1)
    return fa::launch_h16_one((int)dtype, (int)D, causal != 0, a, s) == hipSuccess ? FA_OK : FA_ERR_HIP;
  // workspace: [splits][B*H][Nq][D] float outputs, then [splits][B*H][Nq] log-sum-exps
  a.o_part = (float*)workspace;
  a.lse_part = a.o_part + (size_t)splits * a.n_bh * a.nq * D;
  if (fa::launch_h16<true>((int)dtype, (int)D, causal != 0, a, s) != hipSuccess) return FA_ERR_HIP;
  return fa::launch_combine((int)dtype, (int)D, a, s) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" __attribute__((visibility("default"))) fa_status fa_fwd_split_static(
    const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t Nq,
    int64_t Nk, int64_t D, int causal, float scale, int n_splits, fa_dtype dtype, fa_stream_t stream) {
  // host validation first, in fa_fwd_split's order, then the scratch limit
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  fa_sizes sz;
  int splits = 1;
  fa_status st = fa::check_split_shape(B, H, Nq, Nk, D, causal, n_splits, (int)dtype, &sz, &splits);
  if (st != FA_OK && st != FA_ERR_UNSUPPORTED) return st;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (st == FA_ERR_UNSUPPORTED) return st;
  if (sz.workspace_bytes > FA_STATIC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  if ((st = fa::device_check()) != FA_OK) return st;
  void* ws = nullptr;
  if (sz.workspace_bytes > 0 && (st = fa::scratch_ptr(&ws)) != FA_OK) return st;
  // the same kernels as fa_fwd_split; every partial row and log-sum-exp the
  // merge reads is written by the range kernel first, so nothing is cleared
  return fa_fwd_split(q, k, v, o, lse, ws, sz.workspace_bytes, B, H, Nq, Nk, D, causal, scale, n_splits, dtype,
                      stream);
}
