// Measurement probes for the benchmark (not on the attention path): a clock
// stamp and a register-only MFMA loop.  They let one benchmark run report the
// shader clock the chip held while the attention kernel ran and the bf16
// matrix-core rate the chip attains in that state, beside the published peak
// (ZimaSpace, "Wie reduziert Flash Attention den Speicherverkehr während der
// lokalen Inferenz?", section "Hardware- und Formunterstützung entscheiden
// über die Verwendung des schnellen Pfads": record what the fast path
// actually reached on the hardware).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;  // 4 waves
constexpr int kProbeBlocksPerCu = 2;  // two waves per SIMD
constexpr int kProbeChains = 4;     // independent accumulators per wave

// The shader-clock counter is not one counter shared by the chip: measured,
// stamps read on different XCDs, and on different compute units of one XCD,
// are offset from each other.  A stamp is therefore taken on many compute
// units (kStampBlocks one-wave workgroups, spread over the chip by the
// dispatcher), each tagged with its XCC id and its shader engine / array /
// compute-unit ids, and two stamps are compared only where the tags match.
constexpr int kStampBlocks = FA_PROBE_STAMP_BLOCKS;

__device__ __forceinline__ uint32_t cu_tag() {
  uint32_t x, hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  // HW_ID bits 8-11 CU, 12 shader array, 13-15 shader engine
  return ((x & 0xF) << 8) | ((hw >> 8) & 0xFF);
}

__global__ void fa_probe_stamp_kernel(uint64_t* out) {
  if (threadIdx.x == 0) {
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    uint64_t* o = out + 3 * (size_t)blockIdx.x;
    o[0] = t;
    o[1] = r;
    o[2] = cu_tag();
  }
}

// iters x kProbeChains v_mfma_f32_32x32x16_bf16 per wave on independent
// accumulators, operands in registers.  Lane 0 of wave 0 of every workgroup
// records both counters before and after its loop: stamps[4 b + {0,1,2,3}] =
// {memtime, realtime} at start, then at end.
__global__ __launch_bounds__(kProbeThreads, kProbeBlocksPerCu) void fa_probe_mfma_kernel(int iters,
                                                                                      uint64_t* stamps) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * lane + 0.01f * i);
    b[i] = (__bf16)(0.5f / (i + 1));
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int r = 0; r < kProbeChains; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.0f;
  const bool rec = threadIdx.x == 0;
  uint64_t t0 = 0, r0 = 0;
  if (rec) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kProbeChains; ++r) acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[r], 0, 0, 0);
  }
  // the end stamp waits for the accumulators
#pragma unroll
  for (int r = 0; r < kProbeChains; ++r) asm volatile("" ::"v"(acc[r]));
  if (rec) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* s = stamps + 4 * (size_t)blockIdx.x;
    s[0] = t0;
    s[1] = r0;
    s[2] = t1;
    s[3] = r1;
  }
  // keeps the loop: the accumulators are finite, so nothing is written here
  float x = 0.0f;
#pragma unroll
  for (int r = 0; r < kProbeChains; ++r) x += acc[r][0];
  if (x != x) stamps[4 * (size_t)blockIdx.x] = 0;
}

int probe_blocks() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus * kProbeBlocksPerCu;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int fa_probe_stamp(uint64_t* out, fa_stream_t stream) {
  if (out == nullptr) return -1;
  hipLaunchKernelGGL(fa_probe_stamp_kernel, dim3(kStampBlocks), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

__attribute__((visibility("default"))) int fa_probe_mfma_query(int iters, int* blocks, double* flops) {
  if (blocks == nullptr || flops == nullptr || iters <= 0) return -1;
  const int n = probe_blocks();
  if (n <= 0) return -2;
  *blocks = n;
  *flops = (double)n * (kProbeThreads / 64) * iters * kProbeChains * (2.0 * 32 * 32 * 16);
  return 0;
}

__attribute__((visibility("default"))) int fa_probe_mfma(int iters, uint64_t* stamps, fa_stream_t stream) {
  if (stamps == nullptr || iters <= 0) return -1;
  const int n = probe_blocks();
  if (n <= 0) return -2;
  hipLaunchKernelGGL(fa_probe_mfma_kernel, dim3(n), dim3(kProbeThreads), 0, (hipStream_t)stream, iters, stamps);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

__attribute__((visibility("default"))) int fa_probe_wallclock_khz(int* khz) {
  if (khz == nullptr) return -1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -2;
  return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? 0 : -2;
}

}  // extern "C"
