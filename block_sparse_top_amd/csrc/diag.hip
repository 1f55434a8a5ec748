// Diagnostics, not part of the path: the matrix-core rate this device
// sustains, for reporting kernel rates against a measured peak beside the
// published one.
//
// Every wave runs `iters` rounds of kChains independent MFMA accumulations on
// register operands (no memory traffic inside the loop); the grid puts
// kWavesPerSimd waves on every SIMD of every compute unit.
#include "device_common.hpp"
#include "msa_internal.hpp"

// Written only if an accumulation hits an exact sentinel; external linkage so
// that the loop's results stay live.
__device__ float msa_diag_sink;

namespace msa {
namespace {

constexpr int kChains = 4;
constexpr int kWavesPerSimd = 2;

// FMT 0: bf16 (32x32x16); 1: fp8 e4m3 (32x32x64); 2: E2M1 x E2M1 (32x32x64,
// four-register operands, unit block scales).
template <int FMT>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  if constexpr (FMT == 2) {
    i32x8 a = {}, b = {};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = 0x23232323 + (lane & 3) * 0x01010101;  // E2M1 codes 2..6: 1 .. 4
      b[i] = 0x12121212 + (i & 3) * 0x01010101;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0, 127);
  } else if constexpr (FMT == 1) {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x30303030 + (lane & 7) * 0x01010101;  // e4m3 codes 0x30..0x37: 0.5 .. 0.9375
      b[i] = 0x28282828 + (i & 7) * 0x01010101;     // 0.25 .. 0.46875
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma32x32x64_fp8(a, b, acc[c]);
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (float)(lane + i));
      b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == 1234.5f) msa_diag_sink = s;
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_diag_mfma_rate(int32_t dtype, int32_t iters, double* tflops) {
  using namespace msa;
  if (!tflops || iters < 1 || (dtype != MSA_BF16 && dtype != MSA_FP8_E4M3 && dtype != MSA_MXFP4_QK))
    return MSA_ERR_INVALID_ARG;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return MSA_ERR_HIP;
  const int blocks = ncu * kWavesPerSimd;  // 4 waves per workgroup: one per SIMD
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  float ms = 0.f;
  if (e == hipSuccess) {
    // one warm-up launch, then the timed one
    for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
      if (rep == 1) e = hipEventRecord(e0, nullptr);
      if (e != hipSuccess) break;
      if (dtype == MSA_FP8_E4M3)
        hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(blocks), dim3(256), 0, nullptr, iters);
      else if (dtype == MSA_MXFP4_QK)
        hipLaunchKernelGGL(mfma_loop_kernel<2>, dim3(blocks), dim3(256), 0, nullptr, iters);
      else
        hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(256), 0, nullptr, iters);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess || ms <= 0.f) return MSA_ERR_HIP;
  const double per = dtype == MSA_BF16 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  const double flops = per * kChains * (double)iters * blocks * 4.0;
  *tflops = flops / (ms * 1e-3) / 1e12;
  return MSA_OK;
}
