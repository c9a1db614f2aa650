// MFMA-only throughput probe: a measurement aid for the prefill's roofline, not part of the
// attention method. Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on register
// operands (four independent accumulators, so the matrix core never waits for a result)
// with no memory traffic in the loop; the rate it reaches on a given box and clock is the
// practical ceiling of the dense bf16 contractions the attention kernels issue.
#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;  // 4 waves per workgroup

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(lane + 3 * e + 1));
    b[e] = (__bf16)(1e-3f * (float)(2 * lane - e + 7));
  }
  f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;  // keeps the MFMAs alive
}

}  // namespace
}  // namespace fa

extern "C" fa_status fa_probe_mfma(float* sink, size_t sink_bytes, int blocks, int iters,
                                   void* stream) {
  if (!sink) return FA_ERR_NULL;
  if (blocks < 1 || iters < 1) return FA_ERR_SHAPE;
  if (sink_bytes < (size_t)blocks * fa::kProbeThreads * sizeof(float)) return FA_ERR_WORKSPACE;
  if (((uintptr_t)sink & 3u) != 0) return FA_ERR_ALIGN;
  (void)hipGetLastError();
  hipLaunchKernelGGL(fa::mfma_probe_kernel, dim3(blocks), dim3(fa::kProbeThreads), 0,
                     (hipStream_t)stream, sink, iters);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
