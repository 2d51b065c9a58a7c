// On-device peak probes (include/mka_probe.h): a dense bf16 MFMA loop and a
// streaming read, the measured ceilings beside the published MI355X peaks.
#include "../../include/mka.h"
#include "../../include/mka_probe.h"
#include "common.h"

namespace mka {
namespace {

constexpr int kStreamGrid = 2048;

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * static_cast<float>(lane + i));
    b[i] = static_cast<__bf16>(0.002f * static_cast<float>(lane - i));
  }
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32x32x16(a, b, c0);
    c1 = mfma32x32x16(a, b, c1);
    c2 = mfma32x32x16(a, b, c2);
    c3 = mfma32x32x16(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  s = wave_sum(s);
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_stream_kernel(const u32x4* __restrict__ src, int64_t n,
                                                           float* __restrict__ sink) {
  __shared__ float part[4];
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * 4;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x; i < n; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = min(i + 256 * u, n - 1);  // in bounds; the tail re-reads the last vector
      v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= (i + 256 * u < n) ? (v[u].x ^ v[u].y ^ v[u].z ^ v[u].w) : 0u;
  }
  const float f = wave_sum(static_cast<float>(acc & 0xFFFF));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = f;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

}  // namespace
}  // namespace mka

extern "C" {

int mka_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 24) || sink == nullptr)
    return MKA_ERR_INVALID;
  hipLaunchKernelGGL(mka::probe_mfma_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  return hipGetLastError() == hipSuccess ? MKA_OK : MKA_ERR_HIP;
}

int mka_probe_stream_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return MKA_ERR_INVALID;
  hipLaunchKernelGGL(mka::probe_stream_kernel, dim3(mka::kStreamGrid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const mka::u32x4*>(src),
                     static_cast<int64_t>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MKA_OK : MKA_ERR_HIP;
}

}  // extern "C"
