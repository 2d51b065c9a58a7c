// Route fusion: X_fused[t] = lambda1 * x_t + lambda2 * L2[t] + lambda3 * L3[t],
// with L3[t] the mean of the retrieved block means (zero when none).  MKA
// reading note, method section 3 (fuse the tiers, then project once); the
// landing page's abstract calls the variant broadcast-routed: each lambda is
// one scalar per token and tier, applied to every channel.
//
// Formed in float32 and rounded once to the storage type, which is the operand
// type of the K/V projection that follows.
#include "kernels.h"

namespace mka {

// RMAX = 0: L3 disabled (no index or block read); USE_L2 = false: L2 disabled
// (not read).  A disabled tier contributes an exact zero, as lambda = 0 with a
// zero tier value, so the sum keeps its form and no unread value enters it.
template <typename T, int RMAX, bool USE_L2>
__global__ __launch_bounds__(256) void fuse_mix_kernel(const T* __restrict__ x,
                                                       const float* __restrict__ l2,
                                                       const float* __restrict__ means, int nb_cap,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ lam, Lam3 lam_c,
                                                       int seq, int D, int R, T* __restrict__ xf) {
  const int64_t row = blockIdx.x;  // b * seq + t
  const int b = static_cast<int>(row / seq);
  const int ch = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (ch >= D) return;
  // lambda per token, or one constant vector for every token (lam == nullptr)
  const float l1w = lam ? lam[row * 3 + 0] : lam_c.v[0];
  const float l2w = lam ? lam[row * 3 + 1] : lam_c.v[1];
  const float l3w = lam ? lam[row * 3 + 2] : lam_c.v[2];
  float xv[4], sv[4] = {0.f, 0.f, 0.f, 0.f}, mean[4] = {0.f, 0.f, 0.f, 0.f};
  load4(x + row * D + ch, xv);
  if constexpr (USE_L2) load4(l2 + row * D + ch, sv);
  if constexpr (RMAX > 0) {
    const int32_t* sel = idx + row * R;
    const float* mb = means + static_cast<int64_t>(b) * nb_cap * D + ch;
    int blk[RMAX];
#pragma unroll
    for (int i = 0; i < RMAX; ++i) blk[i] = i < R ? sel[i] : -1;
    // Every retrieved row is loaded unconditionally (unfilled slots read block
    // 0 and are not added), so the loads are in flight together; rank order.
    float m[RMAX][4];
#pragma unroll
    for (int i = 0; i < RMAX; ++i) load4(mb + static_cast<int64_t>(max(blk[i], 0)) * D, m[i]);
    float l3[4] = {0.f, 0.f, 0.f, 0.f};
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
      const bool on = blk[i] >= 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) l3[k] += on ? m[i][k] : 0.f;
      cnt += on;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) mean[k] = cnt ? l3[k] / static_cast<float>(cnt) : 0.f;
  }
  float out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = l1w * xv[k] + l2w * sv[k] + l3w * mean[k];
  store4(xf + row * D + ch, out);
}

template <typename T, bool USE_L2>
hipError_t fuse_mix_launch(dim3 grid, int threads, const T* x, const float* l2,
                           const float* means, int nb_cap, const int32_t* idx, const float* lam,
                           Lam3 lam_c, int seq, int D, int R, bool use_l3, T* xf, hipStream_t s) {
  if (!use_l3)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 0, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else if (R <= 4)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 4, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else if (R <= 8)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 8, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else if (R <= 16)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 16, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else
    hipLaunchKernelGGL((fuse_mix_kernel<T, 32, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  return hipGetLastError();
}

template <typename T>
hipError_t fuse_mix(const T* x, const float* l2, const float* means, int nb_cap,
                    const int32_t* idx, const float* lam, int B, int seq, int D, int R,
                    Routing rt, T* xf, hipStream_t s) {
  // Few tokens: narrow workgroups so that many of them share the row.
  const int threads = static_cast<int64_t>(B) * seq <= 8 ? 64 : 256;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * seq),
                  (D + 4 * threads - 1) / (4 * threads));
  if (rt.l2())
    return fuse_mix_launch<T, true>(grid, threads, x, l2, means, nb_cap, idx, lam, Lam3{}, seq, D,
                                    R, rt.l3(), xf, s);
  return fuse_mix_launch<T, false>(grid, threads, x, l2, means, nb_cap, idx, lam, Lam3{}, seq, D,
                                   R, rt.l3(), xf, s);
}

template <typename T>
hipError_t tier_rows(const T* x, const float* l2, const float* means, int nb_cap,
                     const int32_t* idx, int tier, int B, int seq, int D, int R, T* out,
                     hipStream_t s) {
  const int threads = static_cast<int64_t>(B) * seq <= 8 ? 64 : 256;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * seq),
                  (D + 4 * threads - 1) / (4 * threads));
  Lam3 c{};
  c.v[tier] = 1.0f;
  if (tier == 1)  // L2 alone: no L3 read
    return fuse_mix_launch<T, true>(grid, threads, x, l2, means, nb_cap, idx, nullptr, c, seq, D,
                                    R, false, out, s);
  return fuse_mix_launch<T, false>(grid, threads, x, l2, means, nb_cap, idx, nullptr, c, seq, D, R,
                                   tier == 2, out, s);
}

// ---------------------------------------------------------------------------
// Full MKA's mixture of its attention paths: o = sum_l lambda_l a_l per token,
// lambda broadcast over heads and head dimensions (MKA reading note, method
// section 2).  Paths given as null are disabled tiers and are not read.
// Formed in float32 from the stored path outputs, rounded once.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void mix_paths_kernel(const T* __restrict__ a0,
                                                        const T* __restrict__ a1,
                                                        const T* __restrict__ a2,
                                                        const float* __restrict__ lam, int64_t M,
                                                        int HD, T* __restrict__ o) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= M * HD) return;
  const int64_t row = e / HD;
  const float w0 = lam[row * 3 + 0], w1 = lam[row * 3 + 1], w2 = lam[row * 3 + 2];
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, v[4];
  if (a0) {
    load4(a0 + e, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += w0 * v[k];
  }
  if (a1) {
    load4(a1 + e, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += w1 * v[k];
  }
  if (a2) {
    load4(a2 + e, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += w2 * v[k];
  }
  store4(o + e, acc);
}

template <typename T>
hipError_t mix_paths(const T* a0, const T* a1, const T* a2, const float* lam, int64_t M, int HD,
                     T* o, hipStream_t s) {
  const int64_t n4 = (M * HD + 3) / 4;
  hipLaunchKernelGGL(mix_paths_kernel<T>, dim3(static_cast<unsigned>((n4 + 255) / 256)),
                     dim3(256), 0, s, a0, a1, a2, lam, M, HD, o);
  return hipGetLastError();
}

template hipError_t tier_rows<float>(const float*, const float*, const float*, int,
                                     const int32_t*, int, int, int, int, int, float*, hipStream_t);
template hipError_t tier_rows<bf16_t>(const bf16_t*, const float*, const float*, int,
                                      const int32_t*, int, int, int, int, int, bf16_t*,
                                      hipStream_t);
template hipError_t mix_paths<float>(const float*, const float*, const float*, const float*,
                                     int64_t, int, float*, hipStream_t);
template hipError_t mix_paths<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, const float*,
                                      int64_t, int, bf16_t*, hipStream_t);

template hipError_t fuse_mix<float>(const float*, const float*, const float*, int, const int32_t*,
                                    const float*, int, int, int, int, Routing, float*,
                                    hipStream_t);
template hipError_t fuse_mix<bf16_t>(const bf16_t*, const float*, const float*, int,
                                     const int32_t*, const float*, int, int, int, int, Routing,
                                     bf16_t*, hipStream_t);

}  // namespace mka
