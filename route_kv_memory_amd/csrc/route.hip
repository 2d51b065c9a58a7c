// Router of the FastMKA layer: lambda = softmax(GELU(q W_r1) W_r2), one
// 3-vector per token over the tiers (L1, L2, L3).  MKA reading note, method
// section 2 (routing gate from the query, per token and layer).  The last
// step applies the routing variant (route_weights): the plain softmax, or
// hard top-k / a tier subset as in the abstract page's Tables 9 and 10.
#include "kernels.h"

namespace mka {

// ---------------------------------------------------------------------------
// MFMA router (bf16): a workgroup takes 32 tokens; its NW waves (8 when the
// q width splits into slices of whole 16-wide k-steps, else 4) split the
// q-width reduction, each producing a 32 x r block of hidden pre-activations
// with MFMA 32x32x16 (operands read straight from global: the token's q row
// and the weight row are both contiguous along the reduction).  The slices
// are summed in LDS, GELU applied, then the r -> 3 layer and the softmax run
// one thread per token.
// ---------------------------------------------------------------------------
template <int NB, int NW>  // NB = r / 32 output blocks
__global__ __launch_bounds__(NW * 64) void router_mfma_kernel(const bf16_t* __restrict__ Q, int M, int qw,
                                                          const bf16_t* __restrict__ W1,
                                                          const bf16_t* __restrict__ W2,
                                                          float* __restrict__ lam, Routing rt) {
  constexpr int R = NB * 32;
  __shared__ float part[NW][32][R + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int row0 = blockIdx.x * 32;
  const int row = row0 + l32;
  const int slice = qw / NW;
  const int k_begin = wave * slice;

  f32x16 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x16{};
  const bf16_t* qrow = Q + static_cast<int64_t>(row < M ? row : 0) * qw + 8 * h;
  // U k-steps' loads are issued before their products; steps past the
  // slice re-read its last step (inside the row) and enter as zeros.
  constexpr int U = 32 / NW;
  const int k_end = k_begin + slice;
  for (int k = k_begin; k < k_end; k += 16 * U) {
    bf16x8 a[U], b[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(k + 16 * u, k_end - 16);
      a[u] = *reinterpret_cast<const bf16x8*>(qrow + kk);
      if (row >= M || k + 16 * u >= k_end) a[u] = bf16x8{};
#pragma unroll
      for (int j = 0; j < NB; ++j)
        b[u][j] = *reinterpret_cast<const bf16x8*>(W1 + static_cast<int64_t>(j * 32 + l32) * qw +
                                                   kk + 8 * h);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = mfma32x32x16(a[u], b[u][j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave][acc_row(r, h)][j * 32 + l32] = acc[j][r];
  __syncthreads();
  for (int e = tid; e < 32 * R; e += NW * 64) {
    const int rr = e / R, n = e % R;
    float z = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) z += part[w][rr][n];
    part[0][rr][n] = gelu(z);
  }
  __syncthreads();
  if (tid < 32 && row0 + tid < M) {
    float z[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      float sum = 0.f;
      for (int n = 0; n < R; ++n) sum = fmaf(part[0][tid][n], bf16_to_f32(W2[c * R + n]), sum);
      z[c] = sum;
    }
    float out[3];
    route_weights(z, rt, out);
    float* dst = lam + static_cast<int64_t>(row0 + tid) * 3;
    dst[0] = out[0];
    dst[1] = out[1];
    dst[2] = out[2];
  }
}

hipError_t router_bf16_mfma(const bf16_t* q, int M, int qw, const bf16_t* w1, int r,
                            const bf16_t* w2, float* lam, Routing rt, hipStream_t s) {
  const dim3 grid((M + 31) / 32);
  auto launch = [&](auto kernel, int nw) {
    hipLaunchKernelGGL(kernel, grid, dim3(nw * 64), 0, s, q, M, qw, w1, w2, lam, rt);
  };
  // (qw % 64 == 0 is validated: slices of qw/4 are whole k-steps.)
  if (qw % 128 == 0)
    r == 64 ? launch(router_mfma_kernel<2, 8>, 8) : launch(router_mfma_kernel<1, 8>, 8);
  else
    r == 64 ? launch(router_mfma_kernel<2, 4>, 4) : launch(router_mfma_kernel<1, 4>, 4);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row-wise router: one workgroup per token.  Hidden unit n is a dot product
// computed by one wave (lanes stride the q width), GELU, then thread 0 forms
// the three logits and the softmax.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void router_rowwise_kernel(const T* __restrict__ Q, int qw,
                                                             const T* __restrict__ W1, int r,
                                                             const T* __restrict__ W2,
                                                             float* __restrict__ lam, Routing rt) {
  __shared__ float hid[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const T* q = Q + row * qw;
  constexpr int V = Vec16<T>::kN;
  const int kv = (qw / V) * V;
  for (int n = wave; n < r; n += 4) {
    const T* w = W1 + static_cast<int64_t>(n) * qw;
    float acc = 0.f;
    for (int k = lane * V; k < kv; k += 64 * V) {
      float a[V], b[V];
      Vec16<T>::load(q + k, a);
      Vec16<T>::load(w + k, b);
#pragma unroll
      for (int i = 0; i < V; ++i) acc = fmaf(a[i], b[i], acc);
    }
    for (int k = kv + lane; k < qw; k += 64) acc = fmaf(Elem<T>::to_f32(q[k]), Elem<T>::to_f32(w[k]), acc);
    acc = wave_sum(acc);
    if (lane == 0) hid[n] = gelu(acc);
  }
  __syncthreads();
  if (tid == 0) {
    float z[3];
    for (int c = 0; c < 3; ++c) {
      float sum = 0.f;
      for (int n = 0; n < r; ++n) sum = fmaf(hid[n], Elem<T>::to_f32(W2[c * r + n]), sum);
      z[c] = sum;
    }
    float out[3];
    route_weights(z, rt, out);
    lam[row * 3 + 0] = out[0];
    lam[row * 3 + 1] = out[1];
    lam[row * 3 + 2] = out[2];
  }
}

template <typename T>
hipError_t router_rowwise(const T* q, int M, int qw, const T* w1, int r, const T* w2, float* lam,
                          Routing rt, hipStream_t s) {
  hipLaunchKernelGGL(router_rowwise_kernel<T>, dim3(M), dim3(256), 0, s, q, qw, w1, r, w2, lam, rt);
  return hipGetLastError();
}

// Second router layer and softmax for few tokens, from the hidden layer that
// a small-M product (one wave per hidden unit) left in ``hidden`` [M, r].
template <typename T>
__global__ __launch_bounds__(64) void router_head_kernel(const float* __restrict__ hidden, int r,
                                                         const T* __restrict__ W2,
                                                         float* __restrict__ lam, Routing rt) {
  const int lane = threadIdx.x, row = blockIdx.x;
  float z[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    float sum = 0.f;
    for (int n = lane; n < r; n += 64) sum = fmaf(hidden[static_cast<int64_t>(row) * r + n], Elem<T>::to_f32(W2[c * r + n]), sum);
    z[c] = wave_sum(sum);
  }
  if (lane == 0) {
    float out[3];
    route_weights(z, rt, out);
    lam[static_cast<int64_t>(row) * 3 + 0] = out[0];
    lam[static_cast<int64_t>(row) * 3 + 1] = out[1];
    lam[static_cast<int64_t>(row) * 3 + 2] = out[2];
  }
}

template <typename T>
hipError_t router_head(const float* hidden, int M, int r, const T* w2, float* lam, Routing rt,
                       hipStream_t s) {
  hipLaunchKernelGGL(router_head_kernel<T>, dim3(M), dim3(64), 0, s, hidden, r, w2, lam, rt);
  return hipGetLastError();
}
template hipError_t router_head<float>(const float*, int, int, const float*, float*, Routing,
                                       hipStream_t);
template hipError_t router_head<bf16_t>(const float*, int, int, const bf16_t*, float*, Routing,
                                        hipStream_t);

template hipError_t router_rowwise<float>(const float*, int, int, const float*, int, const float*,
                                          float*, Routing, hipStream_t);
template hipError_t router_rowwise<bf16_t>(const bf16_t*, int, int, const bf16_t*, int,
                                           const bf16_t*, float*, Routing, hipStream_t);

// lambda of the variants that do not use the router (fixed weights, or L1
// alone): the same 3-vector for every token.
__global__ __launch_bounds__(256) void lambda_fixed_kernel(float* __restrict__ lam, int M,
                                                           Routing rt) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < 3 * M) lam[e] = rt.fixed_weight(e % 3);
}

hipError_t lambda_fixed(float* lam, int M, Routing rt, hipStream_t s) {
  hipLaunchKernelGGL(lambda_fixed_kernel, dim3((3 * M + 255) / 256), dim3(256), 0, s, lam, M, rt);
  return hipGetLastError();
}

}  // namespace mka
