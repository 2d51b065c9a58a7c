// Router of the FastMKA layer: lambda = softmax(GELU(q W_r1) W_r2), one
// 3-vector per token over the tiers (L1, L2, L3).  MKA reading note, method
// section 2 (routing gate from the query, per token and layer).  The last
// step applies the routing variant (route_weights): the plain softmax, or
// hard top-k / a tier subset as in the abstract page's Tables 9 and 10.
#include "kernels.h"

namespace mka {

// ---------------------------------------------------------------------------
// MFMA router (bf16).  A workgroup of 4 waves takes TOK = 128 / NB tokens
// (NB = r / 32 blocks of 32 hidden units) and the whole q-width reduction:
// wave w computes the 32 x 32 block (tokens 32 (w / NB) .., hidden units
// 32 (w % NB) ..) with MFMA 32x32x16.  The q rows and W_r1 pass through LDS
// in chunks of 64 channels (128 bytes per row), three chunks in flight, each
// 16-byte piece loaded global -> LDS directly by the lane whose LDS slot it
// fills: a load instruction covers 8 whole 128-byte row segments, so every
// byte of a fetched line is used (a lane-per-token layout read 32 partial
// lines per instruction).  LDS rows are unpadded with 16-byte chunk c of row
// i at slot c ^ ((i / 2) % 8), so the 16 lanes of an operand read (16 rows,
// one chunk) fall in 16 distinct bank groups.  Then GELU, the r -> 3 layer
// and the routing variant, one thread per token.
// ---------------------------------------------------------------------------
constexpr int kRouterKC = 64;      // channels per chunk
constexpr int kRouterStages = 4;  // chunks in flight: kRouterStages - 1

__device__ __forceinline__ int router_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int NB>
__global__ __launch_bounds__(256, 2) void router_mfma_kernel(const bf16_t* __restrict__ Q, int M, int qw,
                                                          const bf16_t* __restrict__ W1,
                                                          const bf16_t* __restrict__ W2,
                                                          float* __restrict__ lam, Routing rt) {
  constexpr int R = NB * 32, TOK = 128 / NB;
  constexpr int A_BYTES = TOK * kRouterKC * 2, W_BYTES = R * kRouterKC * 2;
  constexpr int STAGE = A_BYTES + W_BYTES;
  constexpr int A_LD = A_BYTES / 1024 / 4, W_LD = W_BYTES / 1024 / 4;  // 1 KB loads per wave
  static_assert(A_LD >= 1 && W_LD >= 1 && (A_LD + W_LD) * 4096 == STAGE, "loads split over 4 waves");
  static_assert(TOK * (R + 1) * 4 <= kRouterStages * STAGE, "the hidden block fits the stages");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kRouterStages * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5, l32 = lane & 31;
  const int row0 = blockIdx.x * TOK;
  const int rb = wave / NB, jb = wave % NB;

  // Source of this lane's 16 bytes in load i of a chunk: LDS row 8 i' + lane / 8
  // (i' counts the 1 KB loads of the operand), slot lane % 8.
  // The byte count is made scalar explicitly: the clamp compiles to a vector
  // instruction, and a descriptor with a vector dword turns every load of it
  // into a loop over the lanes' distinct descriptors.
  const uint32_t q_bytes = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(static_cast<int64_t>(max(0, min(TOK, M - row0))) * qw * 2));
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + static_cast<int64_t>(row0) * qw, q_bytes);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(W1, static_cast<uint32_t>(R * qw * 2));
  uint32_t a_src[A_LD], w_src[W_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int row = 8 * (wave * A_LD + i) + (lane >> 3), slot = lane & 7;
    a_src[i] = static_cast<uint32_t>(row * qw + 8 * router_slot(row, slot)) * 2;
  }
#pragma unroll
  for (int i = 0; i < W_LD; ++i) {
    const int row = 8 * (wave * W_LD + i) + (lane >> 3), slot = lane & 7;
    w_src[i] = static_cast<uint32_t>(row * qw + 8 * router_slot(row, slot)) * 2;
  }
  auto issue = [&](int chunk) {
    unsigned char* st = smem + (chunk % kRouterStages) * STAGE;
    const uint32_t k0 = static_cast<uint32_t>(chunk * kRouterKC) * 2;
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      buffer_load_lds16(qrs, (lds_void_t*)(st + (wave * A_LD + i) * 1024), a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < W_LD; ++i)
      buffer_load_lds16(wrs, (lds_void_t*)(st + A_BYTES + (wave * W_LD + i) * 1024), w_src[i] + k0);
  };

  f32x16 acc = f32x16{};
  const int n_chunks = qw / kRouterKC;
  const int arow = 32 * rb + l32, wrow = 32 * jb + l32;
  constexpr int AHEAD = kRouterStages - 1;
#pragma unroll
  for (int c = 0; c < AHEAD; ++c)
    if (c < n_chunks) issue(c);
  for (int c = 0; c < n_chunks; ++c) {
    // chunk c has landed once at most the later chunks' loads are pending
    const int later = min(AHEAD - 1, n_chunks - 1 - c);
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(kVmcntPending<2 * (A_LD + W_LD)>());
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(kVmcntPending<A_LD + W_LD>());
    else
      __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
    __syncthreads();  // every wave's pieces of chunk c are in; chunk c - 1's reads are done
    if (c + AHEAD < n_chunks) issue(c + AHEAD);
    const unsigned char* st = smem + (c % kRouterStages) * STAGE;
    const bf16_t* As = reinterpret_cast<const bf16_t*>(st) + arow * kRouterKC;
    const bf16_t* Ws = reinterpret_cast<const bf16_t*>(st + A_BYTES) + wrow * kRouterKC;
#pragma unroll
    for (int ks = 0; ks < kRouterKC / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + 8 * router_slot(arow, 2 * ks + h));
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Ws + 8 * router_slot(wrow, 2 * ks + h));
      acc = mfma32x32x16(a, b, acc);
    }
  }
  __syncthreads();  // the stages become the hidden block
  float(*hid)[R + 1] = reinterpret_cast<float(*)[R + 1]>(smem);
#pragma unroll
  for (int r = 0; r < 16; ++r) hid[32 * rb + acc_row(r, h)][32 * jb + l32] = gelu(acc[r]);
  __syncthreads();
  if (tid < TOK && row0 + tid < M) {
    float z[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      float sum = 0.f;
      for (int n = 0; n < R; ++n) sum = fmaf(hid[tid][n], bf16_to_f32(W2[c * R + n]), sum);
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
  // (qw % 64 == 0 is validated: the chunks are whole.)
  if (r == 64)
    hipLaunchKernelGGL(router_mfma_kernel<2>, dim3((M + 63) / 64), dim3(256), 0, s, q, M, qw, w1,
                       w2, lam, rt);
  else
    hipLaunchKernelGGL(router_mfma_kernel<1>, dim3((M + 127) / 128), dim3(256), 0, s, q, M, qw,
                       w1, w2, lam, rt);
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
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
