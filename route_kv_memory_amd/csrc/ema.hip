// L2 session summary and L3 block means.
//
// L2 is the exponential moving average s_t = beta * s_{t-1} + (1 - beta) * x_t
// of the token hiddens, prefix inclusive of t.  The MKA reading note, method
// section 1, lets the session tier be either a low-rank summary or an EMA of
// the causal prefix; the EMA is the reading taken.  Block b's mean is the
// mean of x over tokens [b*Bs, (b+1)*Bs).
//
// Chunked scan, channel-parallel and coalesced: a thread owns 4 adjacent
// channels, a workgroup 512 channels of one 64-token chunk.
//   pass 1  each chunk's local result from a zero start: the EMA end value and
//           the block-sum tail (sum since the chunk's last block end);
//   pass 2  per channel, a sequential scan over chunks turns those into the
//           carry entering every chunk (EMA: s <- beta^L s + a; block sum:
//           restart at a chunk that contains a block end);
//   pass 3  each chunk rescans from its carry, writes L2, writes the mean of
//           every block that ends inside it, and the last chunk writes the
//           outgoing EMA state and partial block sum.
// A single-chunk call (decode) skips passes 1-2 and reads the carried state
// directly.
#include "kernels.h"

namespace mka {

constexpr int kEmaThreads = 128, kEmaVec = 4, kEmaSlab = kEmaThreads * kEmaVec;

template <typename T>
__global__ __launch_bounds__(kEmaThreads) void ema_pass1(const T* __restrict__ x, int seq, int D,
                                                          int64_t pos0, int block, float beta,
                                                          float omb, float* __restrict__ agg_s,
                                                          float* __restrict__ agg_a,
                                                          int n_chunks) {
  const int c = blockIdx.x, b = blockIdx.z;
  const int ch = blockIdx.y * kEmaSlab + threadIdx.x * kEmaVec;
  if (ch >= D) return;
  const int t0 = c * kEmaChunk, t1 = min(t0 + kEmaChunk, seq);
  float s[4] = {0.f, 0.f, 0.f, 0.f}, a[4] = {0.f, 0.f, 0.f, 0.f};
  const T* xp = x + (static_cast<int64_t>(b) * seq + t0) * D + ch;
  for (int t = t0; t < t1; ++t, xp += D) {
    float xv[4];
    load4(xp, xv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = fmaf(beta, s[i], omb * xv[i]);
      a[i] += xv[i];
    }
    if ((pos0 + t + 1) % block == 0) a[0] = a[1] = a[2] = a[3] = 0.f;
  }
  const int64_t o = (static_cast<int64_t>(b) * n_chunks + c) * D + ch;
  store4(agg_s + o, s);
  store4(agg_a + o, a);
}

// One thread per (batch, channel): exclusive scan of the chunk results, in place.
__global__ __launch_bounds__(256) void ema_pass2(float* __restrict__ agg_s, float* __restrict__ agg_a,
                                                 const float* __restrict__ state_in,
                                                 const float* __restrict__ acc_in, int B, int D,
                                                 int seq, int64_t pos0, int block, float beta_L,
                                                 int n_chunks) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= B * D) return;
  const int b = e / D, ch = e - b * D;
  // An empty prefix (pos0 == 0) and an empty partial block (pos0 at a block
  // start) contribute zero whatever the buffers hold.
  float cs = pos0 == 0 ? 0.f : state_in[e], ca = pos0 % block == 0 ? 0.f : acc_in[e];
  float* ps = agg_s + static_cast<int64_t>(b) * n_chunks * D + ch;
  float* pa = agg_a + static_cast<int64_t>(b) * n_chunks * D + ch;
  for (int c = 0; c < n_chunks; ++c) {
    const int64_t o = static_cast<int64_t>(c) * D;
    const float sc = ps[o], ac = pa[o];
    ps[o] = cs;
    pa[o] = ca;
    const int64_t t0 = pos0 + static_cast<int64_t>(c) * kEmaChunk;
    const int64_t t1 = pos0 + min((c + 1) * kEmaChunk, seq);
    const bool closes = (t1 / block) > (t0 / block);  // a block ends in [t0, t1)
    cs = fmaf(beta_L, cs, sc);
    ca = closes ? ac : ca + ac;
  }
}

template <typename T>
__global__ __launch_bounds__(kEmaThreads) void ema_pass3(
    const T* __restrict__ x, int seq, int D, int64_t pos0, int block, float beta, float omb,
    const float* carry_s, const float* carry_a, int carry_chunks, float* __restrict__ l2,
    float* __restrict__ means, int nb_cap, float* state_out, float* acc_out, int n_chunks) {
  const int c = blockIdx.x, b = blockIdx.z;
  const int ch = blockIdx.y * kEmaSlab + threadIdx.x * kEmaVec;
  if (ch >= D) return;
  const int t0 = c * kEmaChunk, t1 = min(t0 + kEmaChunk, seq);
  const int64_t co = carry_chunks ? (static_cast<int64_t>(b) * carry_chunks + c) * D + ch
                                  : static_cast<int64_t>(b) * D + ch;
  float s[4] = {0.f, 0.f, 0.f, 0.f}, a[4] = {0.f, 0.f, 0.f, 0.f};
  if (carry_chunks || pos0 != 0) load4(carry_s + co, s);
  if (carry_chunks || pos0 % block != 0) load4(carry_a + co, a);
  const T* xp = x + (static_cast<int64_t>(b) * seq + t0) * D + ch;
  float* lp = l2 + (static_cast<int64_t>(b) * seq + t0) * D + ch;
  for (int t = t0; t < t1; ++t, xp += D, lp += D) {
    float xv[4];
    load4(xp, xv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = fmaf(beta, s[i], omb * xv[i]);
      a[i] += xv[i];
    }
    store4(lp, s);
    const int64_t p = pos0 + t;
    if ((p + 1) % block == 0) {
      const int64_t blk = (p + 1) / block - 1;
      float m[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) m[i] = a[i] / static_cast<float>(block);
      store4(means + (static_cast<int64_t>(b) * nb_cap + blk) * D + ch, m);
      a[0] = a[1] = a[2] = a[3] = 0.f;
    }
  }
  if (c == n_chunks - 1) {
    store4(state_out + static_cast<int64_t>(b) * D + ch, s);
    store4(acc_out + static_cast<int64_t>(b) * D + ch, a);
  }
}

// ---------------------------------------------------------------------------
// Decode: one token per sequence.  A workgroup takes 128 channels of one
// sequence: EMA update (and block mean when the token closes a block), then
// the fp64 partial projections of the new L2 row onto every hyperplane over
// its channels, written to part[(slice * B + b) * 64 + j] for the retrieval's
// selection step to sum in slice order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void ema_hash_decode_kernel(
    const T* __restrict__ x, int D, int64_t pos, int block, float beta, float omb,
    float* __restrict__ state, float* __restrict__ acc, float* __restrict__ l2,
    float* __restrict__ means, int nb_cap, const float* __restrict__ P, int nbits,
    double* __restrict__ part) {
  __shared__ float Ps[64][129];
  __shared__ float Ls[128];
  __shared__ double red[2][64];
  const int tid = threadIdx.x, slice = blockIdx.x, b = blockIdx.y, B = gridDim.y;
  const int c0 = slice * 128, ch = c0 + tid;
  for (int e = tid; e < 64 * 128; e += 128) {
    const int j = e >> 7, c = e & 127;
    Ps[j][c] = (j < nbits && c0 + c < D) ? P[static_cast<int64_t>(j) * D + c0 + c] : 0.f;
  }
  float sv = 0.f;
  if (ch < D) {
    const int64_t o = static_cast<int64_t>(b) * D + ch;
    const float xv = Elem<T>::to_f32(x[o]);
    sv = fmaf(beta, pos == 0 ? 0.f : state[o], omb * xv);
    float a = (pos % block == 0 ? 0.f : acc[o]) + xv;
    state[o] = sv;
    l2[o] = sv;
    if ((pos + 1) % block == 0) {
      means[(static_cast<int64_t>(b) * nb_cap + (pos + 1) / block - 1) * D + ch] =
          a / static_cast<float>(block);
      a = 0.f;
    }
    acc[o] = a;
  }
  Ls[tid] = sv;
  __syncthreads();
  const int j = tid & 63, half = tid >> 6;
  double p = 0.0;
#pragma unroll 8
  for (int c = half * 64; c < half * 64 + 64; ++c)
    p = fma(static_cast<double>(Ls[c]), static_cast<double>(Ps[j][c]), p);
  red[half][j] = p;
  __syncthreads();
  if (tid < 64) part[(static_cast<int64_t>(slice) * B + b) * 64 + tid] = red[0][tid] + red[1][tid];
}

size_t ema_hash_decode_ws_bytes(int B, int D) {
  return sizeof(double) * static_cast<size_t>((D + 127) / 128) * B * 64;
}

template <typename T>
hipError_t ema_hash_decode(const T* x, int B, int D, int64_t pos, int block, float beta,
                           float* state, float* acc, float* l2, float* means, int nb_cap,
                           const float* proj, int nbits, double* part, hipStream_t s) {
  hipLaunchKernelGGL(ema_hash_decode_kernel<T>, dim3((D + 127) / 128, B), dim3(128), 0, s, x, D,
                     pos, block, beta, 1.0f - beta, state, acc, l2, means, nb_cap, proj, nbits,
                     part);
  return hipGetLastError();
}
template hipError_t ema_hash_decode<float>(const float*, int, int, int64_t, int, float, float*,
                                           float*, float*, float*, int, const float*, int, double*,
                                           hipStream_t);
template hipError_t ema_hash_decode<bf16_t>(const bf16_t*, int, int, int64_t, int, float, float*,
                                            float*, float*, float*, int, const float*, int,
                                            double*, hipStream_t);

size_t ema_ws_bytes(int B, int seq, int D) {
  const int n_chunks = (seq + kEmaChunk - 1) / kEmaChunk;
  if (n_chunks <= 1) return 0;
  return 2 * sizeof(float) * static_cast<size_t>(B) * n_chunks * D;
}

template <typename T>
hipError_t ema_scan(const T* x, int B, int seq, int D, int64_t pos0, int block, float beta,
                    float* state_io, float* acc_io, float* l2, float* means, int nb_cap,
                    float* ws, hipStream_t s) {
  const int n_chunks = (seq + kEmaChunk - 1) / kEmaChunk;
  const float omb = 1.0f - beta;
  const dim3 grid(n_chunks, (D + kEmaSlab - 1) / kEmaSlab, B);
  if (n_chunks == 1) {
    hipLaunchKernelGGL(ema_pass3<T>, grid, dim3(kEmaThreads), 0, s, x, seq, D, pos0, block, beta,
                       omb, state_io, acc_io, 0, l2, means, nb_cap, state_io, acc_io, n_chunks);
    return hipGetLastError();
  }
  float* agg_s = ws;
  float* agg_a = ws + static_cast<size_t>(B) * n_chunks * D;
  hipLaunchKernelGGL(ema_pass1<T>, grid, dim3(kEmaThreads), 0, s, x, seq, D, pos0, block, beta, omb,
                     agg_s, agg_a, n_chunks);
  double bl = 1.0;
  for (int i = 0; i < kEmaChunk; ++i) bl *= static_cast<double>(beta);
  hipLaunchKernelGGL(ema_pass2, dim3((B * D + 255) / 256), dim3(256), 0, s, agg_s, agg_a, state_io,
                     acc_io, B, D, seq, pos0, block, static_cast<float>(bl), n_chunks);
  hipLaunchKernelGGL(ema_pass3<T>, grid, dim3(kEmaThreads), 0, s, x, seq, D, pos0, block, beta, omb,
                     agg_s, agg_a, n_chunks, l2, means, nb_cap, state_io, acc_io, n_chunks);
  return hipGetLastError();
}

template hipError_t ema_scan<float>(const float*, int, int, int, int64_t, int, float, float*,
                                    float*, float*, float*, int, float*, hipStream_t);
template hipError_t ema_scan<bf16_t>(const bf16_t*, int, int, int, int64_t, int, float, float*,
                                     float*, float*, float*, int, float*, hipStream_t);

}  // namespace mka
