// L2 session summary and L3 block means.
//
// L2 is the exponential moving average s_t = beta * s_{t-1} + (1 - beta) * x_t
// of the token hiddens, prefix inclusive of t.  The MKA reading note, method
// section 1, lets the session tier be either a low-rank summary or an EMA of
// the causal prefix; the EMA is the reading taken.  Block b's mean is the
// mean of x over tokens [b*Bs, (b+1)*Bs).
//
// Chunked scan, channel-parallel and coalesced: a thread owns 4 adjacent
// channels (8 in pass 1), a workgroup 512 (1024) channels of one 64-token chunk.
//   pass 1  each chunk's local result from a zero start: the EMA end value and
//           the block-sum tail (sum since the chunk's last block end);
//   pass 2  per channel, a scan over chunks (two levels: segments of
//           chunks, then the segments) turns those into the carry entering
//           every chunk (EMA: s <- beta^L s + a; block sum: restart at a
//           chunk that contains a block end);
//   pass 3  each chunk rescans from its carry, writes L2, writes the mean of
//           every block that ends inside it, and the last chunk writes the
//           outgoing EMA state and partial block sum.
// A single-chunk call (decode) skips passes 1-2 and reads the carried state
// directly.
#include "kernels.h"

namespace mka {

constexpr int kEmaThreads = 128, kEmaVec = 4, kEmaSlab = kEmaThreads * kEmaVec;
constexpr int kEmaUnroll = 8, kEmaBatch = 16;

// 8 consecutive values at p as floats, loaded unconditionally (a guarded load
// would be waited for on its own); the upper 4 count only when ``hi`` (the
// row has them).  bf16 rows have D % 64 == 0, so all 8 always exist.
__device__ __forceinline__ void load8(const bf16_t* p, bool, float* out) {
  Vec16<bf16_t>::load(p, out);
}
__device__ __forceinline__ void load8(const float* p, bool hi, float* out) {
  load4(p, out);
  load4(p + (hi ? 4 : 0), out + 4);
  if (!hi) out[4] = out[5] = out[6] = out[7] = 0.f;
}

// Pass 1 takes 8 channels per thread (16-byte loads of bf16 rows).
constexpr int kEma1Vec = 8, kEma1Slab = kEmaThreads * kEma1Vec;

template <typename T>
__global__ __launch_bounds__(kEmaThreads) void ema_pass1(const T* __restrict__ x, int seq, int D,
                                                          int64_t pos0, int block, float beta,
                                                          float omb, float* __restrict__ agg_s,
                                                          float* __restrict__ agg_a,
                                                          int n_chunks) {
  const int c = blockIdx.x, b = blockIdx.z;
  const int ch = blockIdx.y * kEma1Slab + threadIdx.x * kEma1Vec;
  if (ch >= D) return;
  const bool hi = ch + 4 < D;
  const int t0 = c * kEmaChunk, t1 = min(t0 + kEmaChunk, seq);
  float s[8] = {}, a[8] = {};
  const T* xp = x + (static_cast<int64_t>(b) * seq + t0) * D + ch;
  int in_blk = static_cast<int>((pos0 + t0) % block);  // tokens of the current block so far
  // kEmaUnroll tokens' loads are issued before their (sequential) updates
  for (int tb = t0; tb < t1; tb += kEmaUnroll, xp += kEmaUnroll * static_cast<int64_t>(D)) {
    float xv[kEmaUnroll][8];
#pragma unroll
    for (int u = 0; u < kEmaUnroll; ++u)  // rows past the chunk re-read its last row (unused)
      load8(xp + min(u, t1 - 1 - tb) * static_cast<int64_t>(D), hi, xv[u]);
#pragma unroll
    for (int u = 0; u < kEmaUnroll; ++u) {
      if (tb + u < t1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          s[i] = fmaf(beta, s[i], omb * xv[u][i]);
          a[i] += xv[u][i];
        }
        if (++in_blk == block) {
          in_blk = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) a[i] = 0.f;
        }
      }
    }
  }
  const int64_t o = (static_cast<int64_t>(b) * n_chunks + c) * D + ch;
  store4(agg_s + o, s);
  store4(agg_a + o, a);
  if (hi) {
    store4(agg_s + o + 4, s + 4);
    store4(agg_a + o + 4, a + 4);
  }
}

// Exclusive scan of the chunk results, in place, per (batch, channel), in
// two levels: the chunks of a channel split into kEmaSegs segments of
// seg_len chunks; a workgroup holds 16 channels x kEmaSegs segments (lane ->
// channel, so a wave's loads of one chunk are 64 contiguous bytes).  Each
// thread folds its segment from a zero carry (EMA: s <- beta^L s + a; block
// sum: restart at a chunk that contains a block end), one thread per channel
// chains the segments' results, and each thread rewalks its segment from its
// carry, writing the carry entering every chunk.  The sequential depth is
// 2 seg_len + kEmaSegs chunk steps instead of n_chunks.
constexpr int kEmaSegs = 16;

__global__ __launch_bounds__(16 * kEmaSegs) void ema_pass2(float* __restrict__ agg_s,
                                                        float* __restrict__ agg_a,
                                                        const float* __restrict__ state_in,
                                                        const float* __restrict__ acc_in, int B,
                                                        int D, int seq, int64_t pos0, int block,
                                                        float beta_L, int n_chunks, int seg_len) {
  __shared__ float seg_s[kEmaSegs][16], seg_a[kEmaSegs][16], carry_s[kEmaSegs][16],
      carry_a[kEmaSegs][16];
  __shared__ int seg_c[kEmaSegs][16];
  const int chl = threadIdx.x & 15, seg = threadIdx.x >> 4;
  const int e = blockIdx.x * 16 + chl;
  const bool on = e < B * D;
  const int b = on ? e / D : 0, ch = on ? e - b * D : 0;
  float* ps = agg_s + static_cast<int64_t>(b) * n_chunks * D + ch;
  float* pa = agg_a + static_cast<int64_t>(b) * n_chunks * D + ch;
  const int c_begin = min(seg * seg_len, n_chunks), c_end = min(c_begin + seg_len, n_chunks);
  const int step = kEmaChunk % block;
  const int rem0 = static_cast<int>((pos0 + static_cast<int64_t>(c_begin) * kEmaChunk) % block);
  // the segment's chunks, kEmaBatch results loaded before their sequential use
  auto walk = [&](float cs, float ca, bool write, bool& closed) {
    int rem = rem0;
    closed = false;
    for (int c0 = c_begin; c0 < c_end; c0 += kEmaBatch) {
      float sc[kEmaBatch], ac[kEmaBatch];
#pragma unroll
      for (int u = 0; u < kEmaBatch; ++u) {
        const int64_t o = static_cast<int64_t>(min(c0 + u, c_end - 1)) * D;
        sc[u] = on ? ps[o] : 0.f;
        ac[u] = on ? pa[o] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kEmaBatch; ++u) {
        const int c = c0 + u;
        if (c < c_end) {
          if (write && on) {
            const int64_t o = static_cast<int64_t>(c) * D;
            ps[o] = cs;
            pa[o] = ca;
          }
          const int len = min((c + 1) * kEmaChunk, seq) - c * kEmaChunk;
          const bool closes = rem + len >= block;  // a block ends inside this chunk
          closed |= closes;
          cs = fmaf(beta_L, cs, sc[u]);
          ca = closes ? ac[u] : ca + ac[u];
          rem += step;
          if (rem >= block) rem -= block;
        }
      }
    }
    return make_float2(cs, ca);
  };
  bool closed;
  const float2 loc = walk(0.f, 0.f, false, closed);
  seg_s[seg][chl] = loc.x;
  seg_a[seg][chl] = loc.y;
  seg_c[seg][chl] = closed;
  __syncthreads();
  if (seg == 0) {
    // An empty prefix (pos0 == 0) and an empty partial block (pos0 at a block
    // start) contribute zero whatever the buffers hold.
    float cs = pos0 == 0 || !on ? 0.f : state_in[e];
    float ca = pos0 % block == 0 || !on ? 0.f : acc_in[e];
    float pw = 1.f;  // beta^L over a whole segment (only whole segments feed later ones)
    for (int i = 0; i < seg_len; ++i) pw *= beta_L;
    for (int g = 0; g < kEmaSegs; ++g) {
      carry_s[g][chl] = cs;
      carry_a[g][chl] = ca;
      cs = fmaf(pw, cs, seg_s[g][chl]);
      ca = seg_c[g][chl] ? seg_a[g][chl] : ca + seg_a[g][chl];
    }
  }
  __syncthreads();
  walk(carry_s[seg][chl], carry_a[seg][chl], true, closed);
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
  int in_blk = static_cast<int>((pos0 + t0) % block);
  int64_t blk = (pos0 + t0) / block;  // block of the next token
  for (int tb = t0; tb < t1; tb += kEmaUnroll) {
    float xv[kEmaUnroll][4];
#pragma unroll
    for (int u = 0; u < kEmaUnroll; ++u)  // rows past the chunk re-read its last row (unused)
      load4(xp + min(u, t1 - 1 - tb) * static_cast<int64_t>(D), xv[u]);
#pragma unroll
    for (int u = 0; u < kEmaUnroll; ++u) {
      if (tb + u < t1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[i] = fmaf(beta, s[i], omb * xv[u][i]);
          a[i] += xv[u][i];
        }
        store4(lp + u * static_cast<int64_t>(D), s);
        if (++in_blk == block) {
          float m[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) m[i] = a[i] / static_cast<float>(block);
          store4(means + (static_cast<int64_t>(b) * nb_cap + blk) * D + ch, m);
          a[0] = a[1] = a[2] = a[3] = 0.f;
          in_blk = 0;
          ++blk;
        }
      }
    }
    xp += kEmaUnroll * static_cast<int64_t>(D);
    lp += kEmaUnroll * static_cast<int64_t>(D);
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
  const dim3 grid1(n_chunks, (D + kEma1Slab - 1) / kEma1Slab, B);
  hipLaunchKernelGGL(ema_pass1<T>, grid1, dim3(kEmaThreads), 0, s, x, seq, D, pos0, block, beta,
                     omb, agg_s, agg_a, n_chunks);
  double bl = 1.0;
  for (int i = 0; i < kEmaChunk; ++i) bl *= static_cast<double>(beta);
  // one channel per thread, 64-thread workgroups: the scan is spread over many CUs
  const int seg_len = (n_chunks + kEmaSegs - 1) / kEmaSegs;
  hipLaunchKernelGGL(ema_pass2, dim3((B * D + 15) / 16), dim3(16 * kEmaSegs), 0, s, agg_s, agg_a,
                     state_io, acc_io, B, D, seq, pos0, block, static_cast<float>(bl), n_chunks,
                     seg_len);
  hipLaunchKernelGGL(ema_pass3<T>, grid, dim3(kEmaThreads), 0, s, x, seq, D, pos0, block, beta, omb,
                     agg_s, agg_a, n_chunks, l2, means, nb_cap, state_io, acc_io, n_chunks);
  return hipGetLastError();
}

template hipError_t ema_scan<float>(const float*, int, int, int, int64_t, int, float, float*,
                                    float*, float*, float*, int, float*, hipStream_t);
template hipError_t ema_scan<bf16_t>(const bf16_t*, int, int, int, int64_t, int, float, float*,
                                     float*, float*, float*, int, float*, hipStream_t);

}  // namespace mka
