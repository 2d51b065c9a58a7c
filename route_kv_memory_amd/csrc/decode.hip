// Fused kernels of one decode step (one token per sequence, batch B <= 8).
//
// The step's dependencies are: x -> {q, L2 (EMA), key projections};
// q -> router hidden -> lambda; key projections -> key -> top-R blocks;
// (lambda, blocks, L2, x) -> X_fused -> K/V row.  (MKA reading note, method
// sections 1-3; the abstract page's Table 11 counts three launches per token
// for its own kernels.)
//
// bf16 layers use three launches.  The K/V row is linear in X_fused:
//   [K|V] = lambda1 (x W) + lambda2 (L2 W) + lambda3 (L3 W),  W = [W_k; W_v],
// and L3 W is the mean of the retrieved blocks' projected means m_b W, which
// are kept beside the bank (computed when a block is indexed).  So only the
// last kernel waits for the router:
//   decode_inputs   Q = x W_q  |  EMA update, block finalise and fp64
//                   partial key projections per 128 channels
//   decode_attend   split attention over cache rows [0, pos)  |  router
//                   hidden GELU(q W_r1)  |  [x; L2] W  |  per token: key,
//                   top-R, L3 W, EMA state commit
//   decode_merge    lambda, the new K/V row (written to the cache at pos),
//                   its score, and the merge of the attention partials
// float32 layers run the same steps as sequential kernels:
//   decode_front    Q (one wave per output) | EMA, block finalise, key partials
//   decode_mid      router hidden | key, top-R
//   decode_fuse     lambda, X_fused; then the K/V product and attention.
#include "decode.h"
#include "attn_split.h"

namespace mka {

// ---------------------------------------------------------------------------
// Wave-wide minimum of unsigned 32-bit values through DPP lane moves (no LDS
// round trip): xor-1 and xor-2 within quads, mirrors within rows of 16, then
// row broadcasts; the result is read from lane 63.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_min(uint32_t v) {
  const int o = __builtin_amdgcn_update_dpp(static_cast<int>(0xFFFFFFFFu), static_cast<int>(v), CTRL,
                                            ROW_MASK, 0xF, false);
  return min(v, static_cast<uint32_t>(o));
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  v = dpp_min<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_min<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_min<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_min<0x140, 0xF>(v);  // row_mirror
  v = dpp_min<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_min<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint32_t cand_key(uint64_t key, uint64_t code, int b) {
  return (static_cast<uint32_t>(__popcll(key ^ code)) << 24) | (0xFFFFFFu - static_cast<uint32_t>(b));
}
constexpr uint32_t kEmptyKey = 0xFFFFFFFFu;

template <int N>
__device__ __forceinline__ void insert_sorted(uint32_t (&top)[N], uint32_t v) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t lo = min(v, top[i]);
    v = max(v, top[i]);
    top[i] = lo;
  }
}

// ---------------------------------------------------------------------------
// decode_front
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void decode_front_kernel(DecodeArgs<T> a) {
  __shared__ float Ls[kDecSlice];
  __shared__ double red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nq_wg = (a.qw + 3) / 4;
  if (static_cast<int>(blockIdx.x) < nq_wg) {
    // ---- Q projection: one wave per output column, lanes stride D with 16-byte loads.
    const int n = blockIdx.x * 4 + wave;
    if (n >= a.qw) return;
    constexpr int V = Vec16<T>::kN;
    const T* w = a.w_q + static_cast<int64_t>(n) * a.D;
    float acc[kFewRowsDec] = {};
#pragma unroll 4
    for (int k = lane * V; k < a.D; k += 64 * V) {
      float wv[V];
      Vec16<T>::load(w + k, wv);
#pragma unroll
      for (int b = 0; b < kFewRowsDec; ++b) {
        if (b < a.B) {
          float xv[V];
          Vec16<T>::load(a.x + static_cast<int64_t>(b) * a.D + k, xv);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[b] = fmaf(xv[i], wv[i], acc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kFewRowsDec; ++b) {
      if (b < a.B) {
        const float v = wave_sum(acc[b]);
        if (lane == 0) a.q[static_cast<int64_t>(b) * a.qw + n] = Elem<T>::from_f32(v);
      }
    }
    return;
  }
  // ---- EMA update + block finalise + partial key projections for one slice.
  const int e = blockIdx.x - nq_wg;
  const int slice = e % a.n_slices, b = e / a.n_slices;
  const int c0 = slice * kDecSlice;
  float sv = 0.f;
  if (tid < kDecSlice && c0 + tid < a.D) {
    const int64_t o = static_cast<int64_t>(b) * a.D + c0 + tid;
    const float xv = Elem<T>::to_f32(a.x[o]);
    sv = fmaf(a.beta, a.pos == 0 ? 0.f : a.state[o], a.omb * xv);
    float acc = (a.pos % a.block == 0 ? 0.f : a.acc[o]) + xv;
    a.state[o] = sv;
    a.l2[o] = sv;
    if ((a.pos + 1) % a.block == 0) {
      a.means[(static_cast<int64_t>(b) * a.nb_cap + (a.pos + 1) / a.block - 1) * a.D + c0 + tid] =
          acc / static_cast<float>(a.block);
      acc = 0.f;
    }
    a.acc[o] = acc;
  }
  if (!a.rt.l3()) return;  // no retrieval: the key is not needed
  if (tid < kDecSlice) Ls[tid] = sv;
  __syncthreads();
  // thread (j = hyperplane, quarter of the slice): 32 channels of row j of P.
  const int j = lane, quarter = wave;
  double p = 0.0;
  if (j < a.nbits) {
    const float* prow = a.proj + static_cast<int64_t>(j) * a.D + c0 + quarter * 32;
    const int cend = min(32, a.D - c0 - quarter * 32);
#pragma unroll 8
    for (int c = 0; c < 32; ++c)
      if (c < cend) p = fma(static_cast<double>(Ls[quarter * 32 + c]), static_cast<double>(prow[c]), p);
  }
  red[quarter][j] = p;
  __syncthreads();
  if (tid < 64)
    a.part[(static_cast<int64_t>(slice) * a.B + b) * 64 + tid] =
        ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// ---------------------------------------------------------------------------
// decode_mid
// ---------------------------------------------------------------------------
template <typename T, int RMAX>
__global__ __launch_bounds__(256) void decode_mid_kernel(DecodeArgs<T> a) {
  __shared__ uint64_t key_s;
  __shared__ uint32_t cand[4][RMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nh_wg = a.rt.learned() ? (a.r + 3) / 4 : 0;
  if (static_cast<int>(blockIdx.x) < nh_wg) {
    // ---- router hidden unit n for every token: GELU(q . W_r1[n]).
    const int n = blockIdx.x * 4 + wave;
    if (n >= a.r) return;
    constexpr int V = Vec16<T>::kN;
    const T* w = a.w_r1 + static_cast<int64_t>(n) * a.qw;
    float acc[kFewRowsDec] = {};
#pragma unroll 4
    for (int k = lane * V; k < a.qw; k += 64 * V) {
      float wv[V];
      Vec16<T>::load(w + k, wv);
#pragma unroll
      for (int b = 0; b < kFewRowsDec; ++b) {
        if (b < a.B) {
          float qv[V];
          Vec16<T>::load(a.q + static_cast<int64_t>(b) * a.qw + k, qv);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[b] = fmaf(qv[i], wv[i], acc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kFewRowsDec; ++b) {
      if (b < a.B) {
        const float v = wave_sum(acc[b]);
        if (lane == 0) a.hidden[b * a.r + n] = gelu(v);
      }
    }
    return;
  }
  // ---- top-R selection for token b.
  const int b = blockIdx.x - nh_wg;
  if (wave == 0) {
    double p = 0.0;
#pragma unroll 4
    for (int s = 0; s < a.n_slices; ++s) p += a.part[(static_cast<int64_t>(s) * a.B + b) * 64 + lane];
    const uint64_t code = __ballot(lane < a.nbits && p > 0.0);
    if (lane == 0) {
      key_s = code;
      a.key[b] = code;
    }
  }
  __syncthreads();
  const uint64_t key = key_s;
  const int ne = static_cast<int>(a.pos / a.block);
  const uint64_t* codes = a.bhash + static_cast<int64_t>(b) * a.nb_cap;
  uint32_t top[RMAX];
#pragma unroll
  for (int i = 0; i < RMAX; ++i) top[i] = kEmptyKey;
  for (int jb = tid; jb < ne; jb += 256) insert_sorted(top, cand_key(key, codes[jb], jb));
  for (int i = 0; i < a.R; ++i) {
    const uint32_t m = wave_min_dpp(top[0]);
    if (top[0] == m && m != kEmptyKey) {
#pragma unroll
      for (int k = 0; k < RMAX - 1; ++k) top[k] = top[k + 1];
      top[RMAX - 1] = kEmptyKey;
    }
    if (lane == 0) cand[wave][i] = m;
  }
  __syncthreads();
  if (wave != 0) return;
  const uint32_t* flat = &cand[0][0];
  uint32_t c0 = kEmptyKey, c1 = kEmptyKey;
  if (lane < 4 * a.R) c0 = flat[(lane / a.R) * RMAX + lane % a.R];
  if (lane + 64 < 4 * a.R) c1 = flat[((lane + 64) / a.R) * RMAX + (lane + 64) % a.R];
  if (c1 < c0) {
    const uint32_t t = c0;
    c0 = c1;
    c1 = t;
  }
  int32_t* out = a.idx + static_cast<int64_t>(b) * a.R;
  for (int i = 0; i < a.R; ++i) {
    const uint32_t m = wave_min_dpp(c0);
    if (c0 == m && m != kEmptyKey) {
      c0 = c1;
      c1 = kEmptyKey;
    }
    if (lane == 0) out[i] = m == kEmptyKey ? -1 : static_cast<int>(0xFFFFFFu - (m & 0xFFFFFFu));
  }
}

// ---------------------------------------------------------------------------
// decode_fuse: lambda from the hidden layer, then X_fused for 256 channels.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void decode_fuse_kernel(DecodeArgs<T> a) {
  constexpr int RMAX = 32;
  const int lane = threadIdx.x, b = blockIdx.y;
  float z[3] = {0.f, 0.f, 0.f};
  if (a.rt.learned()) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      float sum = 0.f;
      for (int n = lane; n < a.r; n += 64)
        sum = fmaf(a.hidden[b * a.r + n], Elem<T>::to_f32(a.w_r2[c * a.r + n]), sum);
      z[c] = wave_sum(sum);
    }
  }
  float lw[3];
  route_weights(z, a.rt, lw);
  const float l1w = lw[0], l2w = lw[1], l3w = lw[2];
  if (blockIdx.x == 0 && lane == 0) {
    a.lam[b * 3 + 0] = l1w;
    a.lam[b * 3 + 1] = l2w;
    a.lam[b * 3 + 2] = l3w;
  }
  const int ch = (blockIdx.x * 64 + lane) * 4;
  if (ch >= a.D) return;
  const int32_t* sel = a.idx + static_cast<int64_t>(b) * a.R;
  const float* mb = a.means + static_cast<int64_t>(b) * a.nb_cap * a.D + ch;
  int blk[RMAX];
  const int R = a.rt.l3() ? a.R : 0;  // disabled tiers are not read
#pragma unroll
  for (int i = 0; i < RMAX; ++i) blk[i] = i < R ? sel[i] : -1;
  float xv[4], sv[4] = {0.f, 0.f, 0.f, 0.f}, l3[4] = {0.f, 0.f, 0.f, 0.f};
  load4(a.x + static_cast<int64_t>(b) * a.D + ch, xv);
  if (a.rt.l2()) load4(a.l2 + static_cast<int64_t>(b) * a.D + ch, sv);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    if (blk[i] >= 0) {
      float m[4];
      load4(mb + static_cast<int64_t>(blk[i]) * a.D, m);
#pragma unroll
      for (int k = 0; k < 4; ++k) l3[k] += m[k];
      ++cnt;
    }
  }
  float out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float m = cnt ? l3[k] / static_cast<float>(cnt) : 0.f;
    out[k] = l1w * xv[k] + l2w * sv[k] + l3w * m;
  }
  store4(a.xf + static_cast<int64_t>(b) * a.D + ch, out);
}

template <typename T>
hipError_t decode_front(const DecodeArgs<T>& a, hipStream_t s) {
  const int grid = (a.qw + 3) / 4 + (a.rt.ema() ? a.n_slices * a.B : 0);
  hipLaunchKernelGGL(decode_front_kernel<T>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <typename T>
hipError_t decode_mid(const DecodeArgs<T>& a, hipStream_t s) {
  const int grid = (a.rt.learned() ? (a.r + 3) / 4 : 0) + (a.rt.l3() ? a.B : 0);
  if (grid == 0) return hipSuccess;
  if (a.R <= 16)
    hipLaunchKernelGGL((decode_mid_kernel<T, 16>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mid_kernel<T, 32>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <typename T>
hipError_t decode_fuse(const DecodeArgs<T>& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_fuse_kernel<T>, dim3((a.D + 255) / 256, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

template hipError_t decode_front<float>(const DecodeArgs<float>&, hipStream_t);
template hipError_t decode_mid<float>(const DecodeArgs<float>&, hipStream_t);
template hipError_t decode_fuse<float>(const DecodeArgs<float>&, hipStream_t);

// ===========================================================================
// bf16 step in three launches.
// ===========================================================================

// Products of kGemvCols consecutive rows of the weight matrix selected by
// ``wrow`` with the step's token rows: one wave, lanes stride the reduction
// with 16-byte loads.  The weight loads of IT strides are all issued before
// the first product (buffer loads: zero past D), and for each token its IT
// strides of inputs are loaded together; ``feed(b, k, xv)`` supplies NIN rows
// of 8 inputs of token b at k (k <= D - 8).
template <int NIN, typename WRow, typename Feed>
__device__ __forceinline__ void decode_products(int D, int B, WRow wrow, Feed feed,
                                                float (&acc)[NIN][kGemvCols][kFewRowsDec]) {
  constexpr int V = 8, IT = NIN == 1 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  __amdgpu_buffer_rsrc_t wr[kGemvCols];
#pragma unroll
  for (int c = 0; c < kGemvCols; ++c) wr[c] = make_rsrc(wrow(c), static_cast<uint32_t>(D) * 2);
  for (int k0 = 0; k0 < D; k0 += 64 * V * IT) {
    u32x4 wraw[IT][kGemvCols];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int c = 0; c < kGemvCols; ++c)
        wraw[it][c] = buffer_load16(wr[c], static_cast<uint32_t>(k0 + it * 64 * V + lane * V) * 2);
#pragma unroll
    for (int b = 0; b < kFewRowsDec; ++b) {
      if (b < B) {
        float xv[IT][NIN][V];
#pragma unroll
        for (int it = 0; it < IT; ++it) feed(b, min(k0 + it * 64 * V + lane * V, D - V), xv[it]);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          if (k0 + it * 64 * V < D) {  // strides past the end hold no weights
#pragma unroll
            for (int c = 0; c < kGemvCols; ++c) {
              float wv[V];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                wv[2 * e] = __uint_as_float(wraw[it][c][e] << 16);
                wv[2 * e + 1] = __uint_as_float(wraw[it][c][e] & 0xFFFF0000u);
              }
#pragma unroll
              for (int j = 0; j < NIN; ++j)
#pragma unroll
                for (int i = 0; i < V; ++i) acc[j][c][b] = fmaf(xv[it][j][i], wv[i], acc[j][c][b]);
            }
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void decode_inputs_kernel(DecodeArgs<bf16_t> a) {
  __shared__ float Ls[kDecSlice];
  __shared__ double red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nq_wg = (a.qw + 4 * kGemvCols - 1) / (4 * kGemvCols);
  int wg = blockIdx.x;
  if (wg < nq_wg) {
    // ---- Q = x W_q: kGemvCols output columns per wave.
    const int n0 = (wg * 4 + wave) * kGemvCols;
    if (n0 >= a.qw) return;
    float acc[1][kGemvCols][kFewRowsDec] = {};
    decode_products<1>(
        a.D, a.B,
        [&](int c) { return a.w_q + static_cast<int64_t>(min(n0 + c, a.qw - 1)) * a.D; },
        [&](int b, int k, float (&xv)[1][8]) { Vec16<bf16_t>::load(a.x + static_cast<int64_t>(b) * a.D + k, xv[0]); },
        acc);
#pragma unroll
    for (int c = 0; c < kGemvCols; ++c)
#pragma unroll
      for (int b = 0; b < kFewRowsDec; ++b) {
        if (b < a.B) {
          const float v = wave_sum(acc[0][c][b]);
          if (lane == 0 && n0 + c < a.qw) a.q[static_cast<int64_t>(b) * a.qw + n0 + c] = f32_to_bf16(v);
        }
      }
    return;
  }
  wg -= nq_wg;
  // ---- EMA update + block finalise + partial key projections for one slice.
  // The state itself is committed by decode_attend.
  const int slice = wg % a.n_slices, b = wg / a.n_slices;
  const int c0 = slice * kDecSlice;
  float sv = 0.f;
  if (tid < kDecSlice && c0 + tid < a.D) {
    const int64_t o = static_cast<int64_t>(b) * a.D + c0 + tid;
    const float xv = bf16_to_f32(a.x[o]);
    sv = fmaf(a.beta, a.pos == 0 ? 0.f : a.state[o], a.omb * xv);
    float acc = (a.pos % a.block == 0 ? 0.f : a.acc[o]) + xv;
    a.l2[o] = sv;
    if ((a.pos + 1) % a.block == 0) {
      a.means[(static_cast<int64_t>(b) * a.nb_cap + (a.pos + 1) / a.block - 1) * a.D + c0 + tid] =
          acc / static_cast<float>(a.block);
      acc = 0.f;
    }
    a.acc[o] = acc;
  }
  if (!a.rt.l3()) return;  // no retrieval: the key is not needed
  if (tid < kDecSlice) Ls[tid] = sv;
  __syncthreads();
  const int j = lane, quarter = wave;
  double p = 0.0;
  if (j < a.nbits) {
    // the 32 hyperplane entries are loaded before the (in-order) products
    const float* prow = a.proj + static_cast<int64_t>(j) * a.D + c0 + quarter * 32;
    const int cend = min(32, a.D - c0 - quarter * 32);
    float pv[32];
    if (cend == 32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) load4(prow + 4 * i, pv + 4 * i);
    } else {
#pragma unroll
      for (int c = 0; c < 32; ++c) pv[c] = c < cend ? prow[c] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < 32; ++c)
      p = fma(static_cast<double>(Ls[quarter * 32 + c]), static_cast<double>(pv[c]), p);
  }
  red[quarter][j] = p;
  __syncthreads();
  if (tid < 64)
    a.part[(static_cast<int64_t>(slice) * a.B + b) * 64 + tid] =
        ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

template <int DH, int RMAX, bool PAGED>
__global__ __launch_bounds__(256, 2) void decode_attend_kernel(DecodeArgs<bf16_t> a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[split_lds_bytes<DH>()];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nh_wg = a.rt.learned() ? (a.r + 3) / 4 : 0;
  int wg = blockIdx.x;
  if (wg < nh_wg) {
    // ---- router hidden unit n for every token: GELU(q . W_r1[n]).
    const int n = wg * 4 + wave;
    if (n >= a.r) return;
    const bf16_t* w = a.w_r1 + static_cast<int64_t>(n) * a.qw;
    float acc[kFewRowsDec] = {};
#pragma unroll 4
    for (int k = lane * 8; k < a.qw; k += 512) {
      float wv[8];
      Vec16<bf16_t>::load(w + k, wv);
#pragma unroll
      for (int b = 0; b < kFewRowsDec; ++b) {
        if (b < a.B) {
          float qv[8];
          Vec16<bf16_t>::load(a.q + static_cast<int64_t>(b) * a.qw + k, qv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[b] = fmaf(qv[i], wv[i], acc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kFewRowsDec; ++b) {
      if (b < a.B) {
        const float v = wave_sum(acc[b]);
        if (lane == 0) a.hidden[b * a.r + n] = gelu(v);
      }
    }
    return;
  }
  wg -= nh_wg;
  const int nkv = 2 * a.kvw, nkv_wg = (nkv + 4 * kGemvCols - 1) / (4 * kGemvCols);
  if (wg < nkv_wg) {
    // ---- [x; L2] [W_k; W_v]^T (L2 as decode_inputs wrote it); not needed
    // before decode_merge, so it runs beside the attention.
    const int n0 = (wg * 4 + wave) * kGemvCols;
    if (n0 >= nkv) return;
    const auto wrow = [&](int c) {
      const int col = min(n0 + c, nkv - 1);
      return col < a.kvw ? a.w_k + static_cast<int64_t>(col) * a.D
                         : a.w_v + static_cast<int64_t>(col - a.kvw) * a.D;
    };
    if (!a.rt.l2()) {  // L2 not mixed: x W alone
      float acc[1][kGemvCols][kFewRowsDec] = {};
      decode_products<1>(
          a.D, a.B, wrow,
          [&](int b, int k, float (&xv)[1][8]) {
            Vec16<bf16_t>::load(a.x + static_cast<int64_t>(b) * a.D + k, xv[0]);
          },
          acc);
#pragma unroll
      for (int c = 0; c < kGemvCols; ++c)
#pragma unroll
        for (int b = 0; b < kFewRowsDec; ++b) {
          if (b < a.B) {
            const float vx = wave_sum(acc[0][c][b]);
            if (lane == 0 && n0 + c < nkv) a.kvx[static_cast<int64_t>(b) * nkv + n0 + c] = vx;
          }
        }
      return;
    }
    float acc[2][kGemvCols][kFewRowsDec] = {};
    decode_products<2>(
        a.D, a.B, wrow,
        [&](int b, int k, float (&xv)[2][8]) {
          const int64_t o = static_cast<int64_t>(b) * a.D + k;
          Vec16<bf16_t>::load(a.x + o, xv[0]);
          load4(a.l2 + o, xv[1]);
          load4(a.l2 + o + 4, xv[1] + 4);
        },
        acc);
#pragma unroll
    for (int c = 0; c < kGemvCols; ++c)
#pragma unroll
      for (int b = 0; b < kFewRowsDec; ++b) {
        if (b < a.B) {
          const float vx = wave_sum(acc[0][c][b]);
          const float vl = wave_sum(acc[1][c][b]);
          if (lane == 0 && n0 + c < nkv) {
            a.kvx[static_cast<int64_t>(b) * nkv + n0 + c] = vx;
            a.kvl2[static_cast<int64_t>(b) * nkv + n0 + c] = vl;
          }
        }
      }
    return;
  }
  wg -= nkv_wg;
  if (wg < a.B) {
    // ---- token b: key, top-R blocks, L3 W (mean of the projected block means)
    // and the EMA state commit (only the commit without L3; nothing without
    // the EMA).
    if (!a.rt.ema()) return;
    const int b = wg;
    if (a.rt.l3()) {
      uint64_t* key_s = reinterpret_cast<uint64_t*>(lds);
      uint32_t* cand = reinterpret_cast<uint32_t*>(lds + 16);             // [4][RMAX]
      int32_t* sel = reinterpret_cast<int32_t*>(lds + 16 + 16 * RMAX);    // [RMAX]
      const int ne = static_cast<int>(a.pos / a.block);
      const uint64_t* codes = a.bhash + static_cast<int64_t>(b) * a.nb_cap;
      // this thread's first 4 block codes are in flight during the key reduction
      uint64_t cv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) cv[u] = ne > 0 ? codes[min(tid + 256 * u, ne - 1)] : 0;
      if (wave == 0) {
        // partial projections of all slices, loaded first, added in slice order
        double p = 0.0;
        for (int s0 = 0; s0 < a.n_slices; s0 += 8) {
          double v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[u] = a.part[(static_cast<int64_t>(min(s0 + u, a.n_slices - 1)) * a.B + b) * 64 + lane];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (s0 + u < a.n_slices) p += v[u];
        }
        const uint64_t code = __ballot(lane < a.nbits && p > 0.0);
        if (lane == 0) {
          *key_s = code;
          a.key[b] = code;
        }
      }
      __syncthreads();
      const uint64_t key = *key_s;
      uint32_t top[RMAX];
#pragma unroll
      for (int i = 0; i < RMAX; ++i) top[i] = kEmptyKey;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (tid + 256 * u < ne) insert_sorted(top, cand_key(key, cv[u], tid + 256 * u));
      for (int jb = tid + 1024; jb < ne; jb += 256) insert_sorted(top, cand_key(key, codes[jb], jb));
      for (int i = 0; i < a.R; ++i) {
        const uint32_t m = wave_min_dpp(top[0]);
        if (top[0] == m && m != kEmptyKey) {
#pragma unroll
          for (int k = 0; k < RMAX - 1; ++k) top[k] = top[k + 1];
          top[RMAX - 1] = kEmptyKey;
        }
        if (lane == 0) cand[wave * RMAX + i] = m;
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t c0 = kEmptyKey, c1 = kEmptyKey;
        if (lane < 4 * a.R) c0 = cand[(lane / a.R) * RMAX + lane % a.R];
        if (lane + 64 < 4 * a.R) c1 = cand[((lane + 64) / a.R) * RMAX + (lane + 64) % a.R];
        if (c1 < c0) {
          const uint32_t t = c0;
          c0 = c1;
          c1 = t;
        }
        int32_t* out = a.idx + static_cast<int64_t>(b) * a.R;
        for (int i = 0; i < a.R; ++i) {
          const uint32_t m = wave_min_dpp(c0);
          if (c0 == m && m != kEmptyKey) {
            c0 = c1;
            c1 = kEmptyKey;
          }
          const int blk = m == kEmptyKey ? -1 : static_cast<int>(0xFFFFFFu - (m & 0xFFFFFFu));
          if (lane == 0) {
            out[i] = blk;
            sel[i] = blk;
          }
        }
      }
      __syncthreads();
      // L3 W = mean of the selected blocks' projected means, in rank order; the
      // selection is held in registers and every row load is issued up front
      // (rows of unfilled slots are read at block 0 and not added).
      int blk[RMAX], cnt = 0;
#pragma unroll
      for (int i = 0; i < RMAX; ++i) {
        blk[i] = i < a.R ? sel[i] : -1;
        cnt += blk[i] >= 0;
      }
      const float inv = cnt ? 1.0f / static_cast<float>(cnt) : 0.f;
      const float* pb = a.block_kv + static_cast<int64_t>(b) * a.nb_cap * nkv;
      for (int n = tid; n < nkv; n += 256) {
        float v[RMAX];
#pragma unroll
        for (int i = 0; i < RMAX; ++i) v[i] = pb[static_cast<int64_t>(max(blk[i], 0)) * nkv + n];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < RMAX; ++i) sum += blk[i] >= 0 ? v[i] : 0.f;
        a.kvl3[static_cast<int64_t>(b) * nkv + n] = cnt ? sum * inv : 0.f;
      }
    }
    // EMA state commit (the L2 row of this token)
    const float* l2r = a.l2 + static_cast<int64_t>(b) * a.D;
    float* str = a.state + static_cast<int64_t>(b) * a.D;
    for (int c0 = 4 * tid; c0 < a.D; c0 += 4 * 256) {
      float v4[4];
      load4(l2r + c0, v4);
      store4(str + c0, v4);
    }
    return;
  }
  wg -= a.B;
  // ---- attention over cache rows [0, pos): one share per workgroup.
  const int per_b = a.n_chunks * a.G * a.n_hb;
  const int b = wg / per_b, rest = wg % per_b;
  const int c = rest % a.n_chunks, ghb = rest / a.n_chunks;
  decode_split_chunk<DH, PAGED>(a.q, a.k_cache, a.v_cache, a.H, a.G, a.kv, a.pos, a.sl2,
                         a.n_chunks, c, ghb / a.n_hb, ghb % a.n_hb, b, a.part_m, a.part_l,
                         a.part_o, lds);
}

template <int DH>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs<bf16_t> a) {
  __shared__ MergeLds<DH> sm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int hpg = a.H / a.G, g = h / hpg;
  decode_merge_head<DH>(
      a.part_m, a.part_l, a.part_o, a.H, a.n_chunks, h, b, a.q, a.sl2, a.o, sm,
      [&](float* kx, float* vx) {
        const int tid = threadIdx.x, lane = tid & 63;
        // the token's projected rows, loaded before lambda is known
        const int64_t rb = static_cast<int64_t>(b) * 2 * a.kvw;
        const int nk = g * DH + min(tid, DH - 1), nv = a.kvw + nk;
        const float kx1 = a.kvx[rb + nk], kx2 = a.kvl2[rb + nk], kx3 = a.kvl3[rb + nk];
        const float vx1 = a.kvx[rb + nv], vx2 = a.kvl2[rb + nv], vx3 = a.kvl3[rb + nv];
        if (tid < 64) {  // lambda = softmax(hidden W_r2), under the routing variant
          float z[3] = {0.f, 0.f, 0.f};
          if (a.rt.learned()) {
#pragma unroll
            for (int c = 0; c < 3; ++c) {
              float sum = 0.f;
              for (int n = lane; n < a.r; n += 64)
                sum = fmaf(a.hidden[b * a.r + n], bf16_to_f32(a.w_r2[c * a.r + n]), sum);
              z[c] = wave_sum(sum);
            }
          }
          float lw[3];
          route_weights(z, a.rt, lw);
          if (lane == 0) {
            sm.lam[0] = lw[0];
            sm.lam[1] = lw[1];
            sm.lam[2] = lw[2];
            if (h == 0) {
              a.lam[b * 3 + 0] = lw[0];
              a.lam[b * 3 + 1] = lw[1];
              a.lam[b * 3 + 2] = lw[2];
            }
          }
        }
        __syncthreads();
        if (tid < DH) {  // the fused K/V row of the token, rounded as the cache stores it
          const float l1 = sm.lam[0], l2 = sm.lam[1], l3 = sm.lam[2];
          // rows of disabled tiers were not computed this step: exact zeros
          const float k2 = a.rt.l2() ? kx2 : 0.f, v2 = a.rt.l2() ? vx2 : 0.f;
          const float k3 = a.rt.l3() ? kx3 : 0.f, v3 = a.rt.l3() ? vx3 : 0.f;
          const bf16_t kb = f32_to_bf16(l1 * kx1 + l2 * k2 + l3 * k3);
          const bf16_t vb = f32_to_bf16(l1 * vx1 + l2 * v2 + l3 * v3);
          kx[tid] = bf16_to_f32(kb);
          vx[tid] = bf16_to_f32(vb);
          if (h % hpg == 0) {
            const int64_t ro = a.kv.row(b, g, a.pos) + tid;
            a.k_cache[ro] = kb;
            a.v_cache[ro] = vb;
          }
        }
        return true;
      });
}

hipError_t decode_inputs_bf16(const DecodeArgs<bf16_t>& a, hipStream_t s) {
  const int per_wg = 4 * kGemvCols;
  const int grid = (a.qw + per_wg - 1) / per_wg + (a.rt.ema() ? a.n_slices * a.B : 0);
  hipLaunchKernelGGL(decode_inputs_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t decode_attend_bf16(const DecodeArgs<bf16_t>& a, hipStream_t s) {
  const int per_wg = 4 * kGemvCols;
  const int grid = (a.rt.learned() ? (a.r + 3) / 4 : 0) + (2 * a.kvw + per_wg - 1) / per_wg +
                   a.B + a.n_chunks * a.G * a.n_hb * a.B;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, a);
  };
  const bool r16 = a.R <= 16, paged = a.kv.paged();
  if (a.dh == 128) {
    if (paged)
      r16 ? launch(decode_attend_kernel<128, 16, true>) : launch(decode_attend_kernel<128, 32, true>);
    else
      r16 ? launch(decode_attend_kernel<128, 16, false>)
          : launch(decode_attend_kernel<128, 32, false>);
  } else {
    if (paged)
      r16 ? launch(decode_attend_kernel<64, 16, true>) : launch(decode_attend_kernel<64, 32, true>);
    else
      r16 ? launch(decode_attend_kernel<64, 16, false>) : launch(decode_attend_kernel<64, 32, false>);
  }
  return hipGetLastError();
}

hipError_t decode_merge_bf16(const DecodeArgs<bf16_t>& a, hipStream_t s) {
  if (a.dh == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(a.H, a.B), dim3(kMergeThreads), 0, s, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(a.H, a.B), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mka
