// Fused kernels of one decode step (one token per sequence, batch B <= 8).
//
// The step's dependencies are: x -> {q, L2 (EMA), key projections};
// q -> router hidden -> lambda; key projections -> key -> top-R blocks;
// (lambda, blocks, L2, x) -> X_fused -> K/V row.  Each kernel below holds
// workgroups of different roles that share a dependency level, so the step
// needs three launches before the K/V product instead of eight:
//   decode_front   Q = x W_q (one wave per output)  |  EMA update, block
//                  finalise and fp64 partial key projections per 128 channels
//   decode_mid     router hidden GELU(q W_r1) (one wave per unit)  |  per
//                  token: sum key partials, key, top-R selection
//   decode_fuse    lambda = softmax(hidden W_r2) (recomputed by each
//                  workgroup from the 64 hidden values), then X_fused
// (MKA reading note, method sections 1-3; the abstract page's Table 11 counts
// three launches per token for its own kernels.)
#include "decode.h"

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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nh_wg = (a.r + 3) / 4;
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
  float z[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    float sum = 0.f;
    for (int n = lane; n < a.r; n += 64)
      sum = fmaf(a.hidden[b * a.r + n], Elem<T>::to_f32(a.w_r2[c * a.r + n]), sum);
    z[c] = wave_sum(sum);
  }
  const float zm = fmaxf(z[0], fmaxf(z[1], z[2]));
  const float e0 = expf(z[0] - zm), e1 = expf(z[1] - zm), e2 = expf(z[2] - zm);
  const float inv = 1.0f / (e0 + e1 + e2);
  const float l1w = e0 * inv, l2w = e1 * inv, l3w = e2 * inv;
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
#pragma unroll
  for (int i = 0; i < RMAX; ++i) blk[i] = i < a.R ? sel[i] : -1;
  float xv[4], sv[4], l3[4] = {0.f, 0.f, 0.f, 0.f};
  load4(a.x + static_cast<int64_t>(b) * a.D + ch, xv);
  load4(a.l2 + static_cast<int64_t>(b) * a.D + ch, sv);
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
  const int grid = (a.qw + 3) / 4 + a.n_slices * a.B;
  hipLaunchKernelGGL(decode_front_kernel<T>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <typename T>
hipError_t decode_mid(const DecodeArgs<T>& a, hipStream_t s) {
  const int grid = (a.r + 3) / 4 + a.B;
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

template hipError_t decode_front<bf16_t>(const DecodeArgs<bf16_t>&, hipStream_t);
template hipError_t decode_mid<bf16_t>(const DecodeArgs<bf16_t>&, hipStream_t);
template hipError_t decode_fuse<bf16_t>(const DecodeArgs<bf16_t>&, hipStream_t);
template hipError_t decode_front<float>(const DecodeArgs<float>&, hipStream_t);
template hipError_t decode_mid<float>(const DecodeArgs<float>&, hipStream_t);
template hipError_t decode_fuse<float>(const DecodeArgs<float>&, hipStream_t);

}  // namespace mka
