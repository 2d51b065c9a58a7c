// Dense NT products on gfx950: bf16 MFMA tiles, a plain fp32 tiled kernel and a
// small-M (decode) kernel.
#include "gemm.h"

namespace mka {

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.  Workgroup tile 256 (M) x BN (N) x 64 (K), BN = 128 with 4
// waves or 256 with 8 waves; each wave owns 128 x 64 of C as 4 x 2 blocks of
// MFMA 32x32x16, so a k-step reads 6 fragments for 8 MFMAs.  The MFMA computes
// C^T blocks (B rows as its A operand), which leaves 4 consecutive output
// columns of one output row in each lane: the epilogue stores 8 bytes per lane.
// Operand tiles go through registers into double-buffered LDS (rows padded by
// 16 bytes: the fragment reads of 16 consecutive rows hit distinct banks);
// global reads are buffer loads whose range makes rows past M or N read zero.
// ---------------------------------------------------------------------------
template <int BN, class Epi>
__global__ __launch_bounds__(BN * 2) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int n_split, int M, int N, int K, Epi epi) {
  constexpr int BM = 256, BK = kGemmBK, P = BK + 8, NT = BN * 2;
  constexpr int ACH = BM * BK / 8 / NT, BCH = BN * BK / 8 / NT;  // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * P];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * P];

  const int tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_n * ((M + BM - 1) / BM);
  const int item = xcd_contiguous(blockIdx.x, tiles);
  const int tm = item / tiles_n, tn = item % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, h = lane >> 5, l32 = lane & 31;

  // A rows [m0, min(M, m0 + BM)) and B rows of this tile as buffer ranges.
  const uint32_t a_rows = static_cast<uint32_t>(min(BM, M - m0));
  const __amdgpu_buffer_rsrc_t ars =
      make_rsrc(A + static_cast<int64_t>(m0) * lda, a_rows * static_cast<uint32_t>(lda) * 2);
  // B rows come from b0 below n_split and b1 above; a tile never straddles
  // n_split when n_split % BN == 0, otherwise rows are fetched one by one.
  const bool straddle = n0 < n_split && n0 + BN > n_split;
  const bf16_t* bbase = n0 < n_split ? B0 + static_cast<int64_t>(n0) * K
                                     : B1 + static_cast<int64_t>(n0 - n_split) * K;
  const int b_valid = min(BN, (n0 < n_split ? n_split : N) - n0);
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(bbase, static_cast<uint32_t>(b_valid) * static_cast<uint32_t>(K) * 2);

  u32x4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + NT * i, row = c >> 3, col = (c & 7) * 8;
      ra[i] = buffer_load16(ars, static_cast<uint32_t>(row * lda + k0 + col) * 2);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + NT * i, row = c >> 3, col = (c & 7) * 8;
      if (!straddle) {
        rb[i] = buffer_load16(brs, static_cast<uint32_t>(row * K + k0 + col) * 2);
      } else {
        const int gn = n0 + row;
        const bf16_t* br = gn < n_split ? B0 + static_cast<int64_t>(gn) * K
                                        : B1 + static_cast<int64_t>(gn - n_split) * K;
        rb[i] = gn < N ? *reinterpret_cast<const u32x4*>(br + k0 + col) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + NT * i, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[buf][row * P + col]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + NT * i, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&Bs[buf][row * P + col]) = rb[i];
    }
  };

  // acc[i][j]: C^T block of output rows m0 + wm*128 + 32i .., columns n0 + wn*64 + 32j ..
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * 128 + i * 32 + l32) * P + ks * 16 + 8 * h]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * 64 + j * 32 + l32) * P + ks * 16 + 8 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(fb[j], fa[i], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Lane holds output row m = ... + l32 and columns n = ... + 8*(r/4) + 4h + (r%4).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + i * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int n = n0 + wn * 64 + j * 32 + 8 * rq + 4 * h;
        const float v[4] = {acc[i][j][4 * rq], acc[i][j][4 * rq + 1], acc[i][j][4 * rq + 2],
                            acc[i][j][4 * rq + 3]};
        epi.store4(m, n, v, N);
      }
  }
}

template <class Epi>
hipError_t gemm_bf16(const bf16_t* a, int lda, const bf16_t* b0, const bf16_t* b1, int n_split,
                     int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int tiles256 = ((N + 255) / 256) * ((M + 255) / 256);
  if (tiles256 >= 256) {
    hipLaunchKernelGGL((gemm_bf16_kernel<256, Epi>), dim3(tiles256), dim3(512), 0, s, a, lda, b0,
                       b1, n_split, M, N, K, epi);
  } else {
    const int tiles = ((N + 127) / 128) * ((M + 255) / 256);
    hipLaunchKernelGGL((gemm_bf16_kernel<128, Epi>), dim3(tiles), dim3(256), 0, s, a, lda, b0, b1,
                       n_split, M, N, K, epi);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 GEMM: 64 x 64 tile, 16 x 16 threads with 4 x 4 outputs each, k-tile 16.
// ---------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int lda, const float* __restrict__ B0,
    const float* __restrict__ B1, int n_split, int M, int N, int K, Epi epi) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i, kk = tid & 15;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? A[static_cast<int64_t>(gm) * lda + gk] : 0.f;
      float bv = 0.f;
      if (gn < N && gk < K)
        bv = gn < n_split ? B0[static_cast<int64_t>(gn) * K + gk]
                          : B1[static_cast<int64_t>(gn - n_split) * K + gk];
      Bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) epi(m, n, acc[i][j]);
    }
}

template <class Epi>
hipError_t gemm_f32(const float* a, int lda, const float* b0, const float* b1, int n_split, int M,
                    int N, int K, const Epi& epi, hipStream_t s) {
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel<Epi>, grid, dim3(256), 0, s, a, lda, b0, b1, n_split, M, N, K,
                     epi);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small-M product: one wave per output column n, lanes stride the reduction
// with 16-byte loads, every one of the M <= 8 rows reuses the weight row.
// ---------------------------------------------------------------------------
template <typename T, class Epi>
__global__ __launch_bounds__(256) void gemv_kernel(const T* __restrict__ A, int lda, int M,
                                                   const T* __restrict__ B0,
                                                   const T* __restrict__ B1, int n_split, int N,
                                                   int K, Epi epi) {
  constexpr int V = Vec16<T>::kN;
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const T* brow = n < n_split ? B0 + static_cast<int64_t>(n) * K
                              : B1 + static_cast<int64_t>(n - n_split) * K;
  float acc[8] = {};
  const int kv = (K / V) * V;
  constexpr int STEP = 64 * V, U = 4;
  int k = lane * V;
  // Four 16-byte weight loads in flight per lane before any arithmetic.
  for (; k + (U - 1) * STEP < kv; k += U * STEP) {
    float w[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) Vec16<T>::load(brow + k + u * STEP, w[u]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < M) {
        float a[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) Vec16<T>::load(A + static_cast<int64_t>(m) * lda + k + u * STEP, a[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < V; ++i) acc[m] = fmaf(a[u][i], w[u][i], acc[m]);
      }
    }
  }
  for (; k < kv; k += STEP) {
    float w[V];
    Vec16<T>::load(brow + k, w);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < M) {
        float a[V];
        Vec16<T>::load(A + static_cast<int64_t>(m) * lda + k, a);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[m] = fmaf(a[i], w[i], acc[m]);
      }
    }
  }
  for (int k = kv + lane; k < K; k += 64) {
    const float w = Elem<T>::to_f32(brow[k]);
#pragma unroll
    for (int m = 0; m < 8; ++m)
      if (m < M) acc[m] = fmaf(Elem<T>::to_f32(A[static_cast<int64_t>(m) * lda + k]), w, acc[m]);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < M) {
      const float v = wave_sum(acc[m]);
      if (lane == 0) epi(m, n, v);
    }
  }
}

template <typename T, class Epi>
hipError_t gemv(const T* a, int lda, int M, const T* b0, const T* b1, int n_split, int N, int K,
                const Epi& epi, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<T, Epi>), dim3((N + 3) / 4), dim3(256), 0, s, a, lda, M, b0, b1,
                     n_split, N, K, epi);
  return hipGetLastError();
}

// Instantiations used by the host layer.
template hipError_t gemm_bf16<EpiStore<bf16_t>>(const bf16_t*, int, const bf16_t*, const bf16_t*,
                                                 int, int, int, int, const EpiStore<bf16_t>&,
                                                 hipStream_t);
template hipError_t gemm_bf16<EpiKV<bf16_t>>(const bf16_t*, int, const bf16_t*, const bf16_t*, int,
                                              int, int, int, const EpiKV<bf16_t>&, hipStream_t);
template hipError_t gemm_f32<EpiStore<float>>(const float*, int, const float*, const float*, int,
                                               int, int, int, const EpiStore<float>&, hipStream_t);
template hipError_t gemm_f32<EpiKV<float>>(const float*, int, const float*, const float*, int, int,
                                            int, int, const EpiKV<float>&, hipStream_t);
template hipError_t gemv<bf16_t, EpiStore<bf16_t>>(const bf16_t*, int, int, const bf16_t*,
                                                    const bf16_t*, int, int, int,
                                                    const EpiStore<bf16_t>&, hipStream_t);
template hipError_t gemv<bf16_t, EpiKV<bf16_t>>(const bf16_t*, int, int, const bf16_t*,
                                                 const bf16_t*, int, int, int,
                                                 const EpiKV<bf16_t>&, hipStream_t);
template hipError_t gemv<float, EpiStore<float>>(const float*, int, int, const float*, const float*,
                                                  int, int, int, const EpiStore<float>&,
                                                  hipStream_t);
template hipError_t gemv<float, EpiKV<float>>(const float*, int, int, const float*, const float*,
                                               int, int, int, const EpiKV<float>&, hipStream_t);
template hipError_t gemv<bf16_t, EpiGelu>(const bf16_t*, int, int, const bf16_t*, const bf16_t*, int,
                                          int, int, const EpiGelu&, hipStream_t);
template hipError_t gemv<float, EpiGelu>(const float*, int, int, const float*, const float*, int,
                                         int, int, const EpiGelu&, hipStream_t);

}  // namespace mka
