// Dense NT products on gfx950: bf16 MFMA tiles, a plain fp32 tiled kernel and a
// small-M (decode) kernel.
#include "gemm.h"

namespace mka {

// s_waitcnt immediate that waits for every LDS operation of the wave
// (vmcnt and expcnt left at their maxima).
constexpr int kLgkmcntZero = 0xF | (0x3 << 14) | (0x7 << 4);

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.  Workgroup tile 256 (M) x BN (N), 8 waves; each wave owns
// 128 x BN/4 of C as 4 x BN/128 blocks of MFMA 32x32x16.  The MFMA computes
// C^T blocks (B rows as its A operand), which leaves 4 consecutive output
// columns of one output row in each lane: the epilogue stores 8 bytes per lane.
//
// Operands stream global -> LDS directly (global_load_lds, 16 bytes per lane,
// no registers) through a ring of STAGES k-slices of 32, so the loads of a
// slice are issued STAGES-1 slices before it is used.  A row of a slice is 64
// bytes (4 chunks of 16); chunk c of row r is stored at position
// c ^ ((r >> 2) & 3), which keeps both the 1 KB contiguous LDS writes of a
// load instruction and the 16-row fragment reads of the MFMA free of bank
// conflicts.  Rows past M or N are read from the last valid row; their outputs
// are not stored.
// ---------------------------------------------------------------------------
template <int BN, int NW>
struct GemmCfg {
  static constexpr int BM = 256, BK = 32, ROWB = BK * 2;  // bytes per row per slice
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int SLICE = A_BYTES + B_BYTES;
  static constexpr int STAGES = (160 * 1024) / SLICE;      // 5 for BN=256, 6 for BN=128
  static constexpr int LOADS = SLICE / 1024 / NW;           // load instructions per wave per slice
  static constexpr int WN = BN / (NW / 2);                  // wave tile: 128 x WN
  static constexpr int NB = WN / 32;                        // MFMA blocks per wave in N
};

// blockIdx.y selects a range of K_len reduction indices starting at
// blockIdx.y * K_len (split-K; K is the row length of B).  DB: fragments
// double-buffered in registers (below); without it a slice's fragments are
// read after its barrier, in fewer registers (room for other kernels' waves
// on the same SIMDs).
template <int BN, int NW, bool DB, class Epi>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int n_split, int M, int N, int K, int K_len, Epi epi) {
  using C = GemmCfg<BN, NW>;
  constexpr int BM = C::BM, BK = C::BK, ROWB = C::ROWB, STAGES = C::STAGES, NB = C::NB;
  constexpr int WN = C::WN;
  static_assert(C::LOADS * NW * 1024 == C::SLICE, "slice must split evenly over the waves");
  static_assert(STAGES >= 3, "the ring holds the slice in use, the next one and one in flight");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES * C::SLICE];

  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  if (tiles_m % 4 == 0 && tiles_n % 2 == 0) {
    // Workgroups reach the 8 XCDs round-robin; XCD x takes the block of tiles
    // rows [x/2 * tiles_m/4, +tiles_m/4) x columns [x%2 * tiles_n/2, +tiles_n/2),
    // so its concurrent tiles share few A and B panels in its L2.
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8, bn = tiles_n / 2;
    tm = (xcd >> 1) * (tiles_m / 4) + local / bn;
    tn = (xcd & 1) * bn + local % bn;
  } else {
    const int item = xcd_contiguous(blockIdx.x, tiles_n * tiles_m);
    tm = item / tiles_n;
    tn = item % tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int wm = wave & 1, wn = wave >> 1, h = lane >> 5, l32 = lane & 31;

  // This lane's rows and byte offsets for each of its load instructions of a
  // slice: instruction j of wave w covers 16 rows of A (first A_BYTES/1024
  // instructions) or of B; lane l takes row 16*ri + l/4, chunk (l%4) ^ swizzle.
  const bf16_t* src[C::LOADS];
  int dst[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int gi = wave * C::LOADS + j;  // instruction index within the slice
    const bool is_a = gi < C::A_BYTES / 1024;
    const int ri = is_a ? gi : gi - C::A_BYTES / 1024;
    const int row = 16 * ri + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    if (is_a) {
      const int gm = min(m0 + row, M - 1);
      src[j] = A + static_cast<int64_t>(gm) * lda + blockIdx.y * K_len + chunk * 8;
    } else {
      const int gn = min(n0 + row, N - 1);
      src[j] = (gn < n_split ? B0 + static_cast<int64_t>(gn) * K
                             : B1 + static_cast<int64_t>(gn - n_split) * K) +
               blockIdx.y * K_len + chunk * 8;
    }
    dst[j] = (is_a ? 0 : C::A_BYTES) + ri * 1024;  // lane's 16 bytes land at +16*lane
  }
  auto issue = [&](int slice, int stage) {
    unsigned char* base = lds + stage * C::SLICE;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j)
      global_load_lds16(src[j] + slice * BK, (lds_void_t*)(base + dst[j]));
  };

  // acc[i][j]: C^T block of output rows m0 + wm*128 + 32i .., columns n0 + wn*WN + 32j ..
  f32x16 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  // fragment byte offset of row r, chunk c (16 bytes) within a slice operand
  auto frag = [](int r, int c) { return r * ROWB + ((c ^ ((r >> 2) & 3)) << 4); };

  const int nk_all = K_len / BK;
  if constexpr (DB) {
  const int nk = nk_all;
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s, s);
  // Fragments are double-buffered in registers: a slice's fragments are read
  // from LDS during the previous slice's MFMAs, so no wave starts a slice
  // waiting on LDS.  The barrier of iteration kt therefore waits until slice
  // kt+1 has landed; and since every wave has slice kt in registers by then
  // (reads complete before the barrier), slice kt's stage is refilled with
  // slice kt+STAGES right after it: STAGES-1 slices stay in flight.
  typedef bf16x8 FragA[2][4];
  typedef bf16x8 FragB[2][NB];
  auto read_slice = [&](int kt, FragA& fa, FragB& fb) {
    const unsigned char* As = lds + (kt % STAGES) * C::SLICE;
    const unsigned char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[ks][i] =
            *reinterpret_cast<const bf16x8*>(As + frag(wm * 128 + i * 32 + l32, 2 * ks + h));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[ks][j] = *reinterpret_cast<const bf16x8*>(Bs + frag(wn * WN + j * 32 + l32, 2 * ks + h));
    }
  };
  // One slice: wait for slice kt+1, barrier, refill slice kt's stage, read
  // slice kt+1's fragments into (na, nb) while the MFMAs consume (ca, cb).
  // After the last slice the read takes a stale stage and is not used.
  auto step = [&](int kt, const FragA& ca, const FragB& cb, FragA& na, FragB& nb) {
    if (kt + STAGES - 1 < nk) {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 2)>());
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
    }
    __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
    // A bare barrier: a fence here would wait for the prefetches too.
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES < nk) issue(kt + STAGES, kt % STAGES);
    read_slice(kt + 1, na, nb);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32x32x16(cb[ks][j], ca[ks][i], acc[i][j]);
    // one LDS read after each MFMA, the rest at the end
    constexpr int R = (BK / 16) * (4 + NB), F = (BK / 16) * 4 * NB;
    constexpr int P = R < F ? R : F;
#pragma unroll
    for (int u = 0; u < P; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (F > P) __builtin_amdgcn_sched_group_barrier(0x008, F - P, 0);
    if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
  };
  FragA xa, ya;
  FragB xb, yb;
  if (STAGES - 1 < nk) {
    __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 1)>());
  } else {
    __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
  }
  __builtin_amdgcn_s_barrier();
  read_slice(0, xa, xb);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, xa, xb, ya, yb);
    step(kt + 1, ya, yb, xa, xb);
  }
  if (kt < nk) step(kt, xa, xb, ya, yb);

  } else {
  const int nk = nk_all;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    // slice kt has landed once at most the STAGES-2 younger slices are pending
    if (kt + STAGES - 2 < nk) {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 2)>());
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
    }
    // Every wave's part of slice kt is in LDS (each waited for its own loads)
    // and every wave is done reading slice kt-1.  A bare barrier: a fence here
    // would wait for the prefetches too.
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const unsigned char* As = lds + (kt % STAGES) * C::SLICE;
    const unsigned char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[4], fb[NB];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(As + frag(wm * 128 + i * 32 + l32, 2 * ks + h));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(Bs + frag(wn * WN + j * 32 + l32, 2 * ks + h));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32x32x16(fb[j], fa[i], acc[i][j]);
    }
  }

  }

  // Lane holds output row m = ... + l32 and columns n = ... + 8*(r/4) + 4h + (r%4).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + i * 32 + l32;
    if (m >= M) continue;
    if constexpr (std::is_same<Epi, EpiAdd>::value) {
      // accumulate: the row's 4*NB quads are read together, then written
      float old[NB][4][4];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          epi.load4(m, n0 + wn * WN + j * 32 + 8 * rq + 4 * h, N, old[j][rq]);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = old[j][rq][e] + acc[i][j][4 * rq + e];
          epi.put4(m, n0 + wn * WN + j * 32 + 8 * rq + 4 * h, v, N);
        }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int n = n0 + wn * WN + j * 32 + 8 * rq + 4 * h;
          const float v[4] = {acc[i][j][4 * rq], acc[i][j][4 * rq + 1], acc[i][j][4 * rq + 2],
                              acc[i][j][4 * rq + 3]};
          epi.store4(m, n, v, N);
        }
    }
  }
}

constexpr int kGemmWaves256 = 8;

template <class Epi>
hipError_t gemm_bf16(const bf16_t* a, int lda, const bf16_t* b0, const bf16_t* b1, int n_split,
                     int M, int N, int K, const Epi& epi, hipStream_t s, bool single_buffer) {
  const int tiles256 = ((N + 255) / 256) * ((M + 255) / 256);
  if (tiles256 >= 256) {
    if (single_buffer)
      hipLaunchKernelGGL((gemm_bf16_kernel<256, kGemmWaves256, false, Epi>), dim3(tiles256),
                         dim3(kGemmWaves256 * 64), 0, s, a, lda, b0, b1, n_split, M, N, K, K, epi);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<256, kGemmWaves256, true, Epi>), dim3(tiles256),
                         dim3(kGemmWaves256 * 64), 0, s, a, lda, b0, b1, n_split, M, N, K, K, epi);
  } else {
    const int tiles = ((N + 127) / 128) * ((M + 255) / 256);
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 8, true, Epi>), dim3(tiles), dim3(512), 0, s, a, lda,
                       b0, b1, n_split, M, N, K, K, epi);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K for products with few output tiles (the weight gradients: a few
// hundred rows, thousands of columns, a reduction over all tokens): the
// reduction is cut into S ranges, one grid row each, whose float32 partials go
// to a workspace; a second kernel adds them in range order (deterministic)
// and hands the sum to the epilogue.
// ---------------------------------------------------------------------------
struct EpiPart {  // partial of range blockIdx.y: row-major [S][M][N]
  float* base;
  int ldc;
  int64_t stride;
  __device__ __forceinline__ void store4(int m, int n, const float* v, int N) const {
    float* p = base + blockIdx.y * stride + static_cast<int64_t>(m) * ldc + n;
    if (n + 3 < N) {
      mka::store4(p, v);
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) p[i] = v[i];
    }
  }
};

template <class Epi>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ part, int S,
                                                         int M, int N, Epi epi) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t total = static_cast<int64_t>(M) * N;
  if (e >= total) return;
  const int m = static_cast<int>(e / N), n = static_cast<int>(e - static_cast<int64_t>(m) * N);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < S; ++sp) {
    const float* p = part + sp * total + e;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += p[i];
  }
  epi.store4(m, n, v, N);
}

// Ranges: as many as fill one round of the CUs (at most 8), each a multiple of
// the k-slice; 1 when the product already has a round of tiles.
int gemm_splitk_ranges(int M, int N, int K) {
  const int tm = (M + 255) / 256;
  if (((N + 255) / 256) * tm >= 256 || N % 4 != 0) return 1;
  const int tiles = ((N + 127) / 128) * tm;
  int S = 1;
  for (int c = 2; c <= 8; ++c)
    if (c * tiles <= 256 && K % (c * 32) == 0 && K / c >= 256) S = c;
  return S;
}

size_t gemm_bf16_splitk_ws_bytes(int M, int N, int K) {
  const int S = gemm_splitk_ranges(M, N, K);
  return S > 1 ? sizeof(float) * static_cast<size_t>(S) * M * N : 0;
}

template <class Epi>
hipError_t gemm_bf16_splitk(const bf16_t* a, int lda, const bf16_t* b, int M, int N, int K,
                            const Epi& epi, float* ws, hipStream_t s) {
  const int S = gemm_splitk_ranges(M, N, K);
  if (S == 1) return gemm_bf16(a, lda, b, b, N, M, N, K, epi, s);
  const int tiles = ((N + 127) / 128) * ((M + 255) / 256);
  const EpiPart part{ws, N, static_cast<int64_t>(M) * N};
  hipLaunchKernelGGL((gemm_bf16_kernel<128, 8, true, EpiPart>), dim3(tiles, S), dim3(512), 0, s, a, lda,
                     b, b, N, M, N, K, K / S, part);
  const int64_t quads = (static_cast<int64_t>(M) * N + 3) / 4;
  hipLaunchKernelGGL((splitk_sum_kernel<Epi>), dim3(static_cast<unsigned>((quads + 255) / 256)),
                     dim3(256), 0, s, ws, S, M, N, epi);
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
                                                 hipStream_t, bool);
template hipError_t gemm_bf16<EpiKV<bf16_t>>(const bf16_t*, int, const bf16_t*, const bf16_t*, int,
                                              int, int, int, const EpiKV<bf16_t>&, hipStream_t,
                                              bool);
template hipError_t gemm_bf16<EpiStore<float>>(const bf16_t*, int, const bf16_t*, const bf16_t*,
                                                int, int, int, int, const EpiStore<float>&,
                                                hipStream_t, bool);
template hipError_t gemm_bf16<EpiAdd>(const bf16_t*, int, const bf16_t*, const bf16_t*, int, int,
                                      int, int, const EpiAdd&, hipStream_t, bool);
template hipError_t gemm_bf16_splitk<EpiStore<float>>(const bf16_t*, int, const bf16_t*, int, int,
                                                      int, const EpiStore<float>&, float*,
                                                      hipStream_t);
template hipError_t gemm_bf16_splitk<EpiAdd>(const bf16_t*, int, const bf16_t*, int, int, int,
                                             const EpiAdd&, float*, hipStream_t);
template hipError_t gemm_f32<EpiAdd>(const float*, int, const float*, const float*, int, int, int,
                                     int, const EpiAdd&, hipStream_t);
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
