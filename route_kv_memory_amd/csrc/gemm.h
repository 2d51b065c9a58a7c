// Dense products used by the layer: Q = X W_q and [K|V] = X_fused [W_k|W_v].
// Weights are stored [out, in], so both MFMA operands are contiguous along
// the reduction dimension ("NT" product C[m][n] = sum_k A[m][k] * B[n][k]).
#pragma once

#include "common.h"

namespace mka {

// Row-major store C[m * ldc + n].
template <typename T>
struct EpiStore {
  T* c;
  int ldc;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    c[static_cast<int64_t>(m) * ldc + n] = Elem<T>::from_f32(v);
  }
  // Columns n .. n+3 (n % 4 == 0); those at or past N are dropped.
  __device__ __forceinline__ void store4(int m, int n, const float* v, int N) const {
    T* p = c + static_cast<int64_t>(m) * ldc + n;
    if (n + 3 < N) {
      mka::store4(p, v);
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) p[i] = Elem<T>::from_f32(v[i]);
    }
  }
};

// Row-major accumulate C[m * ldc + n] += v (float32 gradients).
struct EpiAdd {
  float* c;
  int ldc;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    c[static_cast<int64_t>(m) * ldc + n] += v;
  }
  __device__ __forceinline__ void store4(int m, int n, const float* v, int N) const {
    float old[4];
    load4(m, n, N, old);
    const float sum[4] = {old[0] + v[0], old[1] + v[1], old[2] + v[2], old[3] + v[3]};
    put4(m, n, sum, N);
  }
  // The two halves of store4, so that a kernel can issue the reads of many
  // quads before their writes (one wait for the lot instead of one per quad).
  // Columns n .. n+3 (n % 4 == 0); those at or past N are neither read nor written.
  __device__ __forceinline__ void load4(int m, int n, int N, float* old) const {
    const float* p = c + static_cast<int64_t>(m) * ldc + n;
    if (n + 3 < N) {
      mka::load4(p, old);
    } else {
      for (int i = 0; i < 4; ++i) old[i] = n + i < N ? p[i] : 0.f;
    }
  }
  __device__ __forceinline__ void put4(int m, int n, const float* v, int N) const {
    float* p = c + static_cast<int64_t>(m) * ldc + n;
    if (n + 3 < N) {
      mka::store4(p, v);
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) p[i] = v[i];
    }
  }
};

// Scatter into the head-major fused KV cache [B, G, t_cap, dh]: row m is token
// t = m % seq of sequence b = m / seq, stored at cache row pos0 + t; columns
// [0, G*dh) are K and [G*dh, 2*G*dh) are V.
template <typename T>
struct EpiKV {
  T* k;
  T* v;
  int seq;
  int n_kv_heads;
  int head_dim;
  KvLayout kv;    // the cache layout (contiguous or paged)
  int64_t pos0;
  __device__ __forceinline__ void operator()(int m, int n, float val) const {
    const int kvw = n_kv_heads * head_dim;
    T* base = n < kvw ? k : v;
    const int nn = n < kvw ? n : n - kvw;
    const int b = m / seq, t = m - b * seq;
    const int g = nn / head_dim, d = nn - g * head_dim;
    base[kv.row(b, g, pos0 + t) + d] = Elem<T>::from_f32(val);
  }
  // Columns n .. n+3 (n % 4 == 0) lie in one head row since head_dim % 4 == 0.
  __device__ __forceinline__ void store4(int m, int n, const float* vals, int N) const {
    if (n >= N) return;
    const int kvw = n_kv_heads * head_dim;
    T* base = n < kvw ? k : v;
    const int nn = n < kvw ? n : n - kvw;
    const int b = m / seq, t = m - b * seq;
    const int g = nn / head_dim, d = nn - g * head_dim;
    mka::store4(base + kv.row(b, g, pos0 + t) + d, vals);
  }
};

// GELU of the product into a float32 row-major buffer (router hidden layer).
struct EpiGelu {
  float* h;
  int ld;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    h[static_cast<int64_t>(m) * ld + n] = gelu(v);
  }
};

// Launchers (defined in gemm.hip).  B rows [0, n_split) come from b0, rows
// [n_split, N) from b1 (row n - n_split); pass n_split = N for one matrix.
// single_buffer: the register-lean loop, for a product that runs beside other
// kernels (more of their waves fit on its SIMDs).
template <class Epi>
hipError_t gemm_bf16(const bf16_t* a, int lda, const bf16_t* b0, const bf16_t* b1, int n_split,
                     int M, int N, int K, const Epi& epi, hipStream_t s,
                     bool single_buffer = false);
template <class Epi>
hipError_t gemm_f32(const float* a, int lda, const float* b0, const float* b1, int n_split,
                    int M, int N, int K, const Epi& epi, hipStream_t s);
// The same with one B matrix, the reduction split into ranges when the output
// has too few tiles to fill the GPU; the float32 partials take
// gemm_bf16_splitk_ws_bytes(M, N, K) bytes of ``ws`` (none when that is 0).
size_t gemm_bf16_splitk_ws_bytes(int M, int N, int K);
template <class Epi>
hipError_t gemm_bf16_splitk(const bf16_t* a, int lda, const bf16_t* b, int M, int N, int K,
                            const Epi& epi, float* ws, hipStream_t s);
// C[m][n] = sum_k A(m, k) B(n, k) with B stored K-major (element (n, k) at
// b[k * ldb + n]) and A stored K-major (a[k * lda + m]) when ``a_kmajor``, else
// K-contiguous (a[m * lda + k]).  K is a multiple of 32; reduction indices at or
// past k_rows (<= K) count as zeros and are not read (k_rows < K needs both
// operands K-major).  lda and ldb are multiples of 8, a and b 16-byte aligned, N % 4
// == 0; hipErrorInvalidValue otherwise.  The reduction is split as in
// gemm_bf16_splitk, its partials in ``ws`` (gemm_bf16_splitk_ws_bytes(M, N, K)).
template <class Epi>
hipError_t gemm_bf16_km(const bf16_t* a, int lda, bool a_kmajor, const bf16_t* b, int ldb, int M,
                        int N, int K, int k_rows, const Epi& epi, float* ws, hipStream_t s);
// Small-M product (M <= 8), one wave per output column: the decode path.
template <typename T, class Epi>
hipError_t gemv(const T* a, int lda, int M, const T* b0, const T* b1, int n_split, int N, int K,
                const Epi& epi, hipStream_t s);

// k-tile of gemm_bf16; it needs K % kGemmBK == 0, N % 4 == 0 and 16-byte
// aligned rows (checked by the host layer before launching).
constexpr int kGemmBK = 64;

}  // namespace mka
