// L3 long-term memory: SimHash codes and Hamming top-R retrieval.
//
// The MKA reading note (method section 1) recalls R << T past blocks through a
// vectorised hash index; the landing page's Table 8 caption uses the top-8
// retrieved chunks per query.  Reading taken: SimHash of block means (bit j =
// [m . p_j > 0]); the query key is the SimHash of L2[t]; eligible blocks are
// those before t's own block; rank by (Hamming distance ascending, block index
// descending).
//
// The sign of each projection decides an integer, so the dot products are
// accumulated in float64 from the float32 operands (each product is exact in
// float64): the code is then the sign of an almost exact value.
#include "kernels.h"

namespace mka {

// Sort key of a candidate: smaller is better.  Distance in bits 24..30, and
// 0xFFFFFF - b below it so that equal distances prefer the larger block index.
// Never 0 (b < 0xFFFFFF) and never 0xFFFFFFFF (the empty slot).
__device__ __forceinline__ uint32_t cand_key(uint64_t key, uint64_t code, int b) {
  return (static_cast<uint32_t>(__popcll(key ^ code)) << 24) | (0xFFFFFFu - static_cast<uint32_t>(b));
}
__device__ __forceinline__ int cand_block(uint32_t k) { return static_cast<int>(0xFFFFFFu - (k & 0xFFFFFFu)); }
constexpr uint32_t kEmpty = 0xFFFFFFFFu;

// Insert v into the ascending list top[0..N): a compare-exchange chain.
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
// SimHash of many rows: a workgroup takes 32 rows x 64 hyperplanes; k-tiles of
// 64 channels of both operands are staged in LDS; a thread accumulates 4 rows
// x 2 hyperplanes in float64; codes are assembled with wave ballots.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void simhash_rows_kernel(const float* __restrict__ v,
                                                           int64_t v_bstride, int rows, int D,
                                                           const float* __restrict__ P, int nbits,
                                                           uint64_t* __restrict__ codes,
                                                           int64_t c_bstride) {
  __shared__ float Vs[32][65];
  __shared__ float Ps[64][65];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blockIdx.x * 32, b = blockIdx.y;
  const float* vb = v + b * v_bstride;
  const int rg = tid >> 5, bp = tid & 31;
  double acc[4][2] = {};
  for (int k0 = 0; k0 < D; k0 += 64) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + 256 * i, r = e >> 6, kk = e & 63;
      Vs[r][kk] = (row0 + r < rows && k0 + kk < D) ? vb[static_cast<int64_t>(row0 + r) * D + k0 + kk] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = tid + 256 * i, j = e >> 6, kk = e & 63;
      Ps[j][kk] = (j < nbits && k0 + kk < D) ? P[static_cast<int64_t>(j) * D + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 64; ++kk) {
      const double p0 = Ps[bp][kk], p1 = Ps[bp + 32][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = Vs[4 * rg + i][kk];
        acc[i][0] = fma(a, p0, acc[i][0]);
        acc[i][1] = fma(a, p1, acc[i][1]);
      }
    }
    __syncthreads();
  }
  // Lanes 0..31 of wave w hold row group 2w, lanes 32..63 row group 2w+1; lane
  // bit bp of a ballot is hyperplane bp (first ballot) or bp + 32 (second).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t lo = __ballot(acc[i][0] > 0.0);
    const uint64_t hi = __ballot(acc[i][1] > 0.0);
    const int r_even = row0 + 4 * (2 * wave) + i, r_odd = row0 + 4 * (2 * wave + 1) + i;
    if (lane == 0 && r_even < rows)
      codes[b * c_bstride + r_even] = (lo & 0xFFFFFFFFull) | (hi << 32);
    if (lane == 32 && r_odd < rows)
      codes[b * c_bstride + r_odd] = (lo >> 32) | (hi & 0xFFFFFFFF00000000ull);
  }
}

hipError_t simhash_rows(const float* v, int64_t v_bstride, int rows, int B, int D,
                        const float* proj, int nbits, uint64_t* codes, int64_t codes_bstride,
                        hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(simhash_rows_kernel, dim3((rows + 31) / 32, B), dim3(256), 0, s, v, v_bstride,
                     rows, D, proj, nbits, codes, codes_bstride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-R for many tokens: one lane per token keeps its R best candidates in a
// sorted register list.  Tokens of a wave are consecutive, so the block codes
// they scan are the same (a broadcast load).
// ---------------------------------------------------------------------------
template <int RMAX>
__global__ __launch_bounds__(256) void topr_rows_kernel(const uint64_t* __restrict__ keys, int B,
                                                        int seq, int64_t pos0,
                                                        const uint64_t* __restrict__ bh, int nb_cap,
                                                        int block, int R, int32_t* __restrict__ idx) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(B) * seq) return;
  const int b = static_cast<int>(e / seq);
  const int64_t t = e - static_cast<int64_t>(b) * seq;
  const int ne = static_cast<int>((pos0 + t) / block);
  const uint64_t key = keys[e];
  const uint64_t* codes = bh + static_cast<int64_t>(b) * nb_cap;
  uint32_t top[RMAX];
#pragma unroll
  for (int i = 0; i < RMAX; ++i) top[i] = kEmpty;
  for (int j = 0; j < ne; ++j) insert_sorted(top, cand_key(key, codes[j], j));
  int32_t* out = idx + e * R;
#pragma unroll
  for (int i = 0; i < RMAX; ++i)
    if (i < R) out[i] = top[i] == kEmpty ? -1 : cand_block(top[i]);
}

hipError_t topr_rows(const uint64_t* keys, int B, int seq, int64_t pos0, const uint64_t* bh,
                     int nb_cap, int block, int R, int32_t* idx, hipStream_t s) {
  const dim3 grid((static_cast<int64_t>(B) * seq + 255) / 256);
  if (R <= 4)
    hipLaunchKernelGGL(topr_rows_kernel<4>, grid, dim3(256), 0, s, keys, B, seq, pos0, bh, nb_cap, block, R, idx);
  else if (R <= 8)
    hipLaunchKernelGGL(topr_rows_kernel<8>, grid, dim3(256), 0, s, keys, B, seq, pos0, bh, nb_cap, block, R, idx);
  else if (R <= 16)
    hipLaunchKernelGGL(topr_rows_kernel<16>, grid, dim3(256), 0, s, keys, B, seq, pos0, bh, nb_cap, block, R, idx);
  else
    hipLaunchKernelGGL(topr_rows_kernel<32>, grid, dim3(256), 0, s, keys, B, seq, pos0, bh, nb_cap, block, R, idx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Few tokens (decode): the key projections are split over D across many
// workgroups (partial sums in float64 in the workspace), then one workgroup
// per token sums them, forms the key, and selects the top R among all its
// eligible blocks (each thread keeps a sorted list of its own candidates; R
// rounds of a workgroup minimum pop the best head).
// ---------------------------------------------------------------------------
constexpr int kSliceCh = 128;

size_t retrieve_few_ws_bytes(int rows, int D) {
  const int n_slices = (D + kSliceCh - 1) / kSliceCh;
  return sizeof(double) * static_cast<size_t>(n_slices) * rows * 64;
}

__global__ __launch_bounds__(256) void hash_partial_kernel(const float* __restrict__ l2, int rows,
                                                           int D, const float* __restrict__ P,
                                                           int nbits, double* __restrict__ part) {
  __shared__ float Ps[64][kSliceCh + 1];
  __shared__ float Vs[kFewRows][kSliceCh];
  __shared__ double red[4][kFewRows][64];
  const int tid = threadIdx.x, s = blockIdx.x, c0 = s * kSliceCh;
  for (int e = tid; e < 64 * kSliceCh; e += 256) {
    const int j = e / kSliceCh, c = e % kSliceCh;
    Ps[j][c] = (j < nbits && c0 + c < D) ? P[static_cast<int64_t>(j) * D + c0 + c] : 0.f;
  }
  for (int e = tid; e < rows * kSliceCh; e += 256) {
    const int r = e / kSliceCh, c = e % kSliceCh;
    Vs[r][c] = c0 + c < D ? l2[static_cast<int64_t>(r) * D + c0 + c] : 0.f;
  }
  __syncthreads();
  const int j = tid & 63, cg = tid >> 6;
  for (int r = 0; r < rows; ++r) {
    double acc = 0.0;
#pragma unroll 8
    for (int c = cg * 32; c < cg * 32 + 32; ++c)
      acc = fma(static_cast<double>(Vs[r][c]), static_cast<double>(Ps[j][c]), acc);
    red[cg][r][j] = acc;
  }
  __syncthreads();
  for (int e = tid; e < rows * 64; e += 256) {
    const int r = e / 64, jj = e % 64;
    part[(static_cast<int64_t>(s) * rows + r) * 64 + jj] =
        ((red[0][r][jj] + red[1][r][jj]) + red[2][r][jj]) + red[3][r][jj];
  }
}

template <int RMAX>
__global__ __launch_bounds__(256) void select_few_kernel(const double* __restrict__ part, int rows,
                                                         int n_slices, int nbits, int seq,
                                                         int64_t pos0, const uint64_t* __restrict__ bh,
                                                         int nb_cap, int block, int R,
                                                         uint64_t* __restrict__ keys,
                                                         int32_t* __restrict__ idx) {
  __shared__ uint64_t key_s;
  __shared__ uint32_t wmin[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;  // row = b * seq + t
  const int b = r / seq;
  const int64_t t = r - static_cast<int64_t>(b) * seq;
  if (wave == 0) {
    double p = 0.0;
    for (int s = 0; s < n_slices; ++s) p += part[(static_cast<int64_t>(s) * rows + r) * 64 + lane];
    const uint64_t code = __ballot(lane < nbits && p > 0.0);
    if (lane == 0) {
      key_s = code;
      keys[r] = code;
    }
  }
  __syncthreads();
  const uint64_t key = key_s;
  const int ne = static_cast<int>((pos0 + t) / block);
  const uint64_t* codes = bh + static_cast<int64_t>(b) * nb_cap;
  uint32_t top[RMAX];
#pragma unroll
  for (int i = 0; i < RMAX; ++i) top[i] = kEmpty;
  for (int j = tid; j < ne; j += 256) insert_sorted(top, cand_key(key, codes[j], j));
  int32_t* out = idx + static_cast<int64_t>(r) * R;
  for (int i = 0; i < R; ++i) {
    uint32_t m = top[0];
    for (int off = 32; off >= 1; off >>= 1) m = min(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, 64)));
    if (lane == 0) wmin[wave] = m;
    __syncthreads();
    const uint32_t best = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
    __syncthreads();
    if (top[0] == best && best != kEmpty) {
#pragma unroll
      for (int k = 0; k < RMAX - 1; ++k) top[k] = top[k + 1];
      top[RMAX - 1] = kEmpty;
    }
    if (tid == 0) out[i] = best == kEmpty ? -1 : cand_block(best);
  }
}

hipError_t retrieve_few(const float* l2, int B, int seq, int D, const float* proj, int nbits,
                        const uint64_t* bh, int nb_cap, int block, int R, int64_t pos0,
                        uint64_t* keys, int32_t* idx, void* ws, hipStream_t s) {
  const int rows = B * seq;
  const int n_slices = (D + kSliceCh - 1) / kSliceCh;
  double* part = static_cast<double*>(ws);
  hipLaunchKernelGGL(hash_partial_kernel, dim3(n_slices), dim3(256), 0, s, l2, rows, D, proj, nbits,
                     part);
  if (R <= 16)
    hipLaunchKernelGGL(select_few_kernel<16>, dim3(rows), dim3(256), 0, s, part, rows, n_slices,
                       nbits, seq, pos0, bh, nb_cap, block, R, keys, idx);
  else
    hipLaunchKernelGGL(select_few_kernel<32>, dim3(rows), dim3(256), 0, s, part, rows, n_slices,
                       nbits, seq, pos0, bh, nb_cap, block, R, keys, idx);
  return hipGetLastError();
}

}  // namespace mka
