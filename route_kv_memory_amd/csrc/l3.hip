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
// SimHash projections on fp64 MFMA (v_mfma_f64_16x16x4f64).  Operand layout,
// lane l: A[l % 16][l / 16], B[l / 16][l % 16]; accumulator register r holds
// C[4r + l/16][l % 16].  A workgroup computes 64 rows x 64 hyperplanes over one
// slice of D: each wave 16 rows x 4 blocks of 16 hyperplanes.  k-tiles of 64
// channels of both operands are staged in LDS as fp32 and widened to fp64 in
// registers; every product of two fp32 values is exact in fp64.
// With one slice the codes are written directly (signs gathered by ballot);
// with several, each slice writes its partial sums and simhash_finalize adds
// them in slice order.
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kHashKT = 64, kHashPitch = kHashKT + 4;

__global__ __launch_bounds__(256) void simhash_mfma_kernel(
    const float* __restrict__ v, int64_t v_bstride, int rows, int D, const float* __restrict__ P,
    int nbits, int k_per_split, uint64_t* __restrict__ codes, int64_t c_bstride,
    double* __restrict__ part) {
  __shared__ float Vs[64 * kHashPitch];
  __shared__ float Ps[64 * kHashPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blockIdx.x * 64, split = blockIdx.y, b = blockIdx.z;
  const int k_begin = split * k_per_split, k_end = min(D, k_begin + k_per_split);
  const float* vb = v + b * v_bstride;
  f64x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int li = lane & 15, lk = lane >> 4;
  // Tile loads are unconditional (rows and channels past the ends read a
  // valid address and are replaced by zero), and tile k+1 is loaded into
  // registers while tile k is multiplied.
  f32x4 ra[4], rp[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i, r = e >> 4, c = (e & 15) * 4;  // 64 rows x 16 float4
      const bool kin = k0 + c < k_end;
      const int kc = kin ? k0 + c : k_begin;
      ra[i] = *reinterpret_cast<const f32x4*>(vb + static_cast<int64_t>(min(row0 + r, rows - 1)) * D + kc);
      rp[i] = *reinterpret_cast<const f32x4*>(P + static_cast<int64_t>(min(r, nbits - 1)) * D + kc);
      if (!(row0 + r < rows && kin)) ra[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!(r < nbits && kin)) rp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (k_begin < k_end) load_tile(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += kHashKT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i, r = e >> 4, c = (e & 15) * 4;
      *reinterpret_cast<f32x4*>(&Vs[r * kHashPitch + c]) = ra[i];
      *reinterpret_cast<f32x4*>(&Ps[r * kHashPitch + c]) = rp[i];
    }
    __syncthreads();
    if (k0 + kHashKT < k_end) load_tile(k0 + kHashKT);
#pragma unroll 4
    for (int kk = 0; kk < kHashKT; kk += 4) {
      const double a = Vs[(wave * 16 + li) * kHashPitch + kk + lk];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double p = Ps[(j * 16 + li) * kHashPitch + kk + lk];
        acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, p, acc[j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (part != nullptr) {
    // part[((split * B + b) * rows + row) * 64 + bit]
    double* pb = part + (static_cast<int64_t>(split) * gridDim.z + b) * rows * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wave * 16 + 4 * r + lk;
        if (row < rows) pb[static_cast<int64_t>(row) * 64 + 16 * j + li] = acc[j][r];
      }
    return;
  }
  // Lanes 16q..16q+15 of register r hold row 4r + q, hyperplanes 16j + (lane % 16).
  uint64_t bal[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) bal[j][r] = __ballot(acc[j][r] > 0.0);
  if (lane < 16) {
    const int r = lane >> 2, q = lane & 3;
    const int row = row0 + wave * 16 + 4 * r + q;
    uint64_t code = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint64_t bj = 0;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (rr == r) bj = bal[j][rr];
      code |= ((bj >> (16 * q)) & 0xFFFFull) << (16 * j);
    }
    if (row < rows) codes[b * c_bstride + row] = code;
  }
}

// Sum the slice partials in slice order and take the signs: one wave per row.
__global__ __launch_bounds__(256) void simhash_finalize_kernel(const double* __restrict__ part,
                                                               int rows, int B, int nsplit,
                                                               int nbits,
                                                               uint64_t* __restrict__ codes,
                                                               int64_t c_bstride) {
  const int lane = threadIdx.x & 63;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (e >= static_cast<int64_t>(B) * rows) return;
  const int b = static_cast<int>(e / rows), row = static_cast<int>(e - static_cast<int64_t>(b) * rows);
  // partials loaded 8 at a time, added in split order
  double p = 0.0;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = part[((static_cast<int64_t>(min(s0 + u, nsplit - 1)) * B + b) * rows + row) * 64 + lane];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < nsplit) p += v[u];
  }
  const uint64_t code = __ballot(lane < nbits && p > 0.0);
  if (lane == 0) codes[b * c_bstride + row] = code;
}

int simhash_splits(int rows, int B, int D) {
  const int tiles = ((rows + 63) / 64) * B;
  const int ktiles = (D + kHashKT - 1) / kHashKT;
  int ns = (512 + tiles - 1) / tiles;
  return ns < 1 ? 1 : (ns > ktiles ? ktiles : ns);
}

size_t simhash_ws_bytes(int rows, int B, int D) {
  const int ns = simhash_splits(rows, B, D);
  return ns > 1 ? sizeof(double) * static_cast<size_t>(ns) * B * rows * 64 : 0;
}

// Launch the projections; with more than one slice the partials go to ``part``.
static hipError_t simhash_launch(const float* v, int64_t v_bstride, int rows, int B, int D,
                                 const float* proj, int nbits, int nsplit, uint64_t* codes,
                                 int64_t codes_bstride, double* part, hipStream_t s) {
  const int ktiles = (D + kHashKT - 1) / kHashKT;
  const int k_per_split = ((ktiles + nsplit - 1) / nsplit) * kHashKT;
  const int ns = (D + k_per_split - 1) / k_per_split;
  hipLaunchKernelGGL(simhash_mfma_kernel, dim3((rows + 63) / 64, ns, B), dim3(256), 0, s, v,
                     v_bstride, rows, D, proj, nbits, k_per_split, codes, codes_bstride,
                     ns > 1 ? part : nullptr);
  if (ns > 1 && codes != nullptr)
    hipLaunchKernelGGL(simhash_finalize_kernel, dim3((B * rows + 3) / 4), dim3(256), 0, s, part,
                       rows, B, ns, nbits, codes, codes_bstride);
  return hipGetLastError();
}

hipError_t simhash_rows(const float* v, int64_t v_bstride, int rows, int B, int D,
                        const float* proj, int nbits, uint64_t* codes, int64_t codes_bstride,
                        void* ws, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return simhash_launch(v, v_bstride, rows, B, D, proj, nbits, simhash_splits(rows, B, D), codes,
                        codes_bstride, static_cast<double*>(ws), s);
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
// workgroups (fp64 partial sums in the workspace); one workgroup per token
// then sums them in slice order, forms the key, and selects the top R among
// all its eligible blocks (each thread keeps a sorted list of its own
// candidates; R rounds of a workgroup minimum pop the best head).
// ---------------------------------------------------------------------------
size_t retrieve_few_ws_bytes(int rows, int D) {
  const int ns = (D + kHashKT - 1) / kHashKT;
  return sizeof(double) * static_cast<size_t>(ns) * rows * 64;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1)
    v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}

template <int RMAX>
__global__ __launch_bounds__(256) void select_few_kernel(const double* __restrict__ part, int rows,
                                                         int n_slices, int nbits, int seq,
                                                         int64_t pos0, const uint64_t* __restrict__ bh,
                                                         int nb_cap, int block, int R,
                                                         uint64_t* __restrict__ keys,
                                                         int32_t* __restrict__ idx) {
  __shared__ uint64_t key_s;
  __shared__ uint32_t cand[4][RMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;  // row = b * seq + t
  const int b = r / seq;
  const int64_t t = r - static_cast<int64_t>(b) * seq;
  if (wave == 0) {
    double p = 0.0;
#pragma unroll 8
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
  // Each wave pops its R best (keys are unique, so exactly one lane pops).
  for (int i = 0; i < R; ++i) {
    const uint32_t m = wave_min_u32(top[0]);
    if (top[0] == m && m != kEmpty) {
#pragma unroll
      for (int k = 0; k < RMAX - 1; ++k) top[k] = top[k + 1];
      top[RMAX - 1] = kEmpty;
    }
    if (lane == 0) cand[wave][i] = m;
  }
  __syncthreads();
  if (wave != 0) return;
  // Wave 0 merges the 4 sorted lists: lane l holds entries l and l + 64.
  const uint32_t* flat = &cand[0][0];
  uint32_t c0 = kEmpty, c1 = kEmpty;
  {
    const int e0 = lane, e1 = lane + 64;
    if (e0 < 4 * R) c0 = flat[(e0 / R) * RMAX + e0 % R];
    if (e1 < 4 * R) c1 = flat[(e1 / R) * RMAX + e1 % R];
    if (c1 < c0) { const uint32_t tmp = c0; c0 = c1; c1 = tmp; }
  }
  int32_t* out = idx + static_cast<int64_t>(r) * R;
  for (int i = 0; i < R; ++i) {
    const uint32_t m = wave_min_u32(c0);
    if (c0 == m && m != kEmpty) {
      c0 = c1;
      c1 = kEmpty;
    }
    if (lane == 0) out[i] = m == kEmpty ? -1 : cand_block(m);
  }
}

hipError_t select_codes_topr(const double* part, int rows, int n_slices, int nbits, int seq,
                             int64_t pos0, const uint64_t* bh, int nb_cap, int block, int R,
                             uint64_t* keys, int32_t* idx, hipStream_t s) {
  if (R <= 16)
    hipLaunchKernelGGL(select_few_kernel<16>, dim3(rows), dim3(256), 0, s, part, rows, n_slices,
                       nbits, seq, pos0, bh, nb_cap, block, R, keys, idx);
  else
    hipLaunchKernelGGL(select_few_kernel<32>, dim3(rows), dim3(256), 0, s, part, rows, n_slices,
                       nbits, seq, pos0, bh, nb_cap, block, R, keys, idx);
  return hipGetLastError();
}

hipError_t retrieve_few(const float* l2, int B, int seq, int D, const float* proj, int nbits,
                        const uint64_t* bh, int nb_cap, int block, int R, int64_t pos0,
                        uint64_t* keys, int32_t* idx, void* ws, hipStream_t s) {
  const int rows = B * seq;
  const int n_slices = (D + kHashKT - 1) / kHashKT;
  double* part = static_cast<double*>(ws);
  // rows are contiguous [B*seq, D]: one "batch" of B*seq rows, one slice per k-tile
  const hipError_t e = simhash_launch(l2, 0, rows, 1, D, proj, nbits, n_slices, nullptr, 0, part, s);
  if (e != hipSuccess) return e;
  if (R <= 16)
    hipLaunchKernelGGL(select_few_kernel<16>, dim3(rows), dim3(256), 0, s, part, rows, n_slices,
                       nbits, seq, pos0, bh, nb_cap, block, R, keys, idx);
  else
    hipLaunchKernelGGL(select_few_kernel<32>, dim3(rows), dim3(256), 0, s, part, rows, n_slices,
                       nbits, seq, pos0, bh, nb_cap, block, R, keys, idx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Projected block means: block_kv[b, blk, n] = m_blk . W[n] for the columns of
// W = [W_k; W_v] (n < kvw: row n of W_k, else row n - kvw of W_v).  A wave
// computes 4 columns for up to 8 blocks; lanes stride D with 16-byte loads of
// the weights.  Kept beside the bank so that a decode step can form L3 W as a
// mean of R rows instead of a product with W.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void block_kv_kernel(const float* __restrict__ means, int nb_cap,
                                                       int first, int n_blocks,
                                                       const T* __restrict__ w_k,
                                                       const T* __restrict__ w_v, int kvw, int D,
                                                       float* __restrict__ out) {
  constexpr int NC = 4, NB = 8, V = Vec16<T>::kN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nkv = 2 * kvw;
  const int n0 = (blockIdx.x * 4 + wave) * NC;
  if (n0 >= nkv) return;
  const int blk0 = first + blockIdx.y * NB, nb = min(NB, first + n_blocks - blk0);
  const int b = blockIdx.z;
  const T* w[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = min(n0 + c, nkv - 1);
    w[c] = col < kvw ? w_k + static_cast<int64_t>(col) * D : w_v + static_cast<int64_t>(col - kvw) * D;
  }
  const float* mrow = means + (static_cast<int64_t>(b) * nb_cap + blk0) * D;
  float acc[NC][NB] = {};
  for (int k = lane * V; k < D; k += 64 * V) {
    float wv[NC][V];
#pragma unroll
    for (int c = 0; c < NC; ++c) Vec16<T>::load(w[c] + k, wv[c]);
    // the block rows are loaded unconditionally (past the range: the last
    // block again, not stored) so the loads are in flight together
    float mv[NB][V];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < V; i += 4) load4(mrow + static_cast<int64_t>(min(j, nb - 1)) * D + k + i, mv[j] + i);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[c][j] = fmaf(mv[j][i], wv[c][i], acc[c][j]);
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < nb) {
        const float v = wave_sum(acc[c][j]);
        if (lane == 0 && n0 + c < nkv)
          out[(static_cast<int64_t>(b) * nb_cap + blk0 + j) * nkv + n0 + c] = v;
      }
    }
}

template <typename T>
hipError_t block_kv_project(const float* means, int nb_cap, int first, int n_blocks, const T* w_k,
                            const T* w_v, int kvw, int D, int B, float* out, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  const dim3 grid((2 * kvw + 15) / 16, (n_blocks + 7) / 8, B);
  hipLaunchKernelGGL(block_kv_kernel<T>, grid, dim3(256), 0, s, means, nb_cap, first, n_blocks,
                     w_k, w_v, kvw, D, out);
  return hipGetLastError();
}
template hipError_t block_kv_project<float>(const float*, int, int, int, const float*,
                                            const float*, int, int, int, float*, hipStream_t);
template hipError_t block_kv_project<bf16_t>(const float*, int, int, int, const bf16_t*,
                                             const bf16_t*, int, int, int, float*, hipStream_t);

}  // namespace mka
