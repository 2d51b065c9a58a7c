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
#include <cmath>
#include <type_traits>

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

// ---------------------------------------------------------------------------
// SimHash codes of many rows on bf16 MFMA, every sign certified.
//
// Each float32 operand is split into bf16 parts x = h + l + r.  The rows a
// are split by truncation (h is a with its low 16 bits cleared, l the same of
// a - h, both subtractions exact): |a - h| < 2^-7 |a|, |l| < 2^-7 |a|,
// |r| < 2^-14 |a|.  The hyperplanes p are split once per call with rounding
// to nearest even: |p - h| <= 2^-8 |p|, |l| <= 2^-8 (1 + 2^-8) |p|,
// |r| <= 2^-16 |p|.  The product a . p is approximated by
// s = sum_k (h_a h_p + h_a l_p + l_a h_p), the bf16 products being exact in
// float32, on MFMA 32x32x16 with float32 accumulation.  Per channel the
// dropped terms h_a r_p + l_a l_p + l_a r_p + r_a p are below
// (2^-14 + 2^-15 + 2^-16 + 2^-21) |a_k||p_k| and the kept ones below
// (1 + 2^-6) |a_k||p_k|; n float32 additions in any order, each with relative
// error below 2^-23, add at most gamma_n = n 2^-23 / (1 - n 2^-23) times the
// sum of their magnitudes.  So
//   |s - a . p| <= ((1 + 2^-6) gamma_n + 2^-14 + 2^-15 + 2^-16 + 2^-21)
//                  sum_k |a_k||p_k|,
// and over a slice of the channels sum |a_k||p_k| <= ||a|| ||p|| (Cauchy-
// Schwarz).  A bit whose |s| exceeds the bound has the sign of the exact
// product; the others (about one in a hundred) are recomputed in float64 from
// the float32 operands, each product exact, as in the kernel above.
//
// Workgroup: 32 rows x 64 hyperplanes; wave w of 16 sums one sixteenth of
// the channels and the slices are added in float64 in slice order.  Per 32
// channels a lane loads 16 consecutive floats of its row (lanes l and l+32
// share a row), which feed two MFMA k-steps: the order of the channels inside
// a k-step is free as long as both operands use the same one.
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 16, kFixChunk = 8;

// bf16 bits of the high halves of x0 (low) and x1 (high): truncation.
__device__ __forceinline__ uint32_t hi_pair(uint32_t x0, uint32_t x1) {
  return __builtin_amdgcn_perm(x1, x0, 0x07060302u);
}
// Truncated bf16 parts of 8 floats.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  uint32_t wh[4], wl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b0 = __float_as_uint(x[2 * i]), b1 = __float_as_uint(x[2 * i + 1]);
    const float r0 = x[2 * i] - __uint_as_float(b0 & 0xFFFF0000u);
    const float r1 = x[2 * i + 1] - __uint_as_float(b1 & 0xFFFF0000u);
    wh[i] = hi_pair(b0, b1);
    wl[i] = hi_pair(__float_as_uint(r0), __float_as_uint(r1));
  }
  hi = __builtin_bit_cast(bf16x8, u32x4{wh[0], wh[1], wh[2], wh[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], wl[2], wl[3]});
}

// Sum over the wave in a fixed butterfly: every lane ends with the same value.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// bf16 bits of x rounded to nearest even (finite x).
__device__ __forceinline__ uint32_t rne_bf16_bits(uint32_t b) {
  return (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
}

// Hyperplanes split once per call, in the order the MFMA operands are loaded:
// for channel pair-block pb (32 channels) and load q = 4 part + 2 t + st,
// lane l holds 8 channels 32 pb + 16 (l / 32) + 8 st .. of plane 32 t + l % 32
// (part 0: hi, 1: lo), so each load of the main kernel reads 1 KB
// contiguous.  Planes j >= nbits are zero.  Blocks npairs.. compute
// Pn[w][j] = ||proj row j|| over wave w's channel slice instead.
__global__ __launch_bounds__(1024) void simhash_split_prep_kernel(const float* __restrict__ P,
                                                                 int nbits, int D, int slice,
                                                                 bf16_t* __restrict__ Ps,
                                                                 double* __restrict__ Pn) {
  const int npairs = D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  if (static_cast<int>(blockIdx.x) < npairs) {
    if (tid >= 512) return;
    const int pb = blockIdx.x, q = tid >> 6;
    const int part_ = q >> 2, t = (q >> 1) & 1, st = q & 1;
    const int j = 32 * t + (lane & 31), k0 = 32 * pb + 16 * (lane >> 5) + 8 * st;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t half[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float x = j < nbits ? P[static_cast<int64_t>(j) * D + k0 + e + u] : 0.f;
        const uint32_t hb = rne_bf16_bits(__float_as_uint(x));
        const float r = x - __uint_as_float(hb);  // exact
        half[u] = (part_ == 0 ? hb : rne_bf16_bits(__float_as_uint(r))) >> 16;
      }
      w[e / 2] = half[0] | (half[1] << 16);
    }
    *reinterpret_cast<u32x4*>(Ps + ((static_cast<int64_t>(pb) * 8 + q) * 64 + lane) * 8) =
        u32x4{w[0], w[1], w[2], w[3]};
    return;
  }
  const int j = blockIdx.x - npairs, wv = tid >> 6;
  const int k0 = wv * slice, k1 = min(D, k0 + slice);
  double sq = 0.0;
  for (int k = k0 + lane; k < k1; k += 64) {
    const float x = j < nbits ? P[static_cast<int64_t>(j) * D + k] : 0.f;
    sq = fma(static_cast<double>(x), static_cast<double>(x), sq);
  }
  sq = wave_sum_f64(sq);
  if (lane == 0) Pn[wv * 64 + j] = sqrt(sq);
}

// Staged rows: a wave's 32 rows x 32 channels (4 KB) arrive by 4 direct-to-LDS
// loads of 8 rows x 128 bytes; 16-byte chunk c of row r sits at
// (r / 8) * 1024 + (r % 8) * 128 + 16 * (c ^ ((r / 2) % 8)), which keeps the
// operand reads (lane: row l % 32, chunks 4 (l / 32) ..) free of bank conflicts.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) void*)(p)));
}
__device__ __forceinline__ int staged_chunk(int r, int c) {
  return (r >> 3) * 1024 + (r & 7) * 128 + 16 * (c ^ ((r >> 1) & 7));
}

__global__ __launch_bounds__(1024) void simhash_split_kernel(
    const float* __restrict__ v, int64_t v_bstride, int rows, int D, const float* __restrict__ P,
    int nbits, const bf16_t* __restrict__ Ps, const double* __restrict__ Pn, int pairs_per_wave,
    double err_factor, uint64_t* __restrict__ codes, int64_t c_bstride) {
  // staging buffers (2 x 4 KB per wave) during the products, slice sums after
  __shared__ __attribute__((aligned(1024))) float part[kSplitWaves][32][64];
  __shared__ float nrm[kSplitWaves][32];
  // codes of the tile's rows and the list of its undecided (row, hyperplane) bits
  __shared__ uint64_t code_s[32];
  __shared__ uint32_t undecided[32 * 64];
  __shared__ int n_undecided;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int row0 = blockIdx.x * 32, b = blockIdx.y;
  const float* vb = v + b * v_bstride;
  const int npairs = D / 32;
  const int p0 = wave * pairs_per_wave, p1 = min(npairs, p0 + pairs_per_wave);
  unsigned char* stage = reinterpret_cast<unsigned char*>(&part[0][0][0]) + wave * 8192;
  // load i of a pair: lane L fetches row 8i + L/8, chunk (L % 8) ^ ((row / 2) % 8),
  // through a resource over this batch's rows (rows past the end read as zeros)
  const __amdgpu_buffer_rsrc_t rsrc =
      make_rsrc(vb, static_cast<uint32_t>(static_cast<int64_t>(rows) * D * 4));
  const uint32_t row_bytes = static_cast<uint32_t>(D) * 4u;
  uint32_t off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    off[i] = static_cast<uint32_t>(row0 + r) * row_bytes + 16u * ((lane & 7) ^ ((r >> 1) & 7));
  }
  const bf16x8* pq = reinterpret_cast<const bf16x8*>(Ps) + lane;
  // Loads of pair p (its stage buffer and its hyperplane registers).  The last
  // iteration fetches its own pair again (p clamped), so every iteration
  // issues the same loads and the waits below stay exact.
  auto issue = [&](int p, int buf, bf16x8* pw) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      buffer_load_lds16(rsrc, (lds_void_t*)(stage + buf * 4096 + i * 1024), off[i] + 128u * p);
#pragma unroll
    for (int q = 0; q < 8; ++q) pw[q] = pq[(p * 8 + q) * 64];
  };
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  float sq = 0.f;
  // One pair: fetch the next one (into the other stage buffer and register
  // set), wait for this one, multiply.  Unrolled by two so that the register
  // sets alternate without copies.
  auto step = [&](int p, const bf16x8* pw, bf16x8* pn) {
    const int buf = (p - p0) & 1;
    issue(min(p + 1, p1 - 1), buf ^ 1, pn);  // the stage read two pairs ago
    // pair p has landed once at most the 12 loads just issued are pending
    __builtin_amdgcn_s_waitcnt(kVmcntPending<12>());
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // The two chunks of this k-step, read in one block that also waits for
      // them (the compiler would otherwise make every LDS read wait for the
      // direct-to-LDS prefetch issued above as well).
      const uint32_t base = lds_addr(stage + buf * 4096);
      const uint32_t a0 = base + staged_chunk(l32, 4 * h + 2 * st);
      const uint32_t a1 = base + staged_chunk(l32, 4 * h + 2 * st + 1);
      f32x4 t0, t1;
      asm volatile(
          "ds_read_b128 %0, %2\n\t"
          "ds_read_b128 %1, %3\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(t0), "=&v"(t1)
          : "v"(a0), "v"(a1)
          : "memory");
      float x[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = t0[u];
        x[4 + u] = t1[u];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sq = fmaf(x[e], x[e], sq);
      bf16x8 ah, al;
      split8(x, ah, al);
      acc0 = mfma32x32x16(ah, pw[0 + st], acc0);
      acc0 = mfma32x32x16(ah, pw[4 + st], acc0);
      acc0 = mfma32x32x16(al, pw[0 + st], acc0);
      acc1 = mfma32x32x16(ah, pw[2 + st], acc1);
      acc1 = mfma32x32x16(ah, pw[6 + st], acc1);
      acc1 = mfma32x32x16(al, pw[2 + st], acc1);
    }
  };
  bf16x8 pa[8], pb[8];
  if (p0 < p1) issue(p0, 0, pa);
  int p = p0;
  for (; p + 1 < p1; p += 2) {
    step(p, pa, pb);
    step(p + 1, pb, pa);
  }
  if (p < p1) step(p, pa, pb);
  __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());  // the last, repeated fetch too
  __syncthreads();  // every wave is done with its staging buffers
  // slice sums (register r: row acc_row(r, h), hyperplane l32 or 32 + l32)
  // and the squared row norm over the slice
  const float sqr = sq + __shfl_xor(sq, 32);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    part[wave][acc_row(r, h)][l32] = acc0[r];
    part[wave][acc_row(r, h)][32 + l32] = acc1[r];
  }
  if (h == 0) nrm[wave][l32] = sqr;
  if (tid == 0) n_undecided = 0;
  __syncthreads();

  // wave: rows 2*wave, 2*wave+1 of the tile; lane: hyperplane
  constexpr int kRowsPerWave = 32 / kSplitWaves;
  const bool on = lane < nbits;
#pragma unroll 1
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int i = wave * kRowsPerWave + rr;
    double s = 0.0, e = 0.0;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      s += static_cast<double>(part[w][i][lane]);
      // the float32 sum of squares is inflated past its own rounding
      e += sqrt(static_cast<double>(nrm[w][i]) * (1.0 + 1e-4)) * Pn[w * 64 + lane];
    }
    e = e * err_factor + 1e-30;
    const uint64_t code = __ballot(on && s > 0.0);
    const uint64_t amb = __ballot(on && fabs(s) <= e);
    if (lane == 0) code_s[i] = code;
    if (amb != 0) {  // uniform over the wave: list the undecided bits
      int first = 0;
      if (lane == 0) first = atomicAdd(&n_undecided, __popcll(amb));
      first = __shfl(first, 0, 64);
      if ((amb >> lane) & 1)
        undecided[first + __popcll(amb & ((1ull << lane) - 1))] = (i << 8) | lane;
    }
  }
  __syncthreads();
  // Float64 recomputation of the undecided bits, spread over all the waves of
  // the workgroup: the row (up to kFixChunk float4 per lane at a time) and the
  // hyperplane are loaded together, each product exact.
  const int n_fix = n_undecided;
  for (int w = wave; w < n_fix; w += kSplitWaves) {
    const uint32_t entry = undecided[w];
    const int i = static_cast<int>(entry >> 8), j = static_cast<int>(entry & 255);
    const float* full = vb + static_cast<int64_t>(min(row0 + i, rows - 1)) * D;
    const float* pj = P + static_cast<int64_t>(j) * D;
    auto load_chunk = [&](const float* src, int c0, f32x4* dst) {
#pragma unroll
      for (int u = 0; u < kFixChunk; ++u) {
        const int k = c0 + 256 * u + 4 * lane;
        dst[u] = k < D ? *reinterpret_cast<const f32x4*>(src + k) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    double t[4] = {0.0, 0.0, 0.0, 0.0};
    for (int c0 = 0; c0 < D; c0 += 256 * kFixChunk) {
      f32x4 xa[kFixChunk], xp[kFixChunk];
      load_chunk(full, c0, xa);
      load_chunk(pj, c0, xp);
#pragma unroll
      for (int u = 0; u < kFixChunk; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          t[c] = fma(static_cast<double>(xa[u][c]), static_cast<double>(xp[u][c]), t[c]);
    }
    const double tt = wave_sum_f64((t[0] + t[1]) + (t[2] + t[3]));
    if (lane == 0) {
      if (tt > 0.0)
        atomicOr(reinterpret_cast<unsigned long long*>(&code_s[i]), 1ull << j);
      else
        atomicAnd(reinterpret_cast<unsigned long long*>(&code_s[i]), ~(1ull << j));
    }
  }
  __syncthreads();
  if (tid < 32 && row0 + tid < rows) codes[b * c_bstride + row0 + tid] = code_s[tid];
}

// The certified path: D a multiple of 32, enough rows to fill the GPU, and a
// batch's rows addressable with 32-bit byte offsets; otherwise the float64
// kernel.
static bool simhash_use_split(int rows, int B, int D) {
  return static_cast<int64_t>(rows) * B >= 256 && D % 32 == 0 &&
         static_cast<int64_t>(rows) * D * 4 < (int64_t{1} << 31);
}
static int split_pairs_per_wave(int D) { return (D / 32 + kSplitWaves - 1) / kSplitWaves; }
static size_t split_ws_bytes(int D) {
  return static_cast<size_t>(2) * 64 * D * sizeof(bf16_t) + kSplitWaves * 64 * sizeof(double);
}

int simhash_splits(int rows, int B, int D) {
  const int tiles = ((rows + 63) / 64) * B;
  const int ktiles = (D + kHashKT - 1) / kHashKT;
  int ns = (512 + tiles - 1) / tiles;
  return ns < 1 ? 1 : (ns > ktiles ? ktiles : ns);
}

static size_t fp64_ws_bytes(int rows, int B, int D) {
  const int ns = simhash_splits(rows, B, D);
  return ns > 1 ? sizeof(double) * static_cast<size_t>(ns) * B * rows * 64 : 0;
}

// Enough for any call with at most ``rows`` rows: below the certified path's
// row count the float64 partials grow with the rows (the slice count is
// capped there), so the largest such call bounds them.
size_t simhash_ws_bytes(int rows, int B, int D) {
  if (!simhash_use_split(rows, B, D)) return fp64_ws_bytes(rows, B, D);
  const int below = (256 + B - 1) / B - 1;  // most rows that still take the float64 path
  const size_t f = below > 0 ? fp64_ws_bytes(below < rows ? below : rows, B, D) : 0;
  const size_t w = split_ws_bytes(D);
  return f > w ? f : w;
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

bool simhash_prepared_path(int rows, int B, int D) { return simhash_use_split(rows, B, D); }
size_t simhash_prep_bytes(int D) { return split_ws_bytes(D); }

hipError_t simhash_prepare(const float* proj, int nbits, int D, void* prep, hipStream_t s) {
  bf16_t* ps = static_cast<bf16_t*>(prep);
  double* pn = reinterpret_cast<double*>(static_cast<char*>(prep) +
                                         static_cast<size_t>(2) * 64 * D * sizeof(bf16_t));
  hipLaunchKernelGGL(simhash_split_prep_kernel, dim3(D / 32 + 64), dim3(1024), 0, s, proj, nbits, D,
                     32 * split_pairs_per_wave(D), ps, pn);
  return hipGetLastError();
}

hipError_t simhash_rows_prepared(const float* v, int64_t v_bstride, int rows, int B, int D,
                                 const float* proj, int nbits, const void* prep, uint64_t* codes,
                                 int64_t codes_bstride, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const bf16_t* ps = static_cast<const bf16_t*>(prep);
  const double* pn = reinterpret_cast<const double*>(
      static_cast<const char*>(prep) + static_cast<size_t>(2) * 64 * D * sizeof(bf16_t));
  const int ppw = split_pairs_per_wave(D);
  // (1 + 2^-6) gamma_n + 2^-14 + 2^-15 + 2^-16 + 2^-21 for n = 3 * 32 * ppw
  // additions, with 2% margin
  const double n = 3.0 * 32.0 * ppw, u = std::ldexp(1.0, -23);
  const double gamma = n * u / (1.0 - n * u);
  const double factor =
      1.02 * ((1.0 + std::ldexp(1.0, -6)) * gamma + std::ldexp(1.0, -14) + std::ldexp(1.0, -15) +
              std::ldexp(1.0, -16) + std::ldexp(1.0, -21));
  hipLaunchKernelGGL(simhash_split_kernel, dim3((rows + 31) / 32, B), dim3(1024), 0, s, v,
                     v_bstride, rows, D, proj, nbits, ps, pn, ppw, factor, codes, codes_bstride);
  return hipGetLastError();
}

hipError_t simhash_rows(const float* v, int64_t v_bstride, int rows, int B, int D,
                        const float* proj, int nbits, uint64_t* codes, int64_t codes_bstride,
                        void* ws, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (simhash_use_split(rows, B, D)) {
    const hipError_t e = simhash_prepare(proj, nbits, D, ws, s);
    if (e != hipSuccess) return e;
    return simhash_rows_prepared(v, v_bstride, rows, B, D, proj, nbits, ws, codes, codes_bstride,
                                 s);
  }
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
  // block codes loaded 16 at a time before their insertions (one load per
  // insertion had made the loop wait on every code)
  for (int j0 = 0; j0 < ne; j0 += 16) {
    uint64_t cv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) cv[u] = codes[min(j0 + u, ne - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (j0 + u < ne) insert_sorted(top, cand_key(key, cv[u], j0 + u));
  }
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

// The same with bf16 weights, on MFMA 32x32x16: the float32 means are split
// by truncation into bf16 parts m = h + l + r (|r| < 2^-14 |m|) and each part
// meets the bf16 weight row exactly, with float32 accumulation (relative error
// of the result of the order of 1e-5).  Workgroup: 32 blocks x 32 columns;
// 8 waves each sum one eighth of D, loading a group of 4 k-steps ahead, and
// the eighths are added in LDS in wave order.
constexpr int kBkvWaves = 8, kBkvGroup = 4;

__global__ __launch_bounds__(512) void block_kv_mfma_kernel(const float* __restrict__ means,
                                                            int nb_cap, int first, int n_blocks,
                                                            const bf16_t* __restrict__ w_k,
                                                            const bf16_t* __restrict__ w_v,
                                                            int kvw, int D,
                                                            float* __restrict__ out) {
  __shared__ float red[kBkvWaves][32][33];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int nkv = 2 * kvw, n0 = blockIdx.x * 32, blk0 = first + blockIdx.y * 32, b = blockIdx.z;
  const int nb = min(32, first + n_blocks - blk0);
  // lane: block row l32 (past the range: the last block again, not stored) and
  // weight row n0 + l32, channels 8h.. of each k-step of 16
  const float* arow =
      means + (static_cast<int64_t>(b) * nb_cap + blk0 + min(l32, nb - 1)) * D + 8 * h;
  const int col = n0 + l32;
  const bf16_t* wrow =
      (col < kvw ? w_k + static_cast<int64_t>(col) * D : w_v + static_cast<int64_t>(col - kvw) * D) +
      8 * h;
  const int groups = D / (16 * kBkvGroup);
  const int per = (groups + kBkvWaves - 1) / kBkvWaves;
  const int g0 = wave * per, g1 = min(groups, g0 + per);
  struct Grp {
    f32x4 a[2 * kBkvGroup];
    bf16x8 w[kBkvGroup];
  };
  auto load = [&](int g, Grp& t) {
#pragma unroll
    for (int u = 0; u < kBkvGroup; ++u) {
      const int k = 16 * (kBkvGroup * g + u);
      t.a[2 * u] = *reinterpret_cast<const f32x4*>(arow + k);
      t.a[2 * u + 1] = *reinterpret_cast<const f32x4*>(arow + k + 4);
      t.w[u] = *reinterpret_cast<const bf16x8*>(wrow + k);
    }
  };
  f32x16 acc = f32x16{};
  // One group: load the next one into the other buffer (the last group again
  // at the end), multiply this one.  Unrolled by two: the buffers alternate.
  auto step = [&](int g, const Grp& cur, Grp& nxt) {
    load(min(g + 1, g1 - 1), nxt);
#pragma unroll
    for (int u = 0; u < kBkvGroup; ++u) {
      float x[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[c] = cur.a[2 * u][c];
        x[4 + c] = cur.a[2 * u + 1][c];
      }
      bf16x8 mh, ml;
      split8(x, mh, ml);
      acc = mfma32x32x16(mh, cur.w[u], acc);
      acc = mfma32x32x16(ml, cur.w[u], acc);
    }
  };
  Grp ga, gb;
  if (g0 < g1) load(g0, ga);
  int g = g0;
  for (; g + 1 < g1; g += 2) {
    step(g, ga, gb);
    step(g + 1, gb, ga);
  }
  if (g < g1) step(g, ga, gb);
  // register r of lane half h: block row acc_row(r, h), column l32
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][acc_row(r, h)][l32] = acc[r];
  __syncthreads();
  for (int e = tid; e < 32 * 32; e += 512) {
    const int i = e >> 5, j = e & 31;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kBkvWaves; ++w) v += red[w][i][j];
    if (i < nb) out[(static_cast<int64_t>(b) * nb_cap + blk0 + i) * nkv + n0 + j] = v;
  }
}

template <typename T>
hipError_t block_kv_project(const float* means, int nb_cap, int first, int n_blocks, const T* w_k,
                            const T* w_v, int kvw, int D, int B, float* out, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (kvw % 16 == 0 && D % (16 * kBkvGroup) == 0) {
      const dim3 grid(2 * kvw / 32, (n_blocks + 31) / 32, B);
      hipLaunchKernelGGL(block_kv_mfma_kernel, grid, dim3(512), 0, s, means, nb_cap, first,
                         n_blocks, w_k, w_v, kvw, D, out);
      return hipGetLastError();
    }
  }
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
