// Route fusion: X_fused[t] = lambda1 * x_t + lambda2 * L2[t] + lambda3 * L3[t],
// with L3[t] the mean of the retrieved block means (zero when none).  MKA
// reading note, method section 3 (fuse the tiers, then project once); the
// landing page's abstract calls the variant broadcast-routed: each lambda is
// one scalar per token and tier, applied to every channel.
//
// Formed in float32 and rounded once to the storage type, which is the operand
// type of the K/V projection that follows.
#include "kernels.h"

namespace mka {

// RMAX = 0: L3 disabled (no index or block read); USE_L2 = false: L2 disabled
// (not read).  A disabled tier contributes an exact zero, as lambda = 0 with a
// zero tier value, so the sum keeps its form and no unread value enters it.
template <typename T, int RMAX, bool USE_L2>
__global__ __launch_bounds__(256) void fuse_mix_kernel(const T* __restrict__ x,
                                                       const float* __restrict__ l2,
                                                       const float* __restrict__ means, int nb_cap,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ lam, Lam3 lam_c,
                                                       int seq, int D, int R, T* __restrict__ xf) {
  const int64_t row = blockIdx.x;  // b * seq + t
  const int b = static_cast<int>(row / seq);
  const int ch = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (ch >= D) return;
  // lambda per token, or one constant vector for every token (lam == nullptr)
  const float l1w = lam ? lam[row * 3 + 0] : lam_c.v[0];
  const float l2w = lam ? lam[row * 3 + 1] : lam_c.v[1];
  const float l3w = lam ? lam[row * 3 + 2] : lam_c.v[2];
  float xv[4], sv[4] = {0.f, 0.f, 0.f, 0.f}, mean[4] = {0.f, 0.f, 0.f, 0.f};
  load4(x + row * D + ch, xv);
  if constexpr (USE_L2) load4(l2 + row * D + ch, sv);
  if constexpr (RMAX > 0) {
    const int32_t* sel = idx + row * R;
    const float* mb = means + static_cast<int64_t>(b) * nb_cap * D + ch;
    int blk[RMAX];
#pragma unroll
    for (int i = 0; i < RMAX; ++i) blk[i] = i < R ? sel[i] : -1;
    // Every retrieved row is loaded unconditionally (unfilled slots read block
    // 0 and are not added), so the loads are in flight together; rank order.
    float m[RMAX][4];
#pragma unroll
    for (int i = 0; i < RMAX; ++i) load4(mb + static_cast<int64_t>(max(blk[i], 0)) * D, m[i]);
    float l3[4] = {0.f, 0.f, 0.f, 0.f};
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
      const bool on = blk[i] >= 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) l3[k] += on ? m[i][k] : 0.f;
      cnt += on;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) mean[k] = cnt ? l3[k] / static_cast<float>(cnt) : 0.f;
  }
  float out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = l1w * xv[k] + l2w * sv[k] + l3w * mean[k];
  store4(xf + row * D + ch, out);
}

// ---------------------------------------------------------------------------
// L3 through the matrix cores (bf16 layers, many tokens).  L3[t] is the mean of
// at most R of the block means, i.e. row t of S M / cnt_t with S the 0/1
// selection matrix [tokens x blocks] and M the block means [blocks x D].
// Gathered row by row, R whole rows per token go through the L2 cache (16 x
// 16 KB per token at D = 4096); as a product, the means pass through LDS once
// per 128 tokens.  M is split into two bf16 planes, M = hi + lo + r with hi
// its truncation and lo the remainder rounded to nearest (|r| <= 2^-17 |M|),
// stored transposed ([ch][blk], blocks padded to a multiple of 64 with zeros)
// by fuse_split_kernel; S is exact in bf16.  Each product of a 0/1 entry and a
// plane value is exact; the sums are float32 (MFMA 32x32x16).  Blocks at or
// beyond the eligible range (possible for an arbitrary idx) are added from the
// float32 means directly.
// ---------------------------------------------------------------------------
constexpr int kSelTok = 128, kSelCh = 64, kSelKB = 64, kSelMaxBlocks = 256, kSelPad = 8;

// Planes [B][2][D][nbp] (bf16) of the means of blocks [0, n_blk); zeros past
// n_blk.  Workgroup: a 64-block x 64-channel tile through LDS.
__global__ __launch_bounds__(256) void fuse_split_kernel(const float* __restrict__ means,
                                                         int nb_cap, int n_blk, int nbp, int D,
                                                         bf16_t* __restrict__ planes) {
  __shared__ float tile[kSelKB][kSelCh + 1];
  const int tid = threadIdx.x;
  const int blk0 = blockIdx.x * kSelKB, ch0 = blockIdx.y * kSelCh, b = blockIdx.z;
  const float* mb = means + static_cast<int64_t>(b) * nb_cap * D + ch0;
  for (int e = tid; e < kSelKB * kSelCh; e += 256) {
    const int r = e / kSelCh, c = e % kSelCh;
    tile[r][c] = blk0 + r < n_blk ? mb[static_cast<int64_t>(blk0 + r) * D + c] : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < kSelCh * (kSelKB / 2); e += 256) {
    const int c = e / (kSelKB / 2), rp = e % (kSelKB / 2);
    uint32_t hi2 = 0, lo2 = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float m = tile[2 * rp + u][c];
      const uint32_t hb = __float_as_uint(m) & 0xFFFF0000u;  // truncation: m - hi is exact
      const uint32_t lb = f32_to_bf16(m - __uint_as_float(hb));
      hi2 |= (hb >> 16) << (16 * u);
      lo2 |= lb << (16 * u);
    }
    const int64_t o = ((static_cast<int64_t>(b) * 2) * D + ch0 + c) * nbp + blk0 + 2 * rp;
    *reinterpret_cast<uint32_t*>(planes + o) = hi2;
    *reinterpret_cast<uint32_t*>(planes + o + static_cast<int64_t>(D) * nbp) = lo2;
  }
}

// X_fused for 128 tokens x 64 channels per workgroup; wave w takes tokens
// 32w .. 32w+31 and both 32-channel blocks.  Per chunk of 64 blocks: S and the
// two planes' chunk in LDS (rows padded by 16 bytes: the 16 rows of an operand
// read fall in distinct bank groups), 16 MFMAs per wave.
template <int RMAX, bool USE_L2>
__global__ __launch_bounds__(256) void fuse_mix_sel_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ l2, const float* __restrict__ means,
    int nb_cap, const bf16_t* __restrict__ planes, int n_blk, int nbp,
    const int32_t* __restrict__ idx, const float* __restrict__ lam, int seq, int D, int R,
    bf16_t* __restrict__ xf) {
  constexpr int SP = kSelKB + kSelPad;  // padded row length (elements)
  // S [kSelTok][SP] then Ms [2][kSelCh][SP] in one buffer (reused for the L3 tile)
  __shared__ __attribute__((aligned(16))) bf16_t smem[(kSelTok + 2 * kSelCh) * SP];
  bf16_t(*S)[SP] = reinterpret_cast<bf16_t(*)[SP]>(smem);
  bf16_t(*Ms)[kSelCh][SP] = reinterpret_cast<bf16_t(*)[kSelCh][SP]>(smem + kSelTok * SP);
  __shared__ int sel[kSelTok][RMAX];
  __shared__ int cnt[kSelTok], far[kSelTok];
  __shared__ int max_blk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int tok0 = blockIdx.x * kSelTok, ch0 = blockIdx.y * kSelCh, b = blockIdx.z;
  if (tid == 0) max_blk = -1;
  __syncthreads();
  if (tid < kSelTok) {
    const int t = tok0 + tid;
    int c = 0, mx = -1, f = 0;
    if (t < seq) {
      const int32_t* si = idx + (static_cast<int64_t>(b) * seq + t) * R;
#pragma unroll
      for (int i = 0; i < RMAX; ++i) {
        const int blk = i < R ? si[i] : -1;
        sel[tid][i] = blk;
        c += blk >= 0;
        if (blk >= n_blk) f = 1;
        else mx = max(mx, blk);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RMAX; ++i) sel[tid][i] = -1;
    }
    cnt[tid] = c;
    far[tid] = f;
    atomicMax(&max_blk, mx);
  }
  __syncthreads();
  const int n_chunks = (max_blk + kSelKB) / kSelKB;  // chunks holding a selected block
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  const bf16_t* pb = planes + (static_cast<int64_t>(b) * 2 * D + ch0) * nbp;
  // S is zeroed once; a chunk sets its ones and clears them after its products
  // (token row i belongs to thread i).  The next chunk's plane pieces are
  // loaded into registers while the current chunk's products run.
  {
    uint32_t* s32 = reinterpret_cast<uint32_t*>(smem);
    for (int e = tid; e < kSelTok * SP / 2; e += 256) s32[e] = 0u;
  }
  constexpr int PL = 2 * kSelCh * (kSelKB / 8) / 256;  // 16-byte plane pieces per thread
  u32x4 pv[PL];
  auto load_planes = [&](int k0) {
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = tid + 256 * j;
      const int p = e / (kSelCh * (kSelKB / 8)), r = e % (kSelCh * (kSelKB / 8));
      const int c = r / (kSelKB / 8), q = r % (kSelKB / 8);
      pv[j] = *reinterpret_cast<const u32x4*>(pb + (static_cast<int64_t>(p) * D + c) * nbp + k0 +
                                              8 * q);
    }
  };
  auto mark = [&](int k0, bf16_t v) {
    if (tid < kSelTok) {
#pragma unroll
      for (int i = 0; i < RMAX; ++i) {
        const int blk = sel[tid][i];
        if (blk >= k0 && blk < k0 + kSelKB) S[tid][blk - k0] = v;
      }
    }
  };
  if (n_chunks > 0) load_planes(0);
  __syncthreads();  // S zeroed
  for (int ck = 0; ck < n_chunks; ++ck) {
    const int k0 = ck * kSelKB;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = tid + 256 * j;
      const int p = e / (kSelCh * (kSelKB / 8)), r = e % (kSelCh * (kSelKB / 8));
      *reinterpret_cast<u32x4*>(&Ms[p][r / (kSelKB / 8)][8 * (r % (kSelKB / 8))]) = pv[j];
    }
    mark(k0, 0x3F80);  // 1.0
    __syncthreads();
    if (ck + 1 < n_chunks) load_planes(k0 + kSelKB);
#pragma unroll
    for (int ks = 0; ks < kSelKB / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&S[32 * wave + l32][16 * ks + 8 * h]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          acc[nb] = mfma32x32x16(
              a, *reinterpret_cast<const bf16x8*>(&Ms[p][32 * nb + l32][16 * ks + 8 * h]), acc[nb]);
    }
    __syncthreads();  // the chunk's reads are done before S and Ms change
    mark(k0, 0);
  }
  __syncthreads();
  // The L3 sums go through LDS (over S and Ms, no longer read) so that the
  // mix streams x, L2 and X_fused in whole 128-byte row segments: 16 threads
  // per token row, 4 channels each.
  constexpr int LP = kSelCh + 4;
  static_assert(kSelTok * LP * 4 <= static_cast<int>(sizeof(smem)), "the L3 tile fits");
  float* L3s = reinterpret_cast<float*>(smem);  // [kSelTok][LP]
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) L3s[(32 * wave + acc_row(r, h)) * LP + 32 * nb + l32] = acc[nb][r];
  __syncthreads();
  // Each thread takes 8 token rows (16 apart); all their loads are issued
  // before the first row's mix (rows past seq re-read the last row and are
  // not stored).
  const int q = tid & 15, ch = ch0 + 4 * q;
  constexpr int NR = kSelTok / 16;
  const int t_last = min(seq, tok0 + kSelTok) - 1;
  float lw[NR][3], xv[NR][4], sv[NR][4], l3[NR][4];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int i = (tid >> 4) + 16 * u;
    const int64_t row = static_cast<int64_t>(b) * seq + min(tok0 + i, t_last);
    lw[u][0] = lam[row * 3 + 0];
    lw[u][1] = lam[row * 3 + 1];
    lw[u][2] = lam[row * 3 + 2];
    load4(x + row * D + ch, xv[u]);
#pragma unroll
    for (int k = 0; k < 4; ++k) sv[u][k] = 0.f;
    if constexpr (USE_L2) load4(l2 + row * D + ch, sv[u]);
    load4(L3s + i * LP + 4 * q, l3[u]);
  }
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int i = (tid >> 4) + 16 * u, t = tok0 + i;
    if (t > t_last) break;
    const int64_t row = static_cast<int64_t>(b) * seq + t;
    if (far[i]) {  // selected blocks outside the eligible range
#pragma unroll
      for (int j = 0; j < RMAX; ++j) {
        const int blk = sel[i][j];
        if (blk >= n_blk) {
          float m[4];
          load4(means + (static_cast<int64_t>(b) * nb_cap + blk) * D + ch, m);
#pragma unroll
          for (int k = 0; k < 4; ++k) l3[u][k] += m[k];
        }
      }
    }
    const int c = cnt[i];
    const float inv = c ? 1.0f / static_cast<float>(c) : 0.f;
    float out[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[k] = lw[u][0] * xv[u][k] + lw[u][1] * sv[u][k] + lw[u][2] * (c ? l3[u][k] * inv : 0.f);
    store4(xf + row * D + ch, out);
  }
}

template <bool USE_L2>
hipError_t fuse_mix_sel_launch(const bf16_t* x, const float* l2, const float* means, int nb_cap,
                               const bf16_t* planes, int n_blk, int nbp, const int32_t* idx,
                               const float* lam, int B, int seq, int D, int R, bf16_t* xf,
                               hipStream_t s) {
  const dim3 grid((seq + kSelTok - 1) / kSelTok, D / kSelCh, B);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, x, l2, means, nb_cap, planes, n_blk, nbp, idx,
                       lam, seq, D, R, xf);
  };
  if (R <= 4)
    launch(fuse_mix_sel_kernel<4, USE_L2>);
  else if (R <= 8)
    launch(fuse_mix_sel_kernel<8, USE_L2>);
  else if (R <= 16)
    launch(fuse_mix_sel_kernel<16, USE_L2>);
  else
    launch(fuse_mix_sel_kernel<32, USE_L2>);
  return hipGetLastError();
}

size_t fuse_sel_ws_bytes(int B, int D) {
  return static_cast<size_t>(B) * 2 * D * kSelMaxBlocks * sizeof(bf16_t);
}

hipError_t fuse_mix_sel(const bf16_t* x, const float* l2, const float* means, int nb_cap,
                        const int32_t* idx, const float* lam, int B, int seq, int D, int R,
                        Routing rt, bf16_t* xf, int n_blk, void* ws, hipStream_t s) {
  const int nbp = (n_blk + kSelKB - 1) / kSelKB * kSelKB;
  bf16_t* planes = static_cast<bf16_t*>(ws);
  hipLaunchKernelGGL(fuse_split_kernel, dim3(nbp / kSelKB, D / kSelCh, B), dim3(256), 0, s, means,
                     nb_cap, n_blk, nbp, D, planes);
  return rt.l2() ? fuse_mix_sel_launch<true>(x, l2, means, nb_cap, planes, n_blk, nbp, idx, lam,
                                             B, seq, D, R, xf, s)
                 : fuse_mix_sel_launch<false>(x, l2, means, nb_cap, planes, n_blk, nbp, idx, lam,
                                              B, seq, D, R, xf, s);
}

// The product pays for its fixed work per workgroup when each token gathers
// many rows (R >= 8: measured 1014 -> ~840 us at 65536 tokens, R = 16, D = 4096;
// with R = 4 on 2 x 4096 tokens the gather kernel was faster, 110 vs 132 us).
bool fuse_sel_applies(int B, int seq, int D, int R, int n_blk, Routing rt) {
  return rt.l3() && R >= 8 && n_blk >= 1 && n_blk <= kSelMaxBlocks && D % kSelCh == 0 &&
         static_cast<int64_t>(B) * seq >= 1024;
}

template <typename T, bool USE_L2>
hipError_t fuse_mix_launch(dim3 grid, int threads, const T* x, const float* l2,
                           const float* means, int nb_cap, const int32_t* idx, const float* lam,
                           Lam3 lam_c, int seq, int D, int R, bool use_l3, T* xf, hipStream_t s) {
  if (!use_l3)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 0, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else if (R <= 4)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 4, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else if (R <= 8)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 8, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else if (R <= 16)
    hipLaunchKernelGGL((fuse_mix_kernel<T, 16, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  else
    hipLaunchKernelGGL((fuse_mix_kernel<T, 32, USE_L2>), grid, dim3(threads), 0, s, x, l2, means,
                       nb_cap, idx, lam, lam_c, seq, D, R, xf);
  return hipGetLastError();
}

template <typename T>
hipError_t fuse_mix(const T* x, const float* l2, const float* means, int nb_cap,
                    const int32_t* idx, const float* lam, int B, int seq, int D, int R,
                    Routing rt, T* xf, hipStream_t s) {
  // Few tokens: narrow workgroups so that many of them share the row.
  const int threads = static_cast<int64_t>(B) * seq <= 8 ? 64 : 256;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * seq),
                  (D + 4 * threads - 1) / (4 * threads));
  if (rt.l2())
    return fuse_mix_launch<T, true>(grid, threads, x, l2, means, nb_cap, idx, lam, Lam3{}, seq, D,
                                    R, rt.l3(), xf, s);
  return fuse_mix_launch<T, false>(grid, threads, x, l2, means, nb_cap, idx, lam, Lam3{}, seq, D,
                                   R, rt.l3(), xf, s);
}

template <typename T>
hipError_t tier_rows(const T* x, const float* l2, const float* means, int nb_cap,
                     const int32_t* idx, int tier, int B, int seq, int D, int R, T* out,
                     hipStream_t s) {
  const int threads = static_cast<int64_t>(B) * seq <= 8 ? 64 : 256;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * seq),
                  (D + 4 * threads - 1) / (4 * threads));
  Lam3 c{};
  c.v[tier] = 1.0f;
  if (tier == 1)  // L2 alone: no L3 read
    return fuse_mix_launch<T, true>(grid, threads, x, l2, means, nb_cap, idx, nullptr, c, seq, D,
                                    R, false, out, s);
  return fuse_mix_launch<T, false>(grid, threads, x, l2, means, nb_cap, idx, nullptr, c, seq, D, R,
                                   tier == 2, out, s);
}

// ---------------------------------------------------------------------------
// Full MKA's mixture of its attention paths: o = sum_l lambda_l a_l per token,
// lambda broadcast over heads and head dimensions (MKA reading note, method
// section 2).  Paths given as null are disabled tiers and are not read.
// Formed in float32 from the stored path outputs, rounded once.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void mix_paths_kernel(const T* __restrict__ a0,
                                                        const T* __restrict__ a1,
                                                        const T* __restrict__ a2,
                                                        const float* __restrict__ lam, int64_t M,
                                                        int HD, T* __restrict__ o) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= M * HD) return;
  const int64_t row = e / HD;
  const float w0 = lam[row * 3 + 0], w1 = lam[row * 3 + 1], w2 = lam[row * 3 + 2];
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, v[4];
  if (a0) {
    load4(a0 + e, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += w0 * v[k];
  }
  if (a1) {
    load4(a1 + e, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += w1 * v[k];
  }
  if (a2) {
    load4(a2 + e, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += w2 * v[k];
  }
  store4(o + e, acc);
}

template <typename T>
hipError_t mix_paths(const T* a0, const T* a1, const T* a2, const float* lam, int64_t M, int HD,
                     T* o, hipStream_t s) {
  const int64_t n4 = (M * HD + 3) / 4;
  hipLaunchKernelGGL(mix_paths_kernel<T>, dim3(static_cast<unsigned>((n4 + 255) / 256)),
                     dim3(256), 0, s, a0, a1, a2, lam, M, HD, o);
  return hipGetLastError();
}

template hipError_t tier_rows<float>(const float*, const float*, const float*, int,
                                     const int32_t*, int, int, int, int, int, float*, hipStream_t);
template hipError_t tier_rows<bf16_t>(const bf16_t*, const float*, const float*, int,
                                      const int32_t*, int, int, int, int, int, bf16_t*,
                                      hipStream_t);
template hipError_t mix_paths<float>(const float*, const float*, const float*, const float*,
                                     int64_t, int, float*, hipStream_t);
template hipError_t mix_paths<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, const float*,
                                      int64_t, int, bf16_t*, hipStream_t);

template hipError_t fuse_mix<float>(const float*, const float*, const float*, int, const int32_t*,
                                    const float*, int, int, int, int, Routing, float*,
                                    hipStream_t);
template hipError_t fuse_mix<bf16_t>(const bf16_t*, const float*, const float*, int,
                                     const int32_t*, const float*, int, int, int, int, Routing,
                                     bf16_t*, hipStream_t);

}  // namespace mka
