// Backward of the FastMKA layer: the derivative of the forward taken step by
// step in reverse (the pages give none; the abstract page's headline is
// training throughput, Tables 1, 2 and 6).  No gradient flows through the
// SimHash codes, the top-R choice or a hard router's choice of tiers.
//
// Attention (reading note, method sections 3-4; the forward keeps each query
// row's log-sum-exp): with P = softmax(S), S = q k^T / sqrt(dh),
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dq = dS k / sqrt(dh),  dk = dS^T q / sqrt(dh),
// the KV heads' gradients summed over their query heads.  The rest: the
// transposed products of the projections, the fusion's tier products, the
// EMA's adjoint (a reverse scan), the block means' adjoint (a scatter to the
// retrieved blocks, spread over each block's tokens) and the router's chain.
#include "kernels.h"

namespace mka {

// ---------------------------------------------------------------------------
// D[m, h] = sum_d dO[m, h, d] * O[m, h, d]: LPR = DH / V lanes per (row, head),
// V elements (16 bytes) per lane, the lanes' sums added by butterfly shuffles.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const T* __restrict__ O,
                                                            const T* __restrict__ dO, int64_t rows,
                                                            float* __restrict__ dsum) {
  constexpr int V = Vec16<T>::kN, LPR = DH / V, RPB = 256 / LPR;
  static_assert(DH % V == 0 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lanes per row");
  const int sub = threadIdx.x % LPR;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
  float acc = 0.f;
  if (r < rows) {
    float o[V], g[V];
    Vec16<T>::load(O + r * DH + sub * V, o);
    Vec16<T>::load(dO + r * DH + sub * V, g);
#pragma unroll
    for (int i = 0; i < V; ++i) acc = fmaf(o[i], g[i], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off /= 2) acc += __shfl_xor(acc, off);
  if (r < rows && sub == 0) dsum[r] = acc;
}

// ---------------------------------------------------------------------------
// Row-parallel attention backward (any storage type, fp32 arithmetic): one
// thread per query row (dq) or per key row (dk, dv), the other side's rows
// staged through LDS in tiles of 32.  lse and dsum are [B, N, H] (token-major),
// dq [B, N, H, DH] and dkv [B, N, 2, G, DH] (K part, then V part) in float32.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(64) void attn_bwd_dq_rows_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dsum, int N,
    int H, int G, int64_t t_cap, float scale, float* __restrict__ dq) {
  constexpr int TK = 32;
  __shared__ float Ks[TK][DH];
  __shared__ float Vs[TK][DH];
  const int tid = threadIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / (H / G);
  const int t = blockIdx.x * 64 + tid;
  const int tc = min(t, N - 1);
  const int64_t row = (static_cast<int64_t>(b) * N + tc) * H + h;
  float q[DH], go[DH], acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    q[d] = Elem<T>::to_f32(Q[row * DH + d]);
    go[d] = Elem<T>::to_f32(dO[row * DH + d]);
    acc[d] = 0.f;
  }
  const float l = lse[row], dd = dsum[row];
  const T* kb = K + (static_cast<int64_t>(b) * G + g) * t_cap * DH;
  const T* vb = V + (static_cast<int64_t>(b) * G + g) * t_cap * DH;
  const int kv_end = min(static_cast<int>(blockIdx.x) * 64 + 64, N);
  for (int j0 = 0; j0 < kv_end; j0 += TK) {
    for (int e = tid; e < TK * DH; e += 64) {
      const int r = e / DH, d = e % DH;
      const bool ok = j0 + r < kv_end;
      Ks[r][d] = ok ? Elem<T>::to_f32(kb[static_cast<int64_t>(j0 + r) * DH + d]) : 0.f;
      Vs[r][d] = ok ? Elem<T>::to_f32(vb[static_cast<int64_t>(j0 + r) * DH + d]) : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < TK; ++jj) {
      if (j0 + jj > t || j0 + jj >= kv_end) break;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        s = fmaf(q[d], Ks[jj][d], s);
        dp = fmaf(go[d], Vs[jj][d], dp);
      }
      const float p = expf(s * scale - l);
      const float ds = p * (dp - dd);
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] = fmaf(ds, Ks[jj][d], acc[d]);
    }
    __syncthreads();
  }
  if (t < N) {
#pragma unroll
    for (int d = 0; d < DH; ++d) dq[row * DH + d] = acc[d] * scale;
  }
}

// WANT_K: dk (needs k and v rows); otherwise dv (needs k only).
template <typename T, int DH, bool WANT_K>
__global__ __launch_bounds__(64) void attn_bwd_dkv_rows_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dsum, int N,
    int H, int G, int64_t t_cap, float scale, float* __restrict__ dkv) {
  constexpr int TQ = 32;
  __shared__ float Qs[TQ][DH];
  __shared__ float Gs[TQ][DH];
  __shared__ float Ls[TQ], Ds[TQ];
  const int tid = threadIdx.x, g = blockIdx.y, b = blockIdx.z, hpg = H / G;
  const int j = blockIdx.x * 64 + tid;
  const int jc = min(j, N - 1);
  const int64_t kvrow = ((static_cast<int64_t>(b) * G + g) * t_cap + jc) * DH;
  float k[DH], v[DH], acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    k[d] = Elem<T>::to_f32(K[kvrow + d]);
    v[d] = WANT_K ? Elem<T>::to_f32(V[kvrow + d]) : 0.f;
    acc[d] = 0.f;
  }
  const int t_begin = blockIdx.x * 64;  // queries before the block see none of its keys
  for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
    for (int t0 = t_begin; t0 < N; t0 += TQ) {
      for (int e = tid; e < TQ * DH; e += 64) {
        const int r = e / DH, d = e % DH;
        const int t = min(t0 + r, N - 1);
        const int64_t row = (static_cast<int64_t>(b) * N + t) * H + h;
        Qs[r][d] = Elem<T>::to_f32(Q[row * DH + d]);
        Gs[r][d] = Elem<T>::to_f32(dO[row * DH + d]);
      }
      if (tid < TQ) {
        const int t = min(t0 + tid, N - 1);
        const int64_t row = (static_cast<int64_t>(b) * N + t) * H + h;
        Ls[tid] = lse[row];
        Ds[tid] = dsum[row];
      }
      __syncthreads();
      for (int tt = 0; tt < TQ; ++tt) {
        const int t = t0 + tt;
        if (t >= N) break;
        if (t < j) continue;
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < DH; ++d) s = fmaf(Qs[tt][d], k[d], s);
        const float p = expf(s * scale - Ls[tt]);
        if (WANT_K) {
          float dp = 0.f;
#pragma unroll
          for (int d = 0; d < DH; ++d) dp = fmaf(Gs[tt][d], v[d], dp);
          const float ds = p * (dp - Ds[tt]);
#pragma unroll
          for (int d = 0; d < DH; ++d) acc[d] = fmaf(ds, Qs[tt][d], acc[d]);
        } else {
#pragma unroll
          for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, Gs[tt][d], acc[d]);
        }
      }
      __syncthreads();
    }
  }
  if (j < N) {
    float* out = dkv + ((static_cast<int64_t>(b) * N + j) * 2 + (WANT_K ? 0 : 1)) * G * DH +
                 static_cast<int64_t>(g) * DH;
#pragma unroll
    for (int d = 0; d < DH; ++d) out[d] = WANT_K ? acc[d] * scale : acc[d];
  }
}

// ---------------------------------------------------------------------------
// Layout helpers for the transposed products.
// dst[c][r] = src[r][c] for r < R, zero for R <= r < Rp; src rows have stride
// lds_ elements, dst rows ldd.  64 x 64 tiles through LDS, moved as 16-byte
// vectors where the tile lies inside both matrices and the strides and bases
// allow it (VEC), element by element otherwise.
// rows_dst (optional): the source converted to TD in place of a separate
// conversion pass (same layout as src).
// ---------------------------------------------------------------------------
template <typename T> constexpr int kPer16 = 16 / sizeof(T);  // elements per 16 bytes

template <typename TS, typename TD>
__global__ __launch_bounds__(256) void transpose_kernel(const TS* __restrict__ src, int64_t lds_,
                                                        int R, int C, int Rp, int64_t ldd,
                                                        TD* __restrict__ dst,
                                                        TD* __restrict__ rows_dst, bool vec_in,
                                                        bool vec_out) {
  constexpr int T = 64, NS = kPer16<TS>, ND = kPer16<TD>;
  __shared__ float tile[T][T + 1];
  const int r0 = blockIdx.y * T, c0 = blockIdx.x * T, tid = threadIdx.x;
  if (vec_in && r0 + T <= R && c0 + T <= C) {
    // T rows of T / NS vectors each
#pragma unroll
    for (int e = tid; e < T * (T / NS); e += 256) {
      const int i = e / (T / NS), cv = (e % (T / NS)) * NS;
      const int64_t o = static_cast<int64_t>(r0 + i) * lds_ + c0 + cv;
      TS v[NS];
      *reinterpret_cast<u32x4*>(v) = *reinterpret_cast<const u32x4*>(src + o);
      TD w[NS];
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        tile[i][cv + k] = Elem<TS>::to_f32(v[k]);
        w[k] = Elem<TD>::from_f32(tile[i][cv + k]);
      }
      if (rows_dst != nullptr) {
#pragma unroll
        for (int k = 0; k < NS; ++k) rows_dst[o + k] = w[k];
      }
    }
  } else {
    for (int e = tid; e < T * T; e += 256) {
      const int i = e / T, c = e % T, r = r0 + i;
      const bool in = r < R && c0 + c < C;
      const int64_t o = static_cast<int64_t>(r) * lds_ + c0 + c;
      tile[i][c] = in ? Elem<TS>::to_f32(src[o]) : 0.f;
      if (rows_dst != nullptr && in) rows_dst[o] = Elem<TD>::from_f32(tile[i][c]);
    }
  }
  __syncthreads();
  if (vec_out && c0 + T <= C && r0 + T <= Rp) {
    // T destination rows (source columns) of T / ND vectors each
#pragma unroll
    for (int e = tid; e < T * (T / ND); e += 256) {
      const int c = e / (T / ND), rv = (e % (T / ND)) * ND;
      TD w[ND];
#pragma unroll
      for (int k = 0; k < ND; ++k) w[k] = Elem<TD>::from_f32(tile[rv + k][c]);
      *reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(c0 + c) * ldd + r0 + rv) =
          *reinterpret_cast<const u32x4*>(w);
    }
  } else {
    for (int e = tid; e < T * T; e += 256) {
      const int c = e / T, i = e % T, r = r0 + i;
      if (c0 + c < C && r < Rp) dst[static_cast<int64_t>(c0 + c) * ldd + r] = Elem<TD>::from_f32(tile[i][c]);
    }
  }
}

// Four elements per thread as vectors when VEC (n % 4 == 0, aligned), else one.
template <typename TS, typename TD, bool VEC>
__global__ __launch_bounds__(256) void convert_kernel(const TS* __restrict__ src, int64_t n,
                                                      TD* __restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if constexpr (VEC) {
    if (4 * i < n) {
      float v[4];
      load4(src + 4 * i, v);
      store4(dst + 4 * i, v);
    }
  } else {
    if (i < n) dst[i] = Elem<TD>::from_f32(Elem<TS>::to_f32(src[i]));
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Fusion backward, one row per workgroup, 4 channels per thread (D % 4 == 0).
// X_fused = l1 x + l2 L2 + l3 L3 with L3 the mean of the retrieved means:
//   dlam_i = <dxf, L_i>, dx = l1 dxf (written), and, when xf is given,
//   X_fused itself (re-formed as the fusion forms it: float32, rounded once),
//   from the same reads of x, L2 and the retrieved means.  The L2 and L3
//   parts of dx (l2 dxf and l3 dxf / |S_t|) are taken by the EMA adjoint and
//   the block gather straight from dxf and lambda.  RMAX = 0: no L3 (idx is
//   not read); l2 == nullptr: no L2.
// ---------------------------------------------------------------------------
template <typename T, int RMAX>
__global__ __launch_bounds__(256) void fuse_bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ l2, const float* __restrict__ means,
    int nb_cap, const int32_t* __restrict__ idx, const float* __restrict__ lam, int N, int D,
    int R, const float* __restrict__ dxf, float* __restrict__ dx, float* __restrict__ dlam,
    T* __restrict__ xf) {
  __shared__ float red[3][4];
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / N);
  const int tid = threadIdx.x;
  const float w1 = lam[row * 3 + 0], w2 = lam[row * 3 + 1], w3 = lam[row * 3 + 2];
  int blk[RMAX > 0 ? RMAX : 1], cnt = 0;
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    blk[i] = i < R ? idx[row * R + i] : -1;
    cnt += blk[i] >= 0;
  }
  const float* mb = means + static_cast<int64_t>(b) * nb_cap * D;
  float a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int c = 4 * tid; c < D; c += 4 * 256) {
    const int64_t o = row * D + c;
    float gx[4], xv[4], sv[4] = {0.f, 0.f, 0.f, 0.f}, mean[4] = {0.f, 0.f, 0.f, 0.f};
    load4(dxf + o, gx);
    load4(x + o, xv);
    if (l2) load4(l2 + o, sv);
    if constexpr (RMAX > 0) {
      // every retrieved row is loaded (unfilled slots read block 0 and are
      // not added), so the loads are in flight together; rank order
      float m[RMAX][4];
#pragma unroll
      for (int i = 0; i < RMAX; ++i) load4(mb + static_cast<int64_t>(max(blk[i], 0)) * D + c, m[i]);
      float l3[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RMAX; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) l3[k] += blk[i] >= 0 ? m[i][k] : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) mean[k] = cnt ? l3[k] / static_cast<float>(cnt) : 0.f;
    }
    float d1[4], out[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a1 = fmaf(gx[k], xv[k], a1);
      a2 = fmaf(gx[k], sv[k], a2);
      a3 = fmaf(gx[k], mean[k], a3);
      d1[k] = w1 * gx[k];
      out[k] = w1 * xv[k] + w2 * sv[k] + w3 * mean[k];
    }
    store4(dx + o, d1);
    if (xf) store4(xf + o, out);
  }
  a1 = wave_sum(a1);
  a2 = wave_sum(a2);
  a3 = wave_sum(a3);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = a1;
    red[1][tid >> 6] = a2;
    red[2][tid >> 6] = a3;
  }
  __syncthreads();
  if (tid < 3) dlam[row * 3 + tid] = ((red[tid][0] + red[tid][1]) + red[tid][2]) + red[tid][3];
}

// ---------------------------------------------------------------------------
// The block means' adjoint without atomics: dm[b, blk] = sum over the tokens t
// that retrieved blk (in token order) of lambda_3[t] / |S_t| * dxf[t].  One
// workgroup per (block, sequence, 1024 channels, range of kGatherTokens
// tokens), writing that range's partial sum (summed over the ranges in order
// afterwards): popular blocks are retrieved by thousands of tokens, so one
// workgroup per block would be a long serial walk.  Tokens are scanned 256 at
// a time (only t >= (blk + 1) * Bs can retrieve blk), the retrieving ones
// compacted into LDS in order, then summed four channels per thread.
// ---------------------------------------------------------------------------
constexpr int kGatherTokens = 512, kGatherBatch = 8;

template <int RMAX>
__global__ __launch_bounds__(256) void block_gather_kernel(const float* __restrict__ dxf,
                                                           const float* __restrict__ lam,
                                                           const int32_t* __restrict__ idx,
                                                           int N, int D, int R, int block,
                                                           int nbs, int n_slices,
                                                           float* __restrict__ part) {
  __shared__ int list_t[256];
  __shared__ float list_w[256];
  __shared__ int wave_cnt[4];
  const int blk = blockIdx.x, b = blockIdx.y, B = gridDim.y;
  const int slice = blockIdx.z % n_slices, range = blockIdx.z / n_slices;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = (slice * 256 + tid) * 4;
  const int t_lo = max((blk + 1) * block, range * kGatherTokens);
  const int t_hi = min(N, (range + 1) * kGatherTokens);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = t_lo; t0 < t_hi; t0 += 256) {
    const int t = t0 + tid;
    bool hit = false;
    float w = 0.f;
    if (t < t_hi) {
      const int64_t row = static_cast<int64_t>(b) * N + t;
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < RMAX; ++i) {
        const int bi = i < R ? idx[row * R + i] : -1;
        cnt += bi >= 0;
        hit |= bi == blk;
      }
      if (hit) w = lam[row * 3 + 2] / static_cast<float>(cnt);
    }
    const uint64_t m = __ballot(hit);
    if (lane == 0) wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int base = 0, total = 0;
    for (int k = 0; k < 4; ++k) {
      base += k < wave ? wave_cnt[k] : 0;
      total += wave_cnt[k];
    }
    if (hit) {
      const int pos = base + __popcll(m & ((static_cast<uint64_t>(1) << lane) - 1));
      list_t[pos] = t;
      list_w[pos] = w;
    }
    __syncthreads();
    if (c < D) {
      // kGatherBatch listed tokens per step, their loads issued together (a
      // slot past the list reads the first token with weight 0); the sum stays
      // in list order
      for (int k0 = 0; k0 < total; k0 += kGatherBatch) {
        float4 v[kGatherBatch];
        float wk[kGatherBatch];
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u) {
          const int k = k0 + u < total ? k0 + u : 0;
          wk[u] = k0 + u < total ? list_w[k] : 0.f;
          v[u] = *reinterpret_cast<const float4*>(dxf + (static_cast<int64_t>(b) * N + list_t[k]) * D + c);
        }
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u) {
          acc[0] = fmaf(wk[u], v[u].x, acc[0]);
          acc[1] = fmaf(wk[u], v[u].y, acc[1]);
          acc[2] = fmaf(wk[u], v[u].z, acc[2]);
          acc[3] = fmaf(wk[u], v[u].w, acc[3]);
        }
      }
    }
    __syncthreads();
  }
  if (c < D)
    *reinterpret_cast<float4*>(part + ((static_cast<int64_t>(range) * B + b) * nbs + blk) * D + c) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// ---------------------------------------------------------------------------
// EMA adjoint: g_t = u_t + beta g_{t+1} (from the last token back), dx_t +=
// (1 - beta) g_t; then the block means' spread dx_t += dm[t / Bs] / Bs for
// tokens of complete blocks.  Chunks of kBwdChunk tokens: pass 1 sums each
// chunk's contribution to g at its first token, pass 2 carries between chunks
// (from the last), pass 3 rescans each chunk with its incoming carry.
// ---------------------------------------------------------------------------
constexpr int kBwdChunk = 64;

// u_t = lambda_2[t] * dxf[t] (lam2 = &lambda[1], stride 3).  Each thread takes
// 4 channels (D % 4 == 0); the loads of kAdjUnroll tokens are issued before
// their sequential updates.
constexpr int kAdjUnroll = 8;

__global__ __launch_bounds__(256) void ema_adj_pass1(const float* __restrict__ u,
                                                     const float* __restrict__ lam2, int N, int D,
                                                     int n_chunks, float beta,
                                                     float* __restrict__ part) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int ch = blockIdx.y, b = blockIdx.z;
  if (c >= D) return;
  const int t0 = ch * kBwdChunk, t1 = min(N, t0 + kBwdChunk);
  float g[4] = {0.f, 0.f, 0.f, 0.f};
  for (int tb = t1 - 1; tb >= t0; tb -= kAdjUnroll) {
    float uv[kAdjUnroll][4], lw[kAdjUnroll];
#pragma unroll
    for (int k = 0; k < kAdjUnroll; ++k) {  // tokens before the chunk re-read its first (unused)
      const int64_t row = static_cast<int64_t>(b) * N + max(tb - k, t0);
      lw[k] = lam2[row * 3];
      load4(u + row * D + c, uv[k]);
    }
#pragma unroll
    for (int k = 0; k < kAdjUnroll; ++k)
      if (tb - k >= t0)
#pragma unroll
        for (int i = 0; i < 4; ++i) g[i] = fmaf(beta, g[i], lw[k] * uv[k][i]);
  }
  store4(part + (static_cast<int64_t>(b) * n_chunks + ch) * D + c, g);
}

__global__ __launch_bounds__(64) void ema_adj_pass2(float* __restrict__ part, int N, int D,
                                                     int n_chunks, float beta) {
  const int c = blockIdx.x * 64 + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= D) return;
  // carry into chunk ch = g at the first token of chunk ch + 1; the chunk
  // sums of kAdjBatch chunks are loaded before their sequential use
  constexpr int kAdjBatch = 16;
  float* pb = part + static_cast<int64_t>(b) * n_chunks * D + c;
  const float decay_full = powf(beta, static_cast<float>(kBwdChunk));
  float carry = 0.f;
  for (int c1 = n_chunks - 1; c1 >= 0; c1 -= kAdjBatch) {
    float local[kAdjBatch];
#pragma unroll
    for (int k = 0; k < kAdjBatch; ++k) local[k] = pb[static_cast<int64_t>(max(c1 - k, 0)) * D];
#pragma unroll
    for (int k = 0; k < kAdjBatch; ++k) {
      const int ch = c1 - k;
      if (ch >= 0) {
        const int len = min(N, (ch + 1) * kBwdChunk) - ch * kBwdChunk;
        pb[static_cast<int64_t>(ch) * D] = carry;  // now: g at the first token after the chunk
        const float decay = len == kBwdChunk ? decay_full : powf(beta, static_cast<float>(len));
        carry = local[k] + decay * carry;
      }
    }
  }
}

__global__ __launch_bounds__(256) void ema_adj_pass3(const float* __restrict__ u,
                                                     const float* __restrict__ lam2,
                                                     const float* __restrict__ part,
                                                     const float* __restrict__ dm, int nbs,
                                                     int N, int D, int n_chunks, int block,
                                                     float beta, float* __restrict__ dx) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int ch = blockIdx.y, b = blockIdx.z;
  if (c >= D) return;
  const int t0 = ch * kBwdChunk, t1 = min(N, t0 + kBwdChunk);
  const int n_full = (N / block) * block;  // tokens of complete blocks
  const float omb = 1.0f - beta, inv_bs = 1.0f / static_cast<float>(block);
  float g[4];
  load4(part + (static_cast<int64_t>(b) * n_chunks + ch) * D + c, g);
  for (int tb = t1 - 1; tb >= t0; tb -= kAdjUnroll) {
    float uv[kAdjUnroll][4], xv[kAdjUnroll][4], mv[kAdjUnroll][4], lw[kAdjUnroll];
#pragma unroll
    for (int k = 0; k < kAdjUnroll; ++k) {  // tokens before the chunk re-read its first (unused)
      const int t = max(tb - k, t0);
      const int64_t row = static_cast<int64_t>(b) * N + t, o = row * D + c;
      lw[k] = lam2[row * 3];
      load4(u + o, uv[k]);
      load4(dx + o, xv[k]);
      // tokens of the incomplete last block take no block-mean term (row 0 read, unused)
      load4(dm + (static_cast<int64_t>(b) * nbs + (t < n_full ? t / block : 0)) * D + c, mv[k]);
    }
#pragma unroll
    for (int k = 0; k < kAdjUnroll; ++k) {
      const int t = tb - k;
      if (t >= t0) {
        float out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          g[i] = fmaf(beta, g[i], lw[k] * uv[k][i]);
          float add = omb * g[i];
          if (t < n_full) add += mv[k][i] * inv_bs;
          out[i] = xv[k][i] + add;
        }
        store4(dx + (static_cast<int64_t>(b) * N + t) * D + c, out);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Router backward, one wave per token: dz from dlam through the (kept-tier)
// softmax, dpre = (dz W_r2) * GELU'(pre) in float32 and in the storage type.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ lam,
                                                         const float* __restrict__ dlam,
                                                         const float* __restrict__ pre,
                                                         const T* __restrict__ W2, int r,
                                                         int64_t M, Routing rt,
                                                         float* __restrict__ dz_out,
                                                         T* __restrict__ dpre) {
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  float dz[3] = {0.f, 0.f, 0.f};
  if (rt.learned()) {
    const float l0 = lam[m * 3], l1 = lam[m * 3 + 1], l2 = lam[m * 3 + 2];
    const float g0 = dlam[m * 3], g1 = dlam[m * 3 + 1], g2 = dlam[m * 3 + 2];
    const float dot = l0 * g0 + l1 * g1 + l2 * g2;  // tiers outside the kept set have lambda 0
    dz[0] = l0 > 0.f ? l0 * (g0 - dot) : 0.f;
    dz[1] = l1 > 0.f ? l1 * (g1 - dot) : 0.f;
    dz[2] = l2 > 0.f ? l2 * (g2 - dot) : 0.f;
  }
  if (lane < 3) dz_out[m * 3 + lane] = dz[lane];
  for (int n = lane; n < r; n += 64) {
    const float dh = dz[0] * Elem<T>::to_f32(W2[n]) + dz[1] * Elem<T>::to_f32(W2[r + n]) +
                     dz[2] * Elem<T>::to_f32(W2[2 * r + n]);
    const float z = pre[m * r + n];
    const float gp = 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
                     z * 0.39894228040143268f * expf(-0.5f * z * z);
    dpre[m * r + n] = Elem<T>::from_f32(dh * gp);
  }
}

// dW_r2[c][n] = sum_m dz[m][c] * GELU(pre[m][n]): one workgroup per output.
__global__ __launch_bounds__(256) void router_dw2_kernel(const float* __restrict__ dz,
                                                         const float* __restrict__ pre, int r,
                                                         int64_t M, float* __restrict__ dw2) {
  __shared__ float red[4];
  const int c = blockIdx.x / r, n = blockIdx.x % r;
  float acc = 0.f;
  for (int64_t m = threadIdx.x; m < M; m += 256) acc = fmaf(dz[m * 3 + c], gelu(pre[m * r + n]), acc);
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) dw2[blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T>
hipError_t attn_bwd_prep(const T* o, const T* d_o, int64_t rows, int dh, float* dsum,
                         hipStream_t s) {
  auto launch = [&](auto kernel, int lanes_per_row) {
    const int64_t per_block = 256 / lanes_per_row;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>((rows + per_block - 1) / per_block)),
                       dim3(256), 0, s, o, d_o, rows, dsum);
  };
  constexpr int V = Vec16<T>::kN;
  if (dh == 128)
    launch(attn_bwd_prep_kernel<T, 128>, 128 / V);
  else if (dh == 64)
    launch(attn_bwd_prep_kernel<T, 64>, 64 / V);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
hipError_t attn_bwd_rows(const T* q, const T* k, const T* v, const T* d_o, const float* lse,
                         const float* dsum, int B, int N, int H, int G, int dh, int64_t t_cap,
                         float* dq, float* dkv, hipStream_t s) {
  const float scale = 1.0f / sqrtf(static_cast<float>(dh));
  const dim3 gq((N + 63) / 64, H, B), gk((N + 63) / 64, G, B);
  if (dh == 128) {
    hipLaunchKernelGGL((attn_bwd_dq_rows_kernel<T, 128>), gq, dim3(64), 0, s, q, k, v, d_o, lse,
                       dsum, N, H, G, t_cap, scale, dq);
    hipLaunchKernelGGL((attn_bwd_dkv_rows_kernel<T, 128, true>), gk, dim3(64), 0, s, q, k, v, d_o,
                       lse, dsum, N, H, G, t_cap, scale, dkv);
    hipLaunchKernelGGL((attn_bwd_dkv_rows_kernel<T, 128, false>), gk, dim3(64), 0, s, q, k, v, d_o,
                       lse, dsum, N, H, G, t_cap, scale, dkv);
  } else {
    hipLaunchKernelGGL((attn_bwd_dq_rows_kernel<T, 64>), gq, dim3(64), 0, s, q, k, v, d_o, lse,
                       dsum, N, H, G, t_cap, scale, dq);
    hipLaunchKernelGGL((attn_bwd_dkv_rows_kernel<T, 64, true>), gk, dim3(64), 0, s, q, k, v, d_o,
                       lse, dsum, N, H, G, t_cap, scale, dkv);
    hipLaunchKernelGGL((attn_bwd_dkv_rows_kernel<T, 64, false>), gk, dim3(64), 0, s, q, k, v, d_o,
                       lse, dsum, N, H, G, t_cap, scale, dkv);
  }
  return hipGetLastError();
}

// 16-byte vectors apply when the base is 16-byte aligned and the row stride a
// multiple of the vector.
template <typename E>
static bool vec_ok(const E* p, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && ld % kPer16<E> == 0;
}

template <typename TS, typename TD>
hipError_t transpose_copy(const TS* src, int64_t lds_, int R, int C, int Rp, int64_t ldd, TD* dst,
                          TD* rows_dst, hipStream_t s) {
  const dim3 grid((C + 63) / 64, (Rp + 63) / 64);
  const bool vec_in = vec_ok(src, lds_) && (rows_dst == nullptr || vec_ok(rows_dst, lds_));
  hipLaunchKernelGGL((transpose_kernel<TS, TD>), grid, dim3(256), 0, s, src, lds_, R, C, Rp, ldd,
                     dst, rows_dst, vec_in, vec_ok(dst, ldd));
  return hipGetLastError();
}

template <typename TS, typename TD>
hipError_t transpose(const TS* src, int64_t lds_, int R, int C, int Rp, int64_t ldd, TD* dst,
                     hipStream_t s) {
  return transpose_copy(src, lds_, R, C, Rp, ldd, dst, static_cast<TD*>(nullptr), s);
}

template <typename TS, typename TD>
hipError_t convert(const TS* src, int64_t n, TD* dst, hipStream_t s) {
  const bool vec = n % 4 == 0 && (reinterpret_cast<uintptr_t>(src) % (4 * sizeof(TS))) == 0 &&
                   (reinterpret_cast<uintptr_t>(dst) % (4 * sizeof(TD))) == 0;
  if (vec)
    hipLaunchKernelGGL((convert_kernel<TS, TD, true>),
                       dim3(static_cast<unsigned>((n / 4 + 255) / 256)), dim3(256), 0, s, src, n,
                       dst);
  else
    hipLaunchKernelGGL((convert_kernel<TS, TD, false>), dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, s, src, n, dst);
  return hipGetLastError();
}

hipError_t fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, p, n);
  return hipGetLastError();
}

template <typename T>
hipError_t fuse_bwd(const T* x, const float* l2, const float* means, int nb_cap,
                    const int32_t* idx, const float* lam, int B, int N, int D, int R,
                    const float* dxf, float* dx, float* dlam, T* xf, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * N));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, x, l2, means, nb_cap, idx, lam, N, D, R, dxf,
                       dx, dlam, xf);
  };
  if (idx == nullptr || R == 0)
    launch(fuse_bwd_kernel<T, 0>);
  else if (R <= 4)
    launch(fuse_bwd_kernel<T, 4>);
  else if (R <= 8)
    launch(fuse_bwd_kernel<T, 8>);
  else if (R <= 16)
    launch(fuse_bwd_kernel<T, 16>);
  else
    launch(fuse_bwd_kernel<T, 32>);
  return hipGetLastError();
}

size_t block_gather_ws_bytes(int B, int N, int D, int block) {
  return sizeof(float) * static_cast<size_t>((N + kGatherTokens - 1) / kGatherTokens) * B *
         (N / block + 1) * D;
}

hipError_t block_gather(const float* dxf, const float* lam, const int32_t* idx, int B, int N,
                        int D, int R, int block, int nbs, float* part, float* dm, hipStream_t s) {
  const int n_blocks = N / block;  // complete blocks: the only ones retrieved
  if (n_blocks == 0) return hipSuccess;
  const int n_slices = (D + 1023) / 1024, n_ranges = (N + kGatherTokens - 1) / kGatherTokens;
  const dim3 grid(n_blocks, B, n_slices * n_ranges);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, dxf, lam, idx, N, D, R, block, nbs,
                       n_slices, part);
  };
  if (R <= 4) launch(block_gather_kernel<4>);
  else if (R <= 8) launch(block_gather_kernel<8>);
  else if (R <= 16) launch(block_gather_kernel<16>);
  else launch(block_gather_kernel<32>);
  // rows of blocks >= n_blocks stay unset in every range: only rows < n_blocks are read
  return sum_slices(part, n_ranges, static_cast<int64_t>(B) * nbs * D / 4, dm, s);
}

size_t ema_adj_ws_bytes(int B, int N, int D) {
  return sizeof(float) * static_cast<size_t>(B) * ((N + kBwdChunk - 1) / kBwdChunk) * D;
}

hipError_t ema_adjoint_add(const float* u, const float* lam, const float* dm, int nbs, int B,
                           int N, int D, int block, float beta, float* part, float* dx,
                           hipStream_t s) {
  const int n_chunks = (N + kBwdChunk - 1) / kBwdChunk;
  const int cx4 = (D / 4 + 255) / 256;  // D % 4 == 0
  hipLaunchKernelGGL(ema_adj_pass1, dim3(cx4, n_chunks, B), dim3(256), 0, s, u, lam + 1, N, D,
                     n_chunks, beta, part);
  hipLaunchKernelGGL(ema_adj_pass2, dim3((D + 63) / 64, B), dim3(64), 0, s, part, N, D, n_chunks,
                     beta);
  hipLaunchKernelGGL(ema_adj_pass3, dim3(cx4, n_chunks, B), dim3(256), 0, s, u, lam + 1, part, dm,
                     nbs,
                     N, D, n_chunks, block, beta, dx);
  return hipGetLastError();
}

template <typename T>
hipError_t router_bwd(const float* lam, const float* dlam, const float* pre, const T* w2, int r,
                      int64_t M, Routing rt, float* dz, T* dpre, float* dw2, hipStream_t s) {
  hipLaunchKernelGGL(router_bwd_kernel<T>, dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0,
                     s, lam, dlam, pre, w2, r, M, rt, dz, dpre);
  hipLaunchKernelGGL(router_dw2_kernel, dim3(3 * r), dim3(256), 0, s, dz, pre, r, M, dw2);
  return hipGetLastError();
}

#define MKA_BWD_INST(T)                                                                            \
  template hipError_t attn_bwd_prep<T>(const T*, const T*, int64_t, int, float*, hipStream_t);    \
  template hipError_t attn_bwd_rows<T>(const T*, const T*, const T*, const T*, const float*,     \
                                       const float*, int, int, int, int, int, int64_t, float*,    \
                                       float*, hipStream_t);                                      \
  template hipError_t convert<float, T>(const float*, int64_t, T*, hipStream_t);                 \
  template hipError_t fuse_bwd<T>(const T*, const float*, const float*, int, const int32_t*,      \
                                  const float*, int, int, int, int, const float*, float*, float*, \
                                  T*, hipStream_t);                                               \
  template hipError_t router_bwd<T>(const float*, const float*, const float*, const T*, int,      \
                                    int64_t, Routing, float*, T*, float*, hipStream_t);
MKA_BWD_INST(float)
MKA_BWD_INST(bf16_t)
#undef MKA_BWD_INST
template hipError_t transpose<float, float>(const float*, int64_t, int, int, int, int64_t, float*,
                                            hipStream_t);
template hipError_t transpose<bf16_t, bf16_t>(const bf16_t*, int64_t, int, int, int, int64_t,
                                              bf16_t*, hipStream_t);
template hipError_t transpose_copy<float, bf16_t>(const float*, int64_t, int, int, int, int64_t,
                                                  bf16_t*, bf16_t*, hipStream_t);
template hipError_t transpose<float, bf16_t>(const float*, int64_t, int, int, int, int64_t,
                                             bf16_t*, hipStream_t);

}  // namespace mka
