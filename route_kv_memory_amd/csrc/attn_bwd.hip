// Attention backward on the matrix cores (bf16 operands, fp32 accumulation).
//
// With the forward's saved log-sum-exp, P = exp(S - lse) is recomputed tile by
// tile (FlashAttention-style), and D = rowsum(dO * O) is precomputed:
//   dS = P * (dP - D),  dP = dO V^T,  dV = P^T dO,
//   dq = dS K / sqrt(dh),  dK = dS^T q / sqrt(dh)  (reading note, method
//   sections 3-4: one causal attention over the fused K/V; its derivative).
//
// Two kernels, both built like the forward (MFMA 32x32x16, operand rows fed
// to the MFMA in the permuted order that makes accumulator register r of lane
// half hl hold row 16*(r/8) + 8*hl + r%8, so probabilities computed in
// registers are directly the B operand of the next product):
//   dq:  a wave owns 32 query rows of one head and walks the key tiles:
//        S^T = K Q^T and dP^T = V dO^T (K and V rows from LDS, Q and dO in
//        registers), dS^T, then dQ^T += K^T dS^T (a transposed K tile).
//   dkv: a wave owns 32 key rows of one KV head and walks every query tile of
//        the group's heads from its block on: S = Q K^T and dP = dO V^T (Q and
//        dO rows from LDS, K and V in registers), P and dS, then dV^T += dO^T P
//        and dK^T += Q^T dS (transposed Q and dO tiles).
#include "attn_split.h"

namespace mka {
namespace {

// Row j of a 64-row tile is stored at LDS row bperm(j): rows 4..7 and 8..11 of
// every 16 swapped (see the header comment).
__device__ __forceinline__ int bperm(int r) {
  const int q = r & 15;
  const int qq = (q >= 4 && q < 8) ? q + 4 : ((q >= 8 && q < 12) ? q - 4 : q);
  return (r & ~15) | qq;
}

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

// ---------------------------------------------------------------------------
// dq.  Workgroup = 4 waves = 128 query rows of head h; K/V tiles of 64 keys,
// double-buffered in LDS as rows (for S^T, dP^T) and transposed K (for dQ).
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dsum,
    int B, int N, int H, int G, int64_t t_cap, float sl2, float scale, int n_qblk, int n_units,
    float* __restrict__ dq) {
  constexpr int NT = 256, BM = 128, BN = 64, KP = DH + 8, VP = BN + 8, NKS = DH / 16,
                NDB = DH / 32;
  constexpr int KCH = BN * DH / 8 / NT;        // 16-byte V row chunks per thread
  constexpr int VITEMS = (BN / 4) * (DH / 8);  // threads loading 4 K rows x 8 dims
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][BN * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Kt[2][DH * VP];

  const int hpg = H / G;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int hh = slot % hpg, u = (slot / hpg) * 8 + xcd;
  if (u >= n_units) return;
  const int qb = n_qblk - 1 - u / (B * G);
  const int bg = u % (B * G), b = bg / G, g = bg % G, h = g * hpg + hh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  const int q_row = qb * BM + wave * 32 + l32;
  const int qc = min(q_row, N - 1);
  const int64_t lrow = static_cast<int64_t>(b * N + qc) * H + h;
  bf16x8 qf[NKS], gf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = ld8(Q + lrow * DH + 8 * hl + 16 * ks);
    gf[ks] = ld8(dO + lrow * DH + 8 * hl + 16 * ks);
    if (q_row >= N) {
      qf[ks] = bf16x8{};
      gf[ks] = bf16x8{};
    }
  }
  const float lse2 = q_row < N ? lse[lrow] * kLog2e : 0.f;
  const float dd = q_row < N ? dsum[lrow] : 0.f;
  const int wave_pos0 = qb * BM + wave * 32;
  const int kv_end = min(qb * BM + BM, N);
  const int n_tiles = (kv_end + BN - 1) / BN;
  const bf16_t* kbase = Kc + (static_cast<int64_t>(b) * G + g) * t_cap * DH;
  const bf16_t* vbase = Vc + (static_cast<int64_t>(b) * G + g) * t_cap * DH;

  u32x4 rk[4], rv[KCH];
  // keys at or beyond kv_end read as zeros through the buffer range
  auto gload = [&](int j0) {
    const uint32_t bytes = static_cast<uint32_t>(min(BN, kv_end - j0) * DH * 2);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase + static_cast<int64_t>(j0) * DH, bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase + static_cast<int64_t>(j0) * DH, bytes);
    if (tid < VITEMS) {
      const int kq = tid & 15, dc = tid >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rk[r] = buffer_load16(krs, static_cast<uint32_t>((4 * kq + r) * DH + 8 * dc) * 2);
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + NT * i, row = c / (DH / 8), col = (c % (DH / 8)) * 8;
      rv[i] = buffer_load16(vrs, static_cast<uint32_t>(row * DH + col) * 2);
    }
  };
  auto sstore = [&](int buf) {
    if (tid < VITEMS) {
      const int kq = tid & 15, dc = tid >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4*>(&Ks[buf][bperm(4 * kq + r) * KP + 8 * dc]) = rk[r];
      store_v_transposed(Kt[buf], VP, 8 * dc, 4 * kq, rk);
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + NT * i, row = c / (DH / 8), col = (c % (DH / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Vs[buf][bperm(row) * KP + col]) = rv[i];
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  gload(0);
  sstore(0);
  __syncthreads();
  for (int jt = 0; jt < n_tiles; ++jt) {
    const int buf = jt & 1, j0 = jt * BN;
    if (jt + 1 < n_tiles) gload(j0 + BN);
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
      const bf16_t* kr = &Ks[buf][(kb * 32 + l32) * KP + 8 * hl];
      const bf16_t* vr = &Vs[buf][(kb * 32 + l32) * KP + 8 * hl];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        s[kb] = mfma32x32x16(ld8(kr + 16 * ks), qf[ks], s[kb]);
        dp[kb] = mfma32x32x16(ld8(vr + 16 * ks), gf[ks], dp[kb]);
      }
    }
    // dS^T = P^T (dP^T - D); register r of lane half hl holds key
    // kb*32 + 16*(r/8) + 8*hl + r%8 of the lane's query
    const bool diag = (j0 + BN - 1) > wave_pos0;
    const int q_rel = q_row - j0;
    bf16x8 dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * st + j;
          float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -lse2));
          if (diag && kb * 32 + 16 * st + 8 * hl + j > q_rel) p = 0.f;
          v[j] = p * (dp[kb][r] - dd);
        }
        dsf[kb][st] = pack_bf16x8(v);
      }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16_t* ktr = &Kt[buf][(db * 32 + l32) * VP + 8 * hl];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          acc[db] = mfma32x32x16(ld8(ktr + kb * 32 + 16 * st), dsf[kb][st], acc[db]);
    }
    if (jt + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }
  if (q_row < N) {
    float* out = dq + lrow * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float v[4] = {acc[db][4 * rq] * scale, acc[db][4 * rq + 1] * scale,
                            acc[db][4 * rq + 2] * scale, acc[db][4 * rq + 3] * scale};
        store4(out + db * 32 + 8 * rq + 4 * hl, v);
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 4 waves = 128 key rows of one KV head and ONE of the
// group's query heads (units ordered heaviest first: the first key blocks see
// the most queries); query tiles of 64 rows from the key block's first row (no
// earlier query sees these keys), double-buffered in LDS as rows (Q, dO) and
// transposed (Q^T, dO^T), with each row's log-sum-exp (log2 units) and D.  The
// head's share goes to its own slice of ``dkv`` ([hpg][B, N, 2, G, DH]), summed
// over the heads afterwards in a fixed order.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dsum,
    int B, int N, int H, int G, int64_t t_cap, float sl2, float scale, float* __restrict__ dkv) {
  constexpr int BK = 128, BQ = 64, KP = DH + 8, QP = BQ + 8, NKS = DH / 16, NDB = DH / 32;
  constexpr int VITEMS = (BQ / 4) * (DH / 8);  // threads loading 4 rows x 8 dims of Q and dO
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][BQ * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Gs[2][BQ * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Qt[2][DH * QP];
  __shared__ __attribute__((aligned(16))) bf16_t Gt[2][DH * QP];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];

  const int hpg = H / G;
  const int u = blockIdx.x, per_kblk = B * G * hpg;
  const int kblk = u / per_kblk, rest = u % per_kblk;
  const int hh = rest % hpg, b = rest / (G * hpg), g = (rest / hpg) % G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  const int k_row = kblk * BK + wave * 32 + l32;
  const int64_t kvoff =
      ((static_cast<int64_t>(b) * G + g) * t_cap + min(k_row, N - 1)) * DH + 8 * hl;
  bf16x8 kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = ld8(Kc + kvoff + 16 * ks);
    vf[ks] = ld8(Vc + kvoff + 16 * ks);
    if (k_row >= N) {
      kf[ks] = bf16x8{};
      vf[ks] = bf16x8{};
    }
  }
  const int t_first = kblk * BK;
  const int n_it = (N - t_first + BQ - 1) / BQ;  // query tiles of head g*hpg + hh

  u32x4 rq[4], rg[4];
  float rl = 0.f, rd = 0.f;
  // rows past N are loaded from row N-1 and zeroed; their lse is +inf (P = 0)
  const int h = g * hpg + hh;
  auto gload = [&](int it) {
    const int t0 = t_first + it * BQ;
    if (tid < VITEMS) {
      const int kq = tid & 15, dc = tid >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * kq + r;
        const int64_t off = (static_cast<int64_t>(b * N + min(t, N - 1)) * H + h) * DH + 8 * dc;
        const u32x4 a = *reinterpret_cast<const u32x4*>(Q + off);
        const u32x4 c = *reinterpret_cast<const u32x4*>(dO + off);
        rq[r] = t < N ? a : u32x4{0u, 0u, 0u, 0u};
        rg[r] = t < N ? c : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < BQ) {
      const int t = t0 + tid;
      const int64_t row = static_cast<int64_t>(b * N + min(t, N - 1)) * H + h;
      const float l = lse[row], dv = dsum[row];
      rl = t < N ? l * kLog2e : INFINITY;
      rd = t < N ? dv : 0.f;
    }
  };
  auto sstore = [&](int buf) {
    if (tid < VITEMS) {
      const int kq = tid & 15, dc = tid >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<u32x4*>(&Qs[buf][bperm(4 * kq + r) * KP + 8 * dc]) = rq[r];
        *reinterpret_cast<u32x4*>(&Gs[buf][bperm(4 * kq + r) * KP + 8 * dc]) = rg[r];
      }
      store_v_transposed(Qt[buf], QP, 8 * dc, 4 * kq, rq);
      store_v_transposed(Gt[buf], QP, 8 * dc, 4 * kq, rg);
    }
    if (tid < BQ) {
      Ls[buf][tid] = rl;
      Ds[buf][tid] = rd;
    }
  };

  f32x16 adk[NDB], adv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    adk[db] = f32x16{};
    adv[db] = f32x16{};
  }
  gload(0);
  sstore(0);
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int buf = it & 1;
    const int t0 = t_first + it * BQ;
    if (it + 1 < n_it) gload(it + 1);
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
      const bf16_t* qr = &Qs[buf][(qb * 32 + l32) * KP + 8 * hl];
      const bf16_t* gr = &Gs[buf][(qb * 32 + l32) * KP + 8 * hl];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        s[qb] = mfma32x32x16(ld8(qr + 16 * ks), kf[ks], s[qb]);
        dp[qb] = mfma32x32x16(ld8(gr + 16 * ks), vf[ks], dp[qb]);
      }
    }
    // register r of lane half hl holds query qb*32 + 16*(r/8) + 8*hl + r%8 of
    // the tile for the lane's key; P = 0 where the query precedes the key
    bf16x8 pf[2][2], dsf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int q0 = qb * 32 + 16 * st + 8 * hl;
        float pv[8], dv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * st + j;
          float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], sl2, -Ls[buf][q0 + j]));
          if (t0 + q0 + j < k_row) p = 0.f;
          pv[j] = p;
          dv[j] = p * (dp[qb][r] - Ds[buf][q0 + j]);
        }
        pf[qb][st] = pack_bf16x8(pv);
        dsf[qb][st] = pack_bf16x8(dv);
      }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16_t* gtr = &Gt[buf][(db * 32 + l32) * QP + 8 * hl];
      const bf16_t* qtr = &Qt[buf][(db * 32 + l32) * QP + 8 * hl];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          adv[db] = mfma32x32x16(ld8(gtr + qb * 32 + 16 * st), pf[qb][st], adv[db]);
          adk[db] = mfma32x32x16(ld8(qtr + qb * 32 + 16 * st), dsf[qb][st], adk[db]);
        }
    }
    if (it + 1 < n_it) sstore(buf ^ 1);
    __syncthreads();
  }
  if (k_row < N) {
    float* out = dkv + static_cast<int64_t>(hh) * B * N * 2 * G * DH +
                 static_cast<int64_t>(b * N + k_row) * 2 * G * DH + g * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq4 = 0; rq4 < 4; ++rq4) {
        const int d = db * 32 + 8 * rq4 + 4 * hl;
        const float k4[4] = {adk[db][4 * rq4] * scale, adk[db][4 * rq4 + 1] * scale,
                             adk[db][4 * rq4 + 2] * scale, adk[db][4 * rq4 + 3] * scale};
        const float v4[4] = {adv[db][4 * rq4], adv[db][4 * rq4 + 1], adv[db][4 * rq4 + 2],
                             adv[db][4 * rq4 + 3]};
        store4(out + d, k4);
        store4(out + static_cast<int64_t>(G) * DH + d, v4);
      }
  }
}

// dkv[i] = sum over the hpg slices (in slice order), four values per thread.
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, int hpg,
                                                         int64_t n4, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 acc = reinterpret_cast<const float4*>(part)[i];
  for (int k = 1; k < hpg; ++k) {
    const float4 v = reinterpret_cast<const float4*>(part)[k * n4 + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  reinterpret_cast<float4*>(out)[i] = acc;
}

hipError_t sum_slices(const float* part, int n_slices, int64_t n4, float* out, hipStream_t s) {
  hipLaunchKernelGGL(sum_slices_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0,
                     s, part, n_slices, n4, out);
  return hipGetLastError();
}

size_t attn_bwd_mfma_ws_bytes(int B, int N, int H, int G, int dh) {
  return H / G > 1 ? sizeof(float) * static_cast<size_t>(H / G) * B * N * 2 * G * dh : 0;
}

hipError_t attn_bwd_mfma(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* d_o,
                         const float* lse, const float* dsum, int B, int N, int H, int G, int dh,
                         int64_t t_cap, float* dq, float* dkv, float* part, hipStream_t s) {
  const float scale = 1.0f / sqrtf(static_cast<float>(dh));
  const float sl2 = kLog2e * scale;
  const int n_qblk = (N + 127) / 128;
  const int n_units = n_qblk * B * G;
  const int grid_q = ((n_units + 7) / 8) * 8 * (H / G);
  const int hpg = H / G;
  const int grid_k = ((N + 127) / 128) * B * G * hpg;
  float* dst = hpg > 1 ? part : dkv;  // per-head slices, summed below
  if (dh == 128) {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, dim3(grid_q), dim3(256), 0, s, q, k, v, d_o, lse,
                       dsum, B, N, H, G, t_cap, sl2, scale, n_qblk, n_units, dq);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<128>, dim3(grid_k), dim3(256), 0, s, q, k, v, d_o, lse,
                       dsum, B, N, H, G, t_cap, sl2, scale, dst);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, dim3(grid_q), dim3(256), 0, s, q, k, v, d_o, lse,
                       dsum, B, N, H, G, t_cap, sl2, scale, n_qblk, n_units, dq);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<64>, dim3(grid_k), dim3(256), 0, s, q, k, v, d_o, lse,
                       dsum, B, N, H, G, t_cap, sl2, scale, dst);
  }
  if (hpg > 1) {
    const int64_t n4 = static_cast<int64_t>(B) * N * 2 * G * dh / 4;
    hipLaunchKernelGGL(sum_slices_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256),
                       0, s, part, hpg, n4, dkv);
  }
  return hipGetLastError();
}

}  // namespace mka
