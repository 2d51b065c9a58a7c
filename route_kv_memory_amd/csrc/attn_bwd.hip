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

// 16-byte chunk swizzle of LDS row P of a row tile that is read both as MFMA
// row fragments (16 consecutive rows, one chunk) and transposed (4 consecutive
// rows x 32 bytes per 16-lane group, two groups per 32-lane half): both land
// on distinct banks (checked on the CPU for dh = 64 and 128).
template <int DH>
__device__ __forceinline__ int cswz(int P) {
  return DH == 128 ? 4 * (P & 3) + ((P >> 2) & 3) : 4 * ((P >> 1) & 1) + ((P >> 2) & 3);
}

// Transposed operand from a row tile in LDS: the bf16x8 A operand holding dim
// d of rows r0 .. r0+7 (lane l: d = d0 + l%32, rows 8*(l/32) ..), read with two
// ds_read_b64_tr_b16 whose per-lane addresses ``a0``/``a1`` select, in each
// 16-lane group, 4 consecutive dims of row r/4 (see ds_read_tr16_b64).
__device__ __forceinline__ bf16x8 ld_tr8(const bf16_t* a0, const bf16_t* a1) {
  const bf16x4 lo = ds_read_tr16_b64(a0), hi = ds_read_tr16_b64(a1);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

// ---------------------------------------------------------------------------
// dq.  Workgroup = 4 waves = 128 query rows of head h; K/V tiles of 64 keys,
// double-buffered in LDS as rows: row fragments for S^T and dP^T, K read
// transposed for dQ.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dsum,
    int B, int N, int H, int G, int64_t t_cap, float sl2, float scale, int n_qblk, int n_units,
    float* __restrict__ dq) {
  constexpr int BM = 128, BN = 64, NKS = DH / 16, NDB = DH / 32;
  constexpr int TLD = BN * DH * 2 / 1024 / 4;  // 1 KB loads per wave per tile (K and V each)
  constexpr int RPC = 1024 / (DH * 2);         // rows per 1 KB
  __shared__ __attribute__((aligned(1024))) bf16_t Ks[2][BN * DH];
  __shared__ __attribute__((aligned(1024))) bf16_t Vs[2][BN * DH];

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

  // K and V tiles go global -> LDS directly (as in the dK/dV kernel): LDS row
  // P holds tile row bperm(P), chunks swizzled by cswz(P); keys at or beyond
  // kv_end lie outside the buffer range and read as zeros.
  uint32_t t_src[TLD];
#pragma unroll
  for (int i = 0; i < TLD; ++i) {
    const int P = (wave * TLD + i) * RPC + lane / (DH / 8), c = lane % (DH / 8);
    t_src[i] = static_cast<uint32_t>((bperm(P) * DH + 8 * (c ^ cswz<DH>(P))) * 2);
  }
  int t_base[2][NDB];  // transposed K reads (see the dK/dV kernel)
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int r = lane & 15, G2 = (lane >> 4) & 1;
      const int P = bperm(8 * hl + 4 * q + (r >> 2)), d = db * 32 + 16 * G2 + 4 * (r & 3);
      t_base[q][db] = P * DH + 8 * ((d >> 3) ^ cswz<DH>(P)) + (d & 7);
    }
  auto gload = [&](int j0, int buf) {
    const uint32_t bytes = static_cast<uint32_t>(min(BN, kv_end - j0) * DH * 2);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase + static_cast<int64_t>(j0) * DH, bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase + static_cast<int64_t>(j0) * DH, bytes);
#pragma unroll
    for (int i = 0; i < TLD; ++i) {
      buffer_load_lds16(krs, (lds_void_t*)(&Ks[buf][(wave * TLD + i) * 512]), t_src[i]);
      buffer_load_lds16(vrs, (lds_void_t*)(&Vs[buf][(wave * TLD + i) * 512]), t_src[i]);
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  gload(0, 0);
  __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());  // this wave's tile loads have landed
  __syncthreads();
  for (int jt = 0; jt < n_tiles; ++jt) {
    const int buf = jt & 1, j0 = jt * BN;
    if (jt + 1 < n_tiles) gload(j0 + BN, buf ^ 1);
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
      const int P = kb * 32 + l32;
      const bf16_t* kr = &Ks[buf][P * DH];
      const bf16_t* vr = &Vs[buf][P * DH];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c = 8 * ((2 * ks + hl) ^ cswz<DH>(P));
        s[kb] = mfma32x32x16(ld8(kr + c), qf[ks], s[kb]);
        dp[kb] = mfma32x32x16(ld8(vr + c), gf[ks], dp[kb]);
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
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int o = (kb * 32 + 16 * st) * DH;
          acc[db] = mfma32x32x16(ld_tr8(&Ks[buf][t_base[0][db] + o], &Ks[buf][t_base[1][db] + o]),
                                 dsf[kb][st], acc[db]);
        }
    }
    __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());  // this wave's tile loads have landed
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
// MODE 0 computes dK and dV together (K, V fragments and both accumulators in
// registers: one workgroup per CU); MODE 1 computes dK alone and MODE 2 dV
// alone, each recomputing the scores, in few enough registers for two
// workgroups per CU (two waves per SIMD).
// ---------------------------------------------------------------------------
template <int DH, int MODE>
__global__ __launch_bounds__(256, MODE == 0 ? 1 : 2) void attn_bwd_dkv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dsum,
    int B, int N, int H, int G, int64_t t_cap, float sl2, float scale, float* __restrict__ dkv) {
  constexpr int BK = 128, BQ = 64, NKS = DH / 16, NDB = DH / 32;
  constexpr int TLD = BQ * DH * 2 / 1024 / 4;  // 1 KB loads per wave per tile (Q and dO each)
  constexpr int RPC = 1024 / (DH * 2);         // rows per 1 KB
  // Each buffer is an object of its own and the tile loop is unrolled by
  // two, so the compiler sees that the next tile's direct loads do not touch
  // the tile being read (it would otherwise wait for them before each read).
  __shared__ __attribute__((aligned(1024))) bf16_t Qs0[BQ * DH];
  __shared__ __attribute__((aligned(1024))) bf16_t Qs1[BQ * DH];
  __shared__ __attribute__((aligned(1024))) bf16_t Gs0[BQ * DH];
  __shared__ __attribute__((aligned(1024))) bf16_t Gs1[BQ * DH];
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
  constexpr bool WK = MODE != 2, WV = MODE != 1;  // dK / dV computed here
  bf16x8 kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = ld8(Kc + kvoff + 16 * ks);
    if (k_row >= N) kf[ks] = bf16x8{};
    if constexpr (WK) {
      vf[ks] = ld8(Vc + kvoff + 16 * ks);
      if (k_row >= N) vf[ks] = bf16x8{};
    }
  }
  const int t_first = kblk * BK;
  const int n_it = (N - t_first + BQ - 1) / BQ;  // query tiles of head g*hpg + hh

  // Q and dO tiles go global -> LDS directly: load instruction i of wave w
  // fills the 1 KB at LDS chunk w*TLD + i, lane l its 16 bytes at +16*l.  LDS
  // row P holds tile row bperm(P) (the permuted feed), chunks swizzled by
  // cswz(P); the rows of head h are H*DH apart in Q and dO.  Rows past N lie
  // outside the buffer range and read as zeros; their lse is +inf (P = 0).
  const int h = g * hpg + hh;
  uint32_t t_src[TLD];
#pragma unroll
  for (int i = 0; i < TLD; ++i) {
    const int P = (wave * TLD + i) * RPC + lane / (DH / 8), c = lane % (DH / 8);
    t_src[i] = static_cast<uint32_t>((bperm(P) * H * DH + 8 * (c ^ cswz<DH>(P))) * 2);
  }
  // transposed reads: lane (group row r, group G, half hl) addresses dims
  // db*32 + 16G + 4(r%4) .. of tile row 8hl + 4q + r/4 (+ 32qb + 16st)
  int t_base[2][NDB];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int r = lane & 15, G = (lane >> 4) & 1;
      const int P = bperm(8 * hl + 4 * q + (r >> 2)), d = db * 32 + 16 * G + 4 * (r & 3);
      t_base[q][db] = P * DH + 8 * ((d >> 3) ^ cswz<DH>(P)) + (d & 7);
    }
  // rl, rd: the raw log-sum-exp and D of the next tile's rows; they are
  // converted where they are stored to LDS, at the end of the tile, because
  // waiting for these loads earlier would also wait for the tile loads issued
  // before them.
  float rl = 0.f, rd = 0.f;
  auto gload = [&](int it, bf16_t* qs, bf16_t* gs) __attribute__((always_inline)) {
    const int t0 = t_first + it * BQ;
    const int nrow = min(BQ, N - t0);
    const int64_t base = (static_cast<int64_t>(b) * N + t0) * H * DH + static_cast<int64_t>(h) * DH;
    const uint32_t bytes = static_cast<uint32_t>(((nrow - 1) * H + 1) * DH * 2);
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, bytes), grs = make_rsrc(dO + base, bytes);
#pragma unroll
    for (int i = 0; i < TLD; ++i) {
      buffer_load_lds16(qrs, (lds_void_t*)(qs + (wave * TLD + i) * 512), t_src[i]);
      buffer_load_lds16(grs, (lds_void_t*)(gs + (wave * TLD + i) * 512), t_src[i]);
    }
    if (tid < BQ) {
      const int t = t0 + tid;
      const int64_t row = static_cast<int64_t>(b * N + min(t, N - 1)) * H + h;
      rl = lse[row];
      rd = dsum[row];
    }
  };
  auto sstore = [&](int it, int buf) {
    if (tid < BQ) {
      const bool in = t_first + it * BQ + tid < N;
      Ls[buf][tid] = in ? rl * kLog2e : INFINITY;
      Ds[buf][tid] = in ? rd : 0.f;
    }
  };

  f32x16 adk[NDB], adv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    adk[db] = f32x16{};
    adv[db] = f32x16{};
  }
  gload(0, Qs0, Gs0);
  sstore(0, 0);
  __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());  // this wave's tile loads have landed
  __syncthreads();
  auto tile = [&](int it, int buf, const bf16_t* qt, const bf16_t* gt, bf16_t* qn, bf16_t* gn)
                  __attribute__((always_inline)) {
    // An opaque zero offset keeps the LDS address arithmetic inside the loop
    // (hoisted for both buffers it would not fit in the registers); the
    // pointers still derive from their own buffer objects.
    int z = 0;
    asm volatile("" : "+s"(z));
    qt += z;
    gt += z;
    const int t0 = t_first + it * BQ;
    if (it + 1 < n_it) gload(it + 1, qn, gn);
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
      const int P = qb * 32 + l32;
      const bf16_t* qr = qt + P * DH;
      const bf16_t* gr = gt + P * DH;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c = 8 * ((2 * ks + hl) ^ cswz<DH>(P));
        s[qb] = mfma32x32x16(ld8(qr + c), kf[ks], s[qb]);
        if constexpr (WK) dp[qb] = mfma32x32x16(ld8(gr + c), vf[ks], dp[qb]);
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
          if constexpr (WK) dv[j] = p * (dp[qb][r] - Ds[buf][q0 + j]);
        }
        if constexpr (WV) pf[qb][st] = pack_bf16x8(pv);
        if constexpr (WK) dsf[qb][st] = pack_bf16x8(dv);
      }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int o = (qb * 32 + 16 * st) * DH;
          if constexpr (WV)
            adv[db] = mfma32x32x16(ld_tr8(gt + t_base[0][db] + o, gt + t_base[1][db] + o),
                                   pf[qb][st], adv[db]);
          if constexpr (WK)
            adk[db] = mfma32x32x16(ld_tr8(qt + t_base[0][db] + o, qt + t_base[1][db] + o),
                                   dsf[qb][st], adk[db]);
        }
    }
    if (it + 1 < n_it) sstore(it + 1, buf ^ 1);
    __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());  // this wave's tile loads have landed
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);  // the two copies of the body are scheduled apart
  };
  for (int it = 0; it < n_it; it += 2) {
    tile(it, 0, Qs0, Gs0, Qs1, Gs1);
    if (it + 1 < n_it) tile(it + 1, 1, Qs1, Gs1, Qs0, Gs0);
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
        if constexpr (WK) store4(out + d, k4);
        if constexpr (WV) store4(out + static_cast<int64_t>(G) * DH + d, v4);
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

// dK and dV in separate passes (MODE 1 then 2) or together (0).
constexpr int kDkvMode = 1;

size_t attn_bwd_mfma_ws_bytes(int B, int N, int H, int G, int dh) {
  return H / G > 1 ? sizeof(float) * static_cast<size_t>(H / G) * B * N * 2 * G * dh : 0;
}

// A null dq skips the dq kernel and a null dkv the dK/dV passes, so that a
// caller can put the two halves (independent: both only read q, K, V, dO,
// the log-sum-exp and D) on different streams.
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
  if (dq != nullptr) {
    if (dh == 128)
      hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, dim3(grid_q), dim3(256), 0, s, q, k, v, d_o, lse,
                         dsum, B, N, H, G, t_cap, sl2, scale, n_qblk, n_units, dq);
    else
      hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, dim3(grid_q), dim3(256), 0, s, q, k, v, d_o, lse,
                         dsum, B, N, H, G, t_cap, sl2, scale, n_qblk, n_units, dq);
  }
  if (dkv == nullptr) return hipGetLastError();
  if (dh == 128) {
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<128, kDkvMode>), dim3(grid_k), dim3(256), 0, s, q, k, v,
                       d_o, lse, dsum, B, N, H, G, t_cap, sl2, scale, dst);
    if (kDkvMode != 0)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<128, 2>), dim3(grid_k), dim3(256), 0, s, q, k, v, d_o,
                         lse, dsum, B, N, H, G, t_cap, sl2, scale, dst);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<64, kDkvMode>), dim3(grid_k), dim3(256), 0, s, q, k, v,
                       d_o, lse, dsum, B, N, H, G, t_cap, sl2, scale, dst);
    if (kDkvMode != 0)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<64, 2>), dim3(grid_k), dim3(256), 0, s, q, k, v, d_o,
                         lse, dsum, B, N, H, G, t_cap, sl2, scale, dst);
  }
  if (hpg > 1) {
    const int64_t n4 = static_cast<int64_t>(B) * N * 2 * G * dh / 4;
    hipLaunchKernelGGL(sum_slices_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256),
                       0, s, part, hpg, n4, dkv);
  }
  return hipGetLastError();
}

}  // namespace mka
