// One causal grouped-query attention over the fused K/V (MKA reading note,
// method section 3: a single attention path over the fused cache), evaluated
// key tile by key tile with the online max-shift of method section 4: the
// running maximum mu is raised tile by tile and the running numerator and
// denominator are rescaled by exp(mu_old - mu_new).
//
// bf16 path (MFMA 32x32x16 on gfx950).  A wave owns 32 query rows and computes
// S^T = K Q^T for a 64-key tile (keys as MFMA rows), so each lane owns one
// query row: the row max and sum need a single cross-half exchange and the
// rescale factor is lane-local.  K rows are fed to the MFMA in a permuted
// order (rows 4..7 and 8..11 of every 16 swapped) which makes accumulator
// register r of lane half hl hold key 16*(r/8) + 8*hl + r%8; the
// probabilities then form, without any data movement, the B operand of
// O^T = V^T P^T, whose A operand is read from a transposed V tile in LDS.
// Scores use exp2 with log2(e)/sqrt(dh) folded into one fp32 scale per score.
#include "attn_split.h"

#include <type_traits>

namespace mka {

// 16-byte chunk swizzle of LDS row P of a K tile: a row is DH*2 bytes (256 B
// for DH = 128, 128 B for DH = 64), so 16 consecutive rows with the same
// logical chunk land in 16 distinct bank groups.
template <int DH>
__device__ __forceinline__ int kswz(int P) {
  return DH == 128 ? (P & 15) : ((P >> 1) & 7);
}

// 16-byte chunk swizzle of LDS row P of a V tile: the 4 keys x 32 bytes that
// a 16-lane group of a transposing read touches, and the two groups of a
// 32-lane half, fall in distinct bank groups.
template <int DH>
__device__ __forceinline__ int vswz(int P) {
  return DH == 128 ? 4 * (P & 3) : 4 * ((P >> 1) & 1);
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002 | 0x400;  // vector ALU, transcendentals included
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

__device__ __forceinline__ int kperm(int r) {
  const int q = r & 15;
  const int qq = (q >= 4 && q < 8) ? q + 4 : ((q >= 8 && q < 12) ? q - 4 : q);
  return (r & ~15) | qq;
}


// ---------------------------------------------------------------------------
// Prefill, bf16.  Workgroup = NW waves = 32*NW query rows of one head; K/V tiles
// of 64 keys double-buffered in LDS.  Work order: units (query block, batch,
// KV group) heaviest first; the H/G heads of a unit are consecutive slots of
// one XCD so they read the same K/V tiles through that XCD's L2.
// ---------------------------------------------------------------------------
template <int DH, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_prefill_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    bf16_t* __restrict__ O, int B, int seq, int H, int G, KvLayout kv, int64_t pos0, float sl2,
    int n_qblk, int n_units, float* __restrict__ lse) {
  constexpr int BM = 32 * NW, BN = 64, NKS = DH / 16,
                NDB = DH / 32;
  constexpr int KLD = BN * DH * 2 / 1024 / NW;  // 1 KB tile loads per wave (K and V each)
  static_assert(KLD * NW * 1024 == BN * DH * 2, "a tile splits evenly over the waves");
  // The two buffers of each tile are distinct objects and the tile loop is
  // unrolled by two, so every LDS access names a fixed buffer: the compiler
  // then sees that the next tile's direct loads do not touch the tile being
  // read and waits for them only where the loop waits explicitly.
  __shared__ __attribute__((aligned(1024))) bf16_t Ks0[BN * DH];
  __shared__ __attribute__((aligned(1024))) bf16_t Ks1[BN * DH];
  __shared__ __attribute__((aligned(1024))) bf16_t Vs0[BN * DH];
  __shared__ __attribute__((aligned(1024))) bf16_t Vs1[BN * DH];

  const int hpg = H / G;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int hh = slot % hpg, u = (slot / hpg) * 8 + xcd;
  if (u >= n_units) return;
  const int qb = n_qblk - 1 - u / (B * G);
  const int bg = u % (B * G), b = bg / G, g = bg % G, h = g * hpg + hh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  const int q_row = qb * BM + wave * 32 + l32;
  const int64_t q_pos = pos0 + q_row;
  const int64_t wave_pos0 = pos0 + qb * BM + wave * 32;
  const int64_t kv_end = pos0 + min(qb * BM + BM, seq);
  const int n_tiles = static_cast<int>((kv_end + BN - 1) / BN);

  bf16x8 qf[NKS];
  {
    // Q enters the products as stored; the scale log2(e)/sqrt(dh) is applied
    // in fp32 to each score (folding it into Q would round Q to bf16 a second
    // time, which moves peaked softmax weights by up to ~1%).
    const bf16_t* qp = Q + (static_cast<int64_t>(b * seq + min(q_row, seq - 1)) * H + h) * DH + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
      if (q_row >= seq) qf[ks] = bf16x8{};
    }
  }
  PageWindow<PAGED> pw;
  pw.fill(kv, b, 0);
  // K and V tiles go global -> LDS directly (no registers): load instruction
  // i of wave w fills the 1 KB at LDS chunk w*KLD + i, lane l its 16 bytes at
  // +16*l, so each lane fetches the source row and chunk that its slot needs.
  // K: LDS row P holds tile row kperm(P) (kperm is its own inverse), its
  // 16-byte chunks XOR-swizzled by kswz(P) so that the 16 rows of an MFMA
  // fragment read fall in distinct banks.  V: LDS row P holds key P, chunks
  // swizzled by vswz(P) for the transposing fragment reads below.
  constexpr int RPC = 1024 / (DH * 2);  // rows per 1 KB
  uint32_t k_src[KLD], v_src[KLD];
#pragma unroll
  for (int i = 0; i < KLD; ++i) {
    const int P = (wave * KLD + i) * RPC + lane / (DH / 8), c = lane % (DH / 8);
    k_src[i] = static_cast<uint32_t>(kperm(P) * DH + 8 * (c ^ kswz<DH>(P))) * 2;
    v_src[i] = static_cast<uint32_t>(P * DH + 8 * (c ^ vswz<DH>(P))) * 2;
  }
  // V^T fragments for O^T += V^T P^T come from two ds_read_b64_tr_b16 each: in
  // a 16-lane group, lane r of the group addresses 4 consecutive dims of one
  // key and lane i receives one dim of 4 consecutive keys (dim i, keys 0..3 of
  // the group's block when lane r reads key r/4, dims 4*(r%4)..).  Lane l of
  // the wave then holds dim db*32 + l%32 and keys 8*(l/32) .. +7 of a 16-key
  // step, as the MFMA's A operand wants.  The swizzle of a key's row is a
  // per-lane constant here, so per dim block a lane keeps one base address
  // and steps keys by immediate offsets.
  const int vr = lane & 15, vg = (lane >> 4) & 1;
  int v_base[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int key0 = 8 * hl + (vr >> 2), d = db * 32 + 16 * vg + 4 * (vr & 3);
    v_base[db] = key0 * DH + 8 * ((d >> 3) ^ vswz<DH>(key0)) + (d & 7);
  }
  // One tile of BN keys lies in one page (pages hold a multiple of 64 rows);
  // keys at or beyond kv_end read as zeros through the buffer range.
  auto gload = [&](int j0, bf16_t* ks, bf16_t* vs) __attribute__((always_inline)) {
    const int64_t off = pw.row(kv, b, g, j0);
    const uint32_t bytes = static_cast<uint32_t>(min<int64_t>(BN, kv_end - j0) * DH * 2);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kc + off, bytes), vrs = make_rsrc(Vc + off, bytes);
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      buffer_load_lds16(krs, (lds_void_t*)(ks + (wave * KLD + i) * 512), k_src[i]);
      buffer_load_lds16(vrs, (lds_void_t*)(vs + (wave * KLD + i) * 512), v_src[i]);
    }
  };

  // ms: the running reference of the row's scores in the exp2 domain
  // (scores scaled by log2(e)/sqrt(dh)); l_i and acc are relative to it.
  float ms = 0.f, l_i = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  gload(0, Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());  // this wave's tile loads have landed
  __syncthreads();
  // One key tile; MASKED: the tile holds keys after some of the wave's query
  // rows (a diagonal tile), which are masked out.  The tiles without a mask
  // take a separate copy of the body so that nothing branches between the
  // score products and the probabilities.
  auto body = [&](int jt, int j0, const bf16_t* kt, const bf16_t* vt, auto MASKED)
                  __attribute__((always_inline)) {
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int P = kb * 32 + l32;
      const bf16_t* kr = kt + P * DH;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        s[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kr + 8 * ((2 * ks + hl) ^ kswz<DH>(P))),
                             qf[ks], s[kb]);
      if constexpr (!decltype(MASKED)::value) {
        if (kb == 0) {
          // first half's products with their K reads a few ahead; the second
          // half is scheduled together with the first half's probabilities
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
          for (int i = 0; i < NKS; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (i < NKS - 4) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // Online max-shift in the exp2 domain: ms is the running reference.  It
    // is raised only when a tile's maximum exceeds it by more than 8, so most
    // tiles need no rescale; probabilities stay below 2^8, which fp32 sums
    // and bf16 operands carry as well as values below 1.
    if constexpr (decltype(MASKED)::value) {
      const int q_rel = static_cast<int>(q_pos - j0);  // keys of the tile after the query
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 16 * (r >> 3) + 8 * hl + (r & 7) > q_rel) s[kb][r] = -INFINITY;
    }

    // Probabilities of key half kb as the bf16x8 B operands of
    // O^T += V^T P^T; the row sum adds the same bf16 values the products use,
    // two per v_dot2 (each pair is built as a bf16x2 value: bit-casting the
    // words of a packed u32x4 instead made the compiler feed the first word to
    // all four dot products).
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    bf16x8 pf[2][2];
    auto probs = [&](int kb, float nms, float& l) __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2v v = {
              static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[kb][8 * st + 2 * i], sl2, nms))),
              static_cast<__bf16>(
                  __builtin_amdgcn_exp2f(fmaf(s[kb][8 * st + 2 * i + 1], sl2, nms)))};
          l = __builtin_amdgcn_fdot2_f32_bf16(v, ones, l, false);
          w[i] = __builtin_bit_cast(uint32_t, v);
        }
        pf[kb][st] = __builtin_bit_cast(bf16x8, w);
      }
    };
    // The first key half's probabilities are formed with the current
    // reference before the tile's maximum is known, so that they overlap the
    // second half's score products; a tile that raises the reference (the
    // first tile always does) forms them again.  The results are those of
    // forming every probability after the raise decision.
    float l_new = l_i;
    probs(0, -ms, l_new);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
    if constexpr (!decltype(MASKED)::value) {
      // The second half's products (K reads a few ahead) with the first
      // half's probabilities and maximum between them: the matrix cores and
      // the vector ALU work on them at the same time.  The empty asm takes
      // the probabilities as inputs, so that they are formed before the
      // scheduling fence below and not next to their later uses.  With
      // dh = 128, 5 vector instructions per product here and 8 in the value
      // products below (the rest of this half's work goes there) measured
      // best (7 and 6: 1% slower; 9 and 4: 2% slower).
      asm volatile("" ::"v"(pf[0][0]), "v"(pf[0][1]), "v"(l_new), "v"(mx));
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
      for (int i = 0; i < NKS; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < NKS - 4) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, DH == 128 ? 5 : 56 / NKS, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    {  // the two lanes of a query (l and l^32) exchange their maxima by a lane swap
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // The tile's maximum relative to the reference, in the exp2 domain; the
    // reference is raised to it when that exceeds 8 (and on the first tile,
    // whose maximum is finite: key 0 is visible to every query row).
    mx = fmaf(mx, sl2, -ms);
    const bool raise = jt == 0 || mx > 8.0f;
    if (__any(raise)) {
      const float delta = raise ? mx : 0.0f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      l_i *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      ms += delta;
      l_new = l_i;
      probs(0, -ms, l_new);
    }

    // O^T += V^T P^T, first key half while the second half's probabilities
    // are formed.
    auto pv = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16_t* vb = vt + v_base[db];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int k0 = (kb * 32 + 16 * st) * DH;
          const bf16x4 lo = ds_read_tr16_b64(vb + k0), hi = ds_read_tr16_b64(vb + k0 + 4 * DH);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[db] = mfma32x32x16(vf, pf[kb][st], acc[db]);
        }
      }
    };
    pv(0);
    probs(1, -ms, l_new);
    pv(1);
    l_i = l_new;
    if constexpr (!decltype(MASKED)::value) {
      // The first half's value products with the second half's probabilities
      // between them; then the second half's products.  Six V^T fragment
      // reads go out ahead of the first product (two: 2% slower; four: 0.3%).
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, DH == 128 ? 8 : 6, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < 5) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
    }
  };
  auto tile = [&](int jt, const bf16_t* kt, const bf16_t* vt, bf16_t* kn, bf16_t* vn)
                  __attribute__((always_inline)) {
    const int j0 = jt * BN;
    if (jt + 1 < n_tiles) gload(j0 + BN, kn, vn);
    if ((j0 + BN - 1) > wave_pos0)
      body(jt, j0, kt, vt, std::true_type{});
    else
      body(jt, j0, kt, vt, std::false_type{});
    __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());  // this wave's tile loads have landed
    __syncthreads();
  };
  for (int jt = 0; jt < n_tiles; jt += 2) {
    tile(jt, Ks0, Vs0, Ks1, Vs1);
    if (jt + 1 < n_tiles) tile(jt + 1, Ks1, Vs1, Ks0, Vs0);
  }

  l_i += __shfl_xor(l_i, 32, 64);
  if (q_row < seq) {
    const float inv = 1.0f / l_i;
    bf16_t* op = O + (static_cast<int64_t>(b * seq + q_row) * H + h) * DH;
    // natural log-sum-exp of the row's scaled scores, for the backward
    if (lse != nullptr && hl == 0)
      lse[static_cast<int64_t>(b * seq + q_row) * H + h] = (ms + log2f(l_i)) * 0.69314718055994531f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float v[4] = {acc[db][4 * rq] * inv, acc[db][4 * rq + 1] * inv,
                            acc[db][4 * rq + 2] * inv, acc[db][4 * rq + 3] * inv};
        store4(op + db * 32 + 8 * rq + 4 * hl, v);
      }
  }
}

// ---------------------------------------------------------------------------
// Prefill, fp32: one thread per query row with the online max-shift over key
// tiles staged in LDS (the reference-precision path of small fp32 layers).
// ---------------------------------------------------------------------------
template <int DH, bool PAGED>
__global__ __launch_bounds__(64) void attn_prefill_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kc, const float* __restrict__ Vc,
    float* __restrict__ O, int seq, int H, int G, KvLayout kv, int64_t pos0, float scale,
    float* __restrict__ lse) {
  constexpr int TK = 32;
  __shared__ float Ks[TK][DH];
  __shared__ float Vs[TK][DH];
  const int tid = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = blockIdx.x * 64 + tid;
  const int g = h / (H / G);
  const int64_t q_pos = pos0 + t;
  const int64_t kv_end = pos0 + min(static_cast<int>(blockIdx.x) * 64 + 64, seq);
  float q[DH], acc[DH];
  const float* qp = Q + (static_cast<int64_t>(b * seq + min(t, seq - 1)) * H + h) * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    q[d] = qp[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  PageWindow<PAGED> pw;
  pw.fill(kv, b, 0);
  for (int64_t j0 = 0; j0 < kv_end; j0 += TK) {
    // a tile of TK keys lies in one page
    const int64_t off = pw.row(kv, b, g, j0);
    const float* kb = Kc + off;
    const float* vb = Vc + off;
    for (int e = tid; e < TK * DH; e += 64) {
      const int r = e / DH, d = e % DH;
      const bool ok = j0 + r < kv_end;
      Ks[r][d] = ok ? kb[r * DH + d] : 0.f;
      Vs[r][d] = ok ? vb[r * DH + d] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < TK; ++jj) {
      const int64_t j = j0 + jj;
      if (j > q_pos || j >= kv_end) break;
      float sdot = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) sdot = fmaf(q[d], Ks[jj][d], sdot);
      const float sc = sdot * scale;
      const float m_new = fmaxf(m, sc);
      const float corr = expf(m - m_new);
      const float p = expf(sc - m_new);
      l = l * corr + p;
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, Vs[jj][d], acc[d] * corr);
      m = m_new;
    }
    __syncthreads();
  }
  if (t < seq) {
    float* op = O + (static_cast<int64_t>(b * seq + t) * H + h) * DH;
    const float inv = 1.0f / l;
    if (lse != nullptr) lse[static_cast<int64_t>(b * seq + t) * H + h] = m + logf(l);
#pragma unroll
    for (int d = 0; d < DH; ++d) op[d] = acc[d] * inv;
  }
}

// Waves per workgroup (32 query rows each).  4: two workgroups share a CU and
// their softmax and MFMA phases overlap on the SIMDs; 8 waves per workgroup
// measured no faster.
constexpr int kAttnWaves = 4;

template <>
hipError_t attn_prefill<bf16_t>(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o, int B,
                                int seq, int H, int G, int dh, const KvLayout& kv, int64_t pos0,
                                float* lse, hipStream_t s) {
  constexpr int NW = kAttnWaves;
  const int n_qblk = (seq + 32 * NW - 1) / (32 * NW);
  const int n_units = n_qblk * B * G;
  const int grid = ((n_units + 7) / 8) * 8 * (H / G);
  const float sl2 = 1.4426950408889634f / sqrtf(static_cast<float>(dh));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(NW * 64), 0, s, q, k, v, o, B, seq, H, G, kv, pos0,
                       sl2, n_qblk, n_units, lse);
  };
  if (dh == 128)
    kv.paged() ? launch(attn_prefill_bf16_kernel<128, NW, true>)
               : launch(attn_prefill_bf16_kernel<128, NW, false>);
  else
    kv.paged() ? launch(attn_prefill_bf16_kernel<64, NW, true>)
               : launch(attn_prefill_bf16_kernel<64, NW, false>);
  return hipGetLastError();
}

template <>
hipError_t attn_prefill<float>(const float* q, const float* k, const float* v, float* o, int B,
                               int seq, int H, int G, int dh, const KvLayout& kv, int64_t pos0,
                               float* lse, hipStream_t s) {
  const dim3 grid((seq + 63) / 64, H, B);
  const float scale = 1.0f / sqrtf(static_cast<float>(dh));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(64), 0, s, q, k, v, o, seq, H, G, kv, pos0, scale, lse);
  };
  if (dh == 128)
    kv.paged() ? launch(attn_prefill_f32_kernel<128, true>)
               : launch(attn_prefill_f32_kernel<128, false>);
  else
    kv.paged() ? launch(attn_prefill_f32_kernel<64, true>)
               : launch(attn_prefill_f32_kernel<64, false>);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode, bf16: the split kernel (one share of the rows per workgroup, see
// attn_split.h) and the merge of its partials with the last cache row.
// ---------------------------------------------------------------------------
static int decode_units(int B, int H, int G) { return B * G * ((H / G + kSplitHeads - 1) / kSplitHeads); }

size_t attn_decode_ws_bytes(int B, int H, int G, int dh, int64_t n_rows) {
  const int64_t n_chunks = n_rows > 0 ? decode_n_chunks(decode_units(B, H, G), n_rows) : 0;
  return sizeof(float) * static_cast<size_t>(B) * H * n_chunks * (dh + 2);
}

template <int DH, bool PAGED>
__global__ __launch_bounds__(256, 2) void attn_decode_split_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    int H, int G, KvLayout kv, int64_t n_rows, float sl2, int n_chunks, int n_hb,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ part_o) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[split_lds_bytes<DH>()];
  const int g = blockIdx.y / n_hb, hb = blockIdx.y % n_hb;
  decode_split_chunk<DH, PAGED>(Q, Kc, Vc, H, G, kv, n_rows, sl2, n_chunks, blockIdx.x, g, hb,
                         blockIdx.z, part_m, part_l, part_o, lds);
}

// The extra row comes from the cache (row ``extra_row``; none if negative).
template <int DH>
__global__ __launch_bounds__(kMergeThreads) void attn_decode_merge_kernel(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_o, int H, int G, int n_chunks, const bf16_t* __restrict__ Q,
    const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc, KvLayout kv,
    int64_t extra_row, float sl2, bf16_t* __restrict__ O) {
  __shared__ MergeLds<DH> sm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t row = extra_row >= 0 ? kv.row(b, h / (H / G), extra_row) : 0;
  decode_merge_head<DH>(part_m, part_l, part_o, H, n_chunks, h, b, Q, sl2, O, sm,
                        [&](float* kx, float* vx) {
                          if (extra_row < 0) return false;
                          const int tid = threadIdx.x;
                          if (tid < DH) {
                            kx[tid] = bf16_to_f32(Kc[row + tid]);
                            vx[tid] = bf16_to_f32(Vc[row + tid]);
                          }
                          return true;
                        });
}


hipError_t attn_decode_split_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, int B, int H,
                                  int G, int dh, const KvLayout& kv, int64_t n_old, void* ws,
                                  hipStream_t s) {
  if (n_old <= 0) return hipSuccess;
  const int n_chunks = decode_n_chunks(decode_units(B, H, G), n_old);
  if (n_chunks > kMaxDecodeChunks) return hipErrorInvalidValue;
  float* part_m = static_cast<float*>(ws);
  float* part_l = part_m + static_cast<size_t>(B) * H * n_chunks;
  float* part_o = part_l + static_cast<size_t>(B) * H * n_chunks;
  const float sl2 = 1.4426950408889634f / sqrtf(static_cast<float>(dh));
  const int n_hb = (H / G + kSplitHeads - 1) / kSplitHeads;
  const dim3 grid(n_chunks, G * n_hb, B);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, q, k, v, H, G, kv, n_old, sl2, n_chunks,
                       n_hb, part_m, part_l, part_o);
  };
  if (dh == 128)
    kv.paged() ? launch(attn_decode_split_kernel<128, true>)
               : launch(attn_decode_split_kernel<128, false>);
  else
    kv.paged() ? launch(attn_decode_split_kernel<64, true>)
               : launch(attn_decode_split_kernel<64, false>);
  return hipGetLastError();
}

hipError_t attn_decode_merge_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o,
                                  int B, int H, int G, int dh, const KvLayout& kv, int64_t n_old,
                                  int64_t extra_row, void* ws, hipStream_t s) {
  const int n_chunks = n_old > 0 ? decode_n_chunks(decode_units(B, H, G), n_old) : 0;
  if (n_chunks > kMaxDecodeChunks) return hipErrorInvalidValue;
  float* part_m = static_cast<float*>(ws);
  float* part_l = part_m + static_cast<size_t>(B) * H * n_chunks;
  float* part_o = part_l + static_cast<size_t>(B) * H * n_chunks;
  const float sl2 = 1.4426950408889634f / sqrtf(static_cast<float>(dh));
  if (dh == 128)
    hipLaunchKernelGGL(attn_decode_merge_kernel<128>, dim3(H, B), dim3(kMergeThreads), 0, s, part_m,
                       part_l, part_o, H, G, n_chunks, q, k, v, kv, extra_row, sl2, o);
  else
    hipLaunchKernelGGL(attn_decode_merge_kernel<64>, dim3(H, B), dim3(kMergeThreads), 0, s, part_m,
                       part_l, part_o, H, G, n_chunks, q, k, v, kv, extra_row, sl2, o);
  return hipGetLastError();
}

// Rows [0, cache_len - 1) through the split kernel; the last row in the merge.
hipError_t attn_decode_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o, int B,
                            int H, int G, int dh, const KvLayout& kv, int64_t cache_len, void* ws,
                            hipStream_t s) {
  const hipError_t e = attn_decode_split_bf16(q, k, v, B, H, G, dh, kv, cache_len - 1, ws, s);
  if (e != hipSuccess) return e;
  return attn_decode_merge_bf16(q, k, v, o, B, H, G, dh, kv, cache_len - 1, cache_len - 1, ws, s);
}

}  // namespace mka
