// Split-K decode attention over one chunk of the fused KV cache (landing page,
// Table 5: decode streams the single fused K/V tensor; reading note, method
// section 4: online max-shift).  Shared by the standalone decode attention and
// the fused decode-step kernel.
//
// A workgroup takes one share ("chunk" c of n_chunks) of the rows of one
// (batch, KV group) for a block of up to 16 query heads of that group: the
// groups of four 32-key tiles c, c + n_chunks, c + 2 n_chunks, ..., one tile
// of each group per wave, each wave with the K and V loads of its next two
// tiles in flight while the probabilities and P V products of the current
// one are computed.  Interleaving the shares keeps the reads of all
// workgroups of a KV head inside one window of the cache at any time, which
// DRAM serves faster than as many separate streams (contiguous chunks took 8%
// longer on a cache read from HBM).  There are about as many shares as CUs
// (decode_chunk_keys): a CU streams one share at the rate its memory pipeline
// allows, so a second share on any CU would double the launch time.  Scores
// are S^T = K Q^T on MFMA 16x16x32 (keys as rows, the heads as the 16
// columns).  The K rows of a tile are fed in the order key(kb, i) =
// 8*(i/4) + 4*kb + i%4 for MFMA row i of sub-block kb, which leaves lane l
// holding keys 8*(l/16) .. 8*(l/16)+7 of head l%16: exactly the
// B operand of O^T = V^T P^T, so the probabilities go to the second product
// without data movement.  V is transposed through a per-wave LDS region.
// The 4 waves merge in LDS into one partial (max, sum, unnormalised output)
// per head; the partials of all chunks are merged by a second kernel.
#pragma once

#include "kernels.h"

namespace mka {

constexpr int kSplitTile = 32;  // keys per wave per step
constexpr int kSplitHeads = 16; // query heads per workgroup (MFMA columns)
constexpr int kDecodeTargetWgs = 256;  // one workgroup per CU of the MI355X
constexpr int kMinDecodeChunk = 256;

// Keys per chunk for n_rows cache rows split over ``units`` = B * G * (head
// blocks) independent streams: about kDecodeTargetWgs chunks in all, a
// multiple of the tile, at least kMinDecodeChunk.  Host and device.
__host__ __device__ inline int decode_chunk_keys(int units, int64_t n_rows) {
  const int per_unit = units >= kDecodeTargetWgs ? 1 : kDecodeTargetWgs / units;
  int64_t c = (n_rows + per_unit - 1) / per_unit;
  c = (c + kSplitTile - 1) / kSplitTile * kSplitTile;
  return static_cast<int>(c < kMinDecodeChunk ? kMinDecodeChunk : c);
}
__host__ __device__ inline int decode_n_chunks(int units, int64_t n_rows) {
  const int c = decode_chunk_keys(units, n_rows);
  return static_cast<int>((n_rows + c - 1) / c);
}

template <int DH>
constexpr int split_lds_bytes() {
  // per-wave transposed V tiles; the 4-wave merge reuses the region
  return 4 * DH * (kSplitTile + 8) * 2;
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 floats -> bf16x8 (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
  return __builtin_bit_cast(bf16x8, w);
}

// Transpose a 4-key x 8-dim bf16 block (4 x 16-byte rows) into 8 rows of 4
// keys and store them at Vt[(d0 + i) * pitch + k0].
__device__ __forceinline__ void store_v_transposed(bf16_t* Vt, int pitch, int d0, int k0,
                                                   const u32x4* rv) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo01 = (rv[0][j] & 0xFFFFu) | (rv[1][j] << 16);
    const uint32_t lo23 = (rv[2][j] & 0xFFFFu) | (rv[3][j] << 16);
    const uint32_t hi01 = (rv[0][j] >> 16) | (rv[1][j] & 0xFFFF0000u);
    const uint32_t hi23 = (rv[2][j] >> 16) | (rv[3][j] & 0xFFFF0000u);
    *reinterpret_cast<u32x2*>(&Vt[(d0 + 2 * j) * pitch + k0]) = u32x2{lo01, lo23};
    *reinterpret_cast<u32x2*>(&Vt[(d0 + 2 * j + 1) * pitch + k0]) = u32x2{hi01, hi23};
  }
}

// Orders a wave's own LDS accesses: LDS operations of one wave complete in
// issue order and the fence keeps the compiler from moving them across.  The
// V regions are private to their wave, so no workgroup barrier is needed.
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup"); }

// Partials of share c for heads hb*16 .. of KV group g, sequence b, over its
// tiles of cache rows [0, n_rows) (tile groups c, c + n_chunks, ...).  Partial p
// of query head h lives at (b*H + h) * n_chunks + c of part_m / part_l and
// p*DH of part_o.  Uses 256 threads and split_lds_bytes<DH>() bytes of ``lds``.
template <int DH, bool PAGED>
__device__ __forceinline__ void decode_split_chunk(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    int H, int G, const KvLayout& kv, int64_t n_rows, float sl2, int n_chunks, int c,
    int g, int hb, int b, float* __restrict__ part_m, float* __restrict__ part_l,
    float* __restrict__ part_o, unsigned char* lds) {
  constexpr int BN = kSplitTile, VP = BN + 8, NKS = DH / 32, NDB = DH / 16, KQ = BN / 4;
  constexpr int VL = KQ * (DH / 8) / 64;  // V load items per lane per tile
  static_assert(4 * kSplitHeads * (DH + 2) * 4 <= split_lds_bytes<DH>(), "merge buffer must fit");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l16 = lane & 15, q4 = lane >> 4;
  const int hpg = H / G, h_lo = hb * kSplitHeads;
  const int nh = min(kSplitHeads, hpg - h_lo);
  bf16_t* Vt = reinterpret_cast<bf16_t*>(lds) + wave * DH * VP;

  // Q^T fragments: lane holds q[head l16][32*ks + 8*q4 .. +7].
  bf16x8 qf[NKS];
  {
    const bf16_t* qp =
        Q + (static_cast<int64_t>(b) * H + g * hpg + h_lo + min(l16, nh - 1)) * DH + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
      if (l16 >= nh) qf[ks] = bf16x8{};
    }
  }
  // Rows of the wave's tile t: workgroup c takes the groups of 4 tiles c,
  // c + n_chunks, c + 2 n_chunks, ... (wave w the w-th tile of each), so the
  // workgroups of a KV head stream one window of the cache at a time.
  constexpr int SB = 4 * BN;
  const int64_t first = static_cast<int64_t>(c) * SB + wave * BN;
  const int my_tiles =
      first < n_rows
          ? static_cast<int>((n_rows - 1 - first) / (static_cast<int64_t>(n_chunks) * SB)) + 1
          : 0;
  const auto tile_row = [&](int t) -> int64_t {
    return first + static_cast<int64_t>(t) * n_chunks * SB;
  };
  float m_i = -INFINITY, l_i = 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};

  const int krow = 8 * (l16 >> 2) + (l16 & 3);  // key of MFMA row l16 in sub-block 0
  u32x4 kbuf[2][2 * NKS], vbuf[2][VL * 4];
  // Paged cache: a tile of BN rows (tiles start at multiples of BN) lies in
  // one page (pages hold at least 64 rows); lane l of the wave holds the pool
  // page of the wave's tile win + l.  Rows past n_rows read as zeros through
  // the buffer range.
  int win = -(1 << 30), win_page = 0;
  const auto tile_base = [&](int t) -> int64_t {  // element offset of the tile's first row
    const int64_t r0 = tile_row(t);
    if constexpr (!PAGED) {
      return kv.row_as<false>(b, g, r0);
    } else {
      if (t < win || t >= win + 64) {
        win = t;
        const int64_t rl = tile_row(min(t + lane, my_tiles - 1));
        win_page = kv.pt[static_cast<int64_t>(b) * kv.pps + (rl >> kv.page_shift)];
      }
      const int64_t pool = __builtin_amdgcn_readlane(win_page, t - win);
      const int64_t in_page = r0 & ((static_cast<int64_t>(1) << kv.page_shift) - 1);
      return ((pool * kv.G + g) * (static_cast<int64_t>(1) << kv.page_shift) + in_page) * kv.DH;
    }
  };
  auto issue = [&](int tile, u32x4* kb_, u32x4* vb_) {
    const int64_t r0 = tile_row(tile);
    const int64_t base = tile_base(tile);
    const uint32_t bytes = static_cast<uint32_t>(min<int64_t>(BN, n_rows - r0)) * DH * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kc + base, bytes), vrs = make_rsrc(Vc + base, bytes);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t off = static_cast<uint32_t>((krow + 4 * kb) * DH + 8 * q4) * 2;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) kb_[kb * NKS + ks] = buffer_load16(krs, off + 64 * ks);
    }
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int item = lane + 64 * it, kq = item % KQ, dc = item / KQ;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vb_[it * 4 + r] = buffer_load16(vrs, static_cast<uint32_t>((4 * kq + r) * DH + 8 * dc) * 2);
    }
  };
  // A tile in two parts: scores() takes the tile's registers (V to the LDS,
  // K into the score products), so the loads of the wave's tile after next
  // go out before accumulate() forms the probabilities and the P V products.
  auto scores = [&](int tile, const u32x4* kb_, const u32x4* vb_, f32x4 (&s)[2]) {
    if (tile_row(tile) < n_rows) {
#pragma unroll
      for (int it = 0; it < VL; ++it) {
        const int item = lane + 64 * it, kq = item % KQ, dc = item / KQ;
        store_v_transposed(Vt, VP, 8 * dc, 4 * kq, vb_ + it * 4);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        s[kb] = mfma16x16x32(__builtin_bit_cast(bf16x8, kb_[kb * NKS + ks]), qf[ks], s[kb]);
    }
  };
  auto accumulate = [&](int tile, f32x4 (&s)[2]) {
    const int64_t r0 = tile_row(tile);  // first key of the tile
    const bool live = r0 < n_rows;
    wave_lds_sync();  // V tile stores before the wave's reads of them
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r0 + 8 * q4 + 4 * kb + r >= n_rows) s[kb][r] = -INFINITY;
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
    const float m_new = fmaxf(m_i, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_i - m_use);
    float p[8], lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[4 * kb + r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -m_use));
        lsum += p[4 * kb + r];
      }
    const bf16x8 pf = pack_bf16x8(p);
    l_i = l_i * alpha + lsum;
    m_i = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    if (live) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma16x16x32(*reinterpret_cast<const bf16x8*>(&Vt[(16 * db + l16) * VP + 8 * q4]),
                               pf, acc[db]);
    }
    wave_lds_sync();  // the reads of this tile before the next tile's stores
  };
  if (my_tiles > 0) issue(0, kbuf[0], vbuf[0]);
  if (my_tiles > 1) issue(1, kbuf[1], vbuf[1]);
  for (int tile = 0; tile < my_tiles; tile += 2) {
    f32x4 s[2];
    scores(tile, kbuf[0], vbuf[0], s);
    if (tile + 2 < my_tiles) issue(tile + 2, kbuf[0], vbuf[0]);
    accumulate(tile, s);
    if (tile + 1 < my_tiles) {
      scores(tile + 1, kbuf[1], vbuf[1], s);
      if (tile + 3 < my_tiles) issue(tile + 3, kbuf[1], vbuf[1]);
      accumulate(tile + 1, s);
    }
  }

  // Merge the 4 waves (the V regions are reused for the exchange).
  __syncthreads();
  l_i += __shfl_xor(l_i, 16, 64);
  l_i += __shfl_xor(l_i, 32, 64);
  float* red_m = reinterpret_cast<float*>(lds);
  float* red_l = red_m + 4 * kSplitHeads;
  float* red_o = red_l + 4 * kSplitHeads;  // [4][16][DH]
  if (q4 == 0) {
    red_m[wave * kSplitHeads + l16] = m_i;
    red_l[wave * kSplitHeads + l16] = l_i;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * kSplitHeads + l16) * DH + 16 * db + 4 * q4 + r] = acc[db][r];
  __syncthreads();
  for (int e = tid; e < nh * DH; e += 256) {
    const int n = e / DH, d = e % DH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w * kSplitHeads + n]);
    float L = 0.f, acc_o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = red_m[w * kSplitHeads + n];
      const float wt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += wt * red_l[w * kSplitHeads + n];
      acc_o += wt * red_o[(w * kSplitHeads + n) * DH + d];
    }
    const int64_t p = (static_cast<int64_t>(b) * H + g * hpg + h_lo + n) * n_chunks + c;
    part_o[p * DH + d] = acc_o;
    if (d == 0) {
      part_m[p] = M;
      part_l[p] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge for query head h of sequence b (512 threads): the chunk partials and
// one extra key/value row, combined with log-sum-exp weights in a fixed order.
// ``extra(kx, vx)`` is called by every thread; it fills kx[0..DH) and
// vx[0..DH) (LDS, float) and returns whether the extra row exists.  It may use
// __syncthreads.  Output o[b, h, :] = sum / denominator, rounded to bf16.
// Every partial is loaded before the extra row is formed (at most one
// (max, sum) pair per thread: n_chunks <= kMaxDecodeChunks).
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 512;
constexpr int kMaxDecodeChunks = kMergeThreads;

template <int DH>
struct MergeLds {
  float wts[kMaxDecodeChunks];
  float red[kMergeThreads / 64];
  float osum[kMergeThreads / DH][DH];
  float kx[DH], vx[DH];
  float lam[4];
  float sx;
};

template <int DH, typename Extra>
__device__ __forceinline__ void decode_merge_head(const float* __restrict__ part_m,
                                                  const float* __restrict__ part_l,
                                                  const float* __restrict__ part_o, int H,
                                                  int n_chunks, int h, int b,
                                                  const bf16_t* __restrict__ Q, float sl2,
                                                  bf16_t* __restrict__ O, MergeLds<DH>& sm,
                                                  Extra extra) {
  constexpr int NT = kMergeThreads, GR = NT / DH, KO = 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int d = tid % DH, grp = tid / DH;
  const int64_t p0 = (static_cast<int64_t>(b) * H + h) * n_chunks;
  const float pm = tid < n_chunks ? part_m[p0 + tid] : -INFINITY;
  const float pl = tid < n_chunks ? part_l[p0 + tid] : 0.f;
  float po[KO];  // this thread's first KO chunks of output column d
#pragma unroll
  for (int i = 0; i < KO; ++i) {
    const int c = grp + GR * i;
    po[i] = c < n_chunks ? part_o[(p0 + c) * DH + d] : 0.f;
  }
  float qv[DH / 64];  // the query, loaded with the partials
  {
    const bf16_t* qh = Q + (static_cast<int64_t>(b) * H + h) * DH;
#pragma unroll
    for (int i = 0; i < DH / 64; ++i) qv[i] = tid < 64 ? bf16_to_f32(qh[lane + 64 * i]) : 0.f;
  }
  const bool has_extra = extra(sm.kx, sm.vx);
  __syncthreads();
  if (has_extra && tid < 64) {  // score of the extra row, scaled like the partials
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < DH / 64; ++i) dot = fmaf(qv[i], sm.kx[lane + 64 * i], dot);
    dot = wave_sum(dot);
    if (lane == 0) sm.sx = dot * sl2;
  }
  const float mx = wave_max(pm);
  if (lane == 0) sm.red[tid >> 6] = mx;
  __syncthreads();
  const float sx = has_extra ? sm.sx : -INFINITY;
  float M = sx;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) M = fmaxf(M, sm.red[w]);
  __syncthreads();
  const float wgt = tid < n_chunks ? __builtin_amdgcn_exp2f(pm - M) : 0.f;
  if (tid < n_chunks) sm.wts[tid] = wgt;
  const float ls = wave_sum(wgt * pl);
  if (lane == 0) sm.red[tid >> 6] = ls;
  __syncthreads();
  const float wx = has_extra ? __builtin_amdgcn_exp2f(sx - M) : 0.f;
  float L = wx;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) L += sm.red[w];
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < KO; ++i) {
    const int c = grp + GR * i;
    if (c < n_chunks) o += sm.wts[c] * po[i];
  }
  for (int c = grp + GR * KO; c < n_chunks; c += GR) o += sm.wts[c] * part_o[(p0 + c) * DH + d];
  sm.osum[grp][d] = o;
  __syncthreads();
  if (tid < DH) {
    float tot = has_extra ? wx * sm.vx[tid] : 0.f;
#pragma unroll
    for (int gi = 0; gi < GR; ++gi) tot += sm.osum[gi][tid];
    O[(static_cast<int64_t>(b) * H + h) * DH + tid] = f32_to_bf16(tot / L);
  }
}

}  // namespace mka
