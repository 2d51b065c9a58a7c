// Dense NT products on gfx950: bf16 MFMA tiles, a plain fp32 tiled kernel and a
// small-M (decode) kernel.
#include <utility>

#include "gemm.h"

namespace mka {

// s_waitcnt immediate that waits for every LDS operation of the wave
// (vmcnt and expcnt left at their maxima).
constexpr int kLgkmcntZero = 0xF | (0x3 << 14) | (0x7 << 4);

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.  Workgroup tile 256 (M) x BN (N), 8 waves; each wave owns
// 128 x BN/4 of C as 4 x BN/128 blocks of MFMA 32x32x16.  The MFMA computes
// C^T blocks (B rows as its A operand), which leaves 4 consecutive output
// columns of one output row in each lane: the epilogue stores 8 bytes per lane.
//
// Operands stream global -> LDS directly (global_load_lds, 16 bytes per lane,
// no registers) through a ring of STAGES k-slices of 32, so the loads of a
// slice are issued STAGES-1 slices before it is used.  A row of a slice is 64
// bytes (4 chunks of 16); chunk c of row r is stored at position
// c ^ ((r >> 2) & 3), which keeps both the 1 KB contiguous LDS writes of a
// load instruction and the 16-row fragment reads of the MFMA free of bank
// conflicts.  Rows past M or N are read from the last valid row; their outputs
// are not stored.
// ---------------------------------------------------------------------------
template <int BN, int NW>
struct GemmCfg {
  static constexpr int BM = 256, BK = 32, ROWB = BK * 2;  // bytes per row per slice
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int SLICE = A_BYTES + B_BYTES;
  static constexpr int STAGES = (160 * 1024) / SLICE;      // 5 for BN=256, 6 for BN=128
  static constexpr int LOADS = SLICE / 1024 / NW;           // load instructions per wave per slice
  static constexpr int WN = BN / (NW / 2);                  // wave tile: 128 x WN
  static constexpr int NB = WN / 32;                        // MFMA blocks per wave in N
};

// The epilogue of a workgroup's tile: lane (h, l32) of wave (wm, wn) holds
// output row m = m0 + wm*128 + 32i + l32 and columns n = n0 + wn*WN + 32j +
// 8*(r/4) + 4h + (r%4) of accumulator acc[i][j][r].
template <int NB, int WN, class Epi>
__device__ __forceinline__ void gemm_store(const f32x16 (&acc)[4][NB], int m0, int n0, int wm,
                                           int wn, int h, int l32, int M, int N, const Epi& epi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + i * 32 + l32;
    if (m >= M) continue;
    if constexpr (std::is_same<Epi, EpiAdd>::value) {
      // accumulate: the row's 4*NB quads are read together, then written
      float old[NB][4][4];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          epi.load4(m, n0 + wn * WN + j * 32 + 8 * rq + 4 * h, N, old[j][rq]);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = old[j][rq][e] + acc[i][j][4 * rq + e];
          epi.put4(m, n0 + wn * WN + j * 32 + 8 * rq + 4 * h, v, N);
        }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int n = n0 + wn * WN + j * 32 + 8 * rq + 4 * h;
          const float v[4] = {acc[i][j][4 * rq], acc[i][j][4 * rq + 1], acc[i][j][4 * rq + 2],
                              acc[i][j][4 * rq + 3]};
          epi.store4(m, n, v, N);
        }
    }
  }
}

// blockIdx.y selects a range of K_len reduction indices starting at
// blockIdx.y * K_len (split-K; K is the row length of B).  DB: fragments
// double-buffered in registers (below); without it a slice's fragments are
// read after its barrier, in fewer registers (room for other kernels' waves
// on the same SIMDs).
template <int BN, int NW, bool DB, class Epi>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, int n_split, int M, int N, int K, int K_len, Epi epi) {
  using C = GemmCfg<BN, NW>;
  constexpr int BM = C::BM, BK = C::BK, ROWB = C::ROWB, STAGES = C::STAGES, NB = C::NB;
  constexpr int WN = C::WN;
  static_assert(C::LOADS * NW * 1024 == C::SLICE, "slice must split evenly over the waves");
  static_assert(STAGES >= 3, "the ring holds the slice in use, the next one and one in flight");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[STAGES * C::SLICE];

  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  if (tiles_m % 4 == 0 && tiles_n % 2 == 0) {
    // Workgroups reach the 8 XCDs round-robin; XCD x takes the block of tiles
    // rows [x/2 * tiles_m/4, +tiles_m/4) x columns [x%2 * tiles_n/2, +tiles_n/2),
    // so its concurrent tiles share few A and B panels in its L2.
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8, bn = tiles_n / 2;
    tm = (xcd >> 1) * (tiles_m / 4) + local / bn;
    tn = (xcd & 1) * bn + local % bn;
  } else {
    const int item = xcd_contiguous(blockIdx.x, tiles_n * tiles_m);
    tm = item / tiles_n;
    tn = item % tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int wm = wave & 1, wn = wave >> 1, h = lane >> 5, l32 = lane & 31;

  // This lane's rows and byte offsets for each of its load instructions of a
  // slice: instruction j of wave w covers 16 rows of A (first A_BYTES/1024
  // instructions) or of B; lane l takes row 16*ri + l/4, chunk (l%4) ^ swizzle.
  const bf16_t* src[C::LOADS];
  int dst[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int gi = wave * C::LOADS + j;  // instruction index within the slice
    const bool is_a = gi < C::A_BYTES / 1024;
    const int ri = is_a ? gi : gi - C::A_BYTES / 1024;
    const int row = 16 * ri + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    if (is_a) {
      const int gm = min(m0 + row, M - 1);
      src[j] = A + static_cast<int64_t>(gm) * lda + blockIdx.y * K_len + chunk * 8;
    } else {
      const int gn = min(n0 + row, N - 1);
      src[j] = (gn < n_split ? B0 + static_cast<int64_t>(gn) * K
                             : B1 + static_cast<int64_t>(gn - n_split) * K) +
               blockIdx.y * K_len + chunk * 8;
    }
    dst[j] = (is_a ? 0 : C::A_BYTES) + ri * 1024;  // lane's 16 bytes land at +16*lane
  }
  auto issue = [&](int slice, int stage) {
    unsigned char* base = lds + stage * C::SLICE;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j)
      global_load_lds16(src[j] + slice * BK, (lds_void_t*)(base + dst[j]));
  };

  // acc[i][j]: C^T block of output rows m0 + wm*128 + 32i .., columns n0 + wn*WN + 32j ..
  f32x16 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  // fragment byte offset of row r, chunk c (16 bytes) within a slice operand
  auto frag = [](int r, int c) { return r * ROWB + ((c ^ ((r >> 2) & 3)) << 4); };

  const int nk_all = K_len / BK;
  if constexpr (DB) {
  const int nk = nk_all;
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s, s);
  // Fragments are double-buffered in registers: a slice's fragments are read
  // from LDS during the previous slice's MFMAs, so no wave starts a slice
  // waiting on LDS.  The barrier of iteration kt therefore waits until slice
  // kt+1 has landed; and since every wave has slice kt in registers by then
  // (reads complete before the barrier), slice kt's stage is refilled with
  // slice kt+STAGES right after it: STAGES-1 slices stay in flight.
  typedef bf16x8 FragA[2][4];
  typedef bf16x8 FragB[2][NB];
  auto read_slice = [&](int kt, FragA& fa, FragB& fb) {
    const unsigned char* As = lds + (kt % STAGES) * C::SLICE;
    const unsigned char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[ks][i] =
            *reinterpret_cast<const bf16x8*>(As + frag(wm * 128 + i * 32 + l32, 2 * ks + h));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[ks][j] = *reinterpret_cast<const bf16x8*>(Bs + frag(wn * WN + j * 32 + l32, 2 * ks + h));
    }
  };
  // One slice: wait for slice kt+1, barrier, refill slice kt's stage, read
  // slice kt+1's fragments into (na, nb) while the MFMAs consume (ca, cb).
  // After the last slice the read takes a stale stage and is not used.
  auto step = [&](int kt, const FragA& ca, const FragB& cb, FragA& na, FragB& nb) {
    if (kt + STAGES - 1 < nk) {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 2)>());
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
    }
    __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
    // A bare barrier: a fence here would wait for the prefetches too.
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES < nk) issue(kt + STAGES, kt % STAGES);
    read_slice(kt + 1, na, nb);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32x32x16(cb[ks][j], ca[ks][i], acc[i][j]);
    // one LDS read after each MFMA, the rest at the end
    constexpr int R = (BK / 16) * (4 + NB), F = (BK / 16) * 4 * NB;
    constexpr int P = R < F ? R : F;
#pragma unroll
    for (int u = 0; u < P; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (F > P) __builtin_amdgcn_sched_group_barrier(0x008, F - P, 0);
    if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
  };
  FragA xa, ya;
  FragB xb, yb;
  if (STAGES - 1 < nk) {
    __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 1)>());
  } else {
    __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
  }
  __builtin_amdgcn_s_barrier();
  read_slice(0, xa, xb);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, xa, xb, ya, yb);
    step(kt + 1, ya, yb, xa, xb);
  }
  if (kt < nk) step(kt, xa, xb, ya, yb);

  } else {
  const int nk = nk_all;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    // slice kt has landed once at most the STAGES-2 younger slices are pending
    if (kt + STAGES - 2 < nk) {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 2)>());
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
    }
    // Every wave's part of slice kt is in LDS (each waited for its own loads)
    // and every wave is done reading slice kt-1.  A bare barrier: a fence here
    // would wait for the prefetches too.
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const unsigned char* As = lds + (kt % STAGES) * C::SLICE;
    const unsigned char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[4], fb[NB];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(As + frag(wm * 128 + i * 32 + l32, 2 * ks + h));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(Bs + frag(wn * WN + j * 32 + l32, 2 * ks + h));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32x32x16(fb[j], fa[i], acc[i][j]);
    }
  }

  }

  gemm_store<NB, WN>(acc, m0, n0, wm, wn, h, l32, M, N, epi);
}

constexpr int kGemmWaves256 = 8;

template <class Epi>
hipError_t gemm_bf16(const bf16_t* a, int lda, const bf16_t* b0, const bf16_t* b1, int n_split,
                     int M, int N, int K, const Epi& epi, hipStream_t s, bool single_buffer) {
  const int tiles256 = ((N + 255) / 256) * ((M + 255) / 256);
  if (tiles256 >= 256) {
    if (single_buffer)
      hipLaunchKernelGGL((gemm_bf16_kernel<256, kGemmWaves256, false, Epi>), dim3(tiles256),
                         dim3(kGemmWaves256 * 64), 0, s, a, lda, b0, b1, n_split, M, N, K, K, epi);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<256, kGemmWaves256, true, Epi>), dim3(tiles256),
                         dim3(kGemmWaves256 * 64), 0, s, a, lda, b0, b1, n_split, M, N, K, K, epi);
  } else {
    const int tiles = ((N + 127) / 128) * ((M + 255) / 256);
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 8, true, Epi>), dim3(tiles), dim3(512), 0, s, a, lda,
                       b0, b1, n_split, M, N, K, K, epi);
  }
  return hipGetLastError();
}

// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N-1>{}).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// The same product with operands stored K-major: an operand marked so is given
// as [K][rows] (its rows contiguous along the output dimension, ``ld`` apart
// per reduction index), e.g. the token-major activations of a weight gradient
// dW = dY^T X or a weight [in][out] used as stored.  Both operands stream
// global -> LDS through buffer resources (direct loads, 16 bytes per lane):
// - a K-major slice is stored as its 32 reduction rows of BM (or BN) values;
//   16-byte chunk c of slice row kr sits at chunk position c ^ 4*(kr % 4);
// - its MFMA fragment (8 consecutive reduction indices of one output row per
//   lane) comes from two transposing LDS reads (ds_read_b64_tr_b16): in each
//   16-lane group, lane r addresses slice row kb + r/4 at output rows
//   mb + 4*(r%4) .. +3, and lane i receives output row mb + i at slice rows
//   kb .. kb+3.  Within each 32-lane half the 4 slice rows x 64 bytes read fall
//   in distinct banks.
// - K-major reduction rows at or past ``k_rows`` read as zeros (the buffer
//   range ends there), so K_len may run past the valid rows; output rows past
//   M (or N) read whatever follows in memory and are not stored.
// K-contiguous operands use the swizzled row layout of gemm_bf16_kernel.
// ---------------------------------------------------------------------------
template <int BN, bool AK, bool BKM, class Epi>
__global__ __launch_bounds__(512) void gemm_bf16_km_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B, int ldb, int M, int N,
    int K_len, int k_rows, Epi epi) {
  constexpr int NW = 8;
  using C = GemmCfg<BN, NW>;
  constexpr int BM = C::BM, BK = C::BK, ROWB = C::ROWB, NB = C::NB;
  constexpr int WN = C::WN;
  // An even number of stages, each a shared object of its own: the loop is
  // unrolled over the ring, so every load and read names its stage at
  // compile time and the compiler can see that a slice's loads do not write
  // the stage being read (otherwise it waits for all loads in flight before
  // each transposing read).
  constexpr int STAGES = BN == 256 ? 4 : 6;
  constexpr int A_RB = BM * 2, B_RB = BN * 2;  // bytes per K-major slice row
  static_assert(C::LOADS * NW * 1024 == C::SLICE, "slice must split evenly over the waves");
  static_assert(STAGES * C::SLICE <= 160 * 1024, "the ring fits the LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char ra0[C::A_BYTES], rb0[C::B_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char ra1[C::A_BYTES], rb1[C::B_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char ra2[C::A_BYTES], rb2[C::B_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char ra3[C::A_BYTES], rb3[C::B_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char ra4[STAGES > 4 ? C::A_BYTES : 16],
      rb4[STAGES > 4 ? C::B_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char ra5[STAGES > 5 ? C::A_BYTES : 16],
      rb5[STAGES > 5 ? C::B_BYTES : 16];
  // stage u's A and B operands
  auto stage_a = [&](auto u) -> unsigned char* {
    constexpr int k = decltype(u)::value % STAGES;
    if constexpr (k == 0) return ra0;
    else if constexpr (k == 1) return ra1;
    else if constexpr (k == 2) return ra2;
    else if constexpr (k == 3) return ra3;
    else if constexpr (k == 4) return ra4;
    else return ra5;
  };
  auto stage_b = [&](auto u) -> unsigned char* {
    constexpr int k = decltype(u)::value % STAGES;
    if constexpr (k == 0) return rb0;
    else if constexpr (k == 1) return rb1;
    else if constexpr (k == 2) return rb2;
    else if constexpr (k == 3) return rb3;
    else if constexpr (k == 4) return rb4;
    else return rb5;
  };

  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  if (tiles_m % 4 == 0 && tiles_n % 2 == 0) {
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8, bn = tiles_n / 2;
    tm = (xcd >> 1) * (tiles_m / 4) + local / bn;
    tn = (xcd & 1) * bn + local % bn;
  } else {
    const int item = xcd_contiguous(blockIdx.x, tiles_n * tiles_m);
    tm = item / tiles_n;
    tn = item % tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_begin = blockIdx.y * K_len;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1, h = lane >> 5, l32 = lane & 31;

  // Load instruction j of this wave: operand (A first), LDS offset, and the
  // lane's byte offset from the slice's resource base (the same every slice).
  bool is_a[C::LOADS];
  int dst[C::LOADS];
  uint32_t voff[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int gi = wave * C::LOADS + j;
    is_a[j] = gi < C::A_BYTES / 1024;
    const int ri = is_a[j] ? gi : gi - C::A_BYTES / 1024;
    dst[j] = ri * 1024;  // within the operand's stage buffer
    const bool km = is_a[j] ? AK : BKM;
    const int rb = is_a[j] ? A_RB : B_RB, ld = is_a[j] ? lda : ldb;
    if (km) {
      const int kr = ri * (1024 / rb) + (16 * lane) / rb, c = (16 * lane % rb) / 16;
      voff[j] = static_cast<uint32_t>(kr * ld * 2 + 16 * (c ^ (4 * (kr & 3))));
    } else {
      const int row = 16 * ri + (lane >> 2);
      const int chunk = (lane & 3) ^ ((row >> 2) & 3);
      const int r0 = is_a[j] ? m0 : n0, rows = is_a[j] ? M : N;
      voff[j] = static_cast<uint32_t>((min(r0 + row, rows - 1) - r0) * ld * 2 + chunk * 16);
    }
  }
  // The resources of slice `slice`: K-major ones end after the last valid
  // reduction row.  Base and size go through readfirstlane so that the
  // resource lives in scalar registers (the clamp is a vector instruction,
  // and a resource in vector registers makes every load a loop over lanes).
  auto rsrc = [&](bool km, const bf16_t* X, int ld, int r0, int slice) {
    const int k0 = k_begin + slice * BK;
    const bf16_t* p;
    uint32_t bytes;
    if (km) {
      const int rows = max(0, min(BK, k_rows - k0));
      bytes = rows > 0 ? static_cast<uint32_t>((static_cast<int64_t>(rows) * ld - r0) * 2) : 0u;
      p = X + static_cast<int64_t>(k0) * ld + r0;
    } else {
      bytes = 0xFFFFFFFFu;
      p = X + static_cast<int64_t>(r0) * ld + k0;
    }
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    return make_rsrc(reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo),
                     __builtin_amdgcn_readfirstlane(bytes));
  };
  auto issue = [&](int slice, unsigned char* abase, unsigned char* bbase) {
    const __amdgpu_buffer_rsrc_t ra = rsrc(AK, A, lda, m0, slice);
    const __amdgpu_buffer_rsrc_t rb = rsrc(BKM, B, ldb, n0, slice);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      if (wave * C::LOADS + j < C::A_BYTES / 1024)  // uniform: a scalar branch
        buffer_load_lds16(ra, (lds_void_t*)(abase + dst[j]), voff[j]);
      else
        buffer_load_lds16(rb, (lds_void_t*)(bbase + dst[j]), voff[j]);
    }
  };

  f32x16 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  // K-contiguous fragment: 8 reduction indices (chunk c) of slice row r.
  auto frag = [](const unsigned char* Xs, int r, int c) {
    return *reinterpret_cast<const bf16x8*>(Xs + r * ROWB + ((c ^ ((r >> 2) & 3)) << 4));
  };
  // K-major fragment: output rows rb0 + l32, reduction indices 16ks + 8h ..
  const int tq = lane >> 4, tr = lane & 15;
  auto frag_km = [&](const unsigned char* Xs, int row_bytes, int rb0, int ks) {
    bf16x4 v[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kr = 16 * ks + 8 * (tq >> 1) + 4 * t + (tr >> 2);
      const int m = rb0 + 16 * (tq & 1) + 4 * (tr & 3);
      v[t] = ds_read_tr16_b64(reinterpret_cast<const bf16_t*>(
          Xs + kr * row_bytes + (((m >> 3) ^ (4 * (kr & 3))) << 4) + (m & 7) * 2));
    }
    return bf16x8{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
  };

  const int nk = K_len / BK;
  static_for<STAGES>([&](auto u) {
    if (decltype(u)::value < nk) issue(decltype(u)::value, stage_a(u), stage_b(u));
  });
  // Fragments double-buffered in registers, as in gemm_bf16_kernel.
  typedef bf16x8 FragA[2][4];
  typedef bf16x8 FragB[2][NB];
  auto read_slice = [&](const unsigned char* As, const unsigned char* Bs, FragA& fa, FragB& fb) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[ks][i] = AK ? frag_km(As, A_RB, wm * 128 + i * 32, ks)
                       : frag(As, wm * 128 + i * 32 + l32, 2 * ks + h);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[ks][j] = BKM ? frag_km(Bs, B_RB, wn * WN + j * 32, ks)
                        : frag(Bs, wn * WN + j * 32 + l32, 2 * ks + h);
    }
  };
  // Slice kt (kt % STAGES == u): wait for slice kt+1, barrier, refill stage u
  // with slice kt+STAGES, read slice kt+1's fragments while the MFMAs consume
  // slice kt's.  After the last slice the read takes a stale stage and is
  // not used.
  auto step = [&](auto u, int kt, const FragA& ca, const FragB& cb, FragA& na, FragB& nb) {
    constexpr int U = decltype(u)::value;
    if (kt + STAGES - 1 < nk) {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 2)>());
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
    }
    __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES < nk) issue(kt + STAGES, stage_a(u), stage_b(u));
    read_slice(stage_a(std::integral_constant<int, U + 1>{}),
               stage_b(std::integral_constant<int, U + 1>{}), na, nb);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32x32x16(cb[ks][j], ca[ks][i], acc[i][j]);
    // one LDS read after each MFMA, the rest at the end (a K-major fragment
    // is two reads)
    constexpr int R = (BK / 16) * ((AK ? 2 : 1) * 4 + (BKM ? 2 : 1) * NB);
    constexpr int F = (BK / 16) * 4 * NB;
    constexpr int P = R < F ? R : F;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (F > P) __builtin_amdgcn_sched_group_barrier(0x008, F - P, 0);
    if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
  };
  FragA xa, ya;
  FragB xb, yb;
  if (STAGES - 1 < nk) {
    __builtin_amdgcn_s_waitcnt(kVmcntPending<C::LOADS * (STAGES - 1)>());
  } else {
    __builtin_amdgcn_s_waitcnt(kVmcntPending<0>());
  }
  __builtin_amdgcn_s_barrier();
  read_slice(ra0, rb0, xa, xb);
  for (int k0 = 0; k0 < nk; k0 += STAGES) {
    static_for<STAGES>([&](auto u) {
      constexpr int U = decltype(u)::value;
      if (k0 + U < nk) {
        if constexpr (U % 2 == 0)
          step(u, k0 + U, xa, xb, ya, yb);
        else
          step(u, k0 + U, ya, yb, xa, xb);
      }
    });
  }

  gemm_store<NB, WN>(acc, m0, n0, wm, wn, h, l32, M, N, epi);
}

// ---------------------------------------------------------------------------
// Split-K for products with few output tiles (the weight gradients: a few
// hundred rows, thousands of columns, a reduction over all tokens): the
// reduction is cut into S ranges, one grid row each, whose float32 partials go
// to a workspace; a second kernel adds them in range order (deterministic)
// and hands the sum to the epilogue.
// ---------------------------------------------------------------------------
struct EpiPart {  // partial of range blockIdx.y: row-major [S][M][N]
  float* base;
  int ldc;
  int64_t stride;
  __device__ __forceinline__ void store4(int m, int n, const float* v, int N) const {
    float* p = base + blockIdx.y * stride + static_cast<int64_t>(m) * ldc + n;
    if (n + 3 < N) {
      mka::store4(p, v);
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) p[i] = v[i];
    }
  }
};

template <class Epi>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ part, int S,
                                                         int M, int N, Epi epi) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t total = static_cast<int64_t>(M) * N;
  if (e >= total) return;
  const int m = static_cast<int>(e / N), n = static_cast<int>(e - static_cast<int64_t>(m) * N);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < S; ++sp) {
    const float* p = part + sp * total + e;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += p[i];
  }
  epi.store4(m, n, v, N);
}

// Ranges: as many as fill one round of the CUs (at most 8), each a multiple of
// the k-slice; 1 when the product already has a round of tiles.
int gemm_splitk_ranges(int M, int N, int K) {
  const int tm = (M + 255) / 256;
  if (((N + 255) / 256) * tm >= 256 || N % 4 != 0) return 1;
  const int tiles = ((N + 127) / 128) * tm;
  int S = 1;
  for (int c = 2; c <= 8; ++c)
    if (c * tiles <= 256 && K % (c * 32) == 0 && K / c >= 256) S = c;
  return S;
}

size_t gemm_bf16_splitk_ws_bytes(int M, int N, int K) {
  const int S = gemm_splitk_ranges(M, N, K);
  return S > 1 ? sizeof(float) * static_cast<size_t>(S) * M * N : 0;
}

template <class Epi>
hipError_t gemm_bf16_splitk(const bf16_t* a, int lda, const bf16_t* b, int M, int N, int K,
                            const Epi& epi, float* ws, hipStream_t s) {
  const int S = gemm_splitk_ranges(M, N, K);
  if (S == 1) return gemm_bf16(a, lda, b, b, N, M, N, K, epi, s);
  const int tiles = ((N + 127) / 128) * ((M + 255) / 256);
  const EpiPart part{ws, N, static_cast<int64_t>(M) * N};
  hipLaunchKernelGGL((gemm_bf16_kernel<128, 8, true, EpiPart>), dim3(tiles, S), dim3(512), 0, s, a, lda,
                     b, b, N, M, N, K, K / S, part);
  const int64_t quads = (static_cast<int64_t>(M) * N + 3) / 4;
  hipLaunchKernelGGL((splitk_sum_kernel<Epi>), dim3(static_cast<unsigned>((quads + 255) / 256)),
                     dim3(256), 0, s, ws, S, M, N, epi);
  return hipGetLastError();
}

template <class Epi>
hipError_t gemm_bf16_km(const bf16_t* a, int lda, bool a_kmajor, const bf16_t* b, int ldb, int M,
                        int N, int K, int k_rows, const Epi& epi, float* ws, hipStream_t s) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) == 0;
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0 || N % 4 != 0 || lda % 8 != 0 || ldb % 8 != 0 ||
      !aligned || k_rows < 0 || k_rows > K || (a_kmajor && lda < M) || ldb < N ||
      (!a_kmajor && k_rows != K))
    return hipErrorInvalidValue;
  const int S = gemm_splitk_ranges(M, N, K);
  const int tm = (M + 255) / 256;
  auto run = [&](auto kernel, int tiles, int ranges, auto e) {
    hipLaunchKernelGGL(kernel, dim3(tiles, ranges), dim3(512), 0, s, a, lda, b, ldb, M, N,
                       K / ranges, k_rows, e);
  };
  if (S > 1) {
    const int tiles = ((N + 127) / 128) * tm;
    const EpiPart part{ws, N, static_cast<int64_t>(M) * N};
    if (a_kmajor)
      run(gemm_bf16_km_kernel<128, true, true, EpiPart>, tiles, S, part);
    else
      run(gemm_bf16_km_kernel<128, false, true, EpiPart>, tiles, S, part);
    const int64_t quads = (static_cast<int64_t>(M) * N + 3) / 4;
    hipLaunchKernelGGL((splitk_sum_kernel<Epi>), dim3(static_cast<unsigned>((quads + 255) / 256)),
                       dim3(256), 0, s, ws, S, M, N, epi);
  } else if (((N + 255) / 256) * tm >= 256) {
    if (a_kmajor)
      run(gemm_bf16_km_kernel<256, true, true, Epi>, ((N + 255) / 256) * tm, 1, epi);
    else
      run(gemm_bf16_km_kernel<256, false, true, Epi>, ((N + 255) / 256) * tm, 1, epi);
  } else {
    if (a_kmajor)
      run(gemm_bf16_km_kernel<128, true, true, Epi>, ((N + 127) / 128) * tm, 1, epi);
    else
      run(gemm_bf16_km_kernel<128, false, true, Epi>, ((N + 127) / 128) * tm, 1, epi);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 GEMM: 64 x 64 tile, 16 x 16 threads with 4 x 4 outputs each, k-tile 16.
// ---------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int lda, const float* __restrict__ B0,
    const float* __restrict__ B1, int n_split, int M, int N, int K, Epi epi) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i, kk = tid & 15;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? A[static_cast<int64_t>(gm) * lda + gk] : 0.f;
      float bv = 0.f;
      if (gn < N && gk < K)
        bv = gn < n_split ? B0[static_cast<int64_t>(gn) * K + gk]
                          : B1[static_cast<int64_t>(gn - n_split) * K + gk];
      Bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) epi(m, n, acc[i][j]);
    }
}

template <class Epi>
hipError_t gemm_f32(const float* a, int lda, const float* b0, const float* b1, int n_split, int M,
                    int N, int K, const Epi& epi, hipStream_t s) {
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel<Epi>, grid, dim3(256), 0, s, a, lda, b0, b1, n_split, M, N, K,
                     epi);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small-M product: one wave per output column n, lanes stride the reduction
// with 16-byte loads, every one of the M <= 8 rows reuses the weight row.
// ---------------------------------------------------------------------------
template <typename T, class Epi>
__global__ __launch_bounds__(256) void gemv_kernel(const T* __restrict__ A, int lda, int M,
                                                   const T* __restrict__ B0,
                                                   const T* __restrict__ B1, int n_split, int N,
                                                   int K, Epi epi) {
  constexpr int V = Vec16<T>::kN;
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const T* brow = n < n_split ? B0 + static_cast<int64_t>(n) * K
                              : B1 + static_cast<int64_t>(n - n_split) * K;
  float acc[8] = {};
  const int kv = (K / V) * V;
  constexpr int STEP = 64 * V, U = 4;
  int k = lane * V;
  // Four 16-byte weight loads in flight per lane before any arithmetic.
  for (; k + (U - 1) * STEP < kv; k += U * STEP) {
    float w[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) Vec16<T>::load(brow + k + u * STEP, w[u]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < M) {
        float a[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) Vec16<T>::load(A + static_cast<int64_t>(m) * lda + k + u * STEP, a[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < V; ++i) acc[m] = fmaf(a[u][i], w[u][i], acc[m]);
      }
    }
  }
  for (; k < kv; k += STEP) {
    float w[V];
    Vec16<T>::load(brow + k, w);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < M) {
        float a[V];
        Vec16<T>::load(A + static_cast<int64_t>(m) * lda + k, a);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[m] = fmaf(a[i], w[i], acc[m]);
      }
    }
  }
  for (int k = kv + lane; k < K; k += 64) {
    const float w = Elem<T>::to_f32(brow[k]);
#pragma unroll
    for (int m = 0; m < 8; ++m)
      if (m < M) acc[m] = fmaf(Elem<T>::to_f32(A[static_cast<int64_t>(m) * lda + k]), w, acc[m]);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < M) {
      const float v = wave_sum(acc[m]);
      if (lane == 0) epi(m, n, v);
    }
  }
}

template <typename T, class Epi>
hipError_t gemv(const T* a, int lda, int M, const T* b0, const T* b1, int n_split, int N, int K,
                const Epi& epi, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<T, Epi>), dim3((N + 3) / 4), dim3(256), 0, s, a, lda, M, b0, b1,
                     n_split, N, K, epi);
  return hipGetLastError();
}

// Instantiations used by the host layer.
template hipError_t gemm_bf16<EpiStore<bf16_t>>(const bf16_t*, int, const bf16_t*, const bf16_t*,
                                                 int, int, int, int, const EpiStore<bf16_t>&,
                                                 hipStream_t, bool);
template hipError_t gemm_bf16<EpiKV<bf16_t>>(const bf16_t*, int, const bf16_t*, const bf16_t*, int,
                                              int, int, int, const EpiKV<bf16_t>&, hipStream_t,
                                              bool);
template hipError_t gemm_bf16<EpiStore<float>>(const bf16_t*, int, const bf16_t*, const bf16_t*,
                                                int, int, int, int, const EpiStore<float>&,
                                                hipStream_t, bool);
template hipError_t gemm_bf16<EpiAdd>(const bf16_t*, int, const bf16_t*, const bf16_t*, int, int,
                                      int, int, const EpiAdd&, hipStream_t, bool);
template hipError_t gemm_bf16_splitk<EpiStore<float>>(const bf16_t*, int, const bf16_t*, int, int,
                                                      int, const EpiStore<float>&, float*,
                                                      hipStream_t);
template hipError_t gemm_bf16_splitk<EpiAdd>(const bf16_t*, int, const bf16_t*, int, int, int,
                                             const EpiAdd&, float*, hipStream_t);
template hipError_t gemm_bf16_km<EpiStore<float>>(const bf16_t*, int, bool, const bf16_t*, int,
                                                   int, int, int, int, const EpiStore<float>&,
                                                   float*, hipStream_t);
template hipError_t gemm_bf16_km<EpiAdd>(const bf16_t*, int, bool, const bf16_t*, int, int, int,
                                          int, int, const EpiAdd&, float*, hipStream_t);
template hipError_t gemm_f32<EpiAdd>(const float*, int, const float*, const float*, int, int, int,
                                     int, const EpiAdd&, hipStream_t);
template hipError_t gemm_f32<EpiStore<float>>(const float*, int, const float*, const float*, int,
                                               int, int, int, const EpiStore<float>&, hipStream_t);
template hipError_t gemm_f32<EpiKV<float>>(const float*, int, const float*, const float*, int, int,
                                            int, int, const EpiKV<float>&, hipStream_t);
template hipError_t gemv<bf16_t, EpiStore<bf16_t>>(const bf16_t*, int, int, const bf16_t*,
                                                    const bf16_t*, int, int, int,
                                                    const EpiStore<bf16_t>&, hipStream_t);
template hipError_t gemv<bf16_t, EpiKV<bf16_t>>(const bf16_t*, int, int, const bf16_t*,
                                                 const bf16_t*, int, int, int,
                                                 const EpiKV<bf16_t>&, hipStream_t);
template hipError_t gemv<float, EpiStore<float>>(const float*, int, int, const float*, const float*,
                                                  int, int, int, const EpiStore<float>&,
                                                  hipStream_t);
template hipError_t gemv<float, EpiKV<float>>(const float*, int, int, const float*, const float*,
                                               int, int, int, const EpiKV<float>&, hipStream_t);
template hipError_t gemv<bf16_t, EpiGelu>(const bf16_t*, int, int, const bf16_t*, const bf16_t*, int,
                                          int, int, const EpiGelu&, hipStream_t);
template hipError_t gemv<float, EpiGelu>(const float*, int, int, const float*, const float*, int,
                                         int, int, const EpiGelu&, hipStream_t);

}  // namespace mka
