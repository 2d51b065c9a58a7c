// Device-side helpers shared by the FastMKA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mka {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bfloat16 values travel as their 16-bit patterns.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Element-type traits: storage type T <-> float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// ---------------------------------------------------------------------------
// MFMA 32x32x16 bf16 -> f32 (gfx950).  Operand layout for a wave of 64 lanes,
// lane l, half h = l / 32:
//   A (32 x 16): lane holds A[l % 32][8h .. 8h+7]
//   B (16 x 32): lane holds B[8h .. 8h+7][l % 32]
//   C (32 x 32): lane holds C[8*(r/4) + 4h + (r%4)][l % 32], r = 0..15
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within the 32x32 block) of accumulator register r for lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Wave-wide reductions through DPP lane moves (xor-1 and xor-2 within quads,
// mirrors within rows of 16, row broadcasts), read back from lane 63: every lane
// gets the result.  Lanes without a DPP source contribute the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1, 0xF>(0.f, v);
  v += dpp_f32<0x4E, 0xF>(0.f, v);
  v += dpp_f32<0x141, 0xF>(0.f, v);
  v += dpp_f32<0x140, 0xF>(0.f, v);
  v += dpp_f32<0x142, 0xA>(0.f, v);
  v += dpp_f32<0x143, 0xC>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1, 0xF>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x4E, 0xF>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x141, 0xF>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x140, 0xF>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x142, 0xA>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x143, 0xC>(-INFINITY, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// 16-byte vector load widened to float: 8 bf16 or 4 fp32 values.
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
  static constexpr int kN = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* out) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int kN = 4;
  static __device__ __forceinline__ void load(const float* p, float* out) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = w[i];
  }
};

// 4 consecutive values widened to float (8-byte or 16-byte load).
__device__ __forceinline__ void load4(const bf16_t* p, float* out) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  out[0] = __uint_as_float(w[0] << 16);
  out[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  out[2] = __uint_as_float(w[1] << 16);
  out[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* p, float* out) {
  const f32x4 w = *reinterpret_cast<const f32x4*>(p);
  out[0] = w[0]; out[1] = w[1]; out[2] = w[2]; out[3] = w[3];
}
__device__ __forceinline__ void store4(bf16_t* p, const float* v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at ``lds`` + 16*l (``lds`` must be the same for the whole wave).  A plain
// device function, so that kernel templates using it keep their host stubs.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void global_load_lds16(const void* src, lds_void_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane r supplies the address of 4 consecutive 16-bit values (row r of a
// 16 x 4 block) and lane i receives column i % 4 of rows i/4, i/4+4, i/4+8,
// i/4+12 (lane layout measured on the GPU).  ``p`` points into LDS.
__device__ __forceinline__ bf16x4 ds_read_tr16_b64(const bf16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// The same through a buffer resource: byte offset ``off`` from its base; lanes
// whose bytes lie outside the resource's range write zeros to LDS (measured).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, lds_void_t* lds,
                                                  uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, static_cast<int>(off), 0, 0, 0);
}

// s_waitcnt immediate that waits until at most N vector-memory operations of
// the wave are outstanding (expcnt and lgkmcnt left at their maxima): vmcnt
// occupies bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int N>
constexpr int kVmcntPending() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// Raw buffer resource over [base, base + bytes): 16-byte loads through it
// return zeros for any part outside the range, with no memory access there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0);
}

// Exact GELU, z * Phi(z), with the device erf.
__device__ __forceinline__ float gelu(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Map a linear workgroup id to a work item so that each of the 8 XCDs (which
// receive workgroups round-robin) works on a contiguous range of items: items
// that share operands then share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
  const int per = n / 8, rem = n % 8;
  const int xcd = bid % 8, local = bid / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
}


// ---- routing variants ------------------------------------------------------
// The abstract page's ablations: Table 10 compares the learned soft router
// with a fixed lambda = 1/3 and hard top-2 / top-1 routing; Table 9 removes
// tiers (L1+L2, L1+L3, L1 alone).  Values equal the C ABI's MKA_ROUTE_* and
// MKA_TIERS_* constants.
constexpr int kRouteSoft = 0, kRouteFixed = 1, kRouteTop1 = 2, kRouteTop2 = 3;
constexpr int kTiersAll = 0, kTiersL1L2 = 1, kTiersL1L3 = 2, kTiersL1 = 3;

// Where row t of KV head g of sequence b lives in a K or V cache (element
// offset).  Contiguous: [B, G, t_cap, dh].  Paged: a pool of pages
// [n_pages, G, page, dh] and a page table [B, pages_per_seq] (int32), logical
// row t of sequence b in page table[b][t >> page_shift] at row t & (page - 1).
struct KvLayout {
  const int32_t* pt = nullptr;  // page table, or null for the contiguous layout
  int page_shift = 0;
  int pps = 0;                  // pages per sequence
  int G = 1, DH = 128;
  int64_t t_cap = 0;            // rows per (b, g) when contiguous
  __host__ __device__ bool paged() const { return pt != nullptr; }
  // The layout fixed at compile time (the attention kernels' inner loops).
  template <bool PAGED>
  __device__ __forceinline__ int64_t row_as(int b, int g, int64_t t) const {
    if constexpr (!PAGED) {
      return ((static_cast<int64_t>(b) * G + g) * t_cap + t) * DH;
    } else {
      const int64_t page = pt[static_cast<int64_t>(b) * pps + (t >> page_shift)];
      const int64_t in_page = t & ((static_cast<int64_t>(1) << page_shift) - 1);
      return ((page * G + g) * (static_cast<int64_t>(1) << page_shift) + in_page) * DH;
    }
  }
  __device__ __forceinline__ int64_t row(int b, int g, int64_t t) const {
    return pt == nullptr ? row_as<false>(b, g, t) : row_as<true>(b, g, t);
  }
  // rows from t to the end of t's page (contiguous: to t_cap)
  __device__ __forceinline__ int64_t rows_to_boundary(int64_t t) const {
    if (pt == nullptr) return t_cap - t;
    const int64_t p = static_cast<int64_t>(1) << page_shift;
    return p - (t & (p - 1));
  }
};

// A wave's window on the page table: lane l holds the pool page of logical
// page first + l, so a tile finds its page with a register read (readlane of a
// wave-uniform index) instead of a memory load on its loads' critical path; the
// window moves (one vector load) when a tile lies outside it.  With the
// contiguous layout it is the plain formula.
template <bool PAGED>
struct PageWindow {
  int first = -(1 << 30);
  int entry = 0;
  __device__ __forceinline__ void fill(const KvLayout& kv, int b, int page) {
    if constexpr (PAGED) {
      first = page;
      const int p = min(page + static_cast<int>(threadIdx.x & 63), kv.pps - 1);
      entry = kv.pt[static_cast<int64_t>(b) * kv.pps + p];
    }
  }
  // Element offset of row t of KV head g; t must be wave-uniform.
  __device__ __forceinline__ int64_t row(const KvLayout& kv, int b, int g, int64_t t) {
    if constexpr (!PAGED) {
      return kv.row_as<false>(b, g, t);
    } else {
      const int page = static_cast<int>(t >> kv.page_shift);
      if (page < first || page >= first + 64) fill(kv, b, page);
      const int64_t pool = __builtin_amdgcn_readlane(entry, page - first);
      const int64_t in_page = t & ((static_cast<int64_t>(1) << kv.page_shift) - 1);
      return ((pool * kv.G + g) * (static_cast<int64_t>(1) << kv.page_shift) + in_page) * kv.DH;
    }
  }
};

// A constant lambda vector passed by value.
struct Lam3 {
  float v[3] = {0.f, 0.f, 0.f};
};

struct Routing {
  int mode = kRouteSoft;
  int tiers = kTiersAll;
  __host__ __device__ bool l2() const { return tiers == kTiersAll || tiers == kTiersL1L2; }
  __host__ __device__ bool l3() const { return tiers == kTiersAll || tiers == kTiersL1L3; }
  // the EMA runs when L2 is mixed or keys the L3 retrieval
  __host__ __device__ bool ema() const { return tiers != kTiersL1; }
  // lambda depends on the router MLP
  __host__ __device__ bool learned() const { return mode != kRouteFixed && tiers != kTiersL1; }
  // lambda when it does not depend on the router: 1 / (enabled tiers) on each
  __host__ __device__ float fixed_weight(int i) const {
    const bool on = i == 0 || (i == 1 && l2()) || (i == 2 && l3());
    return on ? 1.0f / static_cast<float>(1 + l2() + l3()) : 0.0f;
  }
};

// lambda from the three router logits: the k enabled tiers with the largest
// logits (k = 3 soft, 2 or 1 hard; ties to the lower tier index), softmax over
// those, zero elsewhere.  With every tier kept it is the max-shifted softmax
// of the three logits.
__device__ __forceinline__ void route_weights(const float* z, Routing rt, float* out) {
  if (!rt.learned()) {
#pragma unroll
    for (int i = 0; i < 3; ++i) out[i] = rt.fixed_weight(i);
    return;
  }
  const bool on[3] = {true, rt.l2(), rt.l3()};
  const int k = rt.mode == kRouteTop1 ? 1 : rt.mode == kRouteTop2 ? 2 : 3;
  bool keep[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j != i && on[j]) rank += (z[j] > z[i] || (z[j] == z[i] && j < i)) ? 1 : 0;
    keep[i] = on[i] && rank < k;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (keep[i]) m = fmaxf(m, z[i]);
  float e[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) e[i] = keep[i] ? expf(z[i] - m) : 0.0f;
  const float inv = 1.0f / (e[0] + e[1] + e[2]);
#pragma unroll
  for (int i = 0; i < 3; ++i) out[i] = e[i] * inv;
}

}  // namespace mka
