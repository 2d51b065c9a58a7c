// Fused decode-step kernels (see decode.hip).
#pragma once

#include "common.h"

namespace mka {

constexpr int kDecSlice = 128;   // channels per EMA/key-projection workgroup
constexpr int kFewRowsDec = 8;   // tokens per decode step (batch) at most
constexpr int kGemvCols = 2;     // output columns per wave in the decode products

template <typename T>
struct DecodeArgs {
  // token, query projection
  const T* x;      // [B, D]
  const T* w_q;    // [qw, D]
  T* q;            // [B, qw]
  int D, qw, B;
  // EMA state and the L3 bank
  float* state;    // [B, D]
  float* acc;      // [B, D]
  float* l2;       // [B, D]
  float* means;    // [B, nb_cap, D]
  int nb_cap;
  int64_t pos;
  int block;
  float beta, omb;
  const float* proj;  // [nbits, D]
  int nbits, n_slices;
  double* part;       // [n_slices, B, 64] partial key projections
  // router
  const T* w_r1;   // [r, qw]
  const T* w_r2;   // [3, r]
  int r;
  float* hidden;   // [B, r]
  float* lam;      // [B, 3]
  // retrieval
  const uint64_t* bhash;  // [B, nb_cap]
  uint64_t* key;          // [B]
  int32_t* idx;           // [B, R]
  int R;
  // fusion (sequential path): X_fused
  T* xf;           // [B, D]
  // fused K/V row by linearity (overlapped path): the projections of x, L2 and
  // L3 through [W_k; W_v], each [B, 2*kvw] (K columns, then V columns)
  const T* w_k;    // [kvw, D]
  const T* w_v;    // [kvw, D]
  int kvw;
  float* kvx;
  float* kvl2;
  float* kvl3;
  const float* block_kv;  // [B, nb_cap, 2*kvw] projected block means
  // cache and attention
  T* k_cache;      // rows addressed through kv (contiguous or paged)
  T* v_cache;
  int H, G, dh;
  KvLayout kv;
  float sl2;       // log2(e) / sqrt(dh)
  float* part_m;   // split partials over rows [0, pos)
  float* part_l;
  float* part_o;
  int n_chunks, n_hb;  // split shares of the cache rows, 16-head blocks per group
  T* o;            // [B, H, dh] attention output
  // routing variant: steps of disabled tiers are skipped, their inputs unread
  Routing rt;
};

// Sequential path (float32 layers): front, mid, fuse, then the K/V product and
// attention.
template <typename T> hipError_t decode_front(const DecodeArgs<T>& a, hipStream_t s);
template <typename T> hipError_t decode_mid(const DecodeArgs<T>& a, hipStream_t s);
template <typename T> hipError_t decode_fuse(const DecodeArgs<T>& a, hipStream_t s);

// Overlapped path (bf16 layers): three launches per step.
hipError_t decode_inputs_bf16(const DecodeArgs<bf16_t>& a, hipStream_t s);
hipError_t decode_attend_bf16(const DecodeArgs<bf16_t>& a, hipStream_t s);
hipError_t decode_merge_bf16(const DecodeArgs<bf16_t>& a, hipStream_t s);

inline int decode_slices(int D) { return (D + kDecSlice - 1) / kDecSlice; }

}  // namespace mka
