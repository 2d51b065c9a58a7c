// Fused decode-step kernels (see decode.hip).
#pragma once

#include "common.h"

namespace mka {

constexpr int kDecSlice = 128;   // channels per EMA/key-projection workgroup
constexpr int kFewRowsDec = 8;   // tokens per decode step (batch) at most

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
  // fusion
  T* xf;           // [B, D]
};

template <typename T> hipError_t decode_front(const DecodeArgs<T>& a, hipStream_t s);
template <typename T> hipError_t decode_mid(const DecodeArgs<T>& a, hipStream_t s);
template <typename T> hipError_t decode_fuse(const DecodeArgs<T>& a, hipStream_t s);

inline int decode_slices(int D) { return (D + kDecSlice - 1) / kDecSlice; }

}  // namespace mka
