// Launchers of the FastMKA kernels (host side).  Each returns the launch status;
// argument checking is done by the C-ABI layer before any of these is called.
#pragma once

#include "common.h"

namespace mka {

// ---- router: lambda = softmax(GELU(Q W_r1) W_r2) ---------------------------
// MFMA path: bf16, router_hidden in {32, 64}, q_width % 64 == 0.
hipError_t router_bf16_mfma(const bf16_t* q, int M, int qw, const bf16_t* w1, int r,
                            const bf16_t* w2, float* lam, hipStream_t s);
// Few tokens: the hidden layer comes from a small-M product (gemv with a GELU
// epilogue); this applies the second layer and the softmax.
template <typename T>
hipError_t router_head(const float* hidden, int M, int r, const T* w2, float* lam, hipStream_t s);
// One workgroup per token: any type, r <= 256 (fp32 path).
template <typename T>
hipError_t router_rowwise(const T* q, int M, int qw, const T* w1, int r, const T* w2, float* lam,
                          hipStream_t s);

// ---- EMA scan and block means ------------------------------------------------
constexpr int kEmaChunk = 64;  // tokens per scan chunk
template <typename T>
hipError_t ema_scan(const T* x, int B, int seq, int D, int64_t pos0, int block, float beta,
                    float* state_io, float* acc_io, float* l2, float* means, int nb_cap,
                    float* ws, hipStream_t s);
size_t ema_ws_bytes(int B, int seq, int D);

// ---- SimHash codes and top-R retrieval ---------------------------------------
// codes[b * codes_bstride + i] = SimHash(v[b * v_bstride + i * D .. +D]) for i < rows.
// Uses simhash_ws_bytes(rows, B, D) bytes of ``ws`` (none when that is 0).
size_t simhash_ws_bytes(int rows, int B, int D);
hipError_t simhash_rows(const float* v, int64_t v_bstride, int rows, int B, int D,
                        const float* proj, int nbits, uint64_t* codes, int64_t codes_bstride,
                        void* ws, hipStream_t s);
// Few rows (decode): split over D, partial projections in ws, then select.
constexpr int kFewRows = 8;
size_t retrieve_few_ws_bytes(int rows, int D);
hipError_t retrieve_few(const float* l2, int B, int seq, int D, const float* proj, int nbits,
                        const uint64_t* bh, int nb_cap, int block, int R, int64_t pos0,
                        uint64_t* keys, int32_t* idx, void* ws, hipStream_t s);
// Many rows (prefill): keys already computed, one lane per token.
hipError_t topr_rows(const uint64_t* keys, int B, int seq, int64_t pos0, const uint64_t* bh,
                     int nb_cap, int block, int R, int32_t* idx, hipStream_t s);

// ---- route fusion -----------------------------------------------------------------
// xf[row] for rows of B*seq tokens; ``ch_per_wg`` channels per workgroup (a
// multiple of 4, at most 1024).
template <typename T>
hipError_t fuse_mix(const T* x, const float* l2, const float* means, int nb_cap,
                    const int32_t* idx, const float* lam, int B, int seq, int D, int R, T* xf,
                    hipStream_t s);

// ---- attention --------------------------------------------------------------------
template <typename T>
hipError_t attn_prefill(const T* q, const T* k, const T* v, T* o, int B, int seq, int H, int G,
                        int dh, int64_t t_cap, int64_t pos0, hipStream_t s);
// Split decode (bf16): partials in ws, merged by a second kernel.
constexpr int kDecodeChunk = 1024;  // keys per workgroup
size_t attn_decode_ws_bytes(int B, int H, int dh, int64_t cache_len);
hipError_t attn_decode_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o, int B,
                            int H, int G, int dh, int64_t t_cap, int64_t cache_len, void* ws,
                            hipStream_t s);

}  // namespace mka
