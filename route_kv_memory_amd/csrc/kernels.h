// Launchers of the FastMKA kernels (host side).  Each returns the launch status;
// argument checking is done by the C-ABI layer before any of these is called.
#pragma once

#include "common.h"

namespace mka {

// ---- router: lambda = softmax(GELU(Q W_r1) W_r2) ---------------------------
// Every router applies the routing variant ``rt`` to the logits.
// MFMA path: bf16, router_hidden in {32, 64}, q_width % 64 == 0.
hipError_t router_bf16_mfma(const bf16_t* q, int M, int qw, const bf16_t* w1, int r,
                            const bf16_t* w2, float* lam, Routing rt, hipStream_t s);
// Few tokens: the hidden layer comes from a small-M product (gemv with a GELU
// epilogue); this applies the second layer and the softmax.
template <typename T>
hipError_t router_head(const float* hidden, int M, int r, const T* w2, float* lam, Routing rt,
                       hipStream_t s);
// One workgroup per token: any type, r <= 256 (fp32 path).
template <typename T>
hipError_t router_rowwise(const T* q, int M, int qw, const T* w1, int r, const T* w2, float* lam,
                          Routing rt, hipStream_t s);
// Variants whose lambda does not depend on the router: the constant vector.
hipError_t lambda_fixed(float* lam, int M, Routing rt, hipStream_t s);

// ---- EMA scan and block means ------------------------------------------------
constexpr int kEmaChunk = 64;  // tokens per scan chunk
template <typename T>
hipError_t ema_scan(const T* x, int B, int seq, int D, int64_t pos0, int block, float beta,
                    float* state_io, float* acc_io, float* l2, float* means, int nb_cap,
                    float* ws, hipStream_t s);
size_t ema_ws_bytes(int B, int seq, int D);
// Decode (one token per sequence): EMA update + block finalise + fp64 partial
// key projections over 128-channel slices (summed by select_codes_topr).
size_t ema_hash_decode_ws_bytes(int B, int D);
template <typename T>
hipError_t ema_hash_decode(const T* x, int B, int D, int64_t pos, int block, float beta,
                           float* state, float* acc, float* l2, float* means, int nb_cap,
                           const float* proj, int nbits, double* part, hipStream_t s);

// ---- SimHash codes and top-R retrieval ---------------------------------------
// codes[b * codes_bstride + i] = SimHash(v[b * v_bstride + i * D .. +D]) for i < rows.
// Uses simhash_ws_bytes(rows, B, D) bytes of ``ws`` (none when that is 0).
size_t simhash_ws_bytes(int rows, int B, int D);
hipError_t simhash_rows(const float* v, int64_t v_bstride, int rows, int B, int D,
                        const float* proj, int nbits, uint64_t* codes, int64_t codes_bstride,
                        void* ws, hipStream_t s);
// The same in two parts, when the rows take the certified bf16 path
// (simhash_prepared_path): the hyperplanes split into simhash_prep_bytes(D)
// bytes of ``prep`` (depends on proj only), then the codes of the rows.
bool simhash_prepared_path(int rows, int B, int D);
size_t simhash_prep_bytes(int D);
hipError_t simhash_prepare(const float* proj, int nbits, int D, void* prep, hipStream_t s);
hipError_t simhash_rows_prepared(const float* v, int64_t v_bstride, int rows, int B, int D,
                                 const float* proj, int nbits, const void* prep, uint64_t* codes,
                                 int64_t codes_bstride, hipStream_t s);
// Few rows (decode): split over D, partial projections in ws, then select.
constexpr int kFewRows = 8;
size_t retrieve_few_ws_bytes(int rows, int D);
hipError_t retrieve_few(const float* l2, int B, int seq, int D, const float* proj, int nbits,
                        const uint64_t* bh, int nb_cap, int block, int R, int64_t pos0,
                        uint64_t* keys, int32_t* idx, void* ws, hipStream_t s);
// Select from partial key projections already in ``part`` (n_slices slices of
// rows x 64 fp64 sums): one workgroup per token sums, forms the key, picks top R.
hipError_t select_codes_topr(const double* part, int rows, int n_slices, int nbits, int seq,
                             int64_t pos0, const uint64_t* bh, int nb_cap, int block, int R,
                             uint64_t* keys, int32_t* idx, hipStream_t s);
// Many rows (prefill): keys already computed, one lane per token.
hipError_t topr_rows(const uint64_t* keys, int B, int seq, int64_t pos0, const uint64_t* bh,
                     int nb_cap, int block, int R, int32_t* idx, hipStream_t s);

// ---- route fusion -----------------------------------------------------------------
// xf[row] for rows of B*seq tokens; ``ch_per_wg`` channels per workgroup (a
// multiple of 4, at most 1024).
template <typename T>
hipError_t fuse_mix(const T* x, const float* l2, const float* means, int nb_cap,
                    const int32_t* idx, const float* lam, int B, int seq, int D, int R,
                    Routing rt, T* xf, hipStream_t s);
// The same for bf16 layers with many tokens, L3 as a selection product on the
// matrix cores (``n_blk`` = the blocks idx may name, at most 256; ``ws`` holds
// fuse_sel_ws_bytes(B, D) bytes), used where fuse_sel_applies(...).
bool fuse_sel_applies(int B, int seq, int D, int R, int n_blk, Routing rt);
size_t fuse_sel_ws_bytes(int B, int D);
hipError_t fuse_mix_sel(const bf16_t* x, const float* l2, const float* means, int nb_cap,
                        const int32_t* idx, const float* lam, int B, int seq, int D, int R,
                        Routing rt, bf16_t* xf, int n_blk, void* ws, hipStream_t s);
// One tier's rows alone, rounded once to the storage type: tier 1 = L2, tier 2 =
// L3 (mean of the retrieved block means).  Full MKA projects each tier apart.
template <typename T>
hipError_t tier_rows(const T* x, const float* l2, const float* means, int nb_cap,
                     const int32_t* idx, int tier, int B, int seq, int D, int R, T* out,
                     hipStream_t s);
// Full MKA: o[m, :] = sum_l lam[m, l] a_l[m, :] over M rows of HD values; null
// paths are skipped.  HD % 4 == 0.
template <typename T>
hipError_t mix_paths(const T* a0, const T* a1, const T* a2, const float* lam, int64_t M, int HD,
                     T* o, hipStream_t s);

// block_kv[b, blk, :] = m_blk [W_k; W_v]^T (float32) for blocks first .. first+n_blocks-1.
template <typename T>
hipError_t block_kv_project(const float* means, int nb_cap, int first, int n_blocks, const T* w_k,
                            const T* w_v, int kvw, int D, int B, float* out, hipStream_t s);

// ---- attention --------------------------------------------------------------------
template <typename T>
hipError_t attn_prefill(const T* q, const T* k, const T* v, T* o, int B, int seq, int H, int G,
                        int dh, const KvLayout& kv, int64_t pos0, float* lse, hipStream_t s);
// Split decode (bf16): partials in ws (for n_rows rows split into chunks),
// merged by a second kernel.
size_t attn_decode_ws_bytes(int B, int H, int G, int dh, int64_t n_rows);
hipError_t attn_decode_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o, int B,
                            int H, int G, int dh, const KvLayout& kv, int64_t cache_len, void* ws,
                            hipStream_t s);
// The same in two halves, so that work can run between them: the split over
// cache rows [0, n_old) (nothing when n_old == 0), then the merge, which also
// folds in row n_old (written in between) as one more part.
hipError_t attn_decode_split_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, int B, int H,
                                  int G, int dh, const KvLayout& kv, int64_t n_old, void* ws,
                                  hipStream_t s);
hipError_t attn_decode_merge_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* v, bf16_t* o,
                                  int B, int H, int G, int dh, const KvLayout& kv, int64_t n_old,
                                  int64_t extra_row, void* ws, hipStream_t s);

// ---- backward (backward.hip) ------------------------------------------------
// D = rowsum(dO * O) over rows of dh values.
template <typename T>
hipError_t attn_bwd_prep(const T* o, const T* d_o, int64_t rows, int dh, float* dsum,
                         hipStream_t s);
// Row-parallel attention backward over a contiguous cache: dq [B,N,H,dh] and
// dkv [B,N,2,G,dh] (K part, then V part), float32; lse and dsum [B,N,H].
template <typename T>
hipError_t attn_bwd_rows(const T* q, const T* k, const T* v, const T* d_o, const float* lse,
                         const float* dsum, int B, int N, int H, int G, int dh, int64_t t_cap,
                         float* dq, float* dkv, hipStream_t s);
// The same on the matrix cores (bf16), from the forward's log-sum-exp.
// ``part``: attn_bwd_mfma_ws_bytes() of float32 scratch (per-head dK/dV slices).
size_t attn_bwd_mfma_ws_bytes(int B, int N, int H, int G, int dh);
hipError_t attn_bwd_mfma(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* d_o,
                         const float* lse, const float* dsum, int B, int N, int H, int G, int dh,
                         int64_t t_cap, float* dq, float* dkv, float* part, hipStream_t s);
template <typename TS, typename TD>
hipError_t transpose(const TS* src, int64_t lds_, int R, int C, int Rp, int64_t ldd, TD* dst,
                     hipStream_t s);
template <typename TS, typename TD>
hipError_t convert(const TS* src, int64_t n, TD* dst, hipStream_t s);
// transpose that also writes the source converted to TD into rows_dst (same
// layout as src): one read of src for both.
template <typename TS, typename TD>
hipError_t transpose_copy(const TS* src, int64_t lds_, int R, int C, int Rp, int64_t ldd, TD* dst,
                          TD* rows_dst, hipStream_t s);
hipError_t fill_zero(float* p, int64_t n, hipStream_t s);
template <typename T>
hipError_t fuse_bwd(const T* x, const float* l2, const float* means, int nb_cap,
                    const int32_t* idx, const float* lam, int B, int N, int D, int R,
                    const float* dxf, float* dx, float* dlam, T* xf, hipStream_t s);
// dm [B, nbs, D]: rows of the complete blocks (D % 4 == 0), from per-range
// partials in ``part`` (block_gather_ws_bytes()).
size_t block_gather_ws_bytes(int B, int N, int D, int block);
hipError_t block_gather(const float* dxf, const float* lam, const int32_t* idx, int B, int N,
                        int D, int R, int block, int nbs, float* part, float* dm, hipStream_t s);
// out[i] = sum over k < n_slices of part[k * n4 + i] (float4 units, in slice order).
hipError_t sum_slices(const float* part, int n_slices, int64_t n4, float* out, hipStream_t s);
size_t ema_adj_ws_bytes(int B, int N, int D);
// dx += the EMA's adjoint of lambda_2 * dxf, plus dm spread over its blocks' tokens.
hipError_t ema_adjoint_add(const float* u, const float* lam, const float* dm, int nbs, int B,
                           int N, int D, int block, float beta, float* part, float* dx,
                           hipStream_t s);
template <typename T>
hipError_t router_bwd(const float* lam, const float* dlam, const float* pre, const T* w2, int r,
                      int64_t M, Routing rt, float* dz, T* dpre, float* dw2, hipStream_t s);

}  // namespace mka
