// C ABI of the FastMKA layer forward: argument validation, workspace layout and
// dispatch to the kernels.  Every check runs before the first launch of a call,
// so a rejected call has enqueued nothing.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "../../include/mka.h"
#include "decode.h"
#include "gemm.h"
#include "kernels.h"
#include "attn_split.h"

using namespace mka;

static_assert(MKA_ROUTE_SOFT == kRouteSoft && MKA_ROUTE_FIXED == kRouteFixed &&
                  MKA_ROUTE_TOP1 == kRouteTop1 && MKA_ROUTE_TOP2 == kRouteTop2,
              "routing modes");
static_assert(MKA_TIERS_ALL == kTiersAll && MKA_TIERS_L1_L2 == kTiersL1L2 &&
                  MKA_TIERS_L1_L3 == kTiersL1L3 && MKA_TIERS_L1 == kTiersL1,
              "tier sets");

namespace {

thread_local char g_last_error[512] = "";

int hip_fail(const char* where, hipError_t e) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e),
                static_cast<int>(e));
  return MKA_ERR_HIP;
}

#define MKA_CHECK(cond, code) \
  do {                        \
    if (!(cond)) return (code); \
  } while (0)

#define MKA_LAUNCH(where, expr)                     \
  do {                                              \
    const hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return hip_fail(where, e_); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t el_size(const mka_dims* d) { return d->dtype == MKA_BF16 ? 2 : 4; }

size_t round256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// Shape checks shared by every call.
int check_dims(const mka_dims* d) {
  MKA_CHECK(d != nullptr, MKA_ERR_INVALID);
  MKA_CHECK(d->batch >= 1 && d->seq >= 1 && d->d_model >= 1 && d->n_heads >= 1 &&
                d->n_kv_heads >= 1 && d->router_hidden >= 1 && d->block >= 1 && d->top_r >= 1,
            MKA_ERR_INVALID);
  MKA_CHECK(d->n_heads % d->n_kv_heads == 0, MKA_ERR_INVALID);
  MKA_CHECK(d->hash_bits >= 1 && d->hash_bits <= 64, MKA_ERR_INVALID);
  MKA_CHECK(std::isfinite(d->ema_decay) && d->ema_decay >= 0.f && d->ema_decay < 1.f,
            MKA_ERR_INVALID);
  MKA_CHECK(d->dtype == MKA_F32 || d->dtype == MKA_BF16, MKA_ERR_INVALID);
  MKA_CHECK(d->route_mode >= MKA_ROUTE_SOFT && d->route_mode <= MKA_ROUTE_TOP2, MKA_ERR_INVALID);
  MKA_CHECK(d->tiers >= MKA_TIERS_ALL && d->tiers <= MKA_TIERS_L1, MKA_ERR_INVALID);
  MKA_CHECK(d->head_dim == 64 || d->head_dim == 128, MKA_ERR_UNSUPPORTED);
  MKA_CHECK(d->top_r <= 32, MKA_ERR_UNSUPPORTED);
  MKA_CHECK(d->router_hidden <= 256, MKA_ERR_UNSUPPORTED);
  MKA_CHECK(d->n_heads / d->n_kv_heads <= 32, MKA_ERR_UNSUPPORTED);
  const int64_t qw = static_cast<int64_t>(d->n_heads) * d->head_dim;
  MKA_CHECK(static_cast<int64_t>(d->batch) * d->seq <= (1LL << 31) - 1, MKA_ERR_INVALID);
  if (d->dtype == MKA_BF16) {
    MKA_CHECK(d->d_model % 64 == 0 && qw % 64 == 0, MKA_ERR_UNSUPPORTED);
  } else {
    MKA_CHECK(d->d_model % 4 == 0 && qw % 4 == 0, MKA_ERR_UNSUPPORTED);
  }
  return MKA_OK;
}

int rows_of(const mka_dims* d) { return d->batch * d->seq; }

Routing routing_of(const mka_dims* d) { return Routing{d->route_mode, d->tiers}; }

KvLayout contiguous(const mka_dims* d, int64_t t_cap) {
  KvLayout kv;
  kv.G = d->n_kv_heads;
  kv.DH = d->head_dim;
  kv.t_cap = t_cap;
  return kv;
}

// The layer state's cache layout: paged when it carries a page table.
KvLayout layout_of(const mka_dims* d, const mka_state* st) {
  KvLayout kv = contiguous(d, st->t_cap);
  if (st->page_table != nullptr) {
    kv.pt = st->page_table;
    int shift = 0;
    while ((1 << shift) < st->page_size) ++shift;
    kv.page_shift = shift;
    kv.pps = st->pages_per_seq;
  }
  return kv;
}

size_t ema_ws(const mka_dims* d) { return round256(ema_ws_bytes(d->batch, d->seq, d->d_model)); }
// X_fused, then (bf16) the transposed bf16 planes of the block means that the
// selection-product fusion stages.
size_t fuse_ws(const mka_dims* d) {
  return round256(static_cast<size_t>(rows_of(d)) * d->d_model * el_size(d)) +
         (d->dtype == MKA_BF16 ? round256(fuse_sel_ws_bytes(d->batch, d->d_model)) : 0);
}
size_t retrieve_ws(const mka_dims* d) {
  return rows_of(d) <= kFewRows ? round256(retrieve_few_ws_bytes(rows_of(d), d->d_model))
                                : round256(simhash_ws_bytes(d->seq, d->batch, d->d_model));
}
size_t index_ws(const mka_dims* d, int64_t n_blocks) {
  return n_blocks > 0 ? round256(simhash_ws_bytes(static_cast<int>(n_blocks), d->batch, d->d_model))
                      : 0;
}
size_t route_ws(const mka_dims* d) {
  return rows_of(d) <= kFewRows
             ? round256(static_cast<size_t>(rows_of(d)) * d->router_hidden * sizeof(float))
             : 0;
}
size_t decode_ws(const mka_dims* d, int64_t cache_len) {
  if (d->dtype != MKA_BF16) return 0;
  // the split covers rows [0, cache_len - 1); the last row joins in the merge
  return round256(attn_decode_ws_bytes(d->batch, d->n_heads, d->n_kv_heads, d->head_dim,
                                       cache_len - 1));
}

// The split kernel addresses one chunk of a KV head with 32-bit byte offsets.
bool decode_chunk_fits(const mka_dims* d, int64_t n_rows) {
  if (d->dtype != MKA_BF16 || n_rows <= 0) return true;
  const int units = d->batch * d->n_kv_heads *
                    ((d->n_heads / d->n_kv_heads + kSplitHeads - 1) / kSplitHeads);
  return (static_cast<int64_t>(decode_chunk_keys(units, n_rows)) + kSplitTile) * d->head_dim * 2 <
         (static_cast<int64_t>(1) << 31);
}

// ---------------------------------------------------------------- per-step bodies
// Each body assumes check_dims passed and its pointers were validated.

int do_qproj(const mka_dims* d, const void* x, const void* w_q, void* q_out, hipStream_t s) {
  const int M = rows_of(d), D = d->d_model, qw = d->n_heads * d->head_dim;
  if (d->dtype == MKA_BF16) {
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wq = static_cast<const bf16_t*>(w_q);
    const EpiStore<bf16_t> epi{static_cast<bf16_t*>(q_out), qw};
    if (M <= kFewRows)
      MKA_LAUNCH("route/q_gemv", gemv<bf16_t>(xb, D, M, wq, wq, qw, qw, D, epi, s));
    else
      // beside the auxiliary stream's kernels: the register-lean loop
      MKA_LAUNCH("route/q_gemm", gemm_bf16(xb, D, wq, wq, qw, M, qw, D, epi, s, true));
  } else {
    const float* xf = static_cast<const float*>(x);
    const float* wq = static_cast<const float*>(w_q);
    const EpiStore<float> epi{static_cast<float*>(q_out), qw};
    if (M <= kFewRows)
      MKA_LAUNCH("route/q_gemv", gemv<float>(xf, D, M, wq, wq, qw, qw, D, epi, s));
    else
      MKA_LAUNCH("route/q_gemm", gemm_f32(xf, D, wq, wq, qw, M, qw, D, epi, s));
  }
  return MKA_OK;
}

int do_router(const mka_dims* d, const void* q_in, const void* w_r1, const void* w_r2, float* lam,
              void* ws, hipStream_t s) {
  const int M = rows_of(d), qw = d->n_heads * d->head_dim, r = d->router_hidden;
  const Routing rt = routing_of(d);
  if (!rt.learned()) {
    MKA_LAUNCH("route/fixed", lambda_fixed(lam, M, rt, s));
    return MKA_OK;
  }
  if (d->dtype == MKA_BF16) {
    const bf16_t* q = static_cast<const bf16_t*>(q_in);
    const bf16_t* w1 = static_cast<const bf16_t*>(w_r1);
    const bf16_t* w2 = static_cast<const bf16_t*>(w_r2);
    if (M <= kFewRows) {
      float* hid = static_cast<float*>(ws);
      MKA_LAUNCH("route/hidden", gemv<bf16_t>(q, qw, M, w1, w1, r, r, qw, EpiGelu{hid, r}, s));
      MKA_LAUNCH("route/head", router_head<bf16_t>(hid, M, r, w2, lam, rt, s));
    } else if (r == 32 || r == 64) {
      MKA_LAUNCH("route/router", router_bf16_mfma(q, M, qw, w1, r, w2, lam, rt, s));
    } else {
      MKA_LAUNCH("route/router", router_rowwise<bf16_t>(q, M, qw, w1, r, w2, lam, rt, s));
    }
  } else {
    const float* q = static_cast<const float*>(q_in);
    const float* w1 = static_cast<const float*>(w_r1);
    const float* w2 = static_cast<const float*>(w_r2);
    if (M <= kFewRows) {
      float* hid = static_cast<float*>(ws);
      MKA_LAUNCH("route/hidden", gemv<float>(q, qw, M, w1, w1, r, r, qw, EpiGelu{hid, r}, s));
      MKA_LAUNCH("route/head", router_head<float>(hid, M, r, w2, lam, rt, s));
    } else {
      MKA_LAUNCH("route/router", router_rowwise<float>(q, M, qw, w1, r, w2, lam, rt, s));
    }
  }
  return MKA_OK;
}

int do_route(const mka_dims* d, const void* x, const void* w_q, const void* w_r1, const void* w_r2,
             void* q_out, float* lam, void* ws, hipStream_t s) {
  int rc = do_qproj(d, x, w_q, q_out, s);
  if (rc) return rc;
  return do_router(d, q_out, w_r1, w_r2, lam, ws, s);
}

int do_ema(const mka_dims* d, const void* x, int64_t pos0, float* state_io, float* acc_io,
           float* l2, float* means, int nb_cap, void* ws, hipStream_t s) {
  float* w = static_cast<float*>(ws);
  if (d->dtype == MKA_BF16)
    MKA_LAUNCH("ema_scan", ema_scan<bf16_t>(static_cast<const bf16_t*>(x), d->batch, d->seq,
                                            d->d_model, pos0, d->block, d->ema_decay, state_io,
                                            acc_io, l2, means, nb_cap, w, s));
  else
    MKA_LAUNCH("ema_scan", ema_scan<float>(static_cast<const float*>(x), d->batch, d->seq,
                                           d->d_model, pos0, d->block, d->ema_decay, state_io,
                                           acc_io, l2, means, nb_cap, w, s));
  return MKA_OK;
}

int do_index(const mka_dims* d, const float* means, int nb_cap, int first, int n,
             const float* proj, uint64_t* bh, void* ws, hipStream_t s) {
  if (n <= 0) return MKA_OK;
  const int64_t D = d->d_model;
  MKA_LAUNCH("l3_index", simhash_rows(means + first * D, static_cast<int64_t>(nb_cap) * D, n,
                                      d->batch, d->d_model, proj, d->hash_bits, bh + first,
                                      nb_cap, ws, s));
  return MKA_OK;
}

int do_block_kv(const mka_dims* d, const float* means, int nb_cap, int first, int n,
                const void* w_k, const void* w_v, float* block_kv, hipStream_t s) {
  if (n <= 0) return MKA_OK;
  const int kvw = d->n_kv_heads * d->head_dim;
  if (d->dtype == MKA_BF16)
    MKA_LAUNCH("l3_block_kv", block_kv_project<bf16_t>(means, nb_cap, first, n,
                                                       static_cast<const bf16_t*>(w_k),
                                                       static_cast<const bf16_t*>(w_v), kvw,
                                                       d->d_model, d->batch, block_kv, s));
  else
    MKA_LAUNCH("l3_block_kv", block_kv_project<float>(means, nb_cap, first, n,
                                                      static_cast<const float*>(w_k),
                                                      static_cast<const float*>(w_v), kvw,
                                                      d->d_model, d->batch, block_kv, s));
  return MKA_OK;
}

int do_retrieve(const mka_dims* d, const float* l2, const float* proj, const uint64_t* bh,
                int nb_cap, int64_t pos0, uint64_t* keys, int32_t* idx, void* ws, hipStream_t s) {
  const int rows = rows_of(d);
  if (rows <= kFewRows) {
    MKA_LAUNCH("l3_retrieve", retrieve_few(l2, d->batch, d->seq, d->d_model, proj, d->hash_bits, bh,
                                           nb_cap, d->block, d->top_r, pos0, keys, idx, ws, s));
  } else {
    MKA_LAUNCH("l3_retrieve/keys",
               simhash_rows(l2, static_cast<int64_t>(d->seq) * d->d_model, d->seq, d->batch,
                            d->d_model, proj, d->hash_bits, keys, d->seq, ws, s));
    MKA_LAUNCH("l3_retrieve/topr", topr_rows(keys, d->batch, d->seq, pos0, bh, nb_cap, d->block,
                                             d->top_r, idx, s));
  }
  return MKA_OK;
}

int do_kv_proj(const mka_dims* d, const void* src, const void* w_k, const void* w_v, void* kc,
               void* vc, int64_t pos0, const KvLayout& kv, hipStream_t s);

int do_fuse_kv(const mka_dims* d, const void* x, const float* l2, const float* means, int nb_cap,
               const int32_t* idx, const float* lam, const void* w_k, const void* w_v, void* kc,
               void* vc, int64_t pos0, const KvLayout& kv, void* ws, hipStream_t s) {
  const Routing rt = routing_of(d);
  // L1 alone: X_fused = x (lambda = (1, 0, 0)), projected without a fusion pass
  const void* src = x;
  if (rt.ema()) {
    // blocks a token of this call may retrieve: those before the last token's block
    const int64_t n_elig = std::min<int64_t>((pos0 + d->seq - 1) / d->block, nb_cap);
    const size_t xf_bytes = round256(static_cast<size_t>(rows_of(d)) * d->d_model * el_size(d));
    if (d->dtype == MKA_BF16 &&
        fuse_sel_applies(d->batch, d->seq, d->d_model, d->top_r,
                         static_cast<int>(std::min<int64_t>(n_elig, 1 << 30)), rt))
      MKA_LAUNCH("fuse", fuse_mix_sel(static_cast<const bf16_t*>(x), l2, means, nb_cap, idx, lam,
                                      d->batch, d->seq, d->d_model, d->top_r, rt,
                                      static_cast<bf16_t*>(ws), static_cast<int>(n_elig),
                                      static_cast<char*>(ws) + xf_bytes, s));
    else if (d->dtype == MKA_BF16)
      MKA_LAUNCH("fuse", fuse_mix<bf16_t>(static_cast<const bf16_t*>(x), l2, means, nb_cap, idx,
                                          lam, d->batch, d->seq, d->d_model, d->top_r, rt,
                                          static_cast<bf16_t*>(ws), s));
    else
      MKA_LAUNCH("fuse", fuse_mix<float>(static_cast<const float*>(x), l2, means, nb_cap, idx,
                                         lam, d->batch, d->seq, d->d_model, d->top_r, rt,
                                         static_cast<float*>(ws), s));
    src = ws;
  }
  return do_kv_proj(d, src, w_k, w_v, kc, vc, pos0, kv, s);
}

// [K|V] rows pos0 .. pos0+seq-1 of one cache from the rows ``src`` [B, seq, D].
int do_kv_proj(const mka_dims* d, const void* src, const void* w_k, const void* w_v, void* kc,
               void* vc, int64_t pos0, const KvLayout& kv, hipStream_t s) {
  const int M = rows_of(d), D = d->d_model, kvw = d->n_kv_heads * d->head_dim;
  if (d->dtype == MKA_BF16) {
    const bf16_t* xs = static_cast<const bf16_t*>(src);
    const bf16_t* wk = static_cast<const bf16_t*>(w_k);
    const bf16_t* wv = static_cast<const bf16_t*>(w_v);
    const EpiKV<bf16_t> epi{static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), d->seq,
                            d->n_kv_heads, d->head_dim, kv, pos0};
    if (M <= kFewRows)
      MKA_LAUNCH("kv_gemv", gemv<bf16_t>(xs, D, M, wk, wv, kvw, 2 * kvw, D, epi, s));
    else
      MKA_LAUNCH("kv_gemm", gemm_bf16(xs, D, wk, wv, kvw, M, 2 * kvw, D, epi, s));
  } else {
    const float* xs = static_cast<const float*>(src);
    const float* wk = static_cast<const float*>(w_k);
    const float* wv = static_cast<const float*>(w_v);
    const EpiKV<float> epi{static_cast<float*>(kc), static_cast<float*>(vc), d->seq, d->n_kv_heads,
                           d->head_dim, kv, pos0};
    if (M <= kFewRows)
      MKA_LAUNCH("kv_gemv", gemv<float>(xs, D, M, wk, wv, kvw, 2 * kvw, D, epi, s));
    else
      MKA_LAUNCH("kv_gemm", gemm_f32(xs, D, wk, wv, kvw, M, 2 * kvw, D, epi, s));
  }
  return MKA_OK;
}

// One tier's rows (tier 0 = x itself; 1 = L2; 2 = L3) into ``rows`` when they
// need forming; returns the rows to project.
const void* tier_source(const mka_dims* d, int tier, const void* x, const float* l2,
                        const float* means, int nb_cap, const int32_t* idx, void* rows,
                        hipStream_t s, int* rc) {
  *rc = MKA_OK;
  if (tier == 0) return x;
  hipError_t e;
  if (d->dtype == MKA_BF16)
    e = tier_rows<bf16_t>(static_cast<const bf16_t*>(x), l2, means, nb_cap, idx, tier, d->batch,
                          d->seq, d->d_model, d->top_r, static_cast<bf16_t*>(rows), s);
  else
    e = tier_rows<float>(static_cast<const float*>(x), l2, means, nb_cap, idx, tier, d->batch,
                         d->seq, d->d_model, d->top_r, static_cast<float*>(rows), s);
  if (e != hipSuccess) {
    *rc = hip_fail("full/tier_rows", e);
    return nullptr;
  }
  return rows;
}

int do_mix(const mka_dims* d, void* const a[3], const float* lam, void* o, hipStream_t s) {
  const int64_t M = rows_of(d);
  const int HD = d->n_heads * d->head_dim;
  if (d->dtype == MKA_BF16)
    MKA_LAUNCH("full/mix", mix_paths<bf16_t>(static_cast<const bf16_t*>(a[0]),
                                             static_cast<const bf16_t*>(a[1]),
                                             static_cast<const bf16_t*>(a[2]), lam, M, HD,
                                             static_cast<bf16_t*>(o), s));
  else
    MKA_LAUNCH("full/mix", mix_paths<float>(static_cast<const float*>(a[0]),
                                            static_cast<const float*>(a[1]),
                                            static_cast<const float*>(a[2]), lam, M, HD,
                                            static_cast<float*>(o), s));
  return MKA_OK;
}

int do_attn_prefill(const mka_dims* d, const void* q, const void* kc, const void* vc,
                    const KvLayout& kv, int64_t pos0, void* o, hipStream_t s,
                    float* lse = nullptr) {
  if (d->dtype == MKA_BF16)
    MKA_LAUNCH("attn_prefill",
               attn_prefill<bf16_t>(static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(kc),
                                    static_cast<const bf16_t*>(vc), static_cast<bf16_t*>(o),
                                    d->batch, d->seq, d->n_heads, d->n_kv_heads, d->head_dim,
                                    kv, pos0, lse, s));
  else
    MKA_LAUNCH("attn_prefill",
               attn_prefill<float>(static_cast<const float*>(q), static_cast<const float*>(kc),
                                   static_cast<const float*>(vc), static_cast<float*>(o), d->batch,
                                   d->seq, d->n_heads, d->n_kv_heads, d->head_dim, kv, pos0, lse,
                                   s));
  return MKA_OK;
}

int do_attn_decode(const mka_dims* d, const void* q, const void* kc, const void* vc, const KvLayout& kv,
                   int64_t cache_len, void* o, void* ws, hipStream_t s) {
  if (d->dtype == MKA_BF16)
    MKA_LAUNCH("attn_decode",
               attn_decode_bf16(static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(kc),
                                static_cast<const bf16_t*>(vc), static_cast<bf16_t*>(o), d->batch,
                                d->n_heads, d->n_kv_heads, d->head_dim, kv, cache_len, ws, s));
  else  // one query row at position cache_len - 1
    MKA_LAUNCH("attn_decode",
               attn_prefill<float>(static_cast<const float*>(q), static_cast<const float*>(kc),
                                   static_cast<const float*>(vc), static_cast<float*>(o), d->batch,
                                   1, d->n_heads, d->n_kv_heads, d->head_dim, kv, cache_len - 1,
                                   nullptr, s));
  return MKA_OK;
}

// Blocks whose last token lies in [pos0, pos0 + seq): [first, first + n).
void completed_blocks(const mka_dims* d, int64_t pos0, int64_t* first, int64_t* n) {
  *first = pos0 / d->block;
  const int64_t end = (pos0 + d->seq) / d->block;  // one past the last completed block
  *n = end > *first ? end - *first : 0;
}

bool ptrs_ok(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

constexpr int64_t kMaxDecodeCache = static_cast<int64_t>(1) << 26;  // rows

// Per-device auxiliary stream and fork/join/done events of mka_prefill, created on
// a device's first prefill and kept until the process ends.  Enqueueing one
// prefill holds the device's lock, so concurrent callers cannot interleave
// their fork/join records.
struct Aux {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, done = nullptr;
  std::mutex lock;
};

Aux* aux_for_current_device(int* rc) {
  static std::mutex table_lock;
  static std::unordered_map<int, std::unique_ptr<Aux>> table;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *rc = hip_fail("prefill/aux", e);
    return nullptr;
  }
  std::lock_guard<std::mutex> g(table_lock);
  auto it = table.find(dev);
  if (it != table.end()) return it->second.get();
  auto a = std::make_unique<Aux>();
  if ((e = hipStreamCreateWithFlags(&a->stream, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&a->fork, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&a->join, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&a->done, hipEventDisableTiming)) != hipSuccess) {
    *rc = hip_fail("prefill/aux", e);
    return nullptr;
  }
  Aux* p = a.get();
  table.emplace(dev, std::move(a));
  return p;
}

// Workspace of a prefill: the EMA scan and block index run on the auxiliary
// stream beside the query product, so the two streams have disjoint regions:
// [EMA scan, index | route, retrieval, fusion].
size_t prefill_chain_ws(const mka_dims* d) {
  const size_t w = ema_ws(d), wi = index_ws(d, d->seq / d->block + 1);
  return w > wi ? w : wi;
}
// The hyperplane split of the certified SimHash path, prepared on the auxiliary
// stream for the retrieval on the main one: a region of its own.
bool prefill_prepares_codes(const mka_dims* d) {
  return routing_of(d).l3() && rows_of(d) > kFewRows &&
         simhash_prepared_path(d->seq, d->batch, d->d_model);
}
size_t prefill_prep_ws(const mka_dims* d) {
  return prefill_prepares_codes(d) ? round256(simhash_prep_bytes(d->d_model)) : 0;
}
size_t prefill_main_ws(const mka_dims* d) {
  size_t w = fuse_ws(d);
  if (route_ws(d) > w) w = route_ws(d);
  if (retrieve_ws(d) > w) w = retrieve_ws(d);
  return w;
}

// Workspace of a decode step.  bf16: the attention partials over rows [0, pos),
// the router hidden layer, the partial key projections and the three
// projected rows (x, L2, L3) of the new K/V row; float32: hidden, partial key
// projections, X_fused.  Both end with the block index's own workspace.
struct DecodeWs {
  size_t attn, hid, part, kv, xf, index, total;
};
DecodeWs decode_layout(const mka_dims* d, int64_t cache_len) {
  DecodeWs w{};
  const bool bf = d->dtype == MKA_BF16;
  w.attn = bf ? round256(attn_decode_ws_bytes(d->batch, d->n_heads, d->n_kv_heads, d->head_dim,
                                               cache_len - 1))
              : 0;
  w.hid = round256(static_cast<size_t>(d->batch) * d->router_hidden * sizeof(float));
  w.part = round256(sizeof(double) * static_cast<size_t>(decode_slices(d->d_model)) * d->batch * 64);
  w.kv = bf ? round256(3 * sizeof(float) * static_cast<size_t>(d->batch) * 2 * d->n_kv_heads *
                       d->head_dim)
            : 0;
  w.xf = bf ? 0 : fuse_ws(d);
  w.index = index_ws(d, 1);
  w.total = w.attn + w.hid + w.part + w.kv + w.xf + w.index;
  return w;
}

// Workspace of full MKA.  Prefill: [EMA scan, index | route, retrieval | tier
// rows | a_1 | a_2 | a_3]; decode: [the sequential steps' shared region | tier
// rows | a_1 | a_2 | a_3] (the steps run in order on one stream).
struct FullWs {
  size_t chain, main, rows, path, total;
};
FullWs full_layout(const mka_dims* d, bool decode, int64_t cache_len) {
  FullWs w{};
  if (decode) {
    size_t m = route_ws(d);
    for (size_t v : {ema_ws(d), retrieve_ws(d), decode_ws(d, cache_len), index_ws(d, 1)})
      if (v > m) m = v;
    w.main = m;
  } else {
    w.chain = prefill_chain_ws(d);
    w.main = route_ws(d) > retrieve_ws(d) ? route_ws(d) : retrieve_ws(d);
  }
  w.rows = fuse_ws(d);
  w.path = round256(static_cast<size_t>(rows_of(d)) * d->n_heads * d->head_dim * el_size(d));
  w.total = w.chain + w.main + w.rows + 3 * w.path;
  return w;
}

// Workspace of the backward: float32 gradients and scratch, then the storage
// type's product operands (transposed ones padded to Mp = M rounded up to 32
// tokens, the products' reduction dimension).
struct BwdWs {
  size_t dsum, dq, dkv, dxf, dlam, dz, dm, part, pre, heads, gather, splitk, splitk_aux;  // float32
  size_t dkv_a, dkv_t, wkv_t, xf, xf_t, dpre, dpre_t, q_t, wr1_t, wq_t, dq_a, dq_t, x_t;  // dtype
  size_t total;
  int Mp, nbs;
};
BwdWs bwd_layout(const mka_dims* d) {
  BwdWs w{};
  const size_t M = rows_of(d), el = el_size(d), f = sizeof(float);
  const size_t D = d->d_model, qw = static_cast<size_t>(d->n_heads) * d->head_dim;
  const size_t kvw = static_cast<size_t>(d->n_kv_heads) * d->head_dim, r = d->router_hidden;
  const size_t H = d->n_heads;
  w.Mp = static_cast<int>((M + 31) / 32 * 32);
  w.nbs = d->seq / d->block + 1;
  const size_t Mp = w.Mp;
  const bool bf = d->dtype == MKA_BF16;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at += round256(bytes);
    return o;
  };
  w.dsum = take(f * M * H);
  w.dq = take(f * M * qw);
  w.dkv = take(f * M * 2 * kvw);
  w.dxf = take(f * M * D);
  w.dlam = take(f * M * 3);
  w.dz = take(f * M * 3);
  w.dm = take(f * d->batch * w.nbs * D);
  w.part = take(ema_adj_ws_bytes(d->batch, d->seq, d->d_model));
  w.pre = take(f * M * r);
  w.gather = take(block_gather_ws_bytes(d->batch, d->seq, d->d_model, d->block));
  w.heads = bf ? take(attn_bwd_mfma_ws_bytes(d->batch, d->seq, d->n_heads, d->n_kv_heads,
                                             d->head_dim))
               : 0;
  // bf16 layers read the token-major rows as K-major product operands; the
  // transposed copies are for float32 layers only
  w.dkv_a = bf ? take(el * M * 2 * kvw) : 0;
  w.dkv_t = bf ? 0 : take(el * 2 * kvw * Mp);
  w.wkv_t = take(el * D * 2 * kvw);
  w.xf = take(el * M * D);
  w.xf_t = bf ? 0 : take(el * D * Mp);
  w.dpre = take(el * M * r);
  w.dpre_t = bf ? 0 : take(el * r * Mp);
  w.q_t = bf ? 0 : take(el * qw * Mp);
  w.wr1_t = bf ? 0 : take(el * qw * r);
  w.wq_t = bf ? 0 : take(el * D * qw);
  w.dq_a = bf ? take(el * M * qw) : 0;
  w.dq_t = bf ? 0 : take(el * qw * Mp);
  w.x_t = bf ? 0 : take(el * D * Mp);
  if (bf) {  // the largest split-K partials among the products below
    const int m = static_cast<int>(M), mp = w.Mp, dd = static_cast<int>(D);
    const int q = static_cast<int>(qw), kv = static_cast<int>(kvw), rr = static_cast<int>(r);
    size_t sk = 0;
    for (size_t v : {gemm_bf16_splitk_ws_bytes(m, dd, 2 * kv), gemm_bf16_splitk_ws_bytes(kv, dd, mp),
                     gemm_bf16_splitk_ws_bytes(m, rr, q), gemm_bf16_splitk_ws_bytes(rr, q, mp),
                     gemm_bf16_splitk_ws_bytes(m, q, rr), gemm_bf16_splitk_ws_bytes(m, dd, q),
                     gemm_bf16_splitk_ws_bytes(q, dd, mp)})
      if (v > sk) sk = v;
    w.splitk = take(sk);
    // the router's pre-activation, dW_k and dW_v run on the auxiliary stream
    // beside the main stream's products: a partials region of their own
    w.splitk_aux = take(std::max(gemm_bf16_splitk_ws_bytes(kv, dd, mp),
                                 gemm_bf16_splitk_ws_bytes(m, rr, q)));
  }
  w.total = at;
  return w;
}

// The backward's products; bf16 ones split their reduction over ``sk`` (the
// workspace's split-K region) when the output has too few tiles.
template <typename T>
hipError_t gemm_t(const T* a, int lda, const T* b, int M, int N, int K, const EpiStore<float>& e,
                  float* sk, hipStream_t s) {
  if constexpr (std::is_same<T, bf16_t>::value) return gemm_bf16_splitk(a, lda, b, M, N, K, e, sk, s);
  else return gemm_f32(a, lda, b, b, N, M, N, K, e, s);
}
template <typename T>
hipError_t gemm_t(const T* a, int lda, const T* b, int M, int N, int K, const EpiAdd& e, float* sk,
                  hipStream_t s) {
  if constexpr (std::is_same<T, bf16_t>::value) return gemm_bf16_splitk(a, lda, b, M, N, K, e, sk, s);
  else return gemm_f32(a, lda, b, b, N, M, N, K, e, s);
}

// With ``aux`` (bf16 only; its lock held by the caller) the dq kernel runs on
// the auxiliary stream beside the dK/dV passes; the caller joins it (records
// aux->join there and waits for it on s) before dq is next used.
template <typename T>
int attn_backward_steps(const mka_dims* d, const T* q, const T* kc, const T* vc, int64_t t_cap,
                        const T* o, const float* lse, const T* d_o, float* dq, float* dkv,
                        float* dsum, float* heads, hipStream_t s, Aux* aux) {
  const int B = d->batch, N = d->seq, H = d->n_heads, G = d->n_kv_heads, dh = d->head_dim;
  MKA_LAUNCH("bwd/prep", attn_bwd_prep<T>(o, d_o, static_cast<int64_t>(rows_of(d)) * H, dh, dsum,
                                          s));
  if constexpr (std::is_same<T, bf16_t>::value) {
    hipStream_t s_dq = s;
    if (aux != nullptr) {
      MKA_LAUNCH("bwd/fork", hipEventRecord(aux->fork, s));
      MKA_LAUNCH("bwd/fork", hipStreamWaitEvent(aux->stream, aux->fork, 0));
      s_dq = aux->stream;
    }
    MKA_LAUNCH("bwd/attn", attn_bwd_mfma(q, kc, vc, d_o, lse, dsum, B, N, H, G, dh, t_cap, dq,
                                         nullptr, heads, s_dq));
    MKA_LAUNCH("bwd/attn", attn_bwd_mfma(q, kc, vc, d_o, lse, dsum, B, N, H, G, dh, t_cap,
                                         nullptr, dkv, heads, s));
  } else
    MKA_LAUNCH("bwd/attn",
               attn_bwd_rows<T>(q, kc, vc, d_o, lse, dsum, B, N, H, G, dh, t_cap, dq, dkv, s));
  return MKA_OK;
}

// Workspace of the attention backward alone: D, then the per-head dK/dV slices.
size_t attn_bwd_ws(const mka_dims* d) {
  const size_t dsum = round256(sizeof(float) * rows_of(d) * d->n_heads);
  return dsum + (d->dtype == MKA_BF16 ? round256(attn_bwd_mfma_ws_bytes(
                                            d->batch, d->seq, d->n_heads, d->n_kv_heads,
                                            d->head_dim))
                                      : 0);
}

template <typename T>
int backward_body(const mka_dims* d, const void* x_, const mka_weights* w, const mka_state* st,
                  const mka_outputs* fwd, const void* d_o_, const mka_grads* gr, char* ws,
                  hipStream_t s) {
  const BwdWs L = bwd_layout(d);
  const int B = d->batch, N = d->seq, D = d->d_model, H = d->n_heads, G = d->n_kv_heads;
  const int dh = d->head_dim, qw = H * dh, kvw = G * dh, r = d->router_hidden, Mp = L.Mp;
  const int M = rows_of(d);
  const Routing rt = routing_of(d);
  constexpr bool kBf = std::is_same<T, bf16_t>::value;
  const T* x = static_cast<const T*>(x_);
  const T* d_o = static_cast<const T*>(d_o_);
  const T* q = static_cast<const T*>(fwd->q);
  const T* o = static_cast<const T*>(fwd->o);
  const T* wq = static_cast<const T*>(w->w_q);
  const T* wk = static_cast<const T*>(w->w_k);
  const T* wv = static_cast<const T*>(w->w_v);
  const T* wr1 = static_cast<const T*>(w->w_r1);
  const T* wr2 = static_cast<const T*>(w->w_r2);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto E = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
  float *dsum = F(L.dsum), *dq = F(L.dq), *dkv = F(L.dkv), *dxf = F(L.dxf), *dlam = F(L.dlam);
  float *dz = F(L.dz), *dm = F(L.dm), *part = F(L.part), *pre = F(L.pre), *sk = F(L.splitk);
  T *dkv_t = E(L.dkv_t), *wkv_t = E(L.wkv_t), *xf = E(L.xf), *xf_t = E(L.xf_t);
  T *dpre = E(L.dpre), *dpre_t = E(L.dpre_t), *q_t = E(L.q_t), *wr1_t = E(L.wr1_t);
  T *wq_t = E(L.wq_t), *dq_t = E(L.dq_t), *x_t = E(L.x_t);
  // the float32 gradients as product operands of the storage type
  const T* dkv_a = kBf ? E(L.dkv_a) : reinterpret_cast<const T*>(dkv);
  const T* dq_a = kBf ? E(L.dq_a) : reinterpret_cast<const T*>(dq);

  // attention: D = rowsum(dO * O), then dq (bf16: on the auxiliary stream, beside
  // the dK/dV passes and the work below, joined before dq is next used), dK, dV
  Aux* aux = nullptr;
  std::unique_lock<std::mutex> aux_guard;
  if constexpr (kBf) {
    int arc = MKA_OK;
    aux = aux_for_current_device(&arc);
    if (aux == nullptr) return arc;
    aux_guard = std::unique_lock<std::mutex>(aux->lock);
  }
  int rc = attn_backward_steps<T>(d, q, static_cast<const T*>(st->k_cache),
                                  static_cast<const T*>(st->v_cache), st->t_cap, o, fwd->lse, d_o,
                                  dq, dkv, dsum, F(L.heads), s, aux);
  if (rc) return rc;
  if constexpr (kBf) {
    // the router's pre-activation needs only q and W_r1: on the auxiliary
    // stream after the dq kernel
    if (rt.learned())
      MKA_LAUNCH("bwd/pre", gemm_t<T>(q, qw, wr1, M, r, qw, EpiStore<float>{pre, r},
                                      F(L.splitk_aux), aux->stream));
  }
  auto join_dq = [&]() -> int {
    if (aux != nullptr) {
      MKA_LAUNCH("bwd/join", hipEventRecord(aux->join, aux->stream));
      MKA_LAUNCH("bwd/join", hipStreamWaitEvent(s, aux->join, 0));
    }
    return MKA_OK;
  };
  // [K|V] = X_fused [W_k|W_v]^T: dX_fused = dKV [W_k; W_v]; dW = dKV^T X_fused
  MKA_LAUNCH("bwd/t", (transpose<T, T>(wk, D, kvw, D, kvw, 2 * kvw, wkv_t, s)));
  MKA_LAUNCH("bwd/t", (transpose<T, T>(wv, D, kvw, D, kvw, 2 * kvw, wkv_t + kvw, s)));
  // dkv in the storage type: as rows (bf16: the products read the token-major
  // rows directly, K-major where the reduction runs over tokens), or also
  // transposed (float32 products)
  if constexpr (kBf)
    MKA_LAUNCH("bwd/cvt", (convert<float, T>(dkv, static_cast<int64_t>(M) * 2 * kvw,
                                             const_cast<T*>(dkv_a), s)));
  else
    MKA_LAUNCH("bwd/t", (transpose<float, T>(dkv, 2 * kvw, M, 2 * kvw, Mp, Mp, dkv_t, s)));
  MKA_LAUNCH("bwd/dxf", gemm_t<T>(dkv_a, 2 * kvw, wkv_t, M, D, 2 * kvw, EpiStore<float>{dxf, D}, sk, s));
  // the fusion's adjoint (dx = l1 dxf, dlambda) and X_fused re-formed for the
  // weight gradients (with the EMA tiers; otherwise X_fused is x), one pass
  MKA_LAUNCH("bwd/fuse", fuse_bwd<T>(x, rt.l2() ? fwd->l2 : nullptr, st->block_means, st->nb_cap,
                                     rt.l3() ? fwd->idx : nullptr, fwd->lambda, B, N, D,
                                     rt.l3() ? d->top_r : 0, dxf, gr->dx, dlam,
                                     rt.ema() ? xf : nullptr, s));
  const T* xf_src = rt.ema() ? xf : x;
  if constexpr (kBf) {
    // on the auxiliary stream (after the dq kernel there), beside the block
    // gather and the EMA adjoint; joined with dq before the router's steps
    MKA_LAUNCH("bwd/fork", hipEventRecord(aux->done, s));
    MKA_LAUNCH("bwd/fork", hipStreamWaitEvent(aux->stream, aux->done, 0));
    float* sk_aux = F(L.splitk_aux);
    MKA_LAUNCH("bwd/dwk", gemm_bf16_km(dkv_a, 2 * kvw, true, xf_src, D, kvw, D, Mp, M,
                                       EpiStore<float>{gr->dw_k, D}, sk_aux, aux->stream));
    MKA_LAUNCH("bwd/dwv", gemm_bf16_km(dkv_a + kvw, 2 * kvw, true, xf_src, D, kvw, D, Mp, M,
                                       EpiStore<float>{gr->dw_v, D}, sk_aux, aux->stream));
  } else {
    MKA_LAUNCH("bwd/t", (transpose<T, T>(xf_src, D, M, D, Mp, Mp, xf_t, s)));
    MKA_LAUNCH("bwd/dwk", gemm_t<T>(dkv_t, Mp, xf_t, kvw, D, Mp, EpiStore<float>{gr->dw_k, D}, sk, s));
    MKA_LAUNCH("bwd/dwv", gemm_t<T>(dkv_t + static_cast<size_t>(kvw) * Mp, Mp, xf_t, kvw, D, Mp,
                                    EpiStore<float>{gr->dw_v, D}, sk, s));
  }
  // the EMA's adjoint and the block means' adjoint
  if (rt.l3())
    MKA_LAUNCH("bwd/blocks", block_gather(dxf, fwd->lambda, fwd->idx, B, N, D, d->top_r, d->block,
                                          L.nbs, F(L.gather), dm, s));
  else
    MKA_LAUNCH("bwd/zero", fill_zero(dm, static_cast<int64_t>(B) * L.nbs * D, s));
  MKA_LAUNCH("bwd/ema", ema_adjoint_add(dxf, fwd->lambda, dm, L.nbs, B, N, D, d->block,
                                        d->ema_decay, part, gr->dx, s));
  // router: dz, dW_r2, dpre; dW_r1 = dpre^T q; dq += dpre W_r1
  if ((rc = join_dq()) != MKA_OK) return rc;
  if (rt.learned()) {
    if constexpr (!kBf)
      MKA_LAUNCH("bwd/pre", gemm_t<T>(q, qw, wr1, M, r, qw, EpiStore<float>{pre, r}, sk, s));
    MKA_LAUNCH("bwd/router", router_bwd<T>(fwd->lambda, dlam, pre, wr2, r, M, rt, dz, dpre,
                                           gr->dw_r2, s));
    if constexpr (kBf) {
      MKA_LAUNCH("bwd/dwr1", gemm_bf16_km(dpre, r, true, q, qw, r, qw, Mp, M,
                                          EpiStore<float>{gr->dw_r1, qw}, sk, s));
      MKA_LAUNCH("bwd/dqr", gemm_bf16_km(dpre, r, false, wr1, qw, M, qw, r, r, EpiAdd{dq, qw}, sk,
                                         s));
    } else {
      MKA_LAUNCH("bwd/t", (transpose<T, T>(dpre, r, M, r, Mp, Mp, dpre_t, s)));
      MKA_LAUNCH("bwd/t", (transpose<T, T>(q, qw, M, qw, Mp, Mp, q_t, s)));
      MKA_LAUNCH("bwd/dwr1", gemm_t<T>(dpre_t, Mp, q_t, r, qw, Mp, EpiStore<float>{gr->dw_r1, qw}, sk, s));
      MKA_LAUNCH("bwd/t", (transpose<T, T>(wr1, qw, r, qw, r, r, wr1_t, s)));
      MKA_LAUNCH("bwd/dqr", gemm_t<T>(dpre, r, wr1_t, M, qw, r, EpiAdd{dq, qw}, sk, s));
    }
  } else {
    MKA_LAUNCH("bwd/zero", fill_zero(gr->dw_r1, static_cast<int64_t>(r) * qw, s));
    MKA_LAUNCH("bwd/zero", fill_zero(gr->dw_r2, 3 * r, s));
  }
  // Q = x W_q^T: dx += dq W_q; dW_q = dq^T x
  if constexpr (kBf) {
    MKA_LAUNCH("bwd/cvt", (convert<float, T>(dq, static_cast<int64_t>(M) * qw,
                                             const_cast<T*>(dq_a), s)));
    // dW_q on the auxiliary stream beside dx += dq W_q: neither splits its
    // reduction, and each fills the other's partial last round of tiles
    MKA_LAUNCH("bwd/fork", hipEventRecord(aux->fork, s));
    MKA_LAUNCH("bwd/fork", hipStreamWaitEvent(aux->stream, aux->fork, 0));
    MKA_LAUNCH("bwd/dwq", gemm_bf16_km(dq_a, qw, true, x, D, qw, D, Mp, M,
                                       EpiStore<float>{gr->dw_q, D}, F(L.splitk_aux),
                                       aux->stream));
    MKA_LAUNCH("bwd/dx", gemm_bf16_km(dq_a, qw, false, wq, D, M, D, qw, qw, EpiAdd{gr->dx, D}, sk,
                                      s));
    MKA_LAUNCH("bwd/join", hipEventRecord(aux->join, aux->stream));
    MKA_LAUNCH("bwd/join", hipStreamWaitEvent(s, aux->join, 0));
  } else {
    MKA_LAUNCH("bwd/t", (transpose<T, T>(wq, D, qw, D, qw, qw, wq_t, s)));
    MKA_LAUNCH("bwd/t", (transpose<float, T>(dq, qw, M, qw, Mp, Mp, dq_t, s)));
    MKA_LAUNCH("bwd/dx", gemm_t<T>(dq_a, qw, wq_t, M, D, qw, EpiAdd{gr->dx, D}, sk, s));
    MKA_LAUNCH("bwd/t", (transpose<T, T>(x, D, M, D, Mp, Mp, x_t, s)));
    MKA_LAUNCH("bwd/dwq", gemm_t<T>(dq_t, Mp, x_t, qw, D, Mp, EpiStore<float>{gr->dw_q, D}, sk, s));
  }
  return MKA_OK;
}

int check_full_args(const mka_dims* d, const void* x, int64_t pos0, const mka_weights* w,
                    const mka_state* st, const mka_tier_cache* kv, const mka_outputs* out) {
  MKA_CHECK(w != nullptr && st != nullptr && kv != nullptr && out != nullptr, MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({x, w->w_q, w->w_k, w->w_v, w->w_r1, w->w_r2, w->proj}), MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({st->ema_state, st->block_acc, st->block_means}), MKA_ERR_INVALID);
  MKA_CHECK(st->block_hash != nullptr && (reinterpret_cast<uintptr_t>(st->block_hash) & 7u) == 0,
            MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({out->q, out->lambda, out->l2, out->key, out->idx, out->o}), MKA_ERR_INVALID);
  const Routing rt = routing_of(d);
  const bool on[3] = {true, rt.l2(), rt.l3()};
  for (int l = 0; l < 3; ++l)
    if (on[l]) MKA_CHECK(ptrs_ok({kv->k_cache[l], kv->v_cache[l]}), MKA_ERR_INVALID);
  MKA_CHECK(pos0 >= 0 && st->nb_cap >= 1 && st->nb_cap < 0xFFFFFF, MKA_ERR_INVALID);
  MKA_CHECK(pos0 + d->seq <= st->t_cap, MKA_ERR_INVALID);
  MKA_CHECK((pos0 + d->seq) / d->block <= st->nb_cap, MKA_ERR_INVALID);
  MKA_CHECK(st->page_table == nullptr, MKA_ERR_UNSUPPORTED);  // the tier caches are contiguous
  return MKA_OK;
}

}  // namespace

extern "C" {

const char* mka_version(void) { return "mka 0.1.0 (gfx950)"; }

const char* mka_last_error(void) { return g_last_error; }

const char* mka_status_string(int status) {
  switch (status) {
    case MKA_OK: return "ok";
    case MKA_ERR_INVALID: return "invalid argument";
    case MKA_ERR_UNSUPPORTED: return "unsupported shape or type";
    case MKA_ERR_WORKSPACE: return "workspace too small";
    case MKA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

size_t mka_workspace_bytes(const mka_dims* d, int op, int64_t cache_len) {
  if (check_dims(d) != MKA_OK) return 0;
  switch (op) {
    case MKA_OP_EMA_SCAN: return ema_ws(d);
    case MKA_OP_FUSE_KV: return fuse_ws(d);
    case MKA_OP_RETRIEVE: return retrieve_ws(d);
    case MKA_OP_INDEX: return index_ws(d, cache_len);
    case MKA_OP_ROUTE: return route_ws(d);
    case MKA_OP_ATTN_DECODE: return cache_len > 0 ? decode_ws(d, cache_len) : 0;
    case MKA_OP_PREFILL:  // blocks completed by a call at any pos0: at most seq / block + 1
      return prefill_chain_ws(d) + prefill_main_ws(d) + prefill_prep_ws(d);
    case MKA_OP_DECODE_STEP:
      return d->seq == 1 && cache_len > 0 ? decode_layout(d, cache_len).total : 0;
    case MKA_OP_FULL_PREFILL: return full_layout(d, false, 0).total;
    case MKA_OP_BACKWARD: return bwd_layout(d).total;
    case MKA_OP_ATTN_BACKWARD: return attn_bwd_ws(d);
    case MKA_OP_FULL_DECODE_STEP:
      return d->seq == 1 && cache_len > 0 ? full_layout(d, true, cache_len).total : 0;
    default: return 0;
  }
}

int mka_route(const mka_dims* d, const void* x, const void* w_q, const void* w_r1,
              const void* w_r2, void* q_out, float* lambda_out, void* ws, size_t ws_bytes,
              void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(ptrs_ok({x, w_q, w_r1, w_r2, q_out, lambda_out}), MKA_ERR_INVALID);
  if (route_ws(d) > 0) {
    MKA_CHECK(ptrs_ok({ws}), MKA_ERR_WORKSPACE);
    MKA_CHECK(ws_bytes >= route_ws(d), MKA_ERR_WORKSPACE);
  }
  return do_route(d, x, w_q, w_r1, w_r2, q_out, lambda_out, ws, static_cast<hipStream_t>(stream));
}

int mka_ema_scan(const mka_dims* d, const void* x, int64_t pos0, float* state_io,
                 float* block_acc_io, float* l2_out, float* block_means, int32_t nb_cap, void* ws,
                 size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(ptrs_ok({x, state_io, block_acc_io, l2_out}), MKA_ERR_INVALID);
  MKA_CHECK(pos0 >= 0 && nb_cap >= 0, MKA_ERR_INVALID);
  int64_t first, n;
  completed_blocks(d, pos0, &first, &n);
  if (n > 0) {
    MKA_CHECK(ptrs_ok({block_means}), MKA_ERR_INVALID);
    MKA_CHECK(first + n <= nb_cap, MKA_ERR_INVALID);
  }
  if (ema_ws(d) > 0) {
    MKA_CHECK(ptrs_ok({ws}), MKA_ERR_WORKSPACE);
    MKA_CHECK(ws_bytes >= ema_ws(d), MKA_ERR_WORKSPACE);
  }
  return do_ema(d, x, pos0, state_io, block_acc_io, l2_out, block_means, nb_cap, ws,
                static_cast<hipStream_t>(stream));
}

int mka_l3_index(const mka_dims* d, const float* block_means, int32_t nb_cap, int32_t first_block,
                 int32_t n_blocks, const float* proj, uint64_t* block_hash, void* ws,
                 size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(first_block >= 0 && n_blocks >= 0 &&
                static_cast<int64_t>(first_block) + n_blocks <= nb_cap,
            MKA_ERR_INVALID);
  if (n_blocks == 0) return MKA_OK;
  MKA_CHECK(ptrs_ok({block_means, proj}) && block_hash != nullptr &&
                (reinterpret_cast<uintptr_t>(block_hash) & 7u) == 0,
            MKA_ERR_INVALID);
  if (index_ws(d, n_blocks) > 0) {
    MKA_CHECK(ptrs_ok({ws}), MKA_ERR_WORKSPACE);
    MKA_CHECK(ws_bytes >= index_ws(d, n_blocks), MKA_ERR_WORKSPACE);
  }
  return do_index(d, block_means, nb_cap, first_block, n_blocks, proj, block_hash, ws,
                  static_cast<hipStream_t>(stream));
}

int mka_l3_block_kv(const mka_dims* d, const float* block_means, int32_t nb_cap,
                    int32_t first_block, int32_t n_blocks, const void* w_k, const void* w_v,
                    float* block_kv, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(first_block >= 0 && n_blocks >= 0 &&
                static_cast<int64_t>(first_block) + n_blocks <= nb_cap,
            MKA_ERR_INVALID);
  if (n_blocks == 0) return MKA_OK;
  MKA_CHECK(ptrs_ok({block_means, w_k, w_v, block_kv}), MKA_ERR_INVALID);
  return do_block_kv(d, block_means, nb_cap, first_block, n_blocks, w_k, w_v, block_kv,
                     static_cast<hipStream_t>(stream));
}

int mka_l3_retrieve(const mka_dims* d, const float* l2, const float* proj,
                    const uint64_t* block_hash, int32_t nb_cap, int64_t pos0, uint64_t* key_out,
                    int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(ptrs_ok({l2, proj, key_out, idx_out}), MKA_ERR_INVALID);
  MKA_CHECK(pos0 >= 0 && nb_cap >= 0, MKA_ERR_INVALID);
  MKA_CHECK((pos0 + d->seq - 1) / d->block <= nb_cap, MKA_ERR_INVALID);
  MKA_CHECK(nb_cap < 0xFFFFFF, MKA_ERR_UNSUPPORTED);
  if ((pos0 + d->seq - 1) / d->block > 0)
    MKA_CHECK(block_hash != nullptr && (reinterpret_cast<uintptr_t>(block_hash) & 7u) == 0,
              MKA_ERR_INVALID);
  if (retrieve_ws(d) > 0) {
    MKA_CHECK(ptrs_ok({ws}), MKA_ERR_WORKSPACE);
    MKA_CHECK(ws_bytes >= retrieve_ws(d), MKA_ERR_WORKSPACE);
  }
  return do_retrieve(d, l2, proj, block_hash, nb_cap, pos0, key_out, idx_out, ws,
                     static_cast<hipStream_t>(stream));
}

int mka_fuse_kv_proj(const mka_dims* d, const void* x, const float* l2, const float* block_means,
                     int32_t nb_cap, const int32_t* idx, const float* lambda, const void* w_k,
                     const void* w_v, void* k_cache, void* v_cache, int64_t pos0, int64_t t_cap,
                     void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  const Routing rt = routing_of(d);  // inputs of disabled tiers are not read
  MKA_CHECK(ptrs_ok({x, lambda, w_k, w_v, k_cache, v_cache}), MKA_ERR_INVALID);
  MKA_CHECK(!rt.l2() || ptrs_ok({l2}), MKA_ERR_INVALID);
  MKA_CHECK(!rt.l3() || ptrs_ok({idx}), MKA_ERR_INVALID);
  MKA_CHECK(pos0 >= 0 && nb_cap >= 0 && pos0 + d->seq <= t_cap, MKA_ERR_INVALID);
  if (rt.l3() && (pos0 + d->seq - 1) / d->block > 0)
    MKA_CHECK(ptrs_ok({block_means}), MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({ws}), MKA_ERR_WORKSPACE);
  MKA_CHECK(ws_bytes >= fuse_ws(d), MKA_ERR_WORKSPACE);
  return do_fuse_kv(d, x, l2, block_means, nb_cap, idx, lambda, w_k, w_v, k_cache, v_cache, pos0,
                    contiguous(d, t_cap), ws, static_cast<hipStream_t>(stream));
}

int mka_attn_prefill(const mka_dims* d, const void* q, const void* k_cache, const void* v_cache,
                     int64_t t_cap, int64_t pos0, void* o, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(ptrs_ok({q, k_cache, v_cache, o}), MKA_ERR_INVALID);
  MKA_CHECK(pos0 >= 0 && pos0 + d->seq <= t_cap, MKA_ERR_INVALID);
  return do_attn_prefill(d, q, k_cache, v_cache, contiguous(d, t_cap), pos0, o,
                         static_cast<hipStream_t>(stream));
}

int mka_attn_decode(const mka_dims* d, const void* q, const void* k_cache, const void* v_cache,
                    int64_t t_cap, int64_t cache_len, void* o, void* ws, size_t ws_bytes,
                    void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(d->seq == 1, MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({q, k_cache, v_cache, o}), MKA_ERR_INVALID);
  MKA_CHECK(cache_len >= 1 && cache_len <= t_cap, MKA_ERR_INVALID);
  MKA_CHECK(cache_len <= kMaxDecodeCache && decode_chunk_fits(d, cache_len - 1),
            MKA_ERR_UNSUPPORTED);
  if (decode_ws(d, cache_len) > 0) {
    MKA_CHECK(ptrs_ok({ws}), MKA_ERR_WORKSPACE);
    MKA_CHECK(ws_bytes >= decode_ws(d, cache_len), MKA_ERR_WORKSPACE);
  }
  return do_attn_decode(d, q, k_cache, v_cache, contiguous(d, t_cap), cache_len, o, ws,
                        static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Allocation-free decode attention: the split partials live in a file-scope
// device array (one copy per GPU, held until the process ends) instead of a
// caller's workspace.  Host code never passes the array's name to a kernel:
// the name is a host-side stand-in.  Its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static void* scratch_for_current_device(int* rc) {
  static std::mutex lock;
  static std::unordered_map<int, void*> table;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *rc = hip_fail("attn_decode_noalloc/device", e);
    return nullptr;
  }
  std::lock_guard<std::mutex> g(lock);
  auto it = table.find(dev);
  if (it != table.end()) return it->second;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr) {
    *rc = hip_fail("attn_decode_noalloc/scratch", e != hipSuccess ? e : hipErrorInvalidSymbol);
    return nullptr;
  }
  table.emplace(dev, ptr);
  return ptr;
}

int mka_attn_decode_noalloc(const mka_dims* d, const void* q, const void* k_cache,
                            const void* v_cache, int64_t t_cap, int64_t cache_len, void* o,
                            void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(d->seq == 1, MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({q, k_cache, v_cache, o}), MKA_ERR_INVALID);
  MKA_CHECK(cache_len >= 1 && cache_len <= t_cap, MKA_ERR_INVALID);
  MKA_CHECK(cache_len <= kMaxDecodeCache && decode_chunk_fits(d, cache_len - 1),
            MKA_ERR_UNSUPPORTED);
  const size_t need = decode_ws(d, cache_len);
  if (need > kNoAllocScratchBytes) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "attn_decode_noalloc: the split partials need %zu bytes; the library's device "
                  "scratch holds %zu",
                  need, kNoAllocScratchBytes);
    return MKA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_for_current_device(&rc);
    if (ws == nullptr) return rc;
  }
  return do_attn_decode(d, q, k_cache, v_cache, contiguous(d, t_cap), cache_len, o, ws,
                        static_cast<hipStream_t>(stream));
}

size_t mka_attn_decode_noalloc_limit(void) { return kNoAllocScratchBytes; }

static int check_layer_args(const mka_dims* d, const void* x, int64_t pos0, const mka_weights* w,
                            const mka_state* st, const mka_outputs* out) {
  MKA_CHECK(w != nullptr && st != nullptr && out != nullptr, MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({x, w->w_q, w->w_k, w->w_v, w->w_r1, w->w_r2, w->proj}), MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({st->ema_state, st->block_acc, st->block_means, st->block_kv, st->k_cache,
                     st->v_cache}),
            MKA_ERR_INVALID);
  MKA_CHECK(st->block_hash != nullptr && (reinterpret_cast<uintptr_t>(st->block_hash) & 7u) == 0,
            MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({out->q, out->lambda, out->l2, out->key, out->idx, out->o}), MKA_ERR_INVALID);
  MKA_CHECK(pos0 >= 0 && st->nb_cap >= 1 && st->nb_cap < 0xFFFFFF, MKA_ERR_INVALID);
  MKA_CHECK(pos0 + d->seq <= st->t_cap, MKA_ERR_INVALID);
  MKA_CHECK((pos0 + d->seq) / d->block <= st->nb_cap, MKA_ERR_INVALID);
  if (st->page_table != nullptr) {
    MKA_CHECK((reinterpret_cast<uintptr_t>(st->page_table) & 3u) == 0, MKA_ERR_INVALID);
    MKA_CHECK(st->page_size >= 64 && st->page_size <= (1 << 20) &&
                  (st->page_size & (st->page_size - 1)) == 0 && st->pages_per_seq >= 1,
              MKA_ERR_INVALID);
    MKA_CHECK(static_cast<int64_t>(st->pages_per_seq) * st->page_size == st->t_cap,
              MKA_ERR_INVALID);
  }
  return MKA_OK;
}

int mka_prefill(const mka_dims* d, const void* x, int64_t pos0, const mka_weights* w,
                const mka_state* st, const mka_outputs* out, void* ws, size_t ws_bytes,
                void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_layer_args(d, x, pos0, w, st, out);
  if (rc) return rc;
  const size_t need = mka_workspace_bytes(d, MKA_OP_PREFILL, 0);
  MKA_CHECK(ws_bytes >= need, MKA_ERR_WORKSPACE);
  MKA_CHECK(need == 0 || ptrs_ok({ws}), MKA_ERR_WORKSPACE);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Routing rt = routing_of(d);
  int64_t first, n;
  completed_blocks(d, pos0, &first, &n);
  if (!rt.l3()) n = 0;  // no block codes or projections without L3
  char* ws_chain = static_cast<char*>(ws);
  char* ws_main = ws_chain + prefill_chain_ws(d);
  char* ws_prep = ws_main + prefill_main_ws(d);
  const bool prep = prefill_prepares_codes(d);
  // The hyperplane split of the key codes, the EMA scan, the block codes and
  // the retrieval need only the weights and x, so they run on the auxiliary
  // stream beside the query product (register-lean, so the scan's waves share
  // its SIMDs) and the router; the main stream joins them before the fusion.
  Aux* aux = aux_for_current_device(&rc);
  if (aux == nullptr) return rc;
  std::lock_guard<std::mutex> guard(aux->lock);
  hipStream_t s2 = aux->stream;
  MKA_LAUNCH("prefill/fork", hipEventRecord(aux->fork, s));
  MKA_LAUNCH("prefill/fork", hipStreamWaitEvent(s2, aux->fork, 0));
  if (prep)
    MKA_LAUNCH("prefill/prep", simhash_prepare(w->proj, d->hash_bits, d->d_model, ws_prep, s2));
  if (rt.ema() && (rc = do_ema(d, x, pos0, st->ema_state, st->block_acc, out->l2,
                               st->block_means, st->nb_cap, ws_chain, s2)))
    return rc;
  if ((rc = do_index(d, st->block_means, st->nb_cap, static_cast<int>(first), static_cast<int>(n),
                     w->proj, st->block_hash, ws_chain, s2)))
    return rc;
  if (prep) {
    MKA_LAUNCH("l3_retrieve/keys",
               simhash_rows_prepared(out->l2, static_cast<int64_t>(d->seq) * d->d_model, d->seq,
                                     d->batch, d->d_model, w->proj, d->hash_bits, ws_prep,
                                     out->key, d->seq, s2));
    MKA_LAUNCH("l3_retrieve/topr", topr_rows(out->key, d->batch, d->seq, pos0, st->block_hash,
                                             st->nb_cap, d->block, d->top_r, out->idx, s2));
  }
  MKA_LAUNCH("prefill/join", hipEventRecord(aux->join, s2));
  // The block projections serve later decode steps only: they run after the
  // join, beside the fusion and the attention, and the caller's stream waits
  // for them at the end.
  if ((rc = do_block_kv(d, st->block_means, st->nb_cap, static_cast<int>(first),
                        static_cast<int>(n), w->w_k, w->w_v, st->block_kv, s2)))
    return rc;
  MKA_LAUNCH("prefill/join", hipEventRecord(aux->done, s2));
  if ((rc = do_route(d, x, w->w_q, w->w_r1, w->w_r2, out->q, out->lambda, ws_main, s))) return rc;
  MKA_LAUNCH("prefill/join", hipStreamWaitEvent(s, aux->join, 0));
  if (!prep && rt.l3() && (rc = do_retrieve(d, out->l2, w->proj, st->block_hash, st->nb_cap, pos0,
                                            out->key, out->idx, ws_main, s)))
    return rc;
  if ((rc = do_fuse_kv(d, x, out->l2, st->block_means, st->nb_cap, out->idx, out->lambda, w->w_k,
                       w->w_v, st->k_cache, st->v_cache, pos0, layout_of(d, st), ws_main, s)))
    return rc;
  if ((rc = do_attn_prefill(d, out->q, st->k_cache, st->v_cache, layout_of(d, st), pos0, out->o,
                            s, out->lse)))
    return rc;
  MKA_LAUNCH("prefill/join", hipStreamWaitEvent(s, aux->done, 0));
  return MKA_OK;
}

int mka_decode_step(const mka_dims* d, const void* x, int64_t pos, const mka_weights* w,
                    const mka_state* st, const mka_outputs* out, void* ws, size_t ws_bytes,
                    void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(d->seq == 1, MKA_ERR_INVALID);
  rc = check_layer_args(d, x, pos, w, st, out);
  if (rc) return rc;
  MKA_CHECK(pos + 1 <= kMaxDecodeCache && decode_chunk_fits(d, pos), MKA_ERR_UNSUPPORTED);
  const size_t need = mka_workspace_bytes(d, MKA_OP_DECODE_STEP, pos + 1);
  MKA_CHECK(ws_bytes >= need, MKA_ERR_WORKSPACE);
  MKA_CHECK(need == 0 || ptrs_ok({ws}), MKA_ERR_WORKSPACE);
  MKA_CHECK(d->batch <= kFewRowsDec, MKA_ERR_UNSUPPORTED);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DecodeWs L = decode_layout(d, pos + 1);
  char* base = static_cast<char*>(ws);
  float* w_attn = reinterpret_cast<float*>(base);
  float* w_hid = reinterpret_cast<float*>(base + L.attn);
  double* w_part = reinterpret_cast<double*>(base + L.attn + L.hid);
  float* w_kv = reinterpret_cast<float*>(base + L.attn + L.hid + L.part);
  void* w_xf = base + L.attn + L.hid + L.part + L.kv;
  void* w_index = base + L.attn + L.hid + L.part + L.kv + L.xf;
  const int B = d->batch, D = d->d_model, H = d->n_heads, G = d->n_kv_heads, dh = d->head_dim;
  const int qw = H * dh, kvw = G * dh;
  const Routing rt = routing_of(d);
  const bool closes = rt.l3() && (pos + 1) % d->block == 0;
  const int closed_block = static_cast<int>((pos + 1) / d->block - 1);

  auto fill = [&](auto* tag) {
    using T = std::remove_pointer_t<decltype(tag)>;
    DecodeArgs<T> a{};
    a.x = static_cast<const T*>(x);
    a.w_q = static_cast<const T*>(w->w_q);
    a.q = static_cast<T*>(out->q);
    a.D = D;
    a.qw = qw;
    a.B = B;
    a.state = st->ema_state;
    a.acc = st->block_acc;
    a.l2 = out->l2;
    a.means = st->block_means;
    a.nb_cap = st->nb_cap;
    a.pos = pos;
    a.block = d->block;
    a.beta = d->ema_decay;
    a.omb = 1.0f - d->ema_decay;
    a.proj = w->proj;
    a.nbits = d->hash_bits;
    a.n_slices = decode_slices(D);
    a.part = w_part;
    a.w_r1 = static_cast<const T*>(w->w_r1);
    a.w_r2 = static_cast<const T*>(w->w_r2);
    a.r = d->router_hidden;
    a.hidden = w_hid;
    a.lam = out->lambda;
    a.bhash = st->block_hash;
    a.key = out->key;
    a.idx = out->idx;
    a.R = d->top_r;
    a.xf = static_cast<T*>(w_xf);
    a.w_k = static_cast<const T*>(w->w_k);
    a.w_v = static_cast<const T*>(w->w_v);
    a.kvw = kvw;
    a.kvx = w_kv;
    a.kvl2 = w_kv + static_cast<size_t>(B) * 2 * kvw;
    a.kvl3 = w_kv + static_cast<size_t>(2) * B * 2 * kvw;
    a.block_kv = st->block_kv;
    a.k_cache = static_cast<T*>(st->k_cache);
    a.v_cache = static_cast<T*>(st->v_cache);
    a.H = H;
    a.G = G;
    a.dh = dh;
    a.kv = layout_of(d, st);
    a.sl2 = 1.4426950408889634f / sqrtf(static_cast<float>(dh));
    a.n_hb = (H / G + kSplitHeads - 1) / kSplitHeads;
    a.n_chunks = pos > 0 ? decode_n_chunks(B * G * a.n_hb, pos) : 0;
    const size_t np = static_cast<size_t>(B) * H * a.n_chunks;
    a.part_m = w_attn;
    a.part_l = w_attn + np;
    a.part_o = w_attn + 2 * np;
    a.o = static_cast<T*>(out->o);
    a.rt = rt;
    return a;
  };

  if (d->dtype != MKA_BF16) {  // fp32 layers: the sequential kernels in order
    const DecodeArgs<float> a = fill(static_cast<float*>(nullptr));
    MKA_LAUNCH("decode/front", decode_front<float>(a, s));
    MKA_LAUNCH("decode/mid", decode_mid<float>(a, s));
    MKA_LAUNCH("decode/fuse", decode_fuse<float>(a, s));
    const EpiKV<float> epi{static_cast<float*>(st->k_cache), static_cast<float*>(st->v_cache), 1,
                           G, dh, layout_of(d, st), pos};
    MKA_LAUNCH("decode/kv", gemv<float>(a.xf, D, B, static_cast<const float*>(w->w_k),
                                        static_cast<const float*>(w->w_v), kvw, 2 * kvw, D, epi, s));
    if ((rc = do_attn_decode(d, out->q, st->k_cache, st->v_cache, layout_of(d, st), pos + 1, out->o,
                             nullptr, s)))
      return rc;
  } else {
    // bf16: inputs (Q, [x; L2] W, EMA, key partials) -> attention over rows
    // [0, pos) with the router, top-R and L3 W beside it -> merge with the
    // new row, which is formed (lambda applied), cached and scored there.
    const DecodeArgs<bf16_t> a = fill(static_cast<bf16_t*>(nullptr));
    MKA_LAUNCH("decode/inputs", decode_inputs_bf16(a, s));
    MKA_LAUNCH("decode/attend", decode_attend_bf16(a, s));
    MKA_LAUNCH("decode/merge", decode_merge_bf16(a, s));
  }
  if (closes) {  // the block this token closes joins the L3 bank for the next tokens
    if ((rc = do_index(d, st->block_means, st->nb_cap, closed_block, 1, w->proj, st->block_hash,
                       w_index, s)))
      return rc;
    return do_block_kv(d, st->block_means, st->nb_cap, closed_block, 1, w->w_k, w->w_v,
                       st->block_kv, s);
  }
  return MKA_OK;
}

int mka_full_prefill(const mka_dims* d, const void* x, int64_t pos0, const mka_weights* w,
                     const mka_state* st, const mka_tier_cache* kv, const mka_outputs* out,
                     void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_full_args(d, x, pos0, w, st, kv, out);
  if (rc) return rc;
  const FullWs L = full_layout(d, false, 0);
  MKA_CHECK(ws_bytes >= L.total && ptrs_ok({ws}), MKA_ERR_WORKSPACE);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Routing rt = routing_of(d);
  int64_t first, n;
  completed_blocks(d, pos0, &first, &n);
  if (!rt.l3()) n = 0;
  char* base = static_cast<char*>(ws);
  char* ws_chain = base;
  char* ws_main = base + L.chain;
  void* rows = base + L.chain + L.main;
  char* paths = base + L.chain + L.main + L.rows;
  // The scan and block codes run beside the query product, as in mka_prefill.
  Aux* aux = aux_for_current_device(&rc);
  if (aux == nullptr) return rc;
  std::lock_guard<std::mutex> guard(aux->lock);
  hipStream_t s2 = aux->stream;
  MKA_LAUNCH("full/fork", hipEventRecord(aux->fork, s));
  MKA_LAUNCH("full/fork", hipStreamWaitEvent(s2, aux->fork, 0));
  if (rt.ema() && (rc = do_ema(d, x, pos0, st->ema_state, st->block_acc, out->l2,
                               st->block_means, st->nb_cap, ws_chain, s2)))
    return rc;
  if ((rc = do_index(d, st->block_means, st->nb_cap, static_cast<int>(first), static_cast<int>(n),
                     w->proj, st->block_hash, ws_chain, s2)))
    return rc;
  MKA_LAUNCH("full/join", hipEventRecord(aux->join, s2));
  if ((rc = do_route(d, x, w->w_q, w->w_r1, w->w_r2, out->q, out->lambda, ws_main, s))) return rc;
  MKA_LAUNCH("full/join", hipStreamWaitEvent(s, aux->join, 0));
  if (rt.l3() && (rc = do_retrieve(d, out->l2, w->proj, st->block_hash, st->nb_cap, pos0,
                                   out->key, out->idx, ws_main, s)))
    return rc;
  const bool on[3] = {true, rt.l2(), rt.l3()};
  const KvLayout tiers_kv = contiguous(d, st->t_cap);
  void* a[3] = {nullptr, nullptr, nullptr};
  for (int l = 0; l < 3; ++l) {
    if (!on[l]) continue;
    const void* src = tier_source(d, l, x, out->l2, st->block_means, st->nb_cap, out->idx, rows,
                                  s, &rc);
    if (rc) return rc;
    if ((rc = do_kv_proj(d, src, w->w_k, w->w_v, kv->k_cache[l], kv->v_cache[l], pos0, tiers_kv,
                         s)))
      return rc;
    a[l] = paths + l * L.path;
    if ((rc = do_attn_prefill(d, out->q, kv->k_cache[l], kv->v_cache[l], tiers_kv, pos0, a[l],
                              s)))
      return rc;
  }
  return do_mix(d, a, out->lambda, out->o, s);
}

int mka_full_decode_step(const mka_dims* d, const void* x, int64_t pos, const mka_weights* w,
                         const mka_state* st, const mka_tier_cache* kv, const mka_outputs* out,
                         void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(d->seq == 1, MKA_ERR_INVALID);
  rc = check_full_args(d, x, pos, w, st, kv, out);
  if (rc) return rc;
  MKA_CHECK(pos + 1 <= kMaxDecodeCache && decode_chunk_fits(d, pos), MKA_ERR_UNSUPPORTED);
  MKA_CHECK(rows_of(d) <= kFewRows, MKA_ERR_UNSUPPORTED);
  const FullWs L = full_layout(d, true, pos + 1);
  MKA_CHECK(ws_bytes >= L.total && ptrs_ok({ws}), MKA_ERR_WORKSPACE);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Routing rt = routing_of(d);
  char* base = static_cast<char*>(ws);
  void* shared = base;
  void* rows = base + L.main;
  char* paths = base + L.main + L.rows;
  if ((rc = do_route(d, x, w->w_q, w->w_r1, w->w_r2, out->q, out->lambda, shared, s))) return rc;
  if (rt.ema() && (rc = do_ema(d, x, pos, st->ema_state, st->block_acc, out->l2, st->block_means,
                               st->nb_cap, shared, s)))
    return rc;
  if (rt.l3() && (rc = do_retrieve(d, out->l2, w->proj, st->block_hash, st->nb_cap, pos,
                                   out->key, out->idx, shared, s)))
    return rc;
  const bool on[3] = {true, rt.l2(), rt.l3()};
  const KvLayout tiers_kv = contiguous(d, st->t_cap);
  void* a[3] = {nullptr, nullptr, nullptr};
  for (int l = 0; l < 3; ++l) {
    if (!on[l]) continue;
    const void* src = tier_source(d, l, x, out->l2, st->block_means, st->nb_cap, out->idx, rows,
                                  s, &rc);
    if (rc) return rc;
    if ((rc = do_kv_proj(d, src, w->w_k, w->w_v, kv->k_cache[l], kv->v_cache[l], pos, tiers_kv,
                         s)))
      return rc;
    a[l] = paths + l * L.path;
    if ((rc = do_attn_decode(d, out->q, kv->k_cache[l], kv->v_cache[l], tiers_kv, pos + 1, a[l],
                             shared, s)))
      return rc;
  }
  if ((rc = do_mix(d, a, out->lambda, out->o, s))) return rc;
  if (rt.l3() && (pos + 1) % d->block == 0)  // the closed block joins the bank
    return do_index(d, st->block_means, st->nb_cap, static_cast<int>((pos + 1) / d->block - 1), 1,
                    w->proj, st->block_hash, shared, s);
  return MKA_OK;
}

int mka_backward(const mka_dims* d, const void* x, const mka_weights* w, const mka_state* st,
                 const mka_outputs* fwd, const void* d_o, const mka_grads* g, void* ws,
                 size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(w != nullptr && st != nullptr && fwd != nullptr && g != nullptr, MKA_ERR_INVALID);
  const Routing rt = routing_of(d);
  MKA_CHECK(ptrs_ok({x, d_o, w->w_q, w->w_k, w->w_v, w->w_r1, w->w_r2}), MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({fwd->q, fwd->lambda, fwd->o, fwd->lse, st->k_cache, st->v_cache}),
            MKA_ERR_INVALID);
  MKA_CHECK(!rt.ema() || ptrs_ok({fwd->l2}), MKA_ERR_INVALID);
  MKA_CHECK(!rt.l3() || ptrs_ok({fwd->idx, st->block_means}), MKA_ERR_INVALID);
  MKA_CHECK(ptrs_ok({g->dx, g->dw_q, g->dw_k, g->dw_v, g->dw_r1, g->dw_r2}), MKA_ERR_INVALID);
  MKA_CHECK(d->seq <= st->t_cap && st->nb_cap >= 1 && d->seq / d->block <= st->nb_cap,
            MKA_ERR_INVALID);
  MKA_CHECK(st->page_table == nullptr, MKA_ERR_UNSUPPORTED);
  MKA_CHECK(d->dtype != MKA_BF16 || d->router_hidden % 32 == 0, MKA_ERR_UNSUPPORTED);
  const BwdWs L = bwd_layout(d);
  MKA_CHECK(ws_bytes >= L.total && ptrs_ok({ws}), MKA_ERR_WORKSPACE);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  if (d->dtype == MKA_BF16) return backward_body<bf16_t>(d, x, w, st, fwd, d_o, g, base, s);
  return backward_body<float>(d, x, w, st, fwd, d_o, g, base, s);
}

int mka_attn_backward(const mka_dims* d, const void* q, const void* k_cache, const void* v_cache,
                      int64_t t_cap, const void* o, const float* lse, const void* d_o, float* dq,
                      float* dkv, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  MKA_CHECK(ptrs_ok({q, k_cache, v_cache, o, lse, d_o, dq, dkv}), MKA_ERR_INVALID);
  MKA_CHECK(d->seq <= t_cap, MKA_ERR_INVALID);
  const size_t need = attn_bwd_ws(d);
  MKA_CHECK(ws_bytes >= need && ptrs_ok({ws}), MKA_ERR_WORKSPACE);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* dsum = reinterpret_cast<float*>(base);
  float* heads = reinterpret_cast<float*>(base + round256(sizeof(float) * rows_of(d) * d->n_heads));
  if (d->dtype == MKA_BF16) {
    // dq on the auxiliary stream beside the dK/dV passes, joined before returning
    Aux* aux = aux_for_current_device(&rc);
    if (aux == nullptr) return rc;
    std::lock_guard<std::mutex> guard(aux->lock);
    rc = attn_backward_steps<bf16_t>(d, static_cast<const bf16_t*>(q),
                                     static_cast<const bf16_t*>(k_cache),
                                     static_cast<const bf16_t*>(v_cache), t_cap,
                                     static_cast<const bf16_t*>(o), lse,
                                     static_cast<const bf16_t*>(d_o), dq, dkv, dsum, heads, s, aux);
    if (rc) return rc;
    MKA_LAUNCH("attn_bwd/join", hipEventRecord(aux->join, aux->stream));
    MKA_LAUNCH("attn_bwd/join", hipStreamWaitEvent(s, aux->join, 0));
    return MKA_OK;
  }
  return attn_backward_steps<float>(d, static_cast<const float*>(q),
                                    static_cast<const float*>(k_cache),
                                    static_cast<const float*>(v_cache), t_cap,
                                    static_cast<const float*>(o), lse,
                                    static_cast<const float*>(d_o), dq, dkv, dsum, heads, s,
                                    nullptr);
}

}  // extern "C"
