/*
 * mka.h -- C ABI of the FastMKA (route-fused memory-keyed attention) layer
 * forward on MI355X (gfx950).
 *
 * Sources: the Paper-Notes reading note "MKA: Memory-Keyed Attention for
 * Efficient Long-Context Reasoning" (method sections 1-4) and the paper's
 * landing page of the same title (abstract; Tables 4, 5, 11).  Per token a
 * router gives lambda = softmax(MLP(q)) over three memory tiers: L1, the
 * token's own hidden; L2, an exponential moving average of the prefix; L3,
 * the mean of the R past block means whose SimHash codes are nearest (in
 * Hamming distance) to the SimHash of L2[t].  The tiers are fused,
 * X_fused = sum_l lambda_l * L_l; K and V are projected from X_fused
 * (grouped-query heads) and one causal attention runs over them.  Decode
 * caches the fused K/V.
 *
 * Conventions for every call
 *  - Pointers are device pointers unless stated; ``stream`` is a hipStream_t
 *    (NULL = the default stream).  Every call is asynchronous on ``stream``.
 *  - The caller allocates and owns every buffer (inputs, outputs, state,
 *    workspace).  The library allocates no device memory and keeps no pointer
 *    after a call returns.  Its only state is a thread-local string describing
 *    the last HIP error and, per device, one auxiliary stream with three events
 *    that mka_prefill creates on its first call there and keeps until the
 *    process ends.  Calls on different streams are independent; calls that
 *    write the same buffers must be ordered by the caller.
 *  - Arrays are dense, row-major, contiguous.  Token-major activations are
 *    [B, seq, width]; the fused KV cache is head-major [B, G, t_cap, dh].
 *    Weight matrices are stored [out, in] (each output's weights contiguous).
 *  - Storage type ``dtype`` (mka_dims) applies to x, q, o, the weights and
 *    the KV cache.  lambda, L2, EMA state, block sums and means and the
 *    SimHash hyperplanes are always float32; codes are uint64 (low
 *    hash_bits bits used); block indices are int32.
 *  - Return value: MKA_OK (0) or a negative MKA_ERR_* code.  Arguments are
 *    validated before anything is launched: on an error nothing has been
 *    enqueued.  Faults during execution surface at the caller's next
 *    synchronisation of ``stream``.
 */
#ifndef MKA_H
#define MKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MKA_F32 = 0, MKA_BF16 = 1 };

enum {
  MKA_OK = 0,
  MKA_ERR_INVALID = -1,     /* null pointer, inconsistent or out-of-range sizes */
  MKA_ERR_UNSUPPORTED = -2, /* valid but not implemented: head_dim, dtype, alignment */
  MKA_ERR_WORKSPACE = -3,   /* workspace smaller than mka_workspace_bytes() */
  MKA_ERR_HIP = -4          /* a HIP call failed; see mka_last_error() */
};

/* Workspace-using operations, for mka_workspace_bytes(). */
enum { MKA_OP_EMA_SCAN = 0, MKA_OP_FUSE_KV = 1, MKA_OP_ATTN_DECODE = 2, MKA_OP_PREFILL = 3,
       MKA_OP_DECODE_STEP = 4, MKA_OP_RETRIEVE = 5, MKA_OP_INDEX = 6, MKA_OP_ROUTE = 7,
       MKA_OP_FULL_PREFILL = 8, MKA_OP_FULL_DECODE_STEP = 9, MKA_OP_BACKWARD = 10,
       MKA_OP_ATTN_BACKWARD = 11 };

/* Routing variant (mka_dims.route_mode) and enabled tiers (mka_dims.tiers):
 * the ablations of the abstract page, Table 10 (fixed lambda = 1/3, hard
 * top-2 and top-1 routing against the learned soft router) and Table 9
 * (L1+L2, L1+L3, L1 alone = plain multi-head attention).  From the router
 * logits z = GELU(q W_r1) W_r2:
 *   MKA_ROUTE_SOFT   softmax of z over the enabled tiers (with all three
 *                    tiers: the learned router of the reading note, method
 *                    section 2);
 *   MKA_ROUTE_FIXED  1 / (number of enabled tiers) on each, the router unused;
 *   MKA_ROUTE_TOP1/2 the 1 or 2 enabled tiers with the largest logits (ties
 *                    to the lower tier index) and a softmax over those alone:
 *                    top-1 is one-hot; the others get lambda = 0.
 * A disabled tier always has lambda = 0 and its steps do not run: without L3
 * no block codes, block projections or retrieval; with L1 alone also no EMA
 * and no router.  Zero-initialised fields give the full method. */
enum { MKA_ROUTE_SOFT = 0, MKA_ROUTE_FIXED = 1, MKA_ROUTE_TOP1 = 2, MKA_ROUTE_TOP2 = 3 };
enum { MKA_TIERS_ALL = 0, MKA_TIERS_L1_L2 = 1, MKA_TIERS_L1_L3 = 2, MKA_TIERS_L1 = 3 };

/* Shape of one layer call.
 *   batch B >= 1; seq = tokens in this call (1 for a decode step) >= 1;
 *   d_model D; n_heads H and n_kv_heads G with H % G == 0 (query head h uses
 *   KV head h / (H/G)); head_dim dh in {64, 128}; the query width H*dh;
 *   router_hidden r; block = block size Bs of the L3 bank; hash_bits in
 *   [1, 64]; top_r = R >= 1; ema_decay beta in [0, 1); dtype MKA_F32 or
 *   MKA_BF16.  bf16 calls need D % 64 == 0 and H*dh % 64 == 0; fp32 calls need
 *   D % 4 == 0 and H*dh % 4 == 0 (MKA_ERR_UNSUPPORTED otherwise).  top_r <= 32,
 *   router_hidden <= 256, H/G <= 32. */
typedef struct mka_dims {
  int32_t batch;
  int32_t seq;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t router_hidden;
  int32_t block;
  int32_t hash_bits;
  int32_t top_r;
  float ema_decay;
  int32_t dtype;
  int32_t route_mode; /* MKA_ROUTE_* (0 = the learned soft router) */
  int32_t tiers;      /* MKA_TIERS_* (0 = L1, L2 and L3) */
} mka_dims;

/* Router: Q = X W_q and lambda = softmax(GELU(Q W_r1) W_r2).
 * (Reading note, method section 2: lambda = softmax(MLP(q)) in R^{B x S x 3},
 * per token; q is the query projection of the token hidden.)
 *   x       [B, seq, D]            dtype
 *   w_q     [H*dh, D]              dtype
 *   w_r1    [r, H*dh]              dtype
 *   w_r2    [3, r]                 dtype
 *   q_out   [B, seq, H, dh]        dtype (written)
 *   lambda_out [B, seq, 3]         float32 (written; tier 0 = L1, 1 = L2, 2 = L3)
 *   ws      >= mka_workspace_bytes(d, MKA_OP_ROUTE, 0) bytes (may be NULL if 0) */
int mka_route(const mka_dims* d, const void* x, const void* w_q, const void* w_r1,
              const void* w_r2, void* q_out, float* lambda_out, void* ws, size_t ws_bytes,
              void* stream);

/* L2 session summary and block means for tokens at positions pos0 .. pos0+seq-1.
 * (Reading note, method section 1: the L2 tier is a causal summary of the
 * prefix, here the EMA s_t = beta*s_{t-1} + (1-beta)*x_t, prefix inclusive of
 * t, s_{-1} = 0; the L3 bank holds past blocks.)
 *   x            [B, seq, D]   dtype
 *   state_io     [B, D]        in: s_{pos0-1} (not read when pos0 == 0: the prefix is
 *                              empty); out: s_{pos0+seq-1}
 *   block_acc_io [B, D]        in: sum of x over the tokens of pos0's block before pos0 (not
 *                              read when pos0 % block == 0); out: the same sum for the block
 *                              after the last token
 *   l2_out       [B, seq, D]   float32 (written)
 *   block_means  [B, nb_cap, D] float32: row b = mean of x over block b is written
 *                              for every block whose last token is in this call
 *   ws           >= mka_workspace_bytes(d, MKA_OP_EMA_SCAN, 0) bytes (may be NULL if 0)
 * Requires the last completed block index < nb_cap. */
int mka_ema_scan(const mka_dims* d, const void* x, int64_t pos0, float* state_io,
                 float* block_acc_io, float* l2_out, float* block_means, int32_t nb_cap,
                 void* ws, size_t ws_bytes, void* stream);

/* SimHash codes of block means first_block .. first_block+n_blocks-1.
 * (Reading note, method section 1: vectorised hash index of past blocks.)
 * bit j of a code = [m . proj_j > 0], the sign of the exact product of the
 * float32 inputs: accumulated in float64 (fp64 MFMA; split over D, partial
 * sums added in a fixed order, so results are deterministic), or, for
 * B * n_blocks >= 256 rows and D a multiple of 32, from bf16 parts of both
 * operands on bf16 MFMA with an error bound that certifies each sign, the
 * bits it leaves undecided recomputed in float64 (the same codes).
 *   block_means [B, nb_cap, D] float32; proj [hash_bits, D] float32 (row j = hyperplane j)
 *   block_hash  [B, nb_cap]    uint64 (rows written)
 *   ws >= mka_workspace_bytes(d, MKA_OP_INDEX, n_blocks) bytes (may be NULL if 0) */
int mka_l3_index(const mka_dims* d, const float* block_means, int32_t nb_cap,
                 int32_t first_block, int32_t n_blocks, const float* proj,
                 uint64_t* block_hash, void* ws, size_t ws_bytes, void* stream);

/* Projected block means: block_kv[b, blk, :] = block_means[b, blk, :] [W_k; W_v]^T
 * (float32; the first G*dh entries are the K projection, the rest the V projection)
 * for blocks first_block .. first_block+n_blocks-1.  The decode step forms the L3
 * part of the new K/V row as the mean of the retrieved blocks' rows (reading note,
 * method section 3: K and V are linear in X_fused, whose L3 term is a mean of
 * block means).
 *   block_means [B, nb_cap, D] f32;  w_k, w_v [G*dh, D] dtype
 *   block_kv    [B, nb_cap, 2*G*dh] f32 (rows written)
 * Requires first_block + n_blocks <= nb_cap. */
int mka_l3_block_kv(const mka_dims* d, const float* block_means, int32_t nb_cap,
                    int32_t first_block, int32_t n_blocks, const void* w_k, const void* w_v,
                    float* block_kv, void* stream);

/* L3 retrieval for tokens at positions pos0 .. pos0+seq-1.
 * (Reading note, method section 1: recall of R << T past blocks; landing page,
 * Table 8 caption: top-R retrieved chunks per query.)
 * key_t = SimHash(L2[t]) (exact signs, as in mka_l3_index); eligible
 * blocks b < floor(t / block); ranked by (popcount(key_t ^ hash_b) ascending,
 * b descending); the first min(R, #eligible) are written in rank order, the
 * remaining slots hold -1.  top_r <= 32.
 *   l2       [B, seq, D] float32;   proj [hash_bits, D] float32
 *   block_hash [B, nb_cap] uint64, valid for every eligible block
 *   key_out  [B, seq] uint64 (written);  idx_out [B, seq, R] int32 (written)
 *   ws >= mka_workspace_bytes(d, MKA_OP_RETRIEVE, 0) bytes
 * Requires floor((pos0+seq-1)/block) <= nb_cap. */
int mka_l3_retrieve(const mka_dims* d, const float* l2, const float* proj,
                    const uint64_t* block_hash, int32_t nb_cap, int64_t pos0,
                    uint64_t* key_out, int32_t* idx_out, void* ws, size_t ws_bytes,
                    void* stream);

/* Route fusion and K/V projection into the fused KV cache.
 * (Reading note, method section 3: X_fused = sum_l lambda_l * L_l, K = X_fused W_k,
 * V = X_fused W_v, the fused K/V is what the cache holds; landing page, abstract:
 * lambda is broadcast over the hidden dimension.)
 * L3[t] = mean of block_means rows idx[t, :] that are >= 0 (zero if none).
 * X_fused is formed in float32 and rounded once to dtype before the projection.
 *   x [B, seq, D] dtype; l2 [B, seq, D] f32; block_means [B, nb_cap, D] f32;
 *   idx [B, seq, R] int32; lambda [B, seq, 3] f32; w_k, w_v [G*dh, D] dtype
 *   k_cache, v_cache [B, G, t_cap, dh] dtype: rows pos0 .. pos0+seq-1 written
 *   ws >= mka_workspace_bytes(d, MKA_OP_FUSE_KV, 0) bytes
 * Inputs of disabled tiers (d->tiers) are not read and may be NULL: l2 without
 * L2; idx and block_means without L3.  With L1 alone X_fused = x.
 * Requires pos0 + seq <= t_cap. */
int mka_fuse_kv_proj(const mka_dims* d, const void* x, const float* l2,
                     const float* block_means, int32_t nb_cap, const int32_t* idx,
                     const float* lambda, const void* w_k, const void* w_v, void* k_cache,
                     void* v_cache, int64_t pos0, int64_t t_cap, void* ws, size_t ws_bytes,
                     void* stream);

/* Causal grouped-query flash attention for queries at positions pos0 .. pos0+seq-1
 * over cache rows 0 .. pos0+seq-1.
 * (Reading note, method sections 3-4: one standard causal attention over the fused
 * K/V, evaluated blockwise with the online max-shift.)
 * O[t,h] = sum_{j<=t} softmax_j(q_{t,h} . k_{j,g(h)} / sqrt(dh)) v_{j,g(h)}.
 *   q [B, seq, H, dh] dtype; k_cache, v_cache [B, G, t_cap, dh] dtype;
 *   o [B, seq, H, dh] dtype (written).  Requires pos0 + seq <= t_cap. */
int mka_attn_prefill(const mka_dims* d, const void* q, const void* k_cache,
                     const void* v_cache, int64_t t_cap, int64_t pos0, void* o, void* stream);

/* Decode attention of one query token per sequence (d->seq must be 1) over cache rows
 * 0 .. cache_len-1, split over the keys with a log-sum-exp merge of the parts.
 * (Landing page, Table 5: decode reads the single fused KV tensor.)
 *   q [B, 1, H, dh] dtype; o [B, 1, H, dh] dtype (written)
 *   ws >= mka_workspace_bytes(d, MKA_OP_ATTN_DECODE, cache_len) bytes */
int mka_attn_decode(const mka_dims* d, const void* q, const void* k_cache,
                    const void* v_cache, int64_t t_cap, int64_t cache_len, void* o,
                    void* ws, size_t ws_bytes, void* stream);

/* mka_attn_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as mka_attn_decode (the same
 * kernels).  The split partials (4*B*H*n_chunks*(dh+2) bytes, n_chunks ~ 256 /
 * (B*G*ceil(H/G/16)); 0.93 MB for one 128K Qwen2.5-7B-shaped sequence) go to a
 * device array of the library, mka_attn_decode_noalloc_limit() = 4 MiB per
 * GPU, held from the first call on a GPU until the process ends.  Larger
 * requests return MKA_ERR_WORKSPACE (mka_last_error() says the sizes) and
 * enqueue nothing.  Every call on one GPU uses that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be ordered
 * by the caller.  The call allocates nothing (no hipMalloc, no library
 * allocation); its first call on a GPU looks up the array's device address. */
int mka_attn_decode_noalloc(const mka_dims* d, const void* q, const void* k_cache,
                            const void* v_cache, int64_t t_cap, int64_t cache_len, void* o,
                            void* stream);
size_t mka_attn_decode_noalloc_limit(void);

/* Composite: the whole layer over a prompt at positions pos0 .. pos0+seq-1 (the
 * calls above: route, ema_scan, l3_index and l3_block_kv of the blocks completed
 * here, l3_retrieve, fuse_kv_proj, attn_prefill).  ema_scan, l3_index and
 * l3_block_kv need only x, so they run on the device's auxiliary stream
 * (forked from ``stream`` and joined back into it with events) beside route;
 * completion is signalled on ``stream`` alone.  Concurrent calls on one device
 * serialise their enqueueing.  Intermediates go to the caller's
 * buffers, so the call both answers the prompt and leaves the decode state.
 *   weights: w_q, w_k, w_v, w_r1, w_r2 (dtype), proj (f32), as above
 *   state: state_io, block_acc_io [B, D] f32; block_means [B, nb_cap, D] f32;
 *          block_hash [B, nb_cap] u64; block_kv [B, nb_cap, 2*G*dh] f32 (rows of the
 *          completed blocks written, as mka_l3_block_kv); k_cache, v_cache [B, G, t_cap, dh]
 *   outputs: q [B,seq,H,dh], lambda [B,seq,3], l2 [B,seq,D], key [B,seq],
 *            idx [B,seq,R], o [B,seq,H,dh]
 *   ws >= mka_workspace_bytes(d, MKA_OP_PREFILL, 0) bytes
 * Routing variants (d->route_mode, d->tiers): q, lambda, o and the KV cache
 * are always written.  Without L3, key, idx, block_hash and block_kv are not
 * written.  With L1 alone, l2 and the EMA state, block sums and block means
 * are not written either.  A session uses one variant for all its calls: the
 * state a variant does not keep is not valid for another. */
typedef struct mka_weights {
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* w_r1;
  const void* w_r2;
  const float* proj;
} mka_weights;

typedef struct mka_state {
  float* ema_state;      /* [B, D] */
  float* block_acc;      /* [B, D] */
  float* block_means;    /* [B, nb_cap, D] */
  uint64_t* block_hash;  /* [B, nb_cap] */
  float* block_kv;       /* [B, nb_cap, 2*G*dh]: row b = block_means[b] [W_k; W_v]^T */
  void* k_cache;         /* [B, G, t_cap, dh], or a page pool (see page_table) */
  void* v_cache;         /* [B, G, t_cap, dh], or a page pool */
  int32_t nb_cap;
  int64_t t_cap;
  /* Paged fused KV cache (abstract page, Table 4 caption: the measurements use a
   * contiguous KV layout up to 32K tokens and a paged one beyond).  NULL: the
   * contiguous layout above.  Otherwise k_cache and v_cache are pools of pages
   * [n_pages, G, page_size, dh] (dtype) and page_table [B, pages_per_seq]
   * (int32, device) maps logical page p of sequence b to a pool page: row t of
   * sequence b is row t % page_size of page page_table[b][t / page_size].
   * page_size is a power of two in [64, 2^20]; t_cap must equal
   * pages_per_seq * page_size.  Entries must be valid pool pages; the pages
   * of rows a call writes must not be shared by other live rows.  Only
   * mka_prefill and mka_decode_step take a paged state (the full-MKA calls
   * return MKA_ERR_UNSUPPORTED for one; the single-step calls take
   * contiguous caches). */
  const int32_t* page_table;
  int32_t page_size;
  int32_t pages_per_seq;
} mka_state;

typedef struct mka_outputs {
  void* q;          /* [B, seq, H, dh] */
  float* lambda;    /* [B, seq, 3] */
  float* l2;        /* [B, seq, D] */
  uint64_t* key;    /* [B, seq] */
  int32_t* idx;     /* [B, seq, R] */
  void* o;          /* [B, seq, H, dh] */
  float* lse;       /* [B, seq, H] or NULL: natural log of the sum over keys of
                       exp(q . k / sqrt(dh)) per query row and head, written by
                       mka_prefill when not NULL (mka_backward reads it) */
} mka_outputs;

int mka_prefill(const mka_dims* d, const void* x, int64_t pos0, const mka_weights* w,
                const mka_state* st, const mka_outputs* out, void* ws, size_t ws_bytes,
                void* stream);

/* Composite: one decode step for the token at position ``pos`` (d->seq must be 1):
 * route, EMA update, retrieval over the blocks before pos's block, fusion and K/V
 * append at row pos, decode attention over rows 0..pos, and -- when pos closes a
 * block ((pos+1) % block == 0) -- the block mean, its code and its projection
 * (mka_l3_block_kv) appended to the bank.  Same buffers as mka_prefill with
 * seq = 1; ws >= mka_workspace_bytes(d, MKA_OP_DECODE_STEP, pos + 1) bytes.
 * bf16 layers form the K/V row by linearity,
 *   [K|V] = lambda1 (x W) + lambda2 (L2 W) + lambda3 mean_b(block_kv[b]),
 * equal to (X_fused W) up to float32 rounding (the row is not rounded through
 * X_fused), so that the products need no lambda and run beside the attention;
 * float32 layers take the steps in order.  Everything runs on ``stream``.
 * Routing variants write and keep what mka_prefill does under them. */
int mka_decode_step(const mka_dims* d, const void* x, int64_t pos, const mka_weights* w,
                    const mka_state* st, const mka_outputs* out, void* ws, size_t ws_bytes,
                    void* stream);

/* Backward of the layer (training): the gradients of a loss L with respect to x
 * and the weights, given dO = dL/dO, for a whole sequence that mka_prefill
 * processed from pos0 = 0 (its outputs, lse included, and state are the saved
 * forward).  The pages give no backward; this is the derivative of the forward
 * by the chain rule.  The SimHash codes, the top-R choice and a hard router's
 * choice of tiers are discrete: no gradient flows through them (the retrieved
 * blocks and kept tiers are constants); proj and ema_decay are fixed.
 *   attention: dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO O)),
 *              dq = dS K / sqrt(dh), dK = dS^T q / sqrt(dh) (summed per KV head);
 *   [K|V] = X_fused [W_k|W_v]^T: dX_fused, dW_k, dW_v;
 *   X_fused = sum lambda_l L_l: dlambda_l = <dX_fused, L_l>; dx gets lambda_1 dX_fused,
 *              the EMA's adjoint of lambda_2 dX_fused (a reverse scan), and
 *              lambda_3 dX_fused / |S_t| scattered to the retrieved blocks'
 *              means, each spread evenly over its block's tokens;
 *   router: the softmax over the kept tiers, GELU', dW_r2, dW_r1, dq;
 *   Q = x W_q^T: dW_q, dx.
 * Arithmetic: float32 accumulation; bf16 layers feed the products bf16
 * operands (the gradients rounded to bf16 where they enter an MFMA product).
 *   x [B, seq, D] dtype; d_o [B, seq, H, dh] dtype
 *   fwd: q, lambda, o, lse, and l2 (unless tiers == MKA_TIERS_L1) and idx
 *        (with L3) as mka_prefill wrote them; st: k_cache, v_cache (contiguous),
 *        block_means (with L3), t_cap, nb_cap
 *   g: float32 gradients, written (not accumulated): dx [B, seq, D], dw_q
 *      [H*dh, D], dw_k and dw_v [G*dh, D], dw_r1 [r, H*dh], dw_r2 [3, r]
 *   ws >= mka_workspace_bytes(d, MKA_OP_BACKWARD, 0) bytes
 * bf16 layers need router_hidden % 32 == 0 (MKA_ERR_UNSUPPORTED otherwise); a
 * paged state is MKA_ERR_UNSUPPORTED. */
/* The attention part of the backward alone (causal GQA over a contiguous
 * cache, rows 0 .. seq-1, pos0 = 0), as mka_backward runs it:
 *   dq [B, seq, H, dh] and dkv [B, seq, 2, G, dh] (K part, then V part) float32
 *   (written), from q, k_cache, v_cache, o and lse of the forward and d_o.
 *   ws >= mka_workspace_bytes(d, MKA_OP_ATTN_BACKWARD, 0) bytes. */
int mka_attn_backward(const mka_dims* d, const void* q, const void* k_cache, const void* v_cache,
                      int64_t t_cap, const void* o, const float* lse, const void* d_o, float* dq,
                      float* dkv, void* ws, size_t ws_bytes, void* stream);

typedef struct mka_grads {
  float* dx;
  float* dw_q;
  float* dw_k;
  float* dw_v;
  float* dw_r1;
  float* dw_r2;
} mka_grads;

int mka_backward(const mka_dims* d, const void* x, const mka_weights* w, const mka_state* st,
                 const mka_outputs* fwd, const void* d_o, const mka_grads* g, void* ws,
                 size_t ws_bytes, void* stream);

/* Full MKA, the three-path form that FastMKA replaces: each memory tier is
 * attended separately and the outputs are mixed, O_h = sum_l lambda_l a_l with
 * a_l = softmax(q_h k_l^T / sqrt(dh)) v_l (reading note, method section 2; the
 * abstract page's Table 11 counts 3 attention paths and 9 launches for it).
 * Reading: tier l's keys and values at position j are L_l[j] W_k and
 * L_l[j] W_v -- the tiers of FastMKA (L1 = x, L2 = EMA, L3 = mean of the
 * retrieved block means), each rounded once to dtype, the same W_k and W_v --
 * and each path is one causal attention over its own cache.  Provided as the
 * comparison workload of the three-path design.
 *
 * mka_full_prefill: the layer over positions pos0 .. pos0+seq-1 -- route,
 * ema_scan and l3_index on the auxiliary stream (as mka_prefill), retrieval,
 * then per enabled tier: its rows, the K/V product into that tier's cache,
 * causal attention; finally the lambda mix into out->o.  State and outputs as
 * mka_prefill, except: the fused cache st->k_cache / v_cache and st->block_kv
 * are not used (may be NULL); the three tiers' caches are ``kv`` (entries of
 * disabled tiers may be NULL).  Routing variants apply as in mka_prefill.
 *   ws >= mka_workspace_bytes(d, MKA_OP_FULL_PREFILL, 0) bytes
 * mka_full_decode_step: one token at position ``pos`` (d->seq == 1), the same
 * steps in order on ``stream`` (no auxiliary stream), each tier's K/V row
 * appended at row pos and decode attention over rows 0..pos of each cache;
 * when pos closes a block its mean and code join the bank.
 *   ws >= mka_workspace_bytes(d, MKA_OP_FULL_DECODE_STEP, pos + 1) bytes */
typedef struct mka_tier_cache {
  void* k_cache[3]; /* tier l (0 = L1, 1 = L2, 2 = L3): [B, G, t_cap, dh] dtype */
  void* v_cache[3];
} mka_tier_cache;

int mka_full_prefill(const mka_dims* d, const void* x, int64_t pos0, const mka_weights* w,
                     const mka_state* st, const mka_tier_cache* kv, const mka_outputs* out,
                     void* ws, size_t ws_bytes, void* stream);
int mka_full_decode_step(const mka_dims* d, const void* x, int64_t pos, const mka_weights* w,
                         const mka_state* st, const mka_tier_cache* kv, const mka_outputs* out,
                         void* ws, size_t ws_bytes, void* stream);

/* Workspace in bytes that ``op`` needs for the shape ``d``.  ``cache_len`` is the
 * cache length for MKA_OP_ATTN_DECODE / MKA_OP_DECODE_STEP and the number of
 * blocks for MKA_OP_INDEX; it is ignored otherwise. */
size_t mka_workspace_bytes(const mka_dims* d, int op, int64_t cache_len);

/* Static description of a status code. */
const char* mka_status_string(int status);

/* Thread-local description of the last HIP failure seen by this thread ("" if none). */
const char* mka_last_error(void);

/* Library version string. */
const char* mka_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MKA_H */
