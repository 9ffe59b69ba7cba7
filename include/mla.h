/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA decode library, libmla.so.
 *
 * One decode step of Multi-head Latent Attention with weight absorption, as
 * four calls in the order the step runs:
 *
 *   mla_compress_append  new token -> cached row [c_KV ; k_R] at its position
 *   mla_absorb_q         new token -> absorbed query q = [W_UK^T q_C ; q_R]
 *   mla_decode_attn      q x latent cache -> latent-space output o_lat (+ lse)
 *   mla_out_proj         o_lat -> per-head outputs W_UV o_lat -> W_O [..]
 *
 * Sources (pages): "Understanding MLA (Multi-head Latent Attention)" by
 * S. Dong (called [DONG] below), "Multi-Head Latent Attention" in the
 * llm-arch-kb (called [KB]) and the aicassindra "Multi-head latent attention"
 * explainer (called [CASS]). Notation follows [KB] section 2: h_t is the new
 * token's hidden state (width d), c_KV its latent (width d_c), k_R its rotary
 * key (width d_R), H query heads with nope width d_h and value width d_v,
 * and an optional query latent of width d_cq (d_c' on the pages).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Weights are row-major in the orientation W in R^{out x in} (so a vector v
 *    maps to W v), per-head weights as [H][out][in]:
 *      W_DKV [d_c][d]        W_KR [d_R][d]        W_DQ [d_cq][d]
 *      W_UQ  [H][d_h][d_cq]  W_QR [H][d_R][d_cq]   (in = d when d_cq == 0)
 *      W_UK  [H][d_h][d_c]   W_UV [H][d_v][d_c]   W_O [d][H*d_v]
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc'd or equivalent);
 *    the structs mla_dims and mla_cache are HOST memory, read during the call
 *    only. Storage dtype (dims.dtype) applies to h_t, weights, cache, q,
 *    o_heads and out; o_lat and lse are always float32.
 *  - Alignment: every device pointer must be 16-byte aligned.
 *  - The caller owns all memory. The library never allocates device memory
 *    for a call, never frees, and keeps no pointer after returning; scratch
 *    space comes from the caller's workspace (see mla_workspace_bytes).
 *  - Calls are asynchronous: they validate on the host, enqueue kernels on
 *    `stream` (a hipStream_t; NULL = the default stream) and return. A
 *    non-zero status means nothing was enqueued (except MLA_ERR_HIP, which
 *    reports a launch failure). Device faults surface at the caller's
 *    synchronisation. Device-side preconditions (positions below capacity,
 *    block-table entries inside the pool, top-k entries inside a sequence)
 *    are the caller's to keep; mla_check_indices checks host copies of them.
 *  - The calls are re-entrant; calls that share output or workspace buffers
 *    on different streams race.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,         /* a required pointer is NULL                     */
  MLA_ERR_SHAPE = 2,        /* non-positive or inconsistent sizes             */
  MLA_ERR_DTYPE = 3,        /* dtype is not MLA_FP32 or MLA_BF16              */
  MLA_ERR_ALIGN = 4,        /* a device pointer is not 16-byte aligned        */
  MLA_ERR_WORKSPACE = 5,    /* ws_bytes below what the call needs             */
  MLA_ERR_UNSUPPORTED = 6,  /* shape with no compiled kernel                  */
  MLA_ERR_HIP = 7           /* the HIP runtime reported an error              */
} mla_status;

typedef enum { MLA_FP32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Layer geometry and scalars ([KB] section 2; [DONG] section 3). */
typedef struct {
  int32_t d;              /* hidden width                                     */
  int32_t H;              /* query heads                                      */
  int32_t d_h;            /* per-head nope (content) query/key width          */
  int32_t d_v;            /* per-head value width                             */
  int32_t d_c;            /* KV latent width                                  */
  int32_t d_R;            /* decoupled rotary key width (even)                */
  int32_t d_cq;           /* query latent width; 0 = no query low-rank        */
  float softmax_scale;    /* 0 -> 1/sqrt(d_h + d_R) ([DONG] D2)               */
  float rope_theta;       /* rotary base, > 0 (10000 in the DeepSeek configs)  */
  float norm_eps;         /* latent RMSNorm epsilon; 0 -> 1e-6                 */
  int32_t dtype;          /* mla_dtype: storage dtype                          */
} mla_dims;

/*
 * The latent cache: one row of d_c + d_R values per cached token, the latent
 * followed by the already-rotated rotary key ([DONG] section 5: the two
 * objects side by side; [KB] "Per-token cache after decoupling").
 *  - contiguous (block_table == NULL): data is [B][capacity][d_c + d_R];
 *    row u of sequence b is at data + (b*capacity + u) * row_bytes.
 *  - paged (block_table != NULL): data is a pool [n_blocks][block_size][d_c+d_R];
 *    block_table is a DEVICE int32 array [B][max_blocks]; row u of sequence b
 *    is slot u % block_size of block block_table[b*max_blocks + u/block_size].
 */
typedef struct {
  void* data;                 /* device                                        */
  const int32_t* block_table; /* device, or NULL for the contiguous layout     */
  int32_t capacity;           /* contiguous: rows per sequence                 */
  int32_t block_size;         /* paged: rows per block                         */
  int32_t max_blocks;         /* paged: entries per block-table row            */
  int32_t n_blocks;           /* paged: blocks in the pool                     */
} mla_cache;

/*
 * mla_compress_append -- compress the new tokens and append them.
 * For each sequence b, with t = pos[b]:
 *   c   = W_DKV h_t[b]                      ([KB] "Low-rank latent"; [DONG] A1)
 *   c   = c * gamma / sqrt(mean(c^2) + eps) only if gamma_kv != NULL ([DONG] A2)
 *   k_R = RoPE(W_KR h_t[b], t)              ([KB] "Decoupled RoPE head"; [DONG] B2)
 * and stores [c ; k_R], rounded to the storage dtype (nearest-even), as row t
 * of sequence b. RoPE rotates consecutive pairs (x[2j], x[2j+1]) by the angle
 * t * theta^(-2j/d_R).
 *   h_t      [B][d]        storage dtype
 *   gamma_kv [d_c]         storage dtype, or NULL (no latent norm)
 *   pos      [B] int32     device: position of the new token (= rows already
 *                          cached); must be < capacity, or inside the
 *                          sequence's allocated blocks when paged
 *   ws       workspace of at least mla_workspace_bytes(...) bytes
 * Only row pos[b] of each sequence is written.
 */
mla_status mla_compress_append(const mla_dims* dims, int32_t B, const void* h_t,
                               const void* W_DKV, const void* W_KR,
                               const void* gamma_kv, const int32_t* pos,
                               const mla_cache* cache, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * mla_absorb_q -- the absorbed query of the new tokens.
 *   c_Q      = W_DQ h_t[b]          (c_Q = h_t[b] when d_cq == 0, W_DQ NULL)
 *   q_C(i)   = W_UQ(i) c_Q          ([KB] "Query-side compression")
 *   q_R(i)   = RoPE(W_QR(i) c_Q, pos[b])  (same position as the key, [DONG] C2)
 *   q_lat(i) = W_UK(i)^T q_C(i)     (the key up-projection moved onto the
 *                                    query, [DONG] section 4)
 * Output q [B][H][d_c + 2*d_R] in the storage dtype: q_lat, then q_R, then
 * the low term of q_R (the storage-dtype nearest value of q_R minus its
 * first term; zero for float32). The first d_c + d_R values have the width
 * of a cache row, so attention is one contraction over it; the rotary part
 * is carried as two terms because it dominates the scores at the
 * DeepSeek-V3 widths and its rounding to bf16 alone would reach the softmax.
 * c_Q and q_C stay float32 in the workspace for the same reason.
 */
mla_status mla_absorb_q(const mla_dims* dims, int32_t B, const void* h_t,
                        const void* W_DQ, const void* W_UQ, const void* W_QR,
                        const void* W_UK, const int32_t* pos, void* q,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * mla_decode_attn -- every head attends against the shared latent cache.
 * For sequence b, head i and rows u < seq_lens[b]:
 *   s(i,u)   = scale * (q(b,i) . row(b,u))      over all d_c + d_R columns
 *   o_lat(i) = sum_u softmax_u(s(i,u)) * row(b,u)[0:d_c]
 *   lse(i)   = ln sum_u exp(s(i,u))
 * ([CASS] "End-to-end flow": content and rotary dot products summed, softmax
 * over all history, weights applied to the cached latents.)
 *   q          [B][H][d_c + 2*d_R] storage dtype (from mla_absorb_q): per
 *              head q_lat, q_R, low term of q_R; the score uses q_lat and
 *              q_R + low term
 *   seq_lens   [B] int32 device: rows attended, the new token included; 0 gives
 *              an all-zero o_lat row and lse = -inf
 *   max_seq_len host upper bound of seq_lens (sizes the launch)
 *   num_splits context chunks per sequence (at most), 0 = automatic. Each
 *              chunk is a run of whole 32-row tiles handled by one
 *              workgroup; the chunks of a sequence are merged exactly
 *              afterwards. Automatic (bf16 MFMA path, the V3 geometry): the
 *              device reads seq_lens and picks the smallest chunk size (at
 *              least 128 rows) whose chunk count fits one workgroup per
 *              compute unit (or per sequence, if B is larger), so a ragged
 *              batch is balanced. Other geometries cut every sequence into
 *              the same number of equal chunks of max_seq_len.
 *   o_lat      [B][H][d_c] float32 out;  lse [B][H] float32 out, or NULL
 *   ws         workspace of at least mla_workspace_bytes(dims, B, max_seq_len,
 *              num_splits) bytes: chunk partials and the chunk plan
 * Errors: MLA_ERR_UNSUPPORTED if B exceeds 32768 or B * num_splits exceeds
 * 2^22 on the MFMA path.
 */
mla_status mla_decode_attn(const mla_dims* dims, int32_t B, const void* q,
                           const mla_cache* cache, const int32_t* seq_lens,
                           int32_t max_seq_len, int32_t num_splits,
                           float* o_lat, float* lse, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * mla_decode_attn_noalloc -- mla_decode_attn for callers that cannot allocate
 * device memory or hold a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments, results
 * and errors as mla_decode_attn, without ws / ws_bytes: the scratch space
 * (chunk partials, chunk plan) is a fixed array of MLA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends.
 * The call allocates nothing; its first call on a device looks the array's
 * address up once (hipGetSymbolAddress).
 * Limit: the attention's scratch for these sizes (the attention part of
 * mla_workspace_bytes) must fit the array, else MLA_ERR_WORKSPACE. At the
 * DeepSeek-V3 widths (128 heads) the automatic plan fits for up to 560
 * sequences on a 256-CU device.
 * All calls on one device share the array and it keeps the last call's
 * contents (no call relies on them): calls that overlap on one device, from
 * different streams or threads, race and must be serialised by the caller.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (72u << 20)
mla_status mla_decode_attn_noalloc(const mla_dims* dims, int32_t B, const void* q,
                                   const mla_cache* cache, const int32_t* seq_lens,
                                   int32_t max_seq_len, int32_t num_splits, float* o_lat,
                                   float* lse, void* stream);

/*
 * mla_decode_attn_sparse -- every head attends against a given subset of the
 * latent cache: sequence b attends only to the counts[b] rows listed in
 * indices[b][0..counts[b]) (positions in its cache), the top-k pattern of a
 * sparse selector layered above MLA ([KB] section 4, "Scaling to V3.2 +
 * sparse attention": a top-K subset of the cached latents, k = 2048, per
 * query, each candidate a single d_c + d_R row). For head i:
 *   s(i,j)   = scale * (q(b,i) . row(b, indices[b][j]))   j < counts[b]
 *   o_lat(i) = sum_j softmax_j(s(i,j)) * row(b, indices[b][j])[0:d_c]
 *   lse(i)   = ln sum_j exp(s(i,j))
 * Each listed entry is one term of the softmax (a repeated index counts
 * once per listing); the order of the list does not matter.
 *   indices  [B][topk] int32 device; entries past counts[b] are not read.
 *            Device-side precondition: every listed position is a row of
 *            sequence b's cache (contiguous: < capacity; paged: its block
 *            table entry is valid).
 *   topk     row stride of indices (> 0), and the host bound of counts
 *   counts   [B] int32 device, 0 <= counts[b] <= topk; 0 gives an all-zero
 *            o_lat row and lse = -inf
 *   num_splits, o_lat, lse, ws: as for mla_decode_attn with max_seq_len =
 *            topk (the workspace of mla_workspace_bytes(dims, B, topk,
 *            num_splits) suffices)
 * Errors: as for mla_decode_attn; MLA_ERR_SHAPE if topk <= 0, MLA_ERR_NULL
 * if indices or counts is NULL, MLA_ERR_ALIGN unless both are 4-byte aligned.
 */
mla_status mla_decode_attn_sparse(const mla_dims* dims, int32_t B, const void* q,
                                  const mla_cache* cache, const int32_t* indices, int32_t topk,
                                  const int32_t* counts, int32_t num_splits, float* o_lat,
                                  float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * mla_check_indices -- host-side check of the device-side preconditions.
 * The kernels read positions, lengths, block-table entries and top-k lists
 * from device memory without checking them (a check per element would sit
 * in the hot loops); a violation reads or writes outside the cache. This
 * call checks HOST copies of those arrays against the cache description.
 * Any array may be NULL to skip its checks.
 *   pos         [B] append positions (mla_compress_append, mla_absorb_q):
 *               0 <= pos[b] < capacity (contiguous) or < max_blocks *
 *               block_size with a valid block-table entry (paged); and no
 *               two sequences append into the same cache slot (paged)
 *   seq_lens    [B] rows attended (mla_decode_attn, mla_prefill_attn):
 *               0 <= seq_lens[b] <= max_seq_len and <= capacity (contiguous)
 *               or max_blocks * block_size (paged), every block-table entry
 *               that covers rows [0, seq_lens[b]) valid
 *   max_seq_len the host bound passed with seq_lens
 *   block_table [B][max_blocks] host copy of cache->block_table; required
 *               for a paged cache when any of pos, seq_lens, indices is given
 *   indices     [B][topk] and counts [B] (mla_decode_attn_sparse): 0 <=
 *               counts[b] <= topk, every listed position j < counts[b] a row
 *               of the cache (as for pos) and, with seq_lens given, below
 *               seq_lens[b]
 * A valid block-table entry is 0 <= entry < n_blocks. Returns MLA_OK, or
 * MLA_ERR_SHAPE with mla_last_error naming the first violation (array,
 * sequence, value), MLA_ERR_NULL for a missing host block table or indices
 * without counts; dims and cache are validated as by the other calls. Host
 * only: reads host memory, touches no device memory, enqueues nothing.
 */
mla_status mla_check_indices(const mla_dims* dims, int32_t B, const mla_cache* cache,
                             const int32_t* pos, const int32_t* seq_lens, int32_t max_seq_len,
                             const int32_t* block_table, const int32_t* indices, int32_t topk,
                             const int32_t* counts);

/*
 * mla_out_proj -- back to the hidden width.
 *   o_heads(b,i) = W_UV(i) o_lat(b,i)       ([CASS] value projection after the
 *                                            weighted sum)
 *   out(b)       = W_O [o_heads(b,1); ...; o_heads(b,H)]  ([DONG] D2)
 *   o_lat  [B][H][d_c] float32;  o_heads [B][H][d_v] out (storage dtype);
 *   W_O / out may both be NULL to stop after the per-head outputs.
 */
mla_status mla_out_proj(const mla_dims* dims, int32_t B, const float* o_lat,
                        const void* W_UV, const void* W_O, void* o_heads,
                        void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Precomposed weights ([KB] section 2 "Derivation", paragraph "The RoPE
 * obstruction": the key
 * up-projection folded into the query-side matrix once, offline; [CASS]
 * "absorbed-weights box": the value up-projection pre-multiplied into the
 * output projection). The per-head products are formed once:
 *   W_QK(i) = W_UK(i)^T W_UQ(i)   [H][d_c][qin]   (qin = d_cq, or d if 0)
 *   W_OV    = W_O blockdiag(W_UV(1), ..., W_UV(H))   [d][H*d_c]
 *             i.e. W_OV[:, i*d_c:(i+1)*d_c] = W_O[:, i*d_v:(i+1)*d_v] W_UV(i)
 * and the decode step then uses one product per side. The results equal
 * those of mla_absorb_q / mla_out_proj up to rounding: the composed weights
 * are rounded once to the storage dtype, and the two-step path instead
 * rounds the intermediate q_C and o_heads. Which is faster depends on the
 * sizes: the composed weights are d_c/d_h (query) and H*d_c/(H*d_v) (output)
 * times the per-head up-projections they replace, so they pay off only when
 * the batch is large enough for the product to be compute-bound.
 */

/*
 * mla_precompose -- form W_QK and (if W_UV, W_O and W_OV are all given) W_OV.
 * Accumulates in float32 and rounds once to the storage dtype (nearest-even).
 *   W_UQ [H][d_h][qin], W_UK [H][d_h][d_c], W_UV [H][d_v][d_c], W_O [d][H*d_v]
 *   W_QK [H][d_c][qin] out;  W_OV [d][H*d_c] out, or NULL with W_UV, W_O NULL
 * Needs no workspace. Errors: MLA_ERR_NULL if W_UQ, W_UK or W_QK is NULL or
 * only some of W_UV, W_O, W_OV are given.
 */
mla_status mla_precompose(const mla_dims* dims, const void* W_UQ, const void* W_UK,
                          const void* W_UV, const void* W_O, void* W_QK, void* W_OV,
                          void* stream);

/*
 * mla_absorb_q_precomposed -- the absorbed query from precomposed weights:
 *   c_Q      = W_DQ h_t[b]          (h_t[b] when d_cq == 0, W_DQ NULL)
 *   q_lat(i) = W_QK(i) c_Q
 *   q_R(i)   = RoPE(W_QR(i) c_Q, pos[b])
 * Output q [B][H][d_c + 2*d_R] exactly as mla_absorb_q lays it out.
 * ws: mla_workspace_bytes(dims, B, ...) bytes suffice.
 */
mla_status mla_absorb_q_precomposed(const mla_dims* dims, int32_t B, const void* h_t,
                                    const void* W_DQ, const void* W_QK, const void* W_QR,
                                    const int32_t* pos, void* q, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * mla_out_proj_precomposed -- out(b) = W_OV o_lat(b), o_lat [B][H][d_c]
 * float32 read as [B][H*d_c]; out [B][d] storage dtype. No per-head outputs.
 * ws: mla_workspace_bytes(dims, B, ...) bytes suffice.
 */
mla_status mla_out_proj_precomposed(const mla_dims* dims, int32_t B, const float* o_lat,
                                    const void* W_OV, void* out, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * Causal prefill: T new tokens per sequence attend over the cache, the step
 * on the other side of the cache from decode. Two algorithms with the same
 * inputs and outputs ("Understanding MLA", sections 5-6: the training form
 * expands the latent and runs ordinary attention, the decode form keeps the
 * latent and folds the up-projections into query and output; [KB] section 3
 * sketch of the expanded form):
 *   MLA_PREFILL_MATERIALIZED  K(i)_u = [W_UK(i) c_u ; k_R,u], V(i)_u = W_UV(i) c_u
 *                             for every stored row, then per-head causal
 *                             attention over d_h + d_R wide keys
 *   MLA_PREFILL_ABSORBED      q_lat = W_UK(i)^T q_C per token, latent attention
 *                             over the d_c + d_R wide rows (the decode kernel,
 *                             one entry per token), o = W_UV(i) o_lat
 * For token t of sequence b, at position p = seq_lens[b] - T + t (its own row
 * and the earlier tokens' rows are already in the cache):
 *   s(i,u) = scale * ([q_C ; q_R](b,t,i) . K(i)_u)    u = 0..p
 *   o(b,t,i) = sum_u softmax_u(s(i,u)) V(i)_u,   lse(b,t,i) = ln sum_u exp s(i,u)
 *   q      [B][T][H][d_h + d_R] storage dtype: per head [q_C ; q_R], q_R rotated
 *          at the token's position
 *   seq_lens [B] int32 device: rows of sequence b including its T tokens; a
 *          token with p < 0 attends nothing (zeros, lse = -inf)
 *   max_seq_len host upper bound of seq_lens
 *   W_UK [H][d_h][d_c], W_UV [H][d_v][d_c]
 *   o      [B][T][H][d_v] storage dtype out;  lse [B][T][H] float32 out, or NULL
 *   ws     mla_prefill_workspace_bytes(dims, B, T, max_seq_len, cache, algo)
 *          bytes. The materialised form expands every row the cache stores
 *          (contiguous: B * capacity, paged: n_blocks * block_size) into it:
 *          (d_h + d_v) * H elements per row.
 * MLA_PREFILL_AUTO takes the form a cost model expects to be faster. The model
 * is fitted to measurements on MI355X at the DeepSeek-V3 widths. It picks the
 * absorbed form while the attended rows, bounded from T and max_seq_len, stay
 * below 360 per stored row, and the materialised form above that. A form with
 * no kernel for the shape yields to the other. mla_prefill_choose reports
 * the choice; mla_prefill_workspace_bytes with MLA_PREFILL_AUTO sizes it.
 * Errors: MLA_ERR_SHAPE for B, T <= 0, an unknown algo or max_seq_len above
 * the cache; MLA_ERR_UNSUPPORTED if B * T exceeds 32768 (absorbed, V3
 * geometry) or the cache stores more than 8,388,480 rows (materialised).
 */
typedef enum { MLA_PREFILL_MATERIALIZED = 0, MLA_PREFILL_ABSORBED = 1, MLA_PREFILL_AUTO = 2 } mla_prefill_algo;

mla_status mla_prefill_attn(const mla_dims* dims, int32_t B, int32_t T, const void* q,
                            const mla_cache* cache, const int32_t* seq_lens, int32_t max_seq_len,
                            const void* W_UK, const void* W_UV, int32_t algo, void* o, float* lse,
                            void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes mla_prefill_attn needs; 0 on bad arguments. */
size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t B, int32_t T, int32_t max_seq_len,
                                   const mla_cache* cache, int32_t algo);

/* The form MLA_PREFILL_AUTO runs for these arguments (MLA_PREFILL_MATERIALIZED
 * or MLA_PREFILL_ABSORBED); -1 on bad arguments or when neither form has a
 * kernel for the shape. Host only: reads the structs, no device memory. */
int32_t mla_prefill_choose(const mla_dims* dims, int32_t B, int32_t T, int32_t max_seq_len,
                           const mla_cache* cache);

/* Workspace bytes that suffice for every call above except mla_prefill_attn, with these sizes
 * (num_splits as passed to mla_decode_attn, 0 = automatic). 0 on bad dims. */
size_t mla_workspace_bytes(const mla_dims* dims, int32_t B, int32_t max_seq_len,
                           int32_t num_splits);

/* The number of chunks mla_decode_attn gives a sequence of max_seq_len rows
 * when all B sequences have that length (resolves 0 = automatic; with ragged
 * lengths the automatic plan is made on the device from seq_lens); 0 on bad
 * dims. Needs the current device's compute-unit count for the automatic
 * choice. */
int32_t mla_decode_num_splits(const mla_dims* dims, int32_t B, int32_t max_seq_len,
                              int32_t num_splits);

/* Bytes of one cache row: (d_c + d_R) * element size; 0 on bad dims. */
size_t mla_cache_row_bytes(const mla_dims* dims);

/* Which attention kernel mla_decode_attn uses for these dims:
 * 1 = bf16 MFMA kernel (d_c = 512, d_R = 64, H a multiple of 32 up to 128),
 * 2 = general kernel (any other geometry, fp32 or bf16), 0 = bad dims. */
int32_t mla_decode_kernel(const mla_dims* dims);

/*
 * mla_time_next_attn -- kernel timing of the next attention call. The next
 * mla_decode_attn, mla_decode_attn_sparse or mla_decode_attn_noalloc call
 * made on the calling host thread stamps kernel_start with the start of its
 * attention kernel, kernel_end with that kernel's end and call_end with the
 * end of the call's last kernel (the merge of a sequence's chunks, when it
 * runs). The bf16 MFMA path launches its kernels with hipExtLaunchKernel's
 * start and stop events, so no marker command enters the stream; the general
 * kernel (mla_decode_kernel = 2) records the events as markers around its
 * launches instead.
 *   kernel_start, kernel_end, call_end  hipEvent_t handles created by the
 *            caller with timing enabled, or NULL to leave one out; the
 *            caller owns them and reads them with hipEventElapsedTime
 * The setting holds for one attention call and is cleared by it, whether
 * that call succeeds or not; mla_prefill_attn does not take it. A call that
 * enqueues nothing (an error status) stamps nothing. Returns MLA_OK.
 */
mla_status mla_time_next_attn(void* kernel_start, void* kernel_end, void* call_end);

/* Text for a status code (static storage). */
const char* mla_status_str(int32_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
