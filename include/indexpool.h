/*
 * indexpool.h -- C ABI of libindexpool.so: the global-retrieval half of a hybrid
 * attention layer (IndexPool-compressed indexer, block top-k, sparse attention)
 * on AMD Instinct MI355X (gfx950).
 *
 * The four calls are the four stages of the pipeline that the G2C Brief
 * "GLM-5.3-Flash: hybrid attention becomes the product" draws in its section
 * "DSA keeps selected global access in eleven layers": the latent cache of the
 * full token history, IndexPool (four indexer keys -> one pooled key), learned
 * sparse selection (top 2048 tokens = 512 blocks of 4) and attention over the
 * selected history.  Decode and prefill are separate calls because the two phases
 * have very different arithmetic intensity (reading notes "GLM-5.3-Flash: Hybrid
 * Attention, IndexPool, and Vision-in-the-Loop", section 4, "EPD disaggregation").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Memory: every pointer named "device" is device memory owned by the caller.
 *    The library allocates nothing.  Its only state between calls: per host
 *    thread, the text behind ip_last_error() and the benchmarking hook armed by
 *    ip_time_next_launch() (see the end of this header), which no compute call
 *    needs; per GPU, the static workspace of index_score_topk_noalloc and its
 *    device address, set up by that call's first use on the GPU.
 *  - Streams: every call only enqueues work on `stream` (0 = the null stream) and
 *    never synchronises the host.  Outputs are ready when the stream reaches them.
 *  - Errors: arguments the host can check (null pointers, unsupported dtypes or
 *    sizes, a workspace that is too small) make a call return a non-zero
 *    ip_status before anything is enqueued; ip_last_error() then describes it.
 *    A failed launch returns IP_EDEVICE.  Contents of device arrays (lengths,
 *    page ids, positions, selected ids) are not checked: they are the caller's
 *    contract, stated per call below.
 *  - Caches: token t of sequence b lives at physical row
 *        page_table[b * max_pages + t / page_tokens] * page_tokens + t % page_tokens
 *    when a page table is given, else at row  b * seq_stride + t.  Pooled block j
 *    (tokens 4j..4j+3) of sequence b lives at the same formula with
 *    page_tokens / 4 and seq_stride / 4, so pooled row r always covers token rows
 *    4r .. 4r+3.
 */
#ifndef INDEXPOOL_H
#define INDEXPOOL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IP_OK = 0,
  IP_EINVAL = 1,        /* a null pointer or an inconsistent size */
  IP_EUNSUPPORTED = 2,  /* a dtype / geometry / size outside the supported set */
  IP_EWORKSPACE = 3,    /* workspace missing or smaller than *_workspace_bytes() */
  IP_EDEVICE = 4        /* a HIP launch failed */
} ip_status;

typedef enum {
  IP_F32 = 0,
  IP_BF16 = 1,
  IP_FP8_E4M3FN = 2     /* OCP e4m3fn: bias 7, max 448, no infinities */
} ip_dtype;

/* One cache: `rows` rows of `row_dim` elements; row r starts at
 * (char*)data + r * row_stride.  FP8 rows carry one fp32 scale each
 * (value = scale[r] * decode(code)). */
typedef struct ip_cache {
  void*   data;        /* device */
  float*  scale;       /* device [rows] fp32; required iff dtype == IP_FP8_E4M3FN, else NULL */
  int32_t dtype;       /* ip_dtype of the elements */
  int32_t row_dim;     /* elements per row */
  int64_t row_stride;  /* bytes between rows; a multiple of 16 */
} ip_cache;

/* The batch of sequences and how their caches are laid out. */
typedef struct ip_seqs {
  int32_t        batch;        /* number of sequences, >= 1 */
  int32_t        max_seq_len;  /* host-side upper bound on every seq_lens[b] (sizes grids) */
  const int32_t* seq_lens;     /* device [batch]: tokens cached for each sequence */
  const int32_t* page_table;   /* device [batch, max_pages] physical page ids, or NULL */
  int32_t        max_pages;    /* row length of page_table (ignored when NULL) */
  int32_t        page_tokens;  /* tokens per page, a multiple of 4 (ignored when NULL) */
  int64_t        seq_stride;   /* tokens between sequence starts, a multiple of 4 (page_table NULL) */
} ip_seqs;

/* ---------------------------------------------------------------------------------
 * indexpool_compress -- IndexPool.
 * Reading notes, section 2, sub-section "IndexPool": four indexer key vectors are
 * merged into one by weighted pooling with learned weights (QSA's r = 4 block
 * pooling with a plain mean is the equal-weight case), so the resident indexer
 * state shrinks 4x; the FP8 cache tier is from section 4, "The serving stack".
 *
 * For each sequence b and each complete block j in
 *     [begin_b, min(begin_b + max_blocks, seq_lens[b] / 4))      (begin_b = block_begin[b] or 0)
 * with token keys k_i, scales s_i and logits l_i (i = 0..3, tokens 4j+i):
 *     w = softmax(l_0..l_3);   K_j = sum_i w_i * s_i * k_i
 * FP8 output: sigma_j = max_d |K_j[d]| / 448, code_j = e4m3fn(K_j / sigma_j) rounded
 *             to nearest even and saturated at +-448; sigma_j = 0 gives zero codes.
 * F32 output: K_j as is (keys F32, no scales).
 *
 *  keys     token-level index keys, dtype FP8 (with scale) or F32; row_dim D = 128
 *           for FP8, D <= 256 and a multiple of 4 for F32
 *  logits   device [token rows] fp32, one pooling logit per cached token, indexed
 *           like the key rows
 *  pooled   output, same dtype and row_dim as keys; FP8 also writes pooled->scale
 *  block_begin  device [batch] first block to pool per sequence, or NULL (= 0)
 *  max_blocks   host bound on blocks pooled per sequence (grid size); <= 0 means
 *               max_seq_len / 4
 * Only the rows of the pooled blocks are written.
 * ------------------------------------------------------------------------------- */
ip_status indexpool_compress(const ip_seqs* seqs, const int32_t* block_begin, int32_t max_blocks,
                             const ip_cache* keys, const float* logits, const ip_cache* pooled,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * indexpool_append -- one decode step's cache growth.
 * G2C Brief, "DSA keeps selected global access in eleven layers": the DSA layers
 * keep a token-addressable history that grows with the sequence (the MLA latent
 * rows, and the indexer keys that IndexPool pools four at a time); reading notes,
 * section 4 "The serving stack": the FP8 cache tier; reading notes, section 2,
 * sub-section "IndexPool" for the pooling.
 *
 * seq_lens[b] already counts the new token, which goes to position
 * t = seq_lens[b] - 1 of sequence b (sequences with seq_lens[b] < 1 are skipped):
 *     kv[t]     = kv_new[b]       row copy (BF16 or F32 cache, same dtype as kv_new);
 *                                 FP8 cache (the lower-precision latent tier): kv_new
 *                                 is BF16, quantised per token like the FP8 keys
 *                                 below into codes and kv->scale[t]
 *     v[t]      = v_new[b]        only when v is not NULL (separate V cache)
 *     keys[t]   = key_new[b]      FP8 keys: sigma_t = max_d |x_d| / 448 and codes
 *                                 e4m3fn(x / sigma_t), rounded to nearest even and
 *                                 saturated at +-448 (sigma_t = 0: zero codes);
 *                                 F32 keys: copied
 *     logits[t] = logit_new[b]
 * and when seq_lens[b] % 4 == 0 the block t / 4 that the token completes is pooled
 * into `pooled` exactly as indexpool_compress pools it.
 *
 *  kv_new   device [batch, kv->row_dim], kv->dtype; kv->row_dim * element size a
 *           multiple of 16 bytes (the same for v_new / v).  FP8 kv: kv_new BF16,
 *           8-byte aligned, kv->row_dim a multiple of 4 and <= 1024, v NULL
 *  keys NULL: a DSA layer without indexer state (an IndexCache follower, reading
 *           notes, section 2 "IndexPool": the cross-layer variant): only kv (and v)
 *           rows are written; key_new, logit_new, logits and pooled must be NULL too
 *  key_new  device [batch, keys->row_dim], key_dtype BF16 or F32 (F32 for F32 keys)
 *  logit_new  device [batch] fp32;  logits  device [token rows] fp32
 *  keys, pooled  as in indexpool_compress (FP8 with scales, row_dim 128; or F32)
 * Errors: NULL pointers, dtype or shape mismatches -> IP_EINVAL / IP_EUNSUPPORTED
 * before any launch.  Writes only the new token's rows and the pooled row.
 * ------------------------------------------------------------------------------- */
ip_status indexpool_append(const ip_seqs* seqs, const void* kv_new, const ip_cache* kv,
                           const void* v_new, const ip_cache* v, const void* key_new,
                           int32_t key_dtype, const ip_cache* keys, const float* logit_new,
                           float* logits, const ip_cache* pooled, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * index_score_topk -- the lightweight indexer and the learned top-k selection.
 * Reading notes, section 2 "Hybrid Attention: Linear State + Sparse Retrieval"
 * (sparse attention as the global retriever, via a lightweight indexer, in the
 * lineage of DeepSeek-V3.2's DSA indexer); G2C Brief, "DSA keeps selected global
 * access in eleven layers" (learned sparse selection, index_topk = 2048 tokens).
 *
 * Query row r belongs to sequence b = q_seq[r] (NULL: b = r) at position
 * p = q_pos[r] (NULL: seq_lens[b] - 1); its own block is b_q = p / 4.  For every
 * block j < b_q:
 *     S_j = sum_h gates[r, h] * relu(q_idx[r, h, :] . K_j)        (K_j dequantised)
 * The selection keeps b_q plus the k'-1 best blocks j < b_q, k' = min(top_k, b_q+1),
 * ordered by higher S_j then lower j.  out_idx[r, :] lists the kept ids ascending
 * (b_q last), then -1 up to top_k.
 *
 *  q_idx    device [n_q, n_heads, head_dim]; BF16 with FP8 pooled keys (n_heads 32,
 *           head_dim 128), or F32 with F32 pooled keys (n_heads <= 64,
 *           n_heads * head_dim <= 4096)
 *  gates    device [n_q, n_heads] fp32
 *  pooled   pooled keys written by indexpool_compress for blocks j < b_q
 *  top_k    1 .. 2048
 *  out_idx  device [n_q, top_k] int32
 *  scores   device [n_q, ld] fp32 or NULL, ld = index_scores_ld(max_seq_len); when
 *           given, S_j is written at [r, j] for j < b_q (other entries untouched)
 *           and no score workspace is used
 *  ws       device workspace of ws_bytes >= index_score_topk_workspace_bytes(...),
 *           256-byte aligned, zero-filled before its first use; each call leaves
 *           its per-row synchronisation words (counters, and a parity word that
 *           alternates from call to call) in the state the next call expects, so a
 *           workspace serves any number of later calls (one call at a time)
 *           without being cleared again; the caller must not modify it between
 *           calls
 * Contract: 0 <= p < seq_lens[b]; blocks j < b_q were pooled.
 * ------------------------------------------------------------------------------- */
int64_t index_scores_ld(int32_t max_seq_len);   /* >= max_seq_len/4, rounded up to whole top-k chunks */
size_t index_score_topk_workspace_bytes(const ip_seqs* seqs, int32_t n_q, int32_t top_k,
                                        int32_t scores_given);
ip_status index_score_topk(const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                           const int32_t* q_pos, const void* q_idx, int32_t q_dtype,
                           int32_t n_heads, int32_t head_dim, const float* gates,
                           const ip_cache* pooled, int32_t top_k, int32_t* out_idx,
                           float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * index_score_topk_noalloc -- index_score_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and results, without `ws` /
 * `ws_bytes`.  The workspace is a static array inside the library, one per GPU,
 * of index_score_topk_noalloc_max_bytes() bytes (8 MiB), held until the process
 * ends; calls whose index_score_topk_workspace_bytes(seqs, n_q, top_k, scores !=
 * NULL) exceeds it return IP_EWORKSPACE.  The call allocates and frees nothing.
 * The first call on a GPU looks up the array's device address and clears it with
 * a kernel on `stream`.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams, or different host threads)
 * race and must not be issued.
 * ------------------------------------------------------------------------------- */
size_t index_score_topk_noalloc_max_bytes(void);
ip_status index_score_topk_noalloc(const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                                   const int32_t* q_pos, const void* q_idx, int32_t q_dtype,
                                   int32_t n_heads, int32_t head_dim, const float* gates,
                                   const ip_cache* pooled, int32_t top_k, int32_t* out_idx,
                                   float* scores, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * indexpool_decode_index -- one decode step's cache growth and indexer together:
 * exactly indexpool_append(...) followed by index_score_topk(...) for the decode
 * rows (row r = sequence r at p = seq_lens[r] - 1, n_q = batch; q_seq, q_pos NULL),
 * with the same arguments as those two calls (`pooled` serves both).  G2C Brief,
 * "DSA keeps selected global access in eleven layers" (the growing history and the
 * learned selection).
 *
 * The results are those of the two calls in order, bit for bit: scoring reads the
 * pooled rows of blocks j < b_q only, while the append writes the new token's rows
 * and the pooled row of the block it completes, which is b_q itself.  So with FP8
 * keys the append runs as extra workgroups of the first scoring launch (one launch
 * fewer per step); with F32 keys it is launched first.
 * Errors: those of the two calls (keys must not be NULL); workspace as for
 * index_score_topk_workspace_bytes(seqs, batch, top_k, scores != NULL).
 * ------------------------------------------------------------------------------- */
ip_status indexpool_decode_index(const ip_seqs* seqs, const void* kv_new, const ip_cache* kv,
                                 const void* v_new, const ip_cache* v, const void* key_new,
                                 int32_t key_dtype, const ip_cache* keys, const float* logit_new,
                                 float* logits, const ip_cache* pooled, const void* q_idx,
                                 int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                                 const float* gates, int32_t top_k, int32_t* out_idx, float* scores,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * sparse_attn_decode / sparse_attn_prefill -- attention over the selected history.
 * G2C Brief, "DSA keeps selected global access in eleven layers": the layer keeps
 * a token-addressable MLA latent history of rank 512 and attends over the
 * selected subset of it.
 *
 * For query row r (sequence b, position p as in index_score_topk), the tokens are
 * U = { 4j + i : j in sel_idx[r, :], j >= 0, 0 <= i < 4, 4j + i <= p } and, per head h,
 *     l_t = scale * q[r, h, :] . K_t,   O[r, h, :] = sum_t softmax(l)_t V_t,
 *     lse[r, h] = log sum_t exp(l_t).
 * Geometries:
 *   BF16 latent (MQA): q BF16 [n_q, 64, 576]; k is the 576-dim BF16 latent cache,
 *     v must be NULL: V is the first 512 dims of the same rows (dk 576, dv 512);
 *     out BF16 [n_q, 64, 512] (round to nearest even).
 *   FP8 latent tier (reading notes, section 4 "The serving stack": FP8 as a cache
 *     tier): as BF16 latent, but k is FP8 e4m3fn codes with k->scale[row] per token
 *     row, K_t = scale_t * code_t; the products run in bf16 with fp32 accumulation
 *     (codes widen to bf16 exactly; P_t * scale_t is rounded to bf16 for P V).
 *   Latent paths: token rows (physical row indices) must be below 2^29.
 *   F32: q F32 [n_q, n_heads, dk]; separate F32 k [rows, dk] and v [rows, dv]
 *     caches; n_heads <= 16, dk, dv <= 128 and multiples of 4; out F32.
 *  sel_idx  device [n_q, top_k] ascending block ids, -1 entries ignored
 *           (index_score_topk's output; under IndexCache, that of the group's first
 *           layer, passed unchanged to the group's other layers)
 *  lse      device [n_q, n_heads] fp32 or NULL
 *  ws       device workspace of ws_bytes >= sparse_attn_workspace_bytes(...) (may be
 *           0 bytes, then ws may be NULL)
 * Contract: every non-negative id j satisfies 4j <= p, and the own block of each
 * row is among them (so U is never empty).
 * decode:  row r is sequence r at p = seq_lens[r] - 1 (n_q = batch).
 * prefill: rows given by q_seq (NULL: row r is sequence r) and q_pos.
 * ------------------------------------------------------------------------------- */
size_t sparse_attn_workspace_bytes(int32_t n_q, int32_t n_heads, int32_t dv, int32_t top_k,
                                   int32_t q_dtype);
ip_status sparse_attn_decode(const ip_seqs* seqs, const void* q, int32_t q_dtype,
                             int32_t n_heads, int32_t dk, int32_t dv, float scale,
                             const ip_cache* k, const ip_cache* v, const int32_t* sel_idx,
                             int32_t top_k, void* out, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream);
ip_status sparse_attn_prefill(const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                              const int32_t* q_pos, const void* q, int32_t q_dtype,
                              int32_t n_heads, int32_t dk, int32_t dv, float scale,
                              const ip_cache* k, const ip_cache* v, const int32_t* sel_idx,
                              int32_t top_k, void* out, float* lse, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * indexpool_decode_step -- a whole DSA decode step: indexpool_decode_index(...)
 * (append + indexer + selection) followed by sparse_attn_decode(...) over the
 * selected ids, in one call with the arguments of both (k = kv, v as given; the
 * indexer's q_dtype / n_heads / head_dim are idx_dtype / idx_heads / idx_dim).
 * G2C Brief, "DSA keeps selected global access in eleven layers" (the growing
 * latent history, the learned selection and the attention over it).
 *
 * The results are those of the two calls in order: out_idx (and scores when
 * given) bit for bit, out and lse to the attention's rounding.  With FP8 indexer
 * keys and the split BF16 latent attention (decode batches of up to 64 rows) the
 * step is one launch plus the split combine: the scoring workgroups store each
 * wave's best blocks (a per-wave candidate list), and each row's attention
 * workgroups, which start as scoring workgroups finish, fetch their query, merge
 * the row's lists themselves as soon as every list is stored, and attend over
 * their share of the ids (rows whose lists cannot decide the selection take the
 * exact select over the row's scores, published device-coherently by one of
 * them; rows too short or too long for lists wait for the ids published by their
 * last scoring workgroup); the query's own new token is read from kv_new.  Other
 * geometries run the two calls.
 *  ws  device workspace of ws_bytes >= indexpool_decode_step_workspace_bytes(seqs,
 *      top_k, n_heads, dv, q_dtype, scores != NULL), 256-byte aligned, zero-filled
 *      before its first use and not modified between calls (as for index_score_topk);
 *      each call returns its ready words, counters and candidate lists to zero.
 *      The layout depends on seqs->batch, seqs->max_seq_len, top_k, n_heads, dv and
 *      q_dtype: zero-fill it again before a call that changes them.
 * Errors: those of the two calls.  Calls sharing a workspace must not overlap.
 * ------------------------------------------------------------------------------- */
size_t indexpool_decode_step_workspace_bytes(const ip_seqs* seqs, int32_t top_k, int32_t n_heads,
                                             int32_t dv, int32_t q_dtype, int32_t scores_given);
ip_status indexpool_decode_step(const ip_seqs* seqs, const void* kv_new, const ip_cache* kv,
                                const void* v_new, const ip_cache* v, const void* key_new,
                                int32_t key_dtype, const ip_cache* keys, const float* logit_new,
                                float* logits, const ip_cache* pooled, const void* q_idx,
                                int32_t idx_dtype, int32_t idx_heads, int32_t idx_dim,
                                const float* gates, int32_t top_k, int32_t* out_idx, float* scores,
                                const void* q, int32_t q_dtype, int32_t n_heads, int32_t dk,
                                int32_t dv, float scale, void* out, float* lse, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * kda_decode_step -- one decode step of the linear-attention (KDA) half of the
 * hybrid layer.  G2C Brief, section "KDA carries fixed state through most layers":
 * a gated delta-rule recurrence over a fixed matrix state per head, with a short
 * convolution of width 4 and learned gates; the release summary gives 64 heads of
 * width 128 (a 128 x 128 state per head, independent of the context length).
 *
 * For every sequence b and head h (d = 128, channels c of head h = h*128 + 0..127):
 *     y_c = SiLU(w_c0 x_{t-3,c} + w_c1 x_{t-2,c} + w_c2 x_{t-1,c} + w_c3 x_{t,c})
 *           for each of q, k, v, with x_{t-3..t-1} from conv_in; conv_out receives
 *           them shifted by one token (x_{t-2}, x_{t-1}, x_t)
 *     q, k  scaled by 1 / sqrt(|.|^2 + 1e-6) over the head's 128 channels
 *     S'    = Diag(alpha[b, h, :]) S          (row i = key channel i)
 *     S     = S' + beta[b, h] * k (v - S'^T k)^T
 *     out[b, h, :] = S^T q / sqrt(128)
 *
 *  xq, xk, xv  device [batch, n_heads * 128], BF16 (x_dtype = IP_BF16), before the
 *              convolution
 *  alpha    device [batch, n_heads, 128] fp32 decay per key channel, in (0, 1]
 *  beta     device [batch, n_heads] fp32 write strength
 *  conv_w   device [3 (q, k, v), n_heads * 128, 4] fp32 taps (t-3 .. t), 16-byte
 *           aligned
 *  conv_in  device [batch, 3 (q, k, v), 3 (t-3 .. t-1), n_heads * 128] fp32, read
 *  conv_out device, the same layout, written; must not overlap conv_in (the caller
 *           alternates two buffers from step to step)
 *  state    device [batch, n_heads, 128, 128] fp32, read and updated in place,
 *           16-byte aligned
 *  out      device [batch, n_heads, 128] fp32, 16-byte aligned
 * Errors: head_dim other than 128, a dtype other than BF16, NULL or misaligned
 * pointers, overlapping conv buffers -> IP_EUNSUPPORTED / IP_EINVAL before any
 * launch.
 * ------------------------------------------------------------------------------- */
ip_status kda_decode_step(int32_t batch, int32_t n_heads, int32_t head_dim, const void* xq,
                          const void* xk, const void* xv, int32_t x_dtype, const float* alpha,
                          const float* beta, const float* conv_w, const float* conv_in,
                          float* conv_out, float* state, float* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * kda_prefill_chunk -- the KDA half over a chunk of n_tokens consecutive tokens of
 * each sequence (prefill): exactly n_tokens successive kda_decode_step calls (token
 * t of the chunk as the step's input), computed in the chunked form of the gated
 * delta rule (blocks of 16 tokens: the block's writes solve a 16 x 16 triangular
 * system and its outputs and state update are dense products, on fp32 MFMA).  G2C
 * Brief, section "KDA carries fixed state through most layers".
 *
 *  xq, xk, xv  device [batch, n_tokens, n_heads * 128] BF16, 16-byte aligned
 *  alpha    device [batch, n_tokens, n_heads, 128] fp32 in (0, 1], 16-byte aligned
 *  beta     device [batch, n_tokens, n_heads] fp32
 *  conv_w, conv_in, conv_out, state  as for kda_decode_step (conv_in: the taps
 *           before the chunk, conv_out receives those after it; state is read and
 *           updated in place)
 *  out      device [batch, n_tokens, n_heads, 128] fp32
 * Results agree with the token-by-token recurrence to fp32 rounding (the products
 * with the decay are taken as exponentials of running sums of log alpha).
 * n_tokens = 0 copies the taps and leaves the state unchanged.
 * Errors: as kda_decode_step, plus n_tokens < 0 -> IP_EINVAL.
 * ------------------------------------------------------------------------------- */
ip_status kda_prefill_chunk(int32_t batch, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                            const void* xq, const void* xk, const void* xv, int32_t x_dtype,
                            const float* alpha, const float* beta, const float* conv_w,
                            const float* conv_in, float* conv_out, float* state, float* out,
                            hipStream_t stream);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* ip_last_error(void);

/* Timing hook for benchmarks: the next launch (on this thread) of kernel `kernel_id`
 * goes through hipExtLaunchKernelGGL with `start` / `stop`, so the two events
 * receive that dispatch's own start and end times (the timestamps a kernel trace
 * reports).  kernel_id: 1 compress, 2 score, 3 top-k, 4 attention, 5 split
 * combine, 6 append, 7 KDA decode step, 8 fused decode step.  Hooks for different ids may be
 * armed together; each is consumed by one launch.  Passing NULL for one event
 * only is IP_EINVAL; kernel_id 0 with both NULL disarms every hook.  Use it
 * outside stream capture.  Not needed for normal use. */
ip_status ip_time_next_launch(int32_t kernel_id, hipEvent_t start, hipEvent_t stop);

/* Diagnostics: copies the phase stamps of the last fused decode step (up to `bytes`
 * bytes of a [5120][8] uint64 array: rows 0..4095 the step's workgroups by index,
 * rows 4096.. the combine's; slots 0 start, 1 scoring done and its stores
 * acknowledged, 2 ids ready, 3 sub-tile 0 landed, 4 sub-tiles done, 5 end (for the
 * combine: 0 start, 1 end); values of a 100 MHz clock shared by all compute units,
 * 0 where a workgroup recorded nothing) to host memory `host`.  Only a library built
 * with IP_PHASE_STAMPS records them (`python -m long_context_sparse_19_amd.build
 * --stamps`, a library of its own); otherwise IP_EUNSUPPORTED.  Synchronises with
 * the device.  Not needed for normal use. */
ip_status ip_phase_stamps(void* host, size_t bytes);

/* Library version, e.g. "0.1.0". */
const char* ip_version(void);

#ifdef __cplusplus
}
#endif
#endif /* INDEXPOOL_H */
