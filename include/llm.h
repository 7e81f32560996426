/*
 * llm.h -- C ABI of the MI355X (gfx950) Llama-2 decoder forward library.
 *
 * The library runs the decoder-only forward pass described in the
 * walkthrough "Meta Llama 源码深度剖析与生产应用教程" (section 2 data flow,
 * sections 3.2-3.8 for the layer) with the reference's static per-layer KV
 * cache (section 3.1) or a paged block pool (nano-vllm notes, see "paged KV
 * cache" below), as a full-prompt causal prefill followed by one-token
 * decode steps (section 4.2, and the course notes on generate, section 1),
 * and ends in last-position logits with greedy, temperature and top-p
 * sampling (section 4.3).  Every step runs in hand-written HIP kernels on one
 * GPU.
 *
 * Conventions for every call:
 *  - Return value: LLM_OK (0) or a negative llm_status.  Nothing aborts and no
 *    C++ exception crosses this boundary; llm_last_error() returns a message.
 *  - Arguments are validated on the host before any GPU work is queued; an
 *    invalid call changes no state.
 *  - A failing HIP call returns LLM_EDEVICE and poisons the handle: every later
 *    call on it returns LLM_EDEVICE too (destroy is still allowed).
 *  - Pointers without a _d suffix are host pointers; `_d` entry points take
 *    device pointers.  The caller owns everything it passes; the handle owns
 *    all memory it allocates (weights, KV cache, token buffer, logits,
 *    workspace) and frees it in llm_destroy.
 *  - All work is ordered on one HIP stream (the caller's, or the handle's
 *    own).  llm_prefill, llm_decode and the _d calls are asynchronous; calls
 *    that return values into host memory synchronise the stream.
 *  - A handle is not thread-safe.
 */
#ifndef LLM_H
#define LLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LLM_OK = 0,
    LLM_EINVAL = -1,   /* argument out of range or inconsistent */
    LLM_ESTATE = -2,   /* call not allowed in the handle's current state */
    LLM_ENOMEM = -3,   /* device allocation failed */
    LLM_EDEVICE = -4   /* a HIP call failed; the handle is poisoned */
} llm_status;

typedef enum { LLM_F32 = 0, LLM_F16 = 1 } llm_dtype;

/* Model hyper-parameters: the fields of ModelArgs (walkthrough section 3.1)
 * plus the RoPE base (section 3.3) and the storage type.
 *  n_kv_heads <= 0 means n_kv_heads = n_heads (MHA).
 *  ffn_dim_multiplier <= 0 means None.  The FFN width is int(2*4*dim/3),
 *    times the multiplier (int), rounded up to multiple_of (section 3.6).
 *  max_batch_size x max_seq_len fixes the static KV cache extents.
 *  dtype LLM_F16 stores weights, activations and cache in binary16 with fp32
 *    accumulation; LLM_F32 stores them in binary32.
 * Supported shapes: dim divisible by n_heads, n_heads by n_kv_heads,
 * max_batch_size <= 4096.  LLM_F16 models need head_dim 128, dim <= 8192,
 * dim and the FFN width multiples of 64, vocab_size a multiple of 16, max_seq_len a
 * multiple of 64 and n_heads / n_kv_heads <= 16.  LLM_F32 models are limited
 * to dim <= 4096 and max_seq_len <= 8192.  Other shapes give LLM_EINVAL. */
typedef struct {
    int32_t n_layers, dim, n_heads, n_kv_heads;
    int32_t vocab_size, multiple_of;
    float ffn_dim_multiplier;
    float norm_eps, rope_theta;
    int32_t max_batch_size, max_seq_len;
    int32_t dtype;
} llm_params;

typedef struct llm llm_t;

/* ---- sizing (host only, no GPU needed) -------------------------------- */

/* FFN hidden width of the parameters (walkthrough section 3.6), or < 0. */
int64_t llm_ffn_hidden(const llm_params *p);
/* Bytes of the static KV cache: n_layers * 2 * max_batch * n_kv_heads *
 * max_seq_len * head_dim * element size (walkthrough section 3.1). */
int64_t llm_kv_cache_bytes(const llm_params *p);
/* Bytes of all layer matrices plus the output head (what one decode step
 * streams); the embedding table is gathered, not streamed, and excluded. */
int64_t llm_weight_bytes(const llm_params *p);
/* Check parameters without creating anything: LLM_OK or LLM_EINVAL. */
int llm_check_params(const llm_params *p);

/* ---- lifetime ---------------------------------------------------------- */

/* Create a model on the current HIP device.  Every weight is drawn from the
 * seeded generator (SplitMix64 streams per tensor, Irwin-Hall(4) normal with
 * standard deviation 0.02, rounded once to the storage type); RMSNorm weights
 * are 1.  The KV cache is zeroed.  `hip_stream` is a hipStream_t to order all
 * work on, or NULL for a stream owned by the handle.
 * Errors: LLM_EINVAL (parameters), LLM_ENOMEM, LLM_EDEVICE.  On error *out is
 * NULL.
 * Environment read at creation: LLM_NO_GRAPH=1 runs decode steps eagerly
 * instead of replaying a captured graph. */
int llm_create(const llm_params *p, uint64_t seed, void *hip_stream, llm_t **out);

/* A handle that validates arguments and tracks state exactly like a real
 * one but allocates nothing and queues no GPU work; value-returning calls
 * return LLM_ESTATE.  For checking the call protocol without a GPU. */
int llm_create_dry(const llm_params *p, llm_t **out);

void llm_destroy(llm_t *h);
/* The handle's last error message; with h == NULL the calling thread's last
 * message from a handle-free call (llm_sample_logits_static). */
const char *llm_last_error(const llm_t *h);
/* The hipStream_t all of the handle's work is ordered on (owned by the
 * handle unless one was passed to llm_create); NULL for a dry handle. */
void *llm_get_stream(llm_t *h);

/* ---- paged KV cache ------------------------------------------------------
 * The block-pool cache of the nano-vllm notes (model runner,
 * allocate_kv_cache; block tables and slot mapping of prepare_prefill /
 * prepare_decode) in place of the static cache.  The pool holds num_blocks
 * blocks; a block holds block_size consecutive positions of one batch row,
 * K and V of every KV head of every layer.  Row b's positions
 * [i*block_size, (i+1)*block_size) live in the block at entry i of its block
 * table (width ceil(max_seq_len / block_size)).  Results are identical to a
 * static-cache handle of the same parameters, bit for bit.
 *
 * Blocks are handed out on demand: a pass that writes positions [.., end) of
 * row b first gives every empty table entry below ceil(end / block_size) the
 * lowest-numbered free block.  A row keeps its blocks until its table is
 * replaced (llm_kv_set_block_table) or a prefill from position 0 of B rows
 * returns the blocks of rows >= B to the pool.  A pass that needs more free
 * blocks than the pool has fails with LLM_ENOMEM, and a pass that reads
 * cached positions whose table entry is empty fails with LLM_ESTATE, both
 * before anything changes.  Every other call behaves as on a static handle. */
typedef struct {
    int32_t block_size;            /* positions per block: a power of two in [32, 65536] */
    int32_t num_blocks;            /* pool size, at most max_batch_size * table width; 0: from
                                      the memory budget */
    float gpu_memory_utilization;  /* num_blocks == 0: the pool takes
                                      total * gpu_memory_utilization - (memory in use once
                                      weights, buffers and the workspace of the largest pass
                                      are allocated), in (0, 1] */
} llm_paging;

/* Bytes of one block: 2 * n_layers * block_size * n_kv_heads * head_dim *
 * element size (the nano-vllm notes' block_bytes), or < 0. */
int64_t llm_kv_block_bytes(const llm_params *p, int32_t block_size);

/* llm_create with a paged cache; the pool is zeroed.  Errors as llm_create,
 * LLM_EINVAL for paging values out of range, LLM_ENOMEM when the budget
 * leaves no room for one block. */
int llm_create_paged(const llm_params *p, const llm_paging *pg, uint64_t seed, void *hip_stream,
                     llm_t **out);
/* llm_create_dry with a paged cache (num_blocks must be > 0): the block
 * bookkeeping runs as on a real handle. */
int llm_create_paged_dry(const llm_params *p, const llm_paging *pg, llm_t **out);

/* Pool size, free blocks and block-table width; 0 for a static handle. */
int32_t llm_kv_num_blocks(const llm_t *h);
int32_t llm_kv_free_blocks(const llm_t *h);
int32_t llm_kv_table_width(const llm_t *h);

/* Copy the first n entries of row's block table (-1 for empty) into out. */
int llm_kv_block_table(llm_t *h, int32_t row, int32_t *out, int32_t n);

/* Replace row's block table by blocks[0..n) (the rest empty), n <= table
 * width.  The ids must be distinct, in [0, num_blocks) and free or already
 * held by this row; the row's other blocks return to the pool.  A block's
 * contents are what was last written to it: moving cached positions to
 * other blocks makes the row read those.  n == 0 releases the row. */
int llm_kv_set_block_table(llm_t *h, int32_t row, const int32_t *blocks, int32_t n);

/* ---- the forward pass --------------------------------------------------- */

/* Prefill (Transformer.forward(tokens, 0), walkthrough sections 2 and 3.8):
 * tokens[B][T] row-major at positions 0..T-1 with the causal mask.  Writes
 * the KV cache for positions [0, T), stores the tokens in the handle's token
 * buffer tok[B][max_seq_len], and leaves fp32 logits[B][vocab] of position
 * T-1.  Requires 1 <= B <= max_batch_size, 1 <= T <= max_seq_len, every
 * token in [0, vocab).  Host tokens are copied before the call returns. */
int llm_prefill(llm_t *h, const int32_t *tokens, int32_t B, int32_t T);
int llm_prefill_d(llm_t *h, const int32_t *tokens_d, int32_t B, int32_t T);

/* Prefill at an offset (chunked prefill; Transformer.forward(tokens,
 * start_pos) with T tokens, walkthrough section 3.8: the mask is a block of
 * zeros over the cached positions followed by the causal triangle).  Runs
 * tokens[B][T] at positions start_pos..start_pos+T-1 attending to the cache
 * prefix [0, start_pos) and causally to themselves; writes the KV cache and
 * token columns [start_pos, start_pos+T) and leaves the logits of position
 * start_pos+T-1.  start_pos == 0 is llm_prefill.  start_pos > 0 requires an
 * earlier prefill of the same B with KV written up to start_pos-1
 * (start_pos <= last position + 1), else LLM_ESTATE; start_pos + T must not
 * exceed max_seq_len (LLM_EINVAL).  Positions after start_pos+T-1 that an
 * earlier pass wrote stay in the cache but are not attended to until
 * rewritten. */
int llm_prefill_at(llm_t *h, int32_t start_pos, const int32_t *tokens, int32_t B, int32_t T);
int llm_prefill_at_d(llm_t *h, int32_t start_pos, const int32_t *tokens_d, int32_t B, int32_t T);

/* Varlen prefill (ragged prompts; nano-vllm notes, prefill with packed
 * sequences and cumulative lengths): row b has lens[b] tokens (1 <= lens[b]
 * <= max_seq_len, lens on the host), packed row after row in tokens
 * (sum(lens) entries).  Each row runs at positions 0..lens[b]-1 with its own
 * causal mask; writes KV [0, lens[b]) and token columns of row b, and leaves
 * the logits of each row's last prompt position.  The handle then holds rows
 * at different positions ("rows mode"): llm_sample writes column
 * row_last[b] + 1 of row b, llm_decode_rows advances every row, and the
 * uniform-position calls (llm_decode, llm_set_tokens, llm_prefill_at with an
 * offset) return LLM_ESTATE until the next llm_prefill.  Host tokens are
 * copied before the call returns. */
int llm_prefill_varlen(llm_t *h, const int32_t *tokens, const int32_t *lens, int32_t B);
int llm_prefill_varlen_d(llm_t *h, const int32_t *tokens_d, const int32_t *lens, int32_t B);

/* One decode step in rows mode: row b runs the token in its column
 * row_last[b] + 1 at that position (nano-vllm notes: decode with per-sequence
 * context lengths) and leaves its logits.  Every row's next column must be
 * written (llm_sample or llm_set_tokens_rows, else LLM_ESTATE) and below
 * max_seq_len (else LLM_EINVAL).  Captured as a HIP graph per batch size. */
int llm_decode_rows(llm_t *h);

/* Rows mode: write tokens[b] into column row_last[b] + 1 of the rows mask
 * selects (all when mask is NULL); host pointers. */
int llm_set_tokens_rows(llm_t *h, const int32_t *tokens, const uint8_t *mask);

/* One decode step (seqlen 1, no mask: the course notes on generate,
 * section 3): runs tok[:, prev_pos] at position prev_pos against cached keys
 * 0..prev_pos, writes the KV cache at prev_pos, leaves logits of position
 * prev_pos.  Requires a prior prefill, 1 <= prev_pos <= last_pos + 1,
 * prev_pos < max_seq_len, and the token column prev_pos written (by the
 * prefill, llm_sample or llm_set_tokens); else LLM_ESTATE / LLM_EINVAL. */
int llm_decode(llm_t *h, int32_t prev_pos);

/* Sample the next token of every row from the current logits (position
 * last_pos): temperature <= 0 is greedy argmax (lowest id on ties);
 * otherwise P = softmax(logits / temperature) in fp32 and top-p sampling
 * (walkthrough section 4.3) made exact: tokens ordered by (P desc, id asc),
 * Q_i = floor(P_i * 2^48), E_i = sum of Q before i, token i kept iff
 * E_i <= floor(top_p * 2^48); with S the kept mass and U = floor(u * 2^24)
 * the drawn token is the first kept i with E_{i+1} > floor(U * S / 2^24).
 * uniforms[B] are in [0, 1).  The token is written to tok[:, last_pos + 1]
 * when last_pos + 1 < max_seq_len and copied to out_tokens[B] when it is not
 * NULL (then the call synchronises; otherwise it is asynchronous: the host
 * uniforms are staged in pinned memory before it returns).  top_p must lie
 * in (0, 1], temperature must be finite. */
int llm_sample(llm_t *h, float temperature, float top_p, const float *uniforms,
               int32_t *out_tokens);
/* Same with uniforms and output in device memory; never synchronises.
 * out_tokens_d may be NULL. */
int llm_sample_d(llm_t *h, float temperature, float top_p, const float *uniforms_d,
                 int32_t *out_tokens_d);

/* The reference's prompt forcing, where(mask, prompt_token, sampled)
 * (walkthrough section 4.2): tok[b][pos] = tokens[b] for every row b < B of
 * the last prefill whose mask[b] is non-zero (mask NULL: all rows).
 * Requires 0 <= pos < max_seq_len, tokens in [0, vocab). */
int llm_set_tokens(llm_t *h, int32_t pos, const int32_t *tokens, const uint8_t *mask);

/* Same with tokens[B] and mask[B] (or NULL) in device memory; asynchronous.
 * Token ids are not range-checked on the host: the caller guarantees
 * [0, vocab).  The host cannot read a device mask, so with a mask the
 * column counts as written for llm_decode only if it already was (the
 * reference's forcing of some rows over a sampled column); with mask NULL
 * it is written. */
int llm_set_tokens_d(llm_t *h, int32_t pos, const int32_t *tokens_d, const uint8_t *mask_d);

/* Copy fp32 logits[B][vocab] of the last forward into host memory (syncs). */
int llm_get_logits(llm_t *h, float *out);
/* Same into device memory (async). */
int llm_get_logits_d(llm_t *h, float *out_d);
/* Copy the token buffer rows [0, B) columns [0, n_cols) into host memory as
 * int32[B][n_cols] (syncs). */
int llm_get_tokens(llm_t *h, int32_t n_cols, int32_t *out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the draw of
 * llm_sample_d on caller logits, with no handle and no allocation.
 * logits_d[B][V] (fp32), uniforms_d[B] and out_d[B] are device pointers
 * owned by the caller; the work is queued on hip_stream (NULL: the default
 * stream) and the call does not synchronise.  temperature <= 0 is greedy
 * argmax; otherwise the temperature softmax and exact top-p of llm_sample.
 * Vocabularies above 32768 (or not a multiple of 4) stage the probabilities
 * in a static device buffer of 4194304 floats (16 MiB, one per GPU, held
 * until the process ends): B * V beyond that is LLM_EINVAL.  Calls that
 * overlap on one GPU share that buffer and race.  Returns LLM_OK, LLM_EINVAL
 * (arguments; nothing queued) or LLM_EDEVICE (a failed launch);
 * llm_last_error(NULL) gives the calling thread's last message. */
int llm_sample_logits_static(const float *logits_d, int32_t B, int32_t V, float temperature,
                             float top_p, const float *uniforms_d, int32_t *out_d, void *hip_stream);

/* Top-p draw on caller-supplied probabilities probs[B][vocab] (host, fp32)
 * with the exact rule of llm_sample; out[B] receives the token ids (syncs).
 * For checking the sampler on identical inputs. */
int llm_sample_probs(llm_t *h, const float *probs, int32_t B, float top_p,
                     const float *uniforms, int32_t *out);

/* Wait for all queued work. */
int llm_sync(llm_t *h);

/* ---- inspection and single-operation entry points (device pointers) ----
 * These run one kernel of the forward pass in isolation on the handle's
 * stream, for parity checks of each step. */

/* Read `count` logical elements [first, first+count) of a weight tensor in
 * its logical row-major [out][in] order, as stored (uint16 binary16 bit
 * patterns for LLM_F16, float for LLM_F32), into host memory.  Tensor ids:
 * 0 tok_embeddings, 1 output head, 16 + 8*layer + {0 wq, 1 wk, 2 wv, 3 wo,
 * 4 w1, 5 w2, 6 w3}. */
int llm_read_weights(llm_t *h, int32_t tensor_id, int64_t first, int64_t count, void *out);

/* y[M][dim] = RMSNorm(x[M][dim]) (walkthrough section 3.2) in the storage
 * type. */
int llm_op_rmsnorm(llm_t *h, const void *x_d, int32_t M, void *y_d);

/* y[M][N] = round(W x) for one of the model's packed matrices, plain store:
 *  mat 0: layer's [wq; wk; wv] (N = (n_heads + 2 n_kv_heads) * head_dim),
 *  mat 1: layer's wo (N = dim), mat 2: layer's w1/w3 interleaved in blocks of
 *  8 rows (packed row 16j + r is w1 row 8j + r for r < 8, w3 row 8j + r - 8
 *  otherwise; N = 2 * ffn), mat 3: layer's w2 (N = dim), mat 4: output head
 *  (N = vocab; layer ignored).  x is [M][K] in the storage type. */
int llm_op_linear(llm_t *h, int32_t layer, int32_t mat, const void *x_d, int32_t M, void *y_d);

/* Write caller K/V rows into the layer's cache: k_d, v_d are
 * [B][T][n_kv_heads][head_dim] in the storage type, for positions
 * pos0..pos0+T-1 of rows 0..B-1. */
int llm_op_kv_write(llm_t *h, int32_t layer, const void *k_d, const void *v_d, int32_t B,
                    int32_t T, int32_t pos0);

/* Attention of q[B][T][n_heads][head_dim] at positions pos0..pos0+T-1 over
 * the layer's cached keys 0..pos (causal), out in the same shape.  T == 1
 * runs the decode kernel (keys split over the waves of one workgroup per
 * (row, KV head)), T > 1 with pos0 == 0 the causal prefill kernel. */
int llm_op_attention(llm_t *h, int32_t layer, const void *q_d, int32_t B, int32_t T,
                     int32_t pos0, void *out_d);

/* One TransformerBlock (walkthrough section 3.7: h = x +
 * attention(attention_norm(x)), out = h + feed_forward(ffn_norm(h))) of
 * layer `layer` on caller rows: x_d is [B][T][dim] in the storage type, the
 * residual rows entering the layer for positions pos0..pos0+T-1 of batch
 * rows 0..B-1; on return it holds the rows leaving the layer.  The kernels,
 * launch forms and rounding are those a whole pass uses for the same rows:
 * T == 1 with pos0 >= 1 runs the decode-step forms (attention over cached
 * keys 0..pos0), anything else the prefill forms (causal over the T rows
 * after the cached prefix [0, pos0)).  Writes the layer's KV cache at
 * positions pos0..pos0+T-1; keys below pos0 must have been written before
 * (by a pass or by earlier calls for this layer).  Leaves the handle's
 * tokens, logits and positions as they were; overwrites the activation
 * workspace.  For checking the forward pass one layer at a time against
 * the oracle fed the same input.  Synchronises. */
int llm_op_layer(llm_t *h, int32_t layer, void *x_d, int32_t B, int32_t T, int32_t pos0);

/* Run `reps` decode steps at prev_pos without the captured graph, with HIP
 * events on the handle's stream around every kernel, and write the mean
 * milliseconds per step of each kernel class to ms_out[9]: 0 embedding,
 * 1 RMSNorm, 2 wq|wk|wv product (with RoPE and the KV write), 3 attention,
 * 4 wo product, 5 w1|w3 product (with SwiGLU), 6 w2 product, 7 output head,
 * 8 first-to-last event.  Same preconditions and effects as llm_decode;
 * synchronises. */
int llm_profile_decode(llm_t *h, int32_t prev_pos, int32_t reps, float *ms_out);

/* As llm_prefill_d run `reps` times, with the same per-class event timing
 * as llm_profile_decode (ms_out[9], mean per prefill).  Same arguments,
 * preconditions and effects as llm_prefill_d; synchronises. */
int llm_profile_prefill(llm_t *h, const int32_t *tokens_d, int32_t B, int32_t T, int32_t reps, float *ms_out);

/* Time the decode step's weight products on their own, at the current
 * batch and in the launch configuration, epilogue and RMSNorm fusion of a
 * decode step.  Six passes, each captured once as a HIP graph and replayed
 * between two HIP events on the handle's stream: pass k < 5 launches product
 * kind k (0 wq|wk|wv, 1 wo, 2 w1|w3, 3 w2, 4 output head) over every layer
 * (the head once) `reps` times; pass 5 launches all the products of a decode
 * step in forward order `reps` times.  us_out[6] receives the mean
 * microseconds per launch of each pass.  The launches read and write the
 * workspace, the logits and the KV cache at the last decoded position with
 * meaningless values, so the handle needs a new prefill before the next
 * decode.  Requires a prefilled fp16 handle; synchronises. */
int llm_profile_projections(llm_t *h, int32_t reps, float *us_out);

#ifdef __cplusplus
}
#endif

#endif /* LLM_H */
