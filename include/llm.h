/*
 * llm.h - C ABI of the MI355X (gfx950) Llama-family forward pass.
 *
 * The library runs the per-token forward pass of a Llama-family decoder as
 * described by "The Forward Pass in Java" (codeloopback.dev, Examples 3-10 and
 * Project 18) and "What a Llama model computes, and why" (branes-ai synapse
 * pages, sections 2 and 4): embedding-row gather; per layer RMSNorm, the Q/K/V
 * products (+ optional biases), RoPE (normal or NEOX pairs), an F16 KV cache,
 * grouped-query attention, the output product and residual add, RMSNorm, the
 * SwiGLU feed-forward block and residual add; then the final RMSNorm, the
 * vocabulary product and the greedy argmax (first index of the strict maximum).
 *
 * Conventions
 *  - Every call returns an int status: LLM_OK (0) or a negative LLM_ERR_*. No
 *    C++ exception crosses the ABI. Arguments are validated before any device
 *    work is enqueued, so a call that fails validation changes nothing.
 *  - A device failure poisons the context: every later call returns
 *    LLM_ERR_DEVICE until llm_free.
 *  - A context is used by one host thread at a time.
 *  - Pointers named d_* are device pointers (hipMalloc'd or allocated by the
 *    caller's framework on the same device); h_* are host pointers.
 *  - `hip_stream` is a hipStream_t (NULL = the default stream). All work of a
 *    context is enqueued on it.
 */
#ifndef LLM_H
#define LLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tensor type ids of the tensor set, as GGUF numbers them ("Loading GGUF with
 * the FFM API", Example 5 / Project 16): F32, F16 (IEEE binary16), and Q8_0
 * blocks of 32 values stored as {fp16 scale d, int8 qs[32]} = 34 bytes, value j
 * of a block decoding to d * qs[j] ("The Forward Pass in Java", Example 2). */
#define LLM_F32 0
#define LLM_F16 1
#define LLM_Q8_0 8

#define LLM_OK 0
#define LLM_ERR_ARG (-1)       /* NULL or out-of-range argument, bad config */
#define LLM_ERR_SHAPE (-2)     /* tensor dims differ from what the config implies */
#define LLM_ERR_DTYPE (-3)     /* unsupported tensor type, or mixed types where one is required */
#define LLM_ERR_MISSING (-4)   /* a required tensor is absent (or only some of the q/k/v biases) */
#define LLM_ERR_SIZE (-5)      /* nbytes smaller than the dims and type require */
#define LLM_ERR_TOKEN (-6)     /* token id outside [0, vocab) */
#define LLM_ERR_POS (-7)       /* decode position > cache length, or >= n_ctx */
#define LLM_ERR_CTX_FULL (-8)  /* prefill would run past n_ctx */
#define LLM_ERR_NONFINITE (-9) /* a NaN or infinity among the logits */
#define LLM_ERR_DEVICE (-10)   /* a HIP call failed; the context is poisoned */
#define LLM_ERR_OOM (-11)      /* device or host allocation failed */
#define LLM_ERR_LIMIT (-12)    /* a size beyond what these kernels support (see llm_load_weights) */

typedef struct llm_ctx llm_ctx;

/* One tensor of the flat tensor set. `name` follows llama.cpp's names
 * ("token_embd.weight", "blk.3.attn_q.weight", ...). `ne` lists dims innermost
 * first: a matrix of `out` rows of `in` values has n_dims = 2, ne = {in, out},
 * and row r starts at element r * in ("The Forward Pass in Java", Example 5).
 * A vector has n_dims = 1, ne = {n, 1}. `data` is a host pointer to the stored
 * bytes; it is only read during llm_load_weights / llm_plan. */
typedef struct {
    const char* name;
    int32_t dtype;
    int32_t n_dims;
    int64_t ne[2];
    const void* data;
    size_t nbytes;
} llm_tensor;

/* Hyperparameters ("The Forward Pass in Java", Example 1). head_dim is given
 * explicitly; q has n_heads*head_dim values and k, v n_kv_heads*head_dim.
 * rope_dims (n_rot) is the number of rotated dimensions of each head, even,
 * <= head_dim; rope_neox selects NEOX pairs (i, i + n_rot/2) instead of the
 * normal pairs (2i, 2i+1) (Example 6). n_ctx is the KV-cache capacity in
 * positions. eps is the RMSNorm epsilon, rope_base the RoPE frequency base.
 *
 * Attention span ("The Engine", its sliding:N and sink:s,w attentions): with
 * attn_window = 0 the query at position p attends rows 0..p; with
 * attn_window = w > 0 only rows p-w+1..p, plus rows 0..attn_sinks-1
 * (attn_sinks > 0 needs a window). The cache still holds every position.
 * Attention temperature ("What a Llama model computes, and why", section 6,
 * Mistral 3): the query at position p is scaled by
 * 1 + attn_temp_scale * ln(floor(p / attn_temp_len) + 1); attn_temp_scale 0
 * turns it off, Mistral 3 uses 0.1 and 16384. Zero-filled fields give the
 * plain causal attention.
 *
 * YaRN ("What a Llama model computes, and why", section 6; the YaRN paper,
 * Peng et al., 2023): with yarn_factor s >= 1 (0 = off), pair i of base
 * frequency theta_i = rope_base^(-2i/rope_dims) completes
 * r = yarn_orig_ctx * theta_i / (2 pi) turns over the original context; a
 * ramp g(r), 0 below yarn_beta_slow and 1 above yarn_beta_fast (linear in
 * between; Ministral 3 uses 1 and 32), turns the angle a into
 * (1 - g) a / s + g a, and q and k are scaled by 1 + 0.1 ln s.
 *
 * numerics: 0 computes with float activations (the Java engine's numerics);
 * 1 rounds where llama.cpp rounds ("What a Llama model computes, and why",
 * section 8): a Q8_0 product's input to Q8_0 blocks (the quantizer of
 * "Loading GGUF with the FFM API", Example 8),
 * an F16 product's input to binary16, q to binary16 before q.k, and the
 * softmax probabilities to binary16 before they weight V. Both decode paths
 * and prefill implement both modes (the persistent step kernel as a variant
 * compiled for mode 1, with a second attention pass). */
typedef struct {
    int32_t dim, n_layers, n_heads, n_kv_heads, head_dim, ffn, vocab, n_ctx, rope_dims, rope_neox;
    float eps, rope_base;
    int32_t attn_window, attn_sinks;
    float attn_temp_scale;
    int32_t attn_temp_len;
    float yarn_factor;
    int32_t yarn_orig_ctx;
    float yarn_beta_fast, yarn_beta_slow;
    int32_t numerics;
} llm_config;

/*
 * Sizes of the three device arenas a context needs for this config and tensor
 * set (the weight layout depends on the tensor types and on whether
 * output.weight and the biases are present). Any output pointer may be NULL.
 * Returns the same validation errors as llm_load_weights.
 */
int llm_plan(const llm_config* cfg, const llm_tensor* tensors, int32_t n_tensors, size_t* weight_bytes,
             size_t* kv_bytes, size_t* scratch_bytes);

/*
 * Validates the tensor set, packs the weights into the device layout, builds
 * the RoPE table and prepares the per-token launch graph.
 *
 * Required tensors: token_embd.weight [dim, vocab], output_norm.weight [dim],
 * and for every layer l: blk.l.attn_norm.weight [dim], attn_q.weight
 * [dim, n_heads*head_dim], attn_k.weight and attn_v.weight [dim,
 * n_kv_heads*head_dim], attn_output.weight [n_heads*head_dim, dim],
 * ffn_norm.weight [dim], ffn_gate.weight and ffn_up.weight [dim, ffn],
 * ffn_down.weight [ffn, dim]. Optional: output.weight [dim, vocab] (absent means
 * the output product reuses token_embd, "tied embeddings", Example 9) and
 * blk.l.attn_{q,k,v}.bias (all three or none; added after the product and
 * before RoPE, Project 18), and rope_freqs.weight [rope_dims/2]: one divisor
 * per RoPE pair, pair i's angle theta_i becomes theta_i / f_i (Llama 3's
 * frequency factors, "What a Llama model computes, and why", sections 2.4 and
 * 6); its values must be finite and positive (LLM_ERR_ARG from
 * llm_load_weights otherwise). Matrices may be F32, F16 or Q8_0 (q, k and v
 * share one type, as do gate and up); norm gains, biases and divisors are F32.
 *
 * Limits (LLM_ERR_LIMIT): every matrix width (`in`) is a multiple of 32 and at
 * most 16384; head_dim is a multiple of 8 and at most 256; n_heads/n_kv_heads
 * at most 16; n_ctx at most 1<<20.
 *
 * d_weights, d_kv, d_scratch: caller-owned device arenas of at least the sizes
 * llm_plan reports, 256-byte aligned, which must outlive the context; any of
 * them may be NULL, and the library then allocates (and llm_free releases) it.
 * The caller may free the host tensor data after this call returns. On success
 * *out receives the context; on failure *out is NULL and nothing stays
 * allocated.
 */
int llm_load_weights(const llm_config* cfg, const llm_tensor* tensors, int32_t n_tensors, void* d_weights,
                     void* d_kv, void* d_scratch, void* hip_stream, llm_ctx** out);

/*
 * One token at position pos (Project 18, forward(token, pos)): requires
 * 0 <= token < vocab, 0 <= pos <= kv_len and pos < n_ctx. Writes K and V of
 * every layer at row pos, attends rows 0..pos, and sets kv_len = pos + 1 (a pos
 * below kv_len rewinds the sequence). The logits (vocab floats) are left in the
 * context's buffer (llm_logits) and, if d_logits is not NULL, also copied there.
 * If h_next is not NULL the call waits for the stream and stores the greedy
 * next token (first index of the strict maximum, Example 9); then it also
 * returns LLM_ERR_NONFINITE if a logit is NaN or infinite. With h_next NULL the
 * call only enqueues work.
 */
int llm_decode(llm_ctx* ctx, int32_t token, int32_t pos, float* d_logits, int32_t* h_next);

/*
 * Prefill of n tokens at positions kv_len .. kv_len+n-1 ("What a Llama model
 * computes, and why", section 4): the products run as matrix products over the
 * batch, token i attends rows 0..kv_len+i, K and V of all n positions are
 * written, and only the last token's logits are computed. Requires n >= 1,
 * every token in [0, vocab) and kv_len + n <= n_ctx (else LLM_ERR_CTX_FULL).
 * Afterwards kv_len += n. d_logits and h_next as for llm_decode.
 */
int llm_prefill(llm_ctx* ctx, const int32_t* h_tokens, int32_t n, float* d_logits, int32_t* h_next);

/*
 * Prefill with chosen output rows ("What a Llama model computes, and why",
 * section 4: the last layer only needs the rows whose logits are read). Same
 * tokens, positions, K/V writes, requirements and kv_len update as llm_prefill,
 * and the last layer's output product and FFN run only on the chosen rows.
 * h_rows (host, n_rows entries) lists prompt rows in 0..n-1, in any order,
 * repeats allowed; 1 <= n_rows <= n_ctx. h_rows NULL with n_rows == n asks for
 * every row in order. Output j, the logits of prompt row h_rows[j] (vocab
 * floats, before any softmax), goes to d_logits + j*vocab: d_logits is a
 * caller-owned device buffer of n_rows*vocab floats. Any bad argument returns
 * LLM_ERR_ARG (tokens: LLM_ERR_TOKEN; capacity: LLM_ERR_CTX_FULL) before any
 * device work, with kv_len unchanged. The call only enqueues work on the
 * context's stream; the context's own logits buffer (llm_logits) is not
 * written.
 */
int llm_prefill_rows(llm_ctx* ctx, const int32_t* h_tokens, int32_t n, const int32_t* h_rows, int32_t n_rows,
                     float* d_logits);

/*
 * Greedy generation without host round trips ("The Forward Pass in Java",
 * Example 12's loop with the greedy choice of Example 9): decodes `token` at
 * position kv_len, then n_steps-1 more steps, each feeding the previous step's
 * argmax at the next position, all on the device. h_tokens (host, n_steps
 * entries) receives the n_steps generated tokens; the call waits for the stream.
 * Requires kv_len + n_steps <= n_ctx. Afterwards kv_len += n_steps and
 * llm_logits holds the last step's logits.
 */
int llm_generate(llm_ctx* ctx, int32_t token, int32_t n_steps, int32_t* h_tokens);

/* A new sequence: kv_len = 0 ("The Engine", Attention.reset). The cache memory
 * is not cleared; reads are bounded by kv_len. */
int llm_reset(llm_ctx* ctx);

/* Releases the context and any arena the library allocated. NULL is a no-op. */
void llm_free(llm_ctx* ctx);

/* Text of the last error on this context ("" if none). Valid until the next
 * call on the context. A NULL ctx returns the last llm_load_weights error of
 * the calling thread. */
const char* llm_last_error(const llm_ctx* ctx);

/* Device pointer to the context's logits buffer (vocab floats), valid until
 * llm_free; its contents change with every decode/prefill/generate call. */
const float* llm_logits(const llm_ctx* ctx);

/* Current KV-cache length (the number of valid positions), or -1 for NULL. */
int32_t llm_kv_len(const llm_ctx* ctx);

/* Copies the binary16 bits of K and V of one layer at one position, each in the
 * pages' order kv_head * head_dim + i (n_kv_heads*head_dim values), to host
 * memory. Waits for the stream. Requires 0 <= pos < n_ctx; rows at or past
 * kv_len hold whatever was last written there. */
int llm_kv_read(const llm_ctx* ctx, int32_t layer, int32_t pos, uint16_t* h_k, uint16_t* h_v);

#ifdef __cplusplus
}
#endif
#endif /* LLM_H */
