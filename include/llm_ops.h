/*
 * llm_ops.h - per-kernel entry points on a loaded context.
 *
 * Each call runs one of the decode step's fused kernels on its own, with the
 * same kernel, arguments layout and launch configuration the step uses, on
 * caller-given inputs. They exist so a caller can check or time one stage of
 * the forward pass in isolation ("The Forward Pass in Java", Example 11 checks
 * the forward pass tensor by tensor). None of them changes kv_len. All return
 * LLM_OK or a negative LLM_ERR_* (include/llm.h), validate before any device
 * work, enqueue on the context's stream, and do not wait for it unless a host
 * output pointer is given. d_* are device pointers of the sizes named.
 */
#ifndef LLM_OPS_H
#define LLM_OPS_H

#include "llm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stages of one decode step, in order. */
#define LLM_STAGE_QKV 0    /* RMSNorm + Q/K/V products + bias + RoPE + F16 KV store */
#define LLM_STAGE_ATTN 1   /* grouped-query attention over the cache */
#define LLM_STAGE_O 2      /* output product + residual add */
#define LLM_STAGE_FFN_UP 3 /* RMSNorm + gate/up products + SwiGLU */
#define LLM_STAGE_DOWN 4   /* down product + residual add */
#define LLM_STAGE_LOGITS 5 /* final RMSNorm + vocabulary product + greedy argmax */
#define LLM_STAGE_STEP 6   /* one whole decode step (token 0 at position pos) */

/* QKV stage of `layer` at position pos (0 <= pos < n_ctx): h = rmsnorm(d_x)
 * * attn_norm ("The Forward Pass in Java", Example 4), q|k|v = W h (+ bias),
 * RoPE at pos on q and k (Example 6); writes rotated q (n_heads*head_dim floats)
 * to d_q and binary16 k, v to the layer's cache row pos (Example 10).
 * d_x: dim floats. */
int llm_op_qkv(llm_ctx* ctx, int32_t layer, int32_t pos, const float* d_x, float* d_q);

/* Attention stage of `layer` for one token at position pos (0 <= pos < n_ctx):
 * d_q (n_heads*head_dim floats, already rotated) attends cache rows 0..pos
 * (Example 7); writes n_heads*head_dim floats to d_out. */
int llm_op_attention(llm_ctx* ctx, int32_t layer, int32_t pos, const float* d_q, float* d_out);

/* Allocation-free variant of llm_op_attention, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, kernels and result as
 * llm_op_attention; what those kernels write besides d_out (the position
 * state, the per-split partials (m, l, o) and, with numerics = 1, the span
 * maxima and sums) goes to a file-scope device array of
 * LLM_NOALLOC_SCRATCH_BYTES bytes that each device holds until the process
 * ends, instead of the context's scratch arena. Nothing is allocated: no
 * hipMalloc, hipFree or allocating library call. Nothing in the array needs
 * to start at zero (every value a call reads, the call writes first).
 * Requires the context's device to be the current device (else LLM_ERR_ARG);
 * returns LLM_ERR_LIMIT when the context's shape needs more than the array:
 * 256 + n_split * n_kv_heads * (n_heads / n_kv_heads) * (head_dim + 2) * 4
 * + n_heads * 8 bytes (each part rounded up to 256 bytes), n_split = 512 /
 * n_kv_heads position splits. Every call on one device shares that device's
 * array, so calls that overlap on one device (from other streams or threads)
 * race; calls in order on one stream do not. */
#define LLM_NOALLOC_SCRATCH_BYTES (4u << 20)
int llm_op_attention_noalloc(llm_ctx* ctx, int32_t layer, int32_t pos, const float* d_q, float* d_out);

/* Output stage: d_x (dim floats) += W_o d_in (d_in: n_heads*head_dim floats). */
int llm_op_o(llm_ctx* ctx, int32_t layer, const float* d_in, float* d_x);

/* FFN-up stage: h = rmsnorm(d_x) * ffn_norm; d_u[j] = silu(W_gate h)_j *
 * (W_up h)_j (Example 8); d_u: ffn floats. */
int llm_op_ffn_up(llm_ctx* ctx, int32_t layer, const float* d_x, float* d_u);

/* Down stage: d_x (dim floats) += W_down d_u (d_u: ffn floats). */
int llm_op_down(llm_ctx* ctx, int32_t layer, const float* d_u, float* d_x);

/* Logits stage on residual vector d_x (dim floats): final RMSNorm, the
 * vocabulary product into the context's logits buffer (and d_logits if not
 * NULL) and the greedy argmax (Example 9); *h_next (if not NULL) receives it,
 * after waiting for the stream. */
int llm_op_logits(llm_ctx* ctx, const float* d_x, float* d_logits, int32_t* h_next);

/* Writes rows pos0 .. pos0+n_pos-1 of `layer`'s K and V caches from host
 * binary16 bits laid out as the pages' flat cache, [pos][n_kv_heads*head_dim]
 * (Example 7). Requires pos0 >= 0 and pos0 + n_pos <= n_ctx. Waits. */
int llm_op_kv_write(llm_ctx* ctx, int32_t layer, int32_t pos0, int32_t n_pos, const uint16_t* h_k,
                    const uint16_t* h_v);

/* Average device time in milliseconds of one launch of `stage` (LLM_STAGE_*)
 * of `layer`, over n_launch back-to-back launches bracketed by HIP events on
 * the context's stream, with the context's own scratch buffers as inputs
 * (their contents do not affect the time). The attention stage runs at
 * position pos. LLM_STAGE_STEP times a whole decode step at position pos
 * (with layer ignored; on the persistent path one launch of the step kernel,
 * the state being set once before the timed launches); it writes cache row
 * pos of every layer. Waits. */
int llm_op_time(llm_ctx* ctx, int32_t stage, int32_t layer, int32_t pos, int32_t n_launch, float* h_ms);

/* The prompt pass's products of one layer ("What a Llama model computes, and
 * why", section 5: prefill is the same products over a batch of rows). */
#define LLM_PRODUCT_QKV 0     /* q|k|v rows (+ bias), stored */
#define LLM_PRODUCT_O 1       /* output product, added to the residual */
#define LLM_PRODUCT_GATE_UP 2 /* gate|up rows + SwiGLU */
#define LLM_PRODUCT_DOWN 3    /* down product, added to the residual */

/* Average device time in milliseconds of one launch of prefill product
 * `product` (LLM_PRODUCT_*) of `layer` over n_rows rows (1 <= n_rows <=
 * llm_op_prefill_chunk()), over n_launch back-to-back launches bracketed by
 * HIP events on the context's stream: the matrix-core kernel the prompt pass
 * runs for that product, with the same operands (the rounding mode's codes
 * included) and epilogue, over the context's own batch buffers as inputs
 * (their contents do not affect the time). A residual product split over K
 * leaves its partial sums in the workspace, as in the prompt pass, whose next
 * RMSNorm adds them; that reduction is not timed. The context's cache and
 * kv_len are untouched, but the batch buffers are overwritten. Waits. Returns
 * LLM_ERR_ARG for a bad product, layer, row count, launch count or pointer. */
int llm_op_time_prefill_product(llm_ctx* ctx, int32_t product, int32_t layer, int32_t n_rows, int32_t n_launch,
                                float* h_ms);

/* Which kernel runs the context's decode steps: 0 for the captured launch
 * graph (six launches per layer plus the logits), 1 for the persistent step
 * kernel (one launch per token), 2 for a persistent step kernel
 * compiled for the model's shape (the 2048-wide, 64-dim-head, 4-query-heads-
 * per-KV-head shape with 8192 FFN units: Q8_0 layers with F32 vocabulary
 * rows, or F16 layers with F16 vocabulary rows). The persistent kernel is used
 * unless the environment variable LLM_STEP is "graph" at load time, provided
 * the device can co-schedule one block per compute unit, all layer matrices
 * share one weight type and G*head_dim (G = n_heads/n_kv_heads) is a multiple
 * of 32. Returns the kind, or a negative LLM_ERR_* for a NULL context. */
int llm_op_step_kind(llm_ctx* ctx);

/* Rows per prefill batch: llm_prefill and llm_prefill_rows run a prompt
 * through the layers in consecutive chunks of this many rows (the last one
 * shorter), each chunk's rows attending to the cache rows before them and to
 * the chunk's own rows up to themselves ("What a Llama model computes, and
 * why", the prefill/decode section). A context's batch buffers hold this
 * many rows. No context needed; never fails. */
int llm_op_prefill_chunk(void);

/* Whether the context's prefill runs its Q8_0 layer products as integer
 * matrix-core products ("What a Llama model computes, and why", sections 5 and
 * 8: activations rounded to 8-bit Q8_0 blocks and dotted with the 8-bit
 * weights as integers): 1 when the model has Q8_0 layer matrices and
 * numerics = 1 (each 32-deep block's exact int32 sum times the two block
 * scales, from the int8 codes), 0 otherwise (the float numerics' products on
 * the binary16 codes, or F16/F32 layers). Returns a negative LLM_ERR_* for a
 * NULL context. */
int llm_op_prefill_int8(llm_ctx* ctx);

/* Wall-clock stamps (100 MHz device clock) that block 0 of the last decode-step
 * launch took at its start and after each of its 5*n_layers + 1 barriers:
 * stamp k+1 - stamp k is the time of phase k (per layer: QKV, attention,
 * split merge + output, gate/up, down; then the logits; with numerics = 1 the
 * barrier between the two attention passes takes no stamp, so both passes
 * count as the attention phase). h_out receives
 * 5*n_layers + 2 values. Available only when the context was loaded with the
 * environment variable LLM_STEP_TRACE=1 and runs the persistent step kernel;
 * otherwise LLM_ERR_ARG. Waits. */
int llm_op_step_trace(llm_ctx* ctx, uint64_t* h_out, int32_t n);

/* Moves the sequence end back: kv_len = len, for 0 <= len <= kv_len ("The
 * Forward Pass in Java", Example 13: rewritten cache entries give the same
 * results). */
int llm_rewind(llm_ctx* ctx, int32_t len);

#ifdef __cplusplus
}
#endif
#endif /* LLM_OPS_H */
