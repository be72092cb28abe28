/*
 * q3.h -- C ABI of libq3: the forward pass of a Qwen3-0.6B-shaped decoder on
 * one AMD Instinct MI355X (gfx950), in its prefill and greedy-decode phases.
 *
 * The calls follow the generation loop of "Dentro de un LLM: Inferencia en
 * Python puro para Qwen3-0.6B en MLX" (reactapp.top), Paso 9: load the
 * weights once; prefill a whole prompt, which fills the KV cache and yields
 * the logits of its last position and the greedy next token; then decode one
 * token per call, appending its key and value to the cache.
 *
 * Conventions for every call:
 *   - Pointers named d_* are device (HBM) pointers; the others are host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is queued on it; device outputs are valid once it is synchronised.
 *   - The caller owns all device memory (weights, KV arena, workspace,
 *     inputs, outputs) and passes raw pointers; libq3 never allocates device
 *     memory for them.  Borrowed pointers must outlive the model handle.
 *   - Every call returns a q3_status.  On failure a thread-local message is
 *     available from q3_last_error().  Argument, state and capacity errors are
 *     detected on the host before anything is queued, and leave the model
 *     unchanged.  Q3_E_HIP means a HIP call failed; the sequences touched by
 *     that call must then be reset.
 *   - Calls on one handle must not overlap (the caller serialises them).
 */
#ifndef Q3_H
#define Q3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q3_status {
  Q3_OK = 0,
  Q3_E_ARG = -1,          /* a bad argument: NULL pointer, bad shape, token ID out of range */
  Q3_E_STATE = -2,        /* call not valid in the current state (e.g. before q3_load_weights) */
  Q3_E_CAPACITY = -3,     /* the KV cache of a sequence or the arena would overflow */
  Q3_E_HIP = -4,          /* a HIP runtime call failed */
  Q3_E_UNSUPPORTED = -5   /* a shape or option the library does not handle */
} q3_status;

typedef enum q3_dtype { Q3_F32 = 0, Q3_BF16 = 1 } q3_dtype;

/* Most sequences in one prefill or decode call. */
#define Q3_MAX_BATCH 64

/* Model shape and capacity.  Paso 3 fixes rms_eps (1e-6), Paso 4 rope_theta
 * (1e6), Paso 5 the head counts (16 query, 8 key/value, width 128); the
 * vocabulary (151,936) and hidden size (1024) come from Pasos 2 and 7, the
 * SwiGLU width (3072) from Paso 6.
 * Supported: head_dim == 128; n_q_heads % n_kv_heads == 0 with a group of at
 * most 8; hidden, ffn and n_q_heads*128 multiples of 512; vocab a multiple
 * of 16.  `dtype` is the type of the weights, the KV cache and every input of
 * a projection (Q3_BF16), or float32 throughout (Q3_F32, which also limits a
 * sequence to 8192 positions). */
typedef struct q3_config {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;
  float rms_eps;
  double rope_theta;
  int32_t dtype;              /* q3_dtype */
  int32_t max_slots;          /* number of sequence slots */
  int64_t max_positions;      /* longest sequence, in tokens (RoPE table rows) */
  int64_t max_prefill_tokens; /* most tokens in one q3_prefill call (workspace sizing) */
  int64_t kv_tokens;          /* KV arena capacity in tokens, summed over slots */
  int32_t untied_lm_head;     /* 0: the head is the embedding matrix (tied);
                                 1: a separate "lm_head.weight" (vocab, hidden) */
  int32_t weight_bits;        /* 0: projections in the model dtype; 8 or 4: the
                                 q/k/v/o/gate/up/down weights of every block
                                 are stored as affine group codes (groups of
                                 64 along the input dimension, float16 scale
                                 and offset per group, w ~ q * s + b), made at
                                 load time from the bf16 weights (Q3_BF16
                                 models only; embedding, head and norms stay
                                 as they are) */
} q3_config;

/* A named weight tensor in device memory, stored as the page's listings read
 * it: linear weights (out_features, in_features), applied as x @ W^T; norm
 * weights 1-D.  dtype must equal the model's dtype.  Names:
 *   model.embed_tokens.weight                      (vocab, hidden); also the tied lm_head
 *   model.layers.{i}.input_layernorm.weight        (hidden)
 *   model.layers.{i}.self_attn.{q,k,v,o}_proj.weight
 *   model.layers.{i}.self_attn.{q,k}_norm.weight   (head_dim)
 *   model.layers.{i}.post_attention_layernorm.weight
 *   model.layers.{i}.mlp.{gate,up,down}_proj.weight
 *   model.norm.weight                              (hidden)
 *   lm_head.weight                                 (vocab, hidden); only with untied_lm_head = 1 */
typedef struct q3_tensor {
  const char* name;
  const void* data;   /* device pointer, contiguous row-major */
  int32_t dtype;      /* q3_dtype */
  int32_t ndim;       /* 1 or 2 */
  int64_t shape[2];
} q3_tensor;

typedef struct q3_model q3_model;

/* Validate `cfg` and create a handle (host memory only).  *out receives it. */
q3_status q3_create(const q3_config* cfg, q3_model** out);
/* Release the handle and its captured graphs; borrowed memory is untouched. */
void q3_destroy(q3_model* m);

/* Bytes of device memory the caller must provide to q3_bind_memory (0 for an
 * invalid config).  Weights: packed projections, norm weights as float32 and
 * the RoPE cos/sin table.  KV: the arena.  Workspace: activations, partial
 * sums, counters and per-slot state. */
size_t q3_weights_bytes(const q3_config* cfg);
size_t q3_kv_bytes(const q3_config* cfg);
size_t q3_workspace_bytes(const q3_config* cfg);

/* Hand the model its three device regions (each 256-byte aligned and at least
 * the size asked for).  Builds the RoPE table (host float64, stored float32),
 * clears counters and slot state.  Synchronises `stream`. */
q3_status q3_bind_memory(q3_model* m, void* d_weights, size_t weights_bytes, void* d_kv,
                         size_t kv_bytes, void* d_workspace, size_t workspace_bytes,
                         void* stream);

/* Copy the named tensors into the model's layout: q/k/v rows are stacked into
 * one projection, gate and up rows interleaved in runs of 16, norm weights
 * widened to float32.  Every name must be present exactly once with the
 * shape and dtype above.  The source tensors may be freed once `stream` has
 * been synchronised. */
q3_status q3_load_weights(q3_model* m, const q3_tensor* tensors, int32_t n, void* stream);

/* Checkpoints in the safetensors format (one file or shards): an 8-byte
 * little-endian header length, a JSON header of {name: {dtype, shape,
 * data_offsets}}, then the tensor bytes.  Tensors carry the names listed at
 * q3_load_weights ("lm_head.weight" too when untied_lm_head = 1), each exactly
 * once across the files, stored as BF16 for a Q3_BF16 model or F32 for a
 * Q3_F32 model.
 *
 * q3_checkpoint_validate: reads and checks only the headers against `cfg`
 * (host only: no device, no model).  Q3_E_ARG names the first problem (an
 * unreadable or malformed header, an unknown, repeated or missing tensor, a
 * wrong shape, a byte range outside the file); Q3_E_UNSUPPORTED a dtype other
 * than the model's.
 * q3_checkpoint_staging_bytes: size of the device buffer q3_load_safetensors
 * needs (the largest tensor), 0 for an invalid config.
 * q3_load_safetensors: validates as above, then streams every tensor through
 * pinned host memory (allocated and freed by the call) into d_staging and from
 * there into the model's layout, as q3_load_weights does.  Synchronises
 * `stream`; d_staging may be freed afterwards.  On an error the model is left
 * unloaded. */
q3_status q3_checkpoint_validate(const q3_config* cfg, const char* const* paths, int32_t n_paths);
size_t q3_checkpoint_staging_bytes(const q3_config* cfg);
q3_status q3_load_safetensors(q3_model* m, const char* const* paths, int32_t n_paths, void* d_staging,
                              size_t staging_bytes, void* stream);

/* Give slot `slot` a KV region of `capacity_tokens` (rounded up to 64) from
 * the arena, and empty it.  A slot can be allocated once per arena reset. */
q3_status q3_seq_alloc(q3_model* m, int32_t slot, int64_t capacity_tokens, void* stream);
/* Empty the given slots (length 0), keeping their regions.  Queued on
 * `stream` without synchronising it. */
q3_status q3_seq_reset(q3_model* m, int32_t n, const int32_t* slots, void* stream);
/* Free every slot region (the whole arena becomes available again). */
q3_status q3_kv_reset(q3_model* m, void* stream);
/* Host-side length of a slot (tokens cached), as queued so far. */
q3_status q3_seq_length(const q3_model* m, int32_t slot, int64_t* out);

/* Prefill flags. */
#define Q3_PREFILL_ALL_LOGITS 1u  /* d_logits receives [T, vocab]: every position */

/* Prefill n_seqs sequences at once (Paso 9's first forward call, packed as
 * one variable-length batch).  Sequence b consists of tokens
 * d_tokens[h_cu_seqlens[b] .. h_cu_seqlens[b+1]), uses slot h_slots[b] and
 * attends causally to its own tokens.  A slot that already holds P_b tokens
 * (an earlier prefill or decode) is continued: the new tokens sit at
 * positions P_b, P_b + 1, .. and also attend to the cached ones, so a prompt
 * fed in chunks gives what one prefill of the whole prompt gives, up to
 * rounding (chunked prefill).  An empty slot starts at position 0.
 *   h_cu_seqlens: n_seqs+1 non-decreasing offsets, [0] = 0, each length >= 1,
 *                 total T <= max_prefill_tokens.
 *   d_tokens:     int32 [T] in device memory, so IDs are not checked on the
 *                 host (a caller holding a host copy checks it first with
 *                 q3_check_tokens).  An ID outside [0, vocab) reaching the
 *                 kernels gives that row a zero embedding and raises error
 *                 bit 1 (see q3_error_flags); the call still completes and
 *                 advances its slots, so their caches then hold meaningless
 *                 entries: reset them (q3_seq_reset) after bit 1 is seen.
 *   d_logits:     float [n_seqs, vocab] logits of each last position, or
 *                 [T, vocab] with Q3_PREFILL_ALL_LOGITS; may be NULL without
 *                 that flag.
 *   d_next:       int32 [n_seqs] greedy next token (largest logit, lowest
 *                 index on ties; Paso 8).
 * Errors: Q3_E_STATE if a slot is unallocated; Q3_E_CAPACITY if P_b + L_b
 * exceeds the slot or max_positions, or (bf16 model, some P_b > 0) if the
 * sum over the call of roundup(P_b + L_b, 64) exceeds
 * max(max_prefill_tokens, max_positions) + 64 * 64: the fp16 staging of the
 * values every key of the call needs (split such a call). */
q3_status q3_prefill(q3_model* m, int32_t n_seqs, const int32_t* h_slots,
                     const int32_t* h_cu_seqlens, const int32_t* d_tokens, float* d_logits,
                     int32_t* d_next, uint32_t flags, void* stream);

/* One greedy decode step for n_seqs sequences (Paso 9's loop body): token
 * d_tokens[b] goes to slot h_slots[b] at position = that slot's length; its
 * key and value are appended to the cache.
 *   d_tokens: int32 [n_seqs] (typically the previous call's d_next); an ID
 *             outside [0, vocab) is handled as in q3_prefill (error bit 1,
 *             the slots still advance).
 *   d_logits: float [n_seqs, vocab] or NULL.
 *   d_next:   int32 [n_seqs].
 * Positions are read from device-resident slot state, so with graphs enabled
 * (the default, on a non-null stream) the step is recorded once per
 * (n_seqs, slots, pointers, stream) and replayed afterwards.
 * Errors: Q3_E_STATE if a slot is empty; Q3_E_CAPACITY if a slot is full. */
q3_status q3_decode_step(q3_model* m, int32_t n_seqs, const int32_t* h_slots,
                         const int32_t* d_tokens, float* d_logits, int32_t* d_next,
                         void* stream);

/* Host-side check of token IDs (Paso 1: IDs index the vocabulary): Q3_OK
 * when every h_tokens[i], i < n, lies in [0, vocab); Q3_E_ARG naming the first
 * that does not.  For callers that hold the IDs on the host before copying
 * them to d_tokens; touches no device state. */
q3_status q3_check_tokens(const q3_model* m, const int32_t* h_tokens, int64_t n);

/* Temperature + top-p sampling (Paso 8) of n_rows logit rows, e.g. the
 * d_logits of q3_decode_step or q3_prefill; its d_next stays the greedy pick,
 * this call writes the sampled token of row r to d_next[r].
 *   d_logits:    float [n_rows][ld], ld >= vocab; columns 0..vocab-1 used.
 *   temperature: 0 = greedy (largest logit, lowest ID on ties); otherwise a
 *                finite value >= 1e-30 dividing the logits before the softmax.
 *   top_p:       finite; the kept set is the shortest run of tokens, in order
 *                of decreasing probability (equal probabilities by increasing
 *                ID), whose running sum reaches top_p (<= 0: the top token;
 *                >= 1: every token).
 *   d_uniform:   float [n_rows], one uniform number in [0, 1) per row (values
 *                outside are clamped); the sampled token is the kept token
 *                whose renormalised running sum, in the same order, first
 *                exceeds it.  Unused (may be NULL) when temperature is 0.
 * Probabilities are computed in float32 (exp of the shifted logits), their
 * sums exactly on a 2^-40 fixed-point grid, so the result is deterministic.
 * A row with a non-finite logit yields token 0 and raises error bit 2.
 * Queued on `stream`; reads no model state besides the vocabulary size. */
q3_status q3_sample(q3_model* m, int32_t n_rows, const float* d_logits, int64_t ld, float temperature,
                    float top_p, const float* d_uniform, int32_t* d_next, void* stream);

/* Options. */
#define Q3_OPT_DECODE_GRAPH 1  /* value 0/1: record decode steps as HIP graphs (default 1) */
q3_status q3_set_option(q3_model* m, int32_t option, int64_t value);

/* Synchronise `stream`, return and clear the device error bits raised by
 * kernels: 1 = token ID out of range, 2 = non-finite logit, 4 = a position
 * outside its slot. */
q3_status q3_error_flags(q3_model* m, uint32_t* out, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* q3_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* Q3_H */
