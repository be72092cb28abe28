/*
 * q3_ops.h -- single-kernel entry points of libq3, for parity tests and
 * kernel benchmarks.  Each runs one step of the forward pass of "Dentro de un
 * LLM: Inferencia en Python puro para Qwen3-0.6B en MLX" on explicit device
 * buffers, with the same kernels q3_prefill / q3_decode_step use.
 *
 * Conventions are those of q3.h: d_* pointers are device memory, the others
 * host memory; `stream` is a hipStream_t as void*; status codes and
 * q3_last_error() report failures.  No call allocates device memory: kernels
 * that need scratch take `d_ws` of at least the size the matching
 * *_workspace_bytes call returns.  Unlike the model calls, these synchronise
 * the stream after host-to-device copies of small tables (test use only).
 *
 * bf16 data is passed as its 16-bit patterns.
 */
#ifndef Q3_OPS_H
#define Q3_OPS_H

#include <stddef.h>
#include <stdint.h>

#include "q3.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Paso 2: d_out[r][:] = table[ids[r]][:] as float32 (table dtype = dtype).
 * An ID outside [0, vocab) gives a zero row and sets bit 1 of *d_err. */
q3_status q3op_embed(int32_t dtype, const int32_t* d_ids, int32_t n, const void* d_table, int32_t vocab,
                     int32_t dim, float* d_out, uint32_t* d_err, void* stream);

/* Paso 3: d_out[r] = x[r] * rsqrt(mean(x[r]^2) + eps) * w, rows of `dim`
 * (a multiple of 256) float32 values; output float32 or bf16 (out_dtype). */
q3_status q3op_rmsnorm(int32_t out_dtype, const float* d_x, int32_t rows, const float* d_w, int32_t dim,
                       float eps, void* d_out, void* stream);

/* Projection kernels: out = X[M,K] . W[N,K]^T with epilogue `epi`:
 *   0 store float32 out[M][ldo]; 1 add into float32 out[M][ldo];
 *   2 SwiGLU: W rows packed in runs of 16 gate rows then 16 up rows,
 *     out[m][j] = silu(gate_j) * up_j written in X's dtype (ldo >= N/2);
 *   3 logits: store float32 out[M][ldo] and d_next[m] = argmax (lowest index
 *     on ties).  With kernel 1 or 4 and d_next == NULL only the logits and
 *     the kernel's per-block (max, index) partials are produced (one launch).
 * kernel 0 = bf16 MFMA tiled GEMM (prefill; epi 0-2; any M; K % 64 == 0;
 * ldo % 4 == 0 and d_out 16-byte aligned (8 for SwiGLU);
 * the residual epilogue splits K over up to four blocks when the output has
 * fewer than 256 tiles of 64 x 64, merging the slices in a fixed order, and
 * then needs q3op_linear_workspace_bytes of workspace, else Q3_E_ARG);
 * kernel 1 = bf16 weight-streaming kernel (decode and lm_head; M <= 64);
 * kernel 2 = float32 GEMV (float32 model);
 * kernel 3 = bf16 row-per-wavefront GEMV (decode with M <= 4, epi 0 or 1,
 * K a multiple of 512);
 * kernel 4 = bf16 single-row GEMV (M = 1, epi 0-3, K = 512 * {1,2,4,6,8};
 * SwiGLU needs N % 32 == 0; out is dense, ldo is ignored);
 * kernel 5 = bf16 streaming lm_head (epi 0 or 3, M <= 64, N % 16 == 0, K in
 * {512, 1024, 1536, 2048}, 16 * ceil(M/16) rows of K bf16 within 156 KiB; the
 * rows of X stay on chip while the weight rows stream past them once).
 * bf16 kernels take bf16 X and W. */
#define Q3OP_GEMM 0
#define Q3OP_SKINNY 1
#define Q3OP_GEMV_F32 2
#define Q3OP_ROWDOT 3  /* bf16 row-per-wavefront GEMV (decode, M <= 4, epi 0-1) */
#define Q3OP_ROWGEMV 4 /* bf16 single-row GEMV (decode batch 1, epi 0-3) */
#define Q3OP_HEADSTREAM 5 /* bf16 streaming lm_head (decode batches, epi 0 or 3) */
size_t q3op_linear_workspace_bytes(int32_t kernel, int32_t epi, int32_t M, int32_t N, int32_t K);
q3_status q3op_linear(int32_t kernel, int32_t epi, const void* d_x, int32_t M, const void* d_w, int32_t N,
                      int32_t K, void* d_out, int64_t ldo, int32_t* d_next, void* d_ws, size_t ws_bytes,
                      void* stream);

/* q3op_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, epilogues and validation, with the workspace taken from
 * a static device array of Q3OP_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends (its address is looked up
 * once per device, on the first call with that device current).  The caller
 * still passes inputs and outputs.  A call whose
 * q3op_linear_workspace_bytes(kernel, epi, M, N, K) exceeds the scratch
 * returns Q3_E_CAPACITY before anything is queued.  The call allocates
 * nothing and clears what must start at zero (split counters) with a fill
 * kernel on `stream`.  Every call on one GPU shares that GPU's scratch, so
 * calls that overlap on one GPU (different streams or threads without
 * ordering) race; calls queued on one stream are ordered. */
#define Q3OP_NOALLOC_SCRATCH_BYTES (16u << 20)
q3_status q3op_linear_noalloc(int32_t kernel, int32_t epi, const void* d_x, int32_t M, const void* d_w, int32_t N,
                              int32_t K, void* d_out, int64_t ldo, int32_t* d_next, void* stream);

/* Pasos 3 + 5: a decode projection with RMSNorm fused into its prologue:
 * X = bf16(x * rsqrt(mean(x^2) + eps) * g) from float32 rows d_x [M][K] and
 * float32 weight d_gnorm [K], then epilogue `epi` as in q3op_linear.
 * kernel 1 (weight-streaming, M <= 64, epi 0-3) or kernel 4 (single row,
 * M = 1, epi 0 or 2).  Workspace: q3op_linear_workspace_bytes(kernel, ...). */
q3_status q3op_norm_linear(int32_t kernel, int32_t epi, const float* d_x, int32_t M, const float* d_gnorm,
                           float eps, const void* d_w, int32_t N, int32_t K, void* d_out, int64_t ldo,
                           int32_t* d_next, void* d_ws, size_t ws_bytes, void* stream);

/* A one-layer KV arena for the attention ops: sequence b owns the elements
 * [h_base[b], h_base[b] + 2*n_kv*h_cap[b]*128) of d_kv (dtype elements):
 * keys (cap*128 elements per kv head) then values [n_kv][cap/32][128][32]
 * (32-key blocks, each transposed: value dim d of key t at
 * ((t/32)*128 + d)*32 + t%32).  float32 keys are rows [cap][128].  bf16 keys
 * come in 32-key blocks of 4096 elements in MFMA operand order: with
 * k = t%32, dim d of key t sits at (t/32)*4096 + (((sbk*4 + d/32)*4 + (d/8)%4)*16
 * + fr)*8 + d%8, where sbk = (k/4)%2 and fr = (k/8)*4 + k%4.  h_cap[b] and
 * h_base[b] are multiples of 64 and d_kv is 16-byte aligned.  h_len[b] = tokens
 * already cached before the call.
 *
 * Pasos 4-5: per-head RMSNorm (q_norm / k_norm) then rotate-half RoPE at each
 * token's position, queries to d_q_out [T][n_q][128], keys and values into the
 * arena.  Rows of d_qkv [T][(n_q + 2 n_kv)*128] float32 hold q, k, v heads.
 * decode = 0: tokens h_cu[b]..h_cu[b+1] of sequence b sit at positions 0..;
 * decode = 1: token b sits at position h_len[b]. */
size_t q3op_rope_workspace_bytes(int32_t n_seqs, int32_t max_pos);
q3_status q3op_rope_append(int32_t dtype, const float* d_qkv, int32_t n_seqs, const int32_t* h_cu,
                           int32_t decode, const int64_t* h_base, const int32_t* h_cap, const int32_t* h_len,
                           void* d_kv, int32_t n_q, int32_t n_kv, const float* d_qn, const float* d_kn,
                           float eps, double theta, int32_t max_pos, void* d_q_out, void* d_ws,
                           size_t ws_bytes, void* stream);

/* Paso 5 attention over the arena above, output [T][n_q][128] in dtype.
 * kernel 0 = bf16 flash prefill (decode must be 0: query t of sequence b at
 * position t - h_cu[b], keys 0..L_b-1 of that sequence; the call first stages
 * the values as fp16 in the workspace, total_tokens = h_cu[n_seqs]);
 * kernel 1 = bf16 split-K decode (decode must be 1: query b at position
 * h_len[b], keys 0..h_len[b]); `splits` <= 0 picks the library's choice;
 * kernel 2 = float32 (either mode). */
#define Q3OP_ATTN_FLASH 0
#define Q3OP_ATTN_DECODE 1
#define Q3OP_ATTN_F32 2
size_t q3op_attention_workspace_bytes(int32_t kernel, int32_t n_seqs, int32_t total_tokens, int32_t n_q,
                                      int32_t n_kv, int32_t splits);
q3_status q3op_attention(int32_t kernel, const void* d_q, int32_t n_seqs, const int32_t* h_cu, int32_t decode,
                         const int64_t* h_base, const int32_t* h_cap, const int32_t* h_len, const void* d_kv,
                         int32_t n_q, int32_t n_kv, int32_t splits, void* d_out, void* d_ws, size_t ws_bytes,
                         void* stream);

/* Pasos 4-5 for bf16 decode in one kernel: from the fused projection rows
 * d_qkv [n_seqs][(n_q + 2 n_kv)*128] float32, the new token of sequence b sits
 * at position h_len[b]; its key (QK-Norm + RoPE) and value are written into
 * the arena above, and its queries (QK-Norm + RoPE) attend over keys
 * 0..h_len[b]; output d_out [n_seqs][n_q][128] bf16.  `smax` <= 0 picks the
 * library's split count. */
size_t q3op_decode_attn_fused_workspace_bytes(int32_t n_seqs, int32_t n_q, int32_t smax, int32_t max_pos);
q3_status q3op_decode_attn_fused(const float* d_qkv, int32_t n_seqs, const int64_t* h_base, const int32_t* h_cap,
                                 const int32_t* h_len, void* d_kv, int32_t n_q, int32_t n_kv, const float* d_qn,
                                 const float* d_kn, float eps, double theta, int32_t max_pos, int32_t smax,
                                 void* d_out, void* d_ws, size_t ws_bytes, void* stream);

/* The fused decode attention kernel above (Pasos 4-5) on a live bf16 model,
 * exactly as q3_decode_step launches it for layer `layer`: the query, key and
 * value rows are the model's projection workspace as the last call left
 * them, the key and value are written at each slot's current length (which
 * is not advanced, so repeated calls rewrite the same entry), the output goes
 * to the model's attention-output workspace.  Host validation as in
 * q3_decode_step (Q3_E_STATE for an empty slot, Q3_E_CAPACITY for a full
 * one); queued on `stream` without synchronising it, so a benchmark can time
 * repeated launches with events. */
q3_status q3op_model_decode_attention(q3_model* m, int32_t layer, int32_t n, const int32_t* h_slots, void* stream);

/* Paso 8 sampling of n_rows logit rows of width `vocab` (stride ld): the
 * same computation as q3_sample in q3.h, for any vocabulary size.  d_err is a
 * device word that receives error bit 2 for a row with a non-finite logit.
 * d_ws: q3op_sample_workspace_bytes(n_rows) bytes (about 0.6 MB per row, for
 * at most 64 rows; larger calls run 64 rows at a time), unused at
 * temperature 0. */
size_t q3op_sample_workspace_bytes(int32_t n_rows);
q3_status q3op_sample_top_p(const float* d_logits, int32_t n_rows, int32_t vocab, int64_t ld, float temperature,
                            float top_p, const float* d_uniform, int32_t* d_next, uint32_t* d_err, void* d_ws,
                            size_t ws_bytes, void* stream);

/* Weight-only affine group quantization (the page "Investigación de
 * rendimiento de Laya MLX", quantization section): groups of 64 along K,
 * `bits` = 8 or 4.
 * Codes [rows][K * bits / 8] bytes (4-bit: byte j holds k = 2j in its low
 * nibble and 2j + 1 in its high nibble); scale/offset words [rows][K / 64],
 * the float16 scale in the low 16 bits and the float16 offset in the high.
 * q3op_quantize: from bf16 weights [rows][K] (b = fp16(min), s = fp16((max -
 * min) / (2^bits - 1)), q = clamp(floor((w - b) / s + 1/2)), all in float32;
 * q = 0 when s is 0).
 * q3op_dequantize: bf16(q * s + b) into d_out [rows][K].
 * q3op_qlinear: one activation row against the quantized W[N,K] (K = 1024 *
 * 1..4): epi 0 store float32 out[N], 1 add into float32 out[N], 2 SwiGLU on
 * gate/up rows interleaved in runs of 16 (bf16 out[N/2]).  d_x is bf16 [K], or
 * with d_gnorm (epi 0 and 2) the float32 residual row normalised in the
 * kernel: bf16(x * rsqrt(mean(x^2) + eps) * g). */
q3_status q3op_quantize(const void* d_w, int32_t rows, int32_t K, int32_t bits, void* d_codes, void* d_sb,
                        void* stream);
q3_status q3op_dequantize(const void* d_codes, const void* d_sb, int32_t rows, int32_t K, int32_t bits, void* d_out,
                          void* stream);
q3_status q3op_qlinear(int32_t bits, int32_t epi, const void* d_x, const void* d_codes, const void* d_sb, int32_t N,
                       int32_t K, const float* d_gnorm, float eps, void* d_out, void* stream);
/* M = 1..64 activation rows (d_x bf16 [M][K], or with d_gnorm, M <= 16, the
 * float32 residual rows) against the quantized W[N,K] by the weight-streaming
 * kernel (K = 128 * 4..16 * 8 as for q3op_linear kernel 1), output rows of
 * stride ldo: epi 0 float32 store, 1 float32 add (split over K when d_ws is
 * given, q3op_qlinear_rows_workspace_bytes bytes), 2 SwiGLU (bf16). */
size_t q3op_qlinear_rows_workspace_bytes(int32_t M, int32_t N, int32_t K);
q3_status q3op_qlinear_rows(int32_t bits, int32_t epi, const void* d_x, int32_t M, const void* d_codes,
                            const void* d_sb, int32_t N, int32_t K, const float* d_gnorm, float eps, void* d_out,
                            int64_t ldo, void* d_ws, size_t ws_bytes, void* stream);

/* Kernel tuning knobs for benchmarks (process-wide, not thread-safe; they
 * affect q3_prefill too).  Returns Q3_E_ARG for an unknown key or value.
 * Q3OP_TUNE_GEMM_TILES: prefill GEMM tile configuration, -1 = automatic,
 *   0..11 = fixed tile shapes (listed in k_gemm.hip).
 * Q3OP_TUNE_FLASH_ROWS: prefill attention query rows per wavefront / 16,
 *   -1 = automatic, or 1, 2.
 * Q3OP_TUNE_ROWGEMV: single-row GEMV shape, -1 = automatic, else
 *   rows_per_wavefront (1, 2, 4, 8) + 256 * wavefronts_per_block (1..4);
 *   SwiGLU needs an even rows_per_wavefront.
 * Q3OP_TUNE_ATTN_SPLITS: upper bound on the key splits per (sequence, kv
 *   head) of bf16 decode attention, -1 = none, else 1..64; it only lowers
 *   the library's choice, so workspaces sized earlier stay large enough.
 *   Decode graphs captured before the change keep their split count.
 * Q3OP_TUNE_QKV_ROPE: large bf16 prefills fold QK-Norm, RoPE and the key
 *   append into the q/k/v projection's epilogue; -1 = automatic, 0 = never
 *   (the projection writes float32 rows and a separate kernel does the rest;
 *   both give the same bits).
 * Q3OP_TUNE_FLASH_TILES: query tiles per prefill attention block, -1 =
 *   automatic, 1, or 2 (eight wavefronts sharing each key/value tile). */
#define Q3OP_TUNE_GEMM_TILES 1
#define Q3OP_TUNE_FLASH_ROWS 2
#define Q3OP_TUNE_ROWGEMV 3
#define Q3OP_TUNE_ATTN_SPLITS 4
#define Q3OP_TUNE_QKV_ROPE 5
#define Q3OP_TUNE_FLASH_TILES 6
q3_status q3op_tune(int32_t key, int32_t value);

#ifdef __cplusplus
}
#endif
#endif /* Q3_OPS_H */
