// Host-side launchers for the libq3 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace q3k {

enum Dtype { F32 = 0, BF16 = 1 };

// Epilogues of the projection kernels.
enum Epi {
  EPI_STORE = 0,    // out[m][n] = acc                       (float out)
  EPI_RESADD = 1,   // out[m][n] += acc                      (float residual stream)
  EPI_SWIGLU = 2,   // rows packed [gate 16 | up 16]...; out[m][j] = silu(g)*u (act dtype)
  EPI_ARGMAX = 3,   // out[m][n] = acc (float logits) + per-block (max, index) partials
};

// Rows selected from a row-major matrix (n < 0: rows 0..count-1 in order).
struct RowMap {
  int32_t n;
  int32_t row[Q3_MAX_BATCH];
};

// ---------------------------------------------------------------- k_elem.hip
hipError_t embed(int dtype, const int32_t* ids, int n, const void* E, int V, int H, float* x,
                 uint32_t* err, hipStream_t s);
hipError_t rmsnorm(int out_dtype, const float* x, int rows, const RowMap& map, const float* w,
                   int H, float eps, void* out, hipStream_t s);
hipError_t rope_append(int dtype, const float* qkv, int T, const SeqBatch& sb, SeqState* st,
                       void* kv, int layer, int n_q, int n_kv, const float* qn, const float* kn,
                       float eps, const float* cos_t, const float* sin_t, void* q_out,
                       uint32_t* err, hipStream_t s, uint16_t* vstage = nullptr);
// fp16 staging of a bf16 prefill call's values from the cache (vstage_keys(sb)
// keys per kv head: every key 0 .. prior + L - 1 of each sequence);
// rope_append writes the same staging when given one.
hipError_t vstage_from_cache(int T, const SeqBatch& sb, const SeqState* st, const bf16_t* kv, int layer, int n_kv,
                             uint16_t* vstage, hipStream_t s);
// The value half of rope_append for a bf16 prefill whose q/k/v projection ran
// with the fused QK-Norm/RoPE epilogue (gemm_qkv_rope): bf16 value rows
// v [T][n_kv][128] into the cache and the fp16 staging.
hipError_t vt_append_bf16(const bf16_t* v, int T, const SeqBatch& sb, SeqState* st, bf16_t* kv, int layer, int n_kv,
                          uint16_t* vstage, hipStream_t s);
// ---------------------------------------------------------------- k_quant.hip
// Weight-only affine group quantization (groups of 64 along K, 8 or 4 bits,
// fp16 scale and offset per group packed in one 32-bit word).
size_t quant_code_bytes(int rows, int K, int bits);
size_t quant_sb_bytes(int rows, int K);
// Quantize bf16 rows [rows][K] into codes/sb at destination row dst_row0 + r
// (interleave: gate/up runs of 16 rows, up = 0 for gate, 1 for up).
hipError_t quantize_rows(const bf16_t* src, int rows, int K, int bits, uint8_t* codes, uint32_t* sb, int dst_row0,
                         int interleave, int up, hipStream_t s);
// bf16(q * s + b) for every weight of a quantized [N, K] matrix.
hipError_t dequant_rows(const uint8_t* codes, const uint32_t* sb, int N, int K, int bits, bf16_t* out, hipStream_t s);
bool qrowgemv_ok(int K);
// The weight-streaming decode projection (k_skinny.hip) on codes: M <= 64
// rows, EPI_STORE / EPI_RESADD (split over K with the workspace as in
// skinny_bf16) / EPI_SWIGLU, optional RMSNorm prologue.
hipError_t skinny_q(int epi, int bits, const void* X, int M, const uint8_t* codes, const uint32_t* sb, int N, int K,
                    const float* gnorm, float eps, void* out, int64_t ldo, hipStream_t s, float* split_part = nullptr,
                    uint32_t* split_cnt = nullptr);
// One activation row against a quantized matrix: EPI_STORE / EPI_SWIGLU (with
// an optional RMSNorm prologue from the float32 residual when gnorm is given)
// or EPI_RESADD (bf16 activation).
hipError_t qrowgemv(int epi, int bits, const void* X, const uint8_t* codes, const uint32_t* sb, int N, int K,
                    const float* gnorm, float eps, void* out, hipStream_t s);

// ---------------------------------------------------------------- k_sample.hip
// Temperature + top-p sampling of rows 0..n-1 (temperature 0: greedy pick).
// uniform[r] in [0, 1) drives row r's draw; ws holds sample_workspace_bytes(n)
// bytes (rows are processed 64 at a time).
size_t sample_workspace_bytes(int n_rows);
hipError_t sample_top_p(const float* logits, int64_t ld, int n, int V, float temperature, float top_p,
                        const float* uniform, int32_t* next, uint32_t* err, void* ws, hipStream_t s);
hipError_t argmax_rows(const float* logits, int64_t ld, const RowMap& rows, int V, int32_t* next,
                       uint32_t* err, hipStream_t s);
// Reduce per-block (max, index) partials of EPI_ARGMAX ([M][nblocks]) into
// next[m], then advance the lengths of the sequences of `sb` (decode: +1; prefill: = prior + length).
hipError_t argmax_finish(const float* pval, const int32_t* pidx, int nblocks, int M, int32_t* next,
                         const SeqBatch& sb, SeqState* st, uint32_t* err, hipStream_t s);
hipError_t seq_advance(const SeqBatch& sb, SeqState* st, hipStream_t s);
hipError_t seq_set_len(const SeqBatch& sb, SeqState* st, int32_t len, hipStream_t s);
hipError_t widen_bf16(const bf16_t* src, float* dst, int64_t n, hipStream_t s);
hipError_t fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);

// ---------------------------------------------------------------- k_gemm.hip
// C[M,N] = A[M,K] . W[N,K]^T with bf16 operands on MFMA; K % 64 == 0.
hipError_t gemm_bf16(int epi, const bf16_t* A, int M, const bf16_t* W, int N, int K, void* out,
                     int64_t ldo, hipStream_t s, float* split_part = nullptr, uint32_t* split_cnt = nullptr);
// The prefill q/k/v projection with Pasos 4-5's per-token work in its
// epilogue: query heads normalised and rotated into q_out [T][n_q][128]
// (bf16), key heads into the cache at each token's position, value heads
// rounded to bf16 into v_out [T][n_kv][128] (for vt_append_bf16).  Results
// equal gemm_bf16(EPI_STORE) followed by rope_append's query/key work.  Only
// for the tile configuration of large calls (gemm_qkv_rope_ok).
struct QkvRopeArgs {
  SeqBatch sb;
  const SeqState* st;
  bf16_t* kv;
  int layer, n_q, n_kv;
  const float* qn;
  const float* kn;
  float eps;
  const float* cos_t;
  const float* sin_t;
  bf16_t* q_out;
  bf16_t* v_out;
  uint32_t* err;
};
bool gemm_qkv_rope_ok(int M, int N, int K);
hipError_t gemm_qkv_rope(const bf16_t* A, int M, const bf16_t* W, int N, int K, const QkvRopeArgs& ra,
                         hipStream_t s);
void gemm_set_qkv_rope(int mode);  // -1 automatic, 0 never (timing and parity tests)
// Split-K of residual GEMMs on small grids: slices (1 = none) and the float
// workspace their partial tiles need; split_cnt holds one zeroed counter per
// 64 x 64 output tile (every call leaves them zero).
int gemm_splits(int epi, int M, int N, int K);
size_t gemm_split_floats(int M, int N, int K);
void gemm_set_config(int cfg);  // tile configuration override; -1 = automatic
void flash_set_rows(int cb);    // prefill attention rows per wavefront / 16 (1, 2, 4); -1 = automatic
void flash_set_tiles_per_block(int tpb);  // -1 automatic, 1 or 2 query tiles per block

// ---------------------------------------------------------------- k_skinny.hip
struct SkinnyPlan {
  int nst;    // 32-wide K steps per wavefront (4 or 8)
  int waves;  // wavefronts per block; K = waves * nst * 32
};
SkinnyPlan skinny_plan(int epi, int M, int N, int K);
bool skinny_norm_ok(int M);
bool skinny_norm_fuse(int M);  // decode steps fold RMSNorm in for M <= 16
int skinny_argmax_blocks(int N);
// M <= 64 rows times W[N,K]^T (bf16).  gnorm == nullptr: X is bf16 [M][K].
// gnorm != nullptr (M <= 64): X is the float32 residual [M][K] and the kernel
// applies RMSNorm with weight gnorm and eps first.  EPI_ARGMAX also writes
// per-block (max, index) partials, [M][N/16] (each row's partials contiguous).
hipError_t skinny_bf16(int epi, const void* X, int M, const bf16_t* W, int N, int K, const float* gnorm,
                       float eps, void* out, int64_t ldo, float* amax_val, int32_t* amax_idx, hipStream_t s,
                       float* split_part = nullptr, uint32_t* split_cnt = nullptr);
// Streaming lm_head (k_head.hip): M <= 64 rows of bf16 X [M][K] times W[N,K]^T,
// float32 logits out [M][ldo], and per-block (max, index) partials
// [M][headstream_blocks(N)] for argmax_finish.  Needs N % 16 == 0, K in
// {512, 1024, 1536, 2048} and the rows of X (padded to 16) in LDS.
bool headstream_ok(int M, int N, int K);
int headstream_blocks(int N);
hipError_t headstream_bf16(const bf16_t* X, int M, const bf16_t* W, int N, int K, float* out, int64_t ldo,
                           float* amax_val, int32_t* amax_idx, hipStream_t s);
// Split-K for RESADD with few row groups: K slices per row group (1 = none)
// and the float workspace the slices' partial sums need (split_part); the
// split_cnt array holds N/16 counters that must be zero before the first call
// (every call leaves them zero).
int skinny_splits(int epi, int M, int N, int K);
size_t skinny_split_floats(int M, int N, int K);
// Row-parallel bf16 GEMV for decode with M <= 4 rows: one wavefront per
// output row (EPI_STORE / EPI_RESADD), K a multiple of 512 up to 4096.
bool rowdot_ok(int M, int K);

// ---------------------------------------------------------------- k_rowgemv.hip
// One activation row (M = 1), K = 512 * {1,2,4,6,8}.  gnorm != nullptr: X is
// the float32 residual row and RMSNorm is fused (epi STORE or SWIGLU);
// otherwise X is bf16.  ARGMAX writes float32 logits to out and one
// (max, index) partial per block (rowgemv_argmax_blocks(N, K) of them).
bool rowgemv_ok(int M, int K);
int rowgemv_argmax_blocks(int N, int K);
void rowgemv_set_plan(int rows, int waves);  // -1 = automatic
hipError_t rowgemv_bf16(int epi, const void* X, const bf16_t* W, int N, int K, const float* gnorm, float eps,
                        void* out, float* amax_val, int32_t* amax_idx, hipStream_t s);
hipError_t rowdot_bf16(int epi, const bf16_t* X, int M, const bf16_t* W, int N, int K, float* out, int64_t ldo,
                       hipStream_t s);
// float32 weights and activations (the float32 model); any M.
hipError_t gemv_f32(int epi, const float* X, int M, const float* W, int N, int K, void* out,
                    int64_t ldo, hipStream_t s);

// ---------------------------------------------------------------- k_attn.hip
hipError_t flash_prefill(const bf16_t* q, int T, const SeqBatch& sb, const SeqState* st,
                         const bf16_t* kv, const uint16_t* vstage, int layer, int n_q, int n_kv, bf16_t* o,
                         hipStream_t s);
int decode_attn_splits(int B, int n_kv, int64_t max_ctx);
hipError_t decode_attn(const bf16_t* q, const SeqBatch& sb, const SeqState* st, const bf16_t* kv,
                       int layer, int n_q, int n_kv, int splits, float* part, bf16_t* o,
                       hipStream_t s);
// Decode attention with QK-Norm + RoPE + cache append folded in; reads the
// fused projection rows qkv [B][(n_q+2n_kv)*128] float32.  The plan gives
// `smax` splits per (sequence, kv head) at most, and the order in which the
// sequences' blocks are launched (longest context first); partials need
// B * n_q * smax * 130 floats and `counters` B * n_kv zeroed words (left
// zeroed by the kernel).  Results do not depend on the order.
struct AttnPlan {
  int smax;
  uint8_t order[Q3_MAX_BATCH];  // a permutation of 0..B-1
};
// ctx[b]: sequence b's context (cached keys + the new one) at planning time;
// max_cap: the largest slot capacity (bounds the contexts of later steps).
AttnPlan fused_attn_plan(int B, int n_kv, int64_t max_cap, const int64_t* ctx);
int fused_attn_smax_max(int B, int n_kv, int64_t max_ctx);  // ignoring the benchmark cap: for sizing
void decode_attn_set_split_cap(int cap);  // -1 = no cap (benchmarks only)
hipError_t decode_attn_fused(const float* qkv, const SeqBatch& sb, const SeqState* st, bf16_t* kv, int layer,
                             int n_q, int n_kv, const float* qn, const float* kn, float eps, const float* cos_t,
                             const float* sin_t, const AttnPlan& plan, float* part, uint32_t* counters,
                             bf16_t* o, hipStream_t s);
hipError_t attn_f32(const float* q, int T, const SeqBatch& sb, const SeqState* st,
                    const float* kv, int layer, int n_q, int n_kv, float* o, hipStream_t s);

}  // namespace q3k

#include <string>
namespace q3rt {
// Thread-local message returned by q3_last_error().
void set_last_error(const std::string& msg);
}  // namespace q3rt
