// Single-kernel entry points (include/q3_ops.h): the kernels of the forward
// pass on explicit buffers, for parity tests and kernel benchmarks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/q3_ops.h"
#include "kernels.h"

using namespace q3k;

namespace {
q3_status op_fail(q3_status st, const std::string& m) {
  q3rt::set_last_error(m);
  return st;
}
q3_status op_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return Q3_OK;
  return op_fail(Q3_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}
#define OP_TRY(expr)                                  \
  do {                                                \
    q3_status s_ = op_hip((expr), #expr);             \
    if (s_ != Q3_OK) return s_;                       \
  } while (0)

size_t al(size_t v) { return (v + 255) / 256 * 256; }

struct SkinnyWs {
  size_t err, amax_val, amax_idx, split_part, split_cnt, total;
};
SkinnyWs skinny_ws(int M, int N, int K) {
  SkinnyWs w;
  const size_t groups = (size_t)N / 16;
  w.err = 0;
  w.amax_val = al(16);
  w.amax_idx = w.amax_val + al(groups * M * 4);
  w.split_part = w.amax_idx + al(groups * M * 4);
  w.split_cnt = w.split_part + al(skinny_split_floats(M, N, K) * 4);
  w.total = w.split_cnt + al((groups + 1) * 4);
  return w;
}

// Split-K partial tiles and per-tile counters of the residual GEMM.
struct GemmWs {
  size_t part, cnt, total;
  int64_t tiles;
};
GemmWs gemm_ws(int M, int N, int K) {
  GemmWs w;
  w.tiles = (int64_t)((N + 63) / 64) * ((M + 63) / 64);
  w.part = 0;
  w.cnt = al(gemm_split_floats(M, N, K) * 4);
  w.total = std::max<size_t>(256, w.cnt + al(w.tiles * 4));
  return w;
}

// Device tables for the arena-based ops: SeqState[n] then an error word.
q3_status upload_states(int n, const int64_t* base, const int32_t* cap, const int32_t* len, void* d_ws,
                        hipStream_t s) {
  std::vector<SeqState> st(n);
  for (int b = 0; b < n; ++b) {
    if (cap[b] <= 0 || cap[b] % 64 != 0) return op_fail(Q3_E_ARG, "capacities must be positive multiples of 64");
    if (base[b] < 0 || base[b] % 64 != 0) return op_fail(Q3_E_ARG, "bases must be non-negative multiples of 64");
    if (len[b] < 0 || len[b] > cap[b]) return op_fail(Q3_E_ARG, "length outside capacity");
    st[b] = SeqState{base[b], cap[b], len[b]};
  }
  OP_TRY(hipStreamSynchronize(s));
  OP_TRY(hipMemcpy(d_ws, st.data(), n * sizeof(SeqState), hipMemcpyHostToDevice));
  return Q3_OK;
}

q3_status skinny_op(int epi, const void* X, int M, const float* gnorm, float eps, const void* W, int N, int K,
                    void* out, int64_t ldo, int32_t* next, void* d_ws, size_t ws_bytes, hipStream_t s) {
  SkinnyWs w = skinny_ws(M, N, K);
  if (!d_ws || ws_bytes < w.total) return op_fail(Q3_E_ARG, "workspace too small");
  char* ws = (char*)d_ws;
  uint32_t* cnt = (uint32_t*)(ws + w.split_cnt);
  OP_TRY(fill_u32(cnt, 0u, (int64_t)N / 16 + 1, s));
  OP_TRY(skinny_bf16(epi, X, M, (const bf16_t*)W, N, K, gnorm, eps, out, ldo, (float*)(ws + w.amax_val),
                     (int32_t*)(ws + w.amax_idx), s, (float*)(ws + w.split_part), cnt));
  if (epi == EPI_ARGMAX && next) {
    SeqBatch none;
    std::memset(&none, 0, sizeof(none));
    OP_TRY(argmax_finish((const float*)(ws + w.amax_val), (const int32_t*)(ws + w.amax_idx), skinny_argmax_blocks(N),
                         M, next, none, nullptr, (uint32_t*)(ws + w.err), s));
  }
  return Q3_OK;
}

// Partials of the streaming lm_head: [M][blocks] (max, index), an error word.
struct HeadWs {
  size_t err, amax_val, amax_idx, total;
};
HeadWs head_ws(int M, int N) {
  HeadWs w;
  const size_t parts = (size_t)std::max(M, 1) * headstream_blocks(N);
  w.err = 0;
  w.amax_val = al(16);
  w.amax_idx = w.amax_val + al(parts * 4);
  w.total = w.amax_idx + al(parts * 4);
  return w;
}

struct RowWs {
  size_t err, amax_val, amax_idx, total;
};
RowWs row_ws(int N) {
  RowWs w;
  const size_t parts = (size_t)N;  // at most one partial per row, whatever the plan
  w.err = 0;
  w.amax_val = al(16);
  w.amax_idx = w.amax_val + al(parts * 4);
  w.total = w.amax_idx + al(parts * 4);
  return w;
}

q3_status rowgemv_op(int epi, const void* X, const float* gnorm, float eps, const void* W, int N, int K, void* out,
                     int32_t* next, void* d_ws, size_t ws_bytes, hipStream_t s) {
  RowWs w = row_ws(N);
  if (epi == EPI_ARGMAX && (!d_ws || ws_bytes < w.total)) return op_fail(Q3_E_ARG, "workspace too small");
  char* ws = (char*)d_ws;
  float* av = epi == EPI_ARGMAX ? (float*)(ws + w.amax_val) : nullptr;
  int32_t* ai = epi == EPI_ARGMAX ? (int32_t*)(ws + w.amax_idx) : nullptr;
  OP_TRY(rowgemv_bf16(epi, X, (const bf16_t*)W, N, K, gnorm, eps, out, av, ai, s));
  if (epi == EPI_ARGMAX && next) {
    SeqBatch none;
    std::memset(&none, 0, sizeof(none));
    OP_TRY(argmax_finish(av, ai, rowgemv_argmax_blocks(N, K), 1, next, none, nullptr, (uint32_t*)(ws + w.err), s));
  }
  return Q3_OK;
}

// Prefill: sequence b continues after prior[b] cached tokens (NULL: none).
q3_status make_batch(int n, const int32_t* cu, int decode, SeqBatch* sb, const int32_t* prior = nullptr) {
  if (n < 1 || n > Q3_MAX_BATCH) return op_fail(Q3_E_ARG, "n_seqs must be in [1, 64]");
  std::memset(sb, 0, sizeof(*sb));
  sb->n = n;
  sb->decode = decode;
  for (int b = 0; b < n; ++b) sb->slot[b] = b;
  if (decode) {
    for (int b = 0; b <= n; ++b) sb->cu[b] = b;
  } else {
    if (!cu || cu[0] != 0) return op_fail(Q3_E_ARG, "cu_seqlens must start at 0");
    for (int b = 0; b <= n; ++b) sb->cu[b] = cu[b];
    for (int b = 0; b < n; ++b)
      if (cu[b + 1] <= cu[b]) return op_fail(Q3_E_ARG, "empty sequence");
    if (prior)
      for (int b = 0; b < n; ++b) {
        if (prior[b] < 0) return op_fail(Q3_E_ARG, "negative cached length");
        sb->prior[b] = prior[b];
      }
  }
  return Q3_OK;
}
}  // namespace

extern "C" {

q3_status q3op_embed(int32_t dtype, const int32_t* d_ids, int32_t n, const void* d_table, int32_t vocab,
                     int32_t dim, float* d_out, uint32_t* d_err, void* stream) {
  if (n < 0 || !d_ids || !d_table || !d_out || !d_err) return op_fail(Q3_E_ARG, "bad argument");
  OP_TRY(embed(dtype, d_ids, n, d_table, vocab, dim, d_out, d_err, (hipStream_t)stream));
  return Q3_OK;
}

q3_status q3op_rmsnorm(int32_t out_dtype, const float* d_x, int32_t rows, const float* d_w, int32_t dim,
                       float eps, void* d_out, void* stream) {
  if (rows < 0 || dim <= 0 || dim % 256 != 0 || !d_x || !d_w || !d_out) return op_fail(Q3_E_ARG, "bad argument");
  RowMap all;
  all.n = -1;
  OP_TRY(rmsnorm(out_dtype, d_x, rows, all, d_w, dim, eps, d_out, (hipStream_t)stream));
  return Q3_OK;
}

size_t q3op_linear_workspace_bytes(int32_t kernel, int32_t epi, int32_t M, int32_t N, int32_t K) {
  if (kernel == Q3OP_SKINNY) return skinny_ws(M, N, K).total;
  if (kernel == Q3OP_HEADSTREAM) return head_ws(M, N).total;
  if (kernel == Q3OP_ROWGEMV) return row_ws(N).total;
  if (kernel == Q3OP_GEMM && epi == EPI_RESADD) return gemm_ws(M, N, K).total;
  return 256;
}

q3_status q3op_linear(int32_t kernel, int32_t epi, const void* d_x, int32_t M, const void* d_w, int32_t N,
                      int32_t K, void* d_out, int64_t ldo, int32_t* d_next, void* d_ws, size_t ws_bytes,
                      void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (!d_x || !d_w || !d_out || M < 0 || N <= 0 || K <= 0) return op_fail(Q3_E_ARG, "bad argument");
  if (epi < 0 || epi > 3) return op_fail(Q3_E_ARG, "bad epilogue");
  if (epi == EPI_ARGMAX && M > Q3_MAX_BATCH) return op_fail(Q3_E_ARG, "logits epilogue needs M <= 64");
  if (epi == EPI_ARGMAX && !d_next && kernel != Q3OP_SKINNY && kernel != Q3OP_ROWGEMV && kernel != Q3OP_HEADSTREAM)
    return op_fail(Q3_E_ARG, "logits epilogue needs d_next");
  RowMap rows;
  rows.n = M;
  for (int i = 0; i < M && i < Q3_MAX_BATCH; ++i) rows.row[i] = i;
  uint32_t* no_err = nullptr;
  if (kernel == Q3OP_GEMM) {
    float* part = nullptr;
    uint32_t* cnt = nullptr;
    if (epi == EPI_RESADD && gemm_split_floats(M, N, K) > 0) {
      const GemmWs w = gemm_ws(M, N, K);
      if (!d_ws || ws_bytes < w.total) return op_fail(Q3_E_ARG, "workspace smaller than q3op_linear_workspace_bytes");
      part = (float*)((char*)d_ws + w.part);
      cnt = (uint32_t*)((char*)d_ws + w.cnt);
      OP_TRY(fill_u32(cnt, 0u, w.tiles, s));
    }
    OP_TRY(gemm_bf16(epi, (const bf16_t*)d_x, M, (const bf16_t*)d_w, N, K, d_out, ldo, s, part, cnt));
    if (epi == EPI_ARGMAX) {
      if (!d_ws || ws_bytes < 4) return op_fail(Q3_E_ARG, "logits epilogue needs 4 bytes of workspace");
      no_err = (uint32_t*)d_ws;
      OP_TRY(argmax_rows((const float*)d_out, ldo, rows, N, d_next, no_err, s));
    }
    return Q3_OK;
  }
  if (kernel == Q3OP_GEMV_F32) {
    OP_TRY(gemv_f32(epi, (const float*)d_x, M, (const float*)d_w, N, K, d_out, ldo, s));
    if (epi == EPI_ARGMAX) {
      if (!d_ws || ws_bytes < 4) return op_fail(Q3_E_ARG, "logits epilogue needs 4 bytes of workspace");
      OP_TRY(argmax_rows((const float*)d_out, ldo, rows, N, d_next, (uint32_t*)d_ws, s));
    }
    return Q3_OK;
  }
  if (kernel == Q3OP_ROWDOT) {
    if (!rowdot_ok(M, K) || (epi != EPI_STORE && epi != EPI_RESADD))
      return op_fail(Q3_E_UNSUPPORTED, "the row GEMV takes M <= 4, K a multiple of 512, epilogue 0 or 1");
    OP_TRY(rowdot_bf16(epi, (const bf16_t*)d_x, M, (const bf16_t*)d_w, N, K, (float*)d_out, ldo, s));
    return Q3_OK;
  }
  if (kernel == Q3OP_SKINNY) {
    if (M > Q3_MAX_BATCH) return op_fail(Q3_E_UNSUPPORTED, "the weight-streaming kernel takes M <= 64");
    return skinny_op(epi, d_x, M, nullptr, 0.f, d_w, N, K, d_out, ldo, d_next, d_ws, ws_bytes, s);
  }
  if (kernel == Q3OP_HEADSTREAM) {
    if ((epi != EPI_STORE && epi != EPI_ARGMAX) || !headstream_ok(M, N, K))
      return op_fail(Q3_E_UNSUPPORTED,
                     "the streaming lm_head takes epilogue 0 or 3, M <= 64, N % 16 == 0, K in {512, 1024, 1536, "
                     "2048} and 16 * ceil(M/16) rows of K bf16 within 156 KiB");
    const HeadWs w = head_ws(M, N);
    if (!d_ws || ws_bytes < w.total) return op_fail(Q3_E_ARG, "workspace smaller than q3op_linear_workspace_bytes");
    char* ws = (char*)d_ws;
    OP_TRY(headstream_bf16((const bf16_t*)d_x, M, (const bf16_t*)d_w, N, K, (float*)d_out, ldo,
                           (float*)(ws + w.amax_val), (int32_t*)(ws + w.amax_idx), s));
    if (epi == EPI_ARGMAX && d_next) {
      SeqBatch none;
      std::memset(&none, 0, sizeof(none));
      OP_TRY(argmax_finish((const float*)(ws + w.amax_val), (const int32_t*)(ws + w.amax_idx), headstream_blocks(N),
                           M, d_next, none, nullptr, (uint32_t*)(ws + w.err), s));
    }
    return Q3_OK;
  }
  if (kernel == Q3OP_ROWGEMV) {
    if (!rowgemv_ok(M, K)) return op_fail(Q3_E_UNSUPPORTED, "the single-row GEMV takes M = 1, K = 512 * {1,2,4,6,8}");
    if (epi == EPI_SWIGLU && N % 32 != 0) return op_fail(Q3_E_UNSUPPORTED, "SwiGLU needs N % 32 == 0");
    return rowgemv_op(epi, d_x, nullptr, 0.f, d_w, N, K, d_out, d_next, d_ws, ws_bytes, s);
  }
  return op_fail(Q3_E_ARG, "unknown kernel");
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation variant
// The workspace of q3op_linear_noalloc: a file-scope device array, one copy
// per GPU for the life of the process.  In host code `scratch` only names the
// symbol; its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch_ptr.
namespace {
constexpr size_t kScratchBytes = (size_t)Q3OP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

q3_status scratch_for_current_device(void** out) {
  int dev = -1;
  OP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return op_fail(Q3_E_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return op_fail(Q3_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return Q3_OK;
}
}  // namespace

extern "C" {

q3_status q3op_linear_noalloc(int32_t kernel, int32_t epi, const void* d_x, int32_t M, const void* d_w, int32_t N,
                              int32_t K, void* d_out, int64_t ldo, int32_t* d_next, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return op_fail(Q3_E_ARG, "bad argument");
  const size_t need = q3op_linear_workspace_bytes(kernel, epi, M, N, K);
  if (need > kScratchBytes)
    return op_fail(Q3_E_CAPACITY, "q3op_linear_noalloc: the call needs " + std::to_string(need) +
                                      " bytes of workspace, more than the " + std::to_string(kScratchBytes) +
                                      "-byte static scratch; use q3op_linear with a workspace");
  void* ws = nullptr;
  q3_status st = scratch_for_current_device(&ws);
  if (st != Q3_OK) return st;
  return q3op_linear(kernel, epi, d_x, M, d_w, N, K, d_out, ldo, d_next, ws, kScratchBytes, stream);
}

q3_status q3op_norm_linear(int32_t kernel, int32_t epi, const float* d_x, int32_t M, const float* d_gnorm,
                           float eps, const void* d_w, int32_t N, int32_t K, void* d_out, int64_t ldo,
                           int32_t* d_next, void* d_ws, size_t ws_bytes, void* stream) {
  if (!d_x || !d_gnorm || !d_w || !d_out || M <= 0 || N <= 0 || K <= 0) return op_fail(Q3_E_ARG, "bad argument");
  if (epi < 0 || epi > 3) return op_fail(Q3_E_ARG, "bad epilogue");
  if (epi == EPI_ARGMAX && !d_next) return op_fail(Q3_E_ARG, "logits epilogue needs d_next");
  if (kernel == Q3OP_ROWGEMV) {
    if (!rowgemv_ok(M, K)) return op_fail(Q3_E_UNSUPPORTED, "the single-row GEMV takes M = 1, K = 512 * {1,2,4,6,8}");
    if (epi != EPI_STORE && epi != EPI_SWIGLU)
      return op_fail(Q3_E_UNSUPPORTED, "the single-row GEMV fuses RMSNorm for epilogues 0 and 2 only");
    if (epi == EPI_SWIGLU && N % 32 != 0) return op_fail(Q3_E_UNSUPPORTED, "SwiGLU needs N % 32 == 0");
    return rowgemv_op(epi, d_x, d_gnorm, eps, d_w, N, K, d_out, d_next, d_ws, ws_bytes, (hipStream_t)stream);
  }
  if (kernel != Q3OP_SKINNY) return op_fail(Q3_E_ARG, "the fused RMSNorm prologue exists in kernels 1 and 4");
  if (!skinny_norm_ok(M)) return op_fail(Q3_E_UNSUPPORTED, "the fused RMSNorm prologue takes M <= 64");
  return skinny_op(epi, d_x, M, d_gnorm, eps, d_w, N, K, d_out, ldo, d_next, d_ws, ws_bytes, (hipStream_t)stream);
}

size_t q3op_rope_workspace_bytes(int32_t n_seqs, int32_t max_pos) {
  return al(n_seqs * sizeof(SeqState)) + al(16) + 2 * al((size_t)max_pos * 64 * 4);
}

q3_status q3op_rope_append(int32_t dtype, const float* d_qkv, int32_t n, const int32_t* h_cu, int32_t decode,
                           const int64_t* h_base, const int32_t* h_cap, const int32_t* h_len, void* d_kv,
                           int32_t n_q, int32_t n_kv, const float* d_qn, const float* d_kn, float eps,
                           double theta, int32_t max_pos, void* d_q_out, void* d_ws, size_t ws_bytes,
                           void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (!d_qkv || !d_kv || !d_qn || !d_kn || !d_q_out || !h_base || !h_cap || !h_len || max_pos <= 0)
    return op_fail(Q3_E_ARG, "bad argument");
  SeqBatch sb;
  q3_status st = make_batch(n, h_cu, decode, &sb, h_len);
  if (st != Q3_OK) return st;
  if (!d_ws || ws_bytes < q3op_rope_workspace_bytes(n, max_pos)) return op_fail(Q3_E_ARG, "workspace too small");
  for (int b = 0; b < n; ++b) {
    const int last = decode ? h_len[b] : (h_len[b] + sb.cu[b + 1] - sb.cu[b] - 1);
    if (last >= h_cap[b] || last >= max_pos) return op_fail(Q3_E_CAPACITY, "position beyond capacity");
  }
  char* ws = (char*)d_ws;
  st = upload_states(n, h_base, h_cap, h_len, ws, s);
  if (st != Q3_OK) return st;
  uint32_t* err = (uint32_t*)(ws + al(n * sizeof(SeqState)));
  float* cos_t = (float*)(ws + al(n * sizeof(SeqState)) + al(16));
  float* sin_t = (float*)((char*)cos_t + al((size_t)max_pos * 64 * 4));
  std::vector<float> cs((size_t)max_pos * 64), sn((size_t)max_pos * 64);
  for (int p = 0; p < max_pos; ++p)
    for (int i = 0; i < 64; ++i) {
      const double a = (double)p * std::pow(theta, -(double)i / 64.0);
      cs[(size_t)p * 64 + i] = (float)std::cos(a);
      sn[(size_t)p * 64 + i] = (float)std::sin(a);
    }
  OP_TRY(hipMemcpy(cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
  OP_TRY(hipMemcpy(sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
  OP_TRY(fill_u32(err, 0u, 1, s));
  const int T = sb.cu[n];
  OP_TRY(rope_append(dtype, d_qkv, T, sb, (SeqState*)ws, d_kv, 0, n_q, n_kv, d_qn, d_kn, eps, cos_t, sin_t, d_q_out,
                     err, s));
  return Q3_OK;
}

size_t q3op_attention_workspace_bytes(int32_t kernel, int32_t n_seqs, int32_t total_tokens, int32_t n_q,
                                      int32_t n_kv, int32_t splits) {
  size_t b = al(n_seqs * sizeof(SeqState));
  if (kernel == Q3OP_ATTN_DECODE) b += al((size_t)n_seqs * n_q * (splits > 0 ? splits : 2048) * 130 * 4);
  // every sequence's keys rounded up to 64, plus one tile
  if (kernel == Q3OP_ATTN_FLASH)
    b += al(((size_t)std::max(total_tokens, 0) + 64 * (size_t)std::max(n_seqs, 0) + 64) * n_kv * 128 * 2);
  return b;
}

q3_status q3op_attention(int32_t kernel, const void* d_q, int32_t n, const int32_t* h_cu, int32_t decode,
                         const int64_t* h_base, const int32_t* h_cap, const int32_t* h_len, const void* d_kv,
                         int32_t n_q, int32_t n_kv, int32_t splits, void* d_out, void* d_ws, size_t ws_bytes,
                         void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (!d_q || !d_kv || !d_out || !h_base || !h_cap || !h_len) return op_fail(Q3_E_ARG, "bad argument");
  SeqBatch sb;
  q3_status st = make_batch(n, h_cu, decode, &sb, h_len);
  if (st != Q3_OK) return st;
  if (n_kv <= 0 || n_q % n_kv != 0 || n_q / n_kv > 8) return op_fail(Q3_E_UNSUPPORTED, "head grouping");
  if (kernel == Q3OP_ATTN_FLASH && decode) return op_fail(Q3_E_ARG, "flash kernel is the prefill kernel");
  if (kernel == Q3OP_ATTN_DECODE && !decode) return op_fail(Q3_E_ARG, "decode kernel needs decode = 1");
  for (int b = 0; b < n; ++b) {
    const int ctx = decode ? h_len[b] + 1 : h_len[b] + sb.cu[b + 1] - sb.cu[b];
    if (ctx > h_cap[b]) return op_fail(Q3_E_CAPACITY, "context beyond capacity");
  }
  if (kernel == Q3OP_ATTN_DECODE && splits <= 0) {
    int64_t mc = 1;
    for (int b = 0; b < n; ++b) mc = std::max<int64_t>(mc, h_cap[b]);
    splits = decode_attn_splits(n, n_kv, mc);
  }
  const int T = sb.cu[n];
  int64_t keys = 0;  // keys of the call: cached + new
  for (int b = 0; b < n; ++b) keys += (decode ? 0 : h_len[b]) + sb.cu[b + 1] - sb.cu[b];
  if (keys > INT32_MAX) return op_fail(Q3_E_CAPACITY, "too many keys");
  if (!d_ws || ws_bytes < q3op_attention_workspace_bytes(kernel, n, (int32_t)keys, n_q, n_kv, splits))
    return op_fail(Q3_E_ARG, "workspace too small");
  char* ws = (char*)d_ws;
  st = upload_states(n, h_base, h_cap, h_len, ws, s);
  if (st != Q3_OK) return st;
  const SeqState* sst = (const SeqState*)ws;
  if (kernel == Q3OP_ATTN_FLASH) {
    uint16_t* vstage = (uint16_t*)(ws + al(n * sizeof(SeqState)));
    OP_TRY(vstage_from_cache(T, sb, sst, (const bf16_t*)d_kv, 0, n_kv, vstage, s));
    OP_TRY(flash_prefill((const bf16_t*)d_q, T, sb, sst, (const bf16_t*)d_kv, vstage, 0, n_q, n_kv,
                         (bf16_t*)d_out, s));
  } else if (kernel == Q3OP_ATTN_DECODE) {
    float* part = (float*)(ws + al(n * sizeof(SeqState)));
    OP_TRY(decode_attn((const bf16_t*)d_q, sb, sst, (const bf16_t*)d_kv, 0, n_q, n_kv, splits, part,
                       (bf16_t*)d_out, s));
  } else if (kernel == Q3OP_ATTN_F32) {
    OP_TRY(attn_f32((const float*)d_q, T, sb, sst, (const float*)d_kv, 0, n_q, n_kv, (float*)d_out, s));
  } else {
    return op_fail(Q3_E_ARG, "unknown kernel");
  }
  return Q3_OK;
}

q3_status q3op_quantize(const void* d_w, int32_t rows, int32_t K, int32_t bits, void* d_codes, void* d_sb,
                        void* stream) {
  if (rows < 1 || K < 64 || K % 64 != 0 || (bits != 8 && bits != 4)) return op_fail(Q3_E_ARG, "bad shape or bits");
  if (!d_w || !d_codes || !d_sb) return op_fail(Q3_E_ARG, "NULL pointer");
  OP_TRY(quantize_rows((const bf16_t*)d_w, rows, K, bits, (uint8_t*)d_codes, (uint32_t*)d_sb, 0, 0, 0,
                       (hipStream_t)stream));
  return Q3_OK;
}

q3_status q3op_dequantize(const void* d_codes, const void* d_sb, int32_t rows, int32_t K, int32_t bits, void* d_out,
                          void* stream) {
  if (rows < 1 || K < 64 || K % 64 != 0 || (bits != 8 && bits != 4)) return op_fail(Q3_E_ARG, "bad shape or bits");
  if (!d_codes || !d_sb || !d_out) return op_fail(Q3_E_ARG, "NULL pointer");
  OP_TRY(dequant_rows((const uint8_t*)d_codes, (const uint32_t*)d_sb, rows, K, bits, (bf16_t*)d_out,
                      (hipStream_t)stream));
  return Q3_OK;
}

q3_status q3op_qlinear(int32_t bits, int32_t epi, const void* d_x, const void* d_codes, const void* d_sb, int32_t N,
                       int32_t K, const float* d_gnorm, float eps, void* d_out, void* stream) {
  if (bits != 8 && bits != 4) return op_fail(Q3_E_ARG, "bits must be 8 or 4");
  if (!qrowgemv_ok(K) || N < 1) return op_fail(Q3_E_UNSUPPORTED, "K must be 1024, 2048, 3072 or 4096");
  if (epi != EPI_STORE && epi != EPI_RESADD && epi != EPI_SWIGLU) return op_fail(Q3_E_ARG, "epilogue");
  if (epi == EPI_SWIGLU && N % 32 != 0) return op_fail(Q3_E_ARG, "SwiGLU needs N % 32 == 0");
  if (epi == EPI_RESADD && d_gnorm) return op_fail(Q3_E_ARG, "no RMSNorm prologue with the residual epilogue");
  if (!d_x || !d_codes || !d_sb || !d_out) return op_fail(Q3_E_ARG, "NULL pointer");
  OP_TRY(qrowgemv(epi, bits, d_x, (const uint8_t*)d_codes, (const uint32_t*)d_sb, N, K, d_gnorm, eps, d_out,
                  (hipStream_t)stream));
  return Q3_OK;
}

size_t q3op_qlinear_rows_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 1 || N < 16 || K < 64) return 0;
  return al(std::max<size_t>(16, skinny_split_floats(M, N, K)) * 4) + al((size_t)(N / 16 + 1) * 4);
}

q3_status q3op_qlinear_rows(int32_t bits, int32_t epi, const void* d_x, int32_t M, const void* d_codes,
                            const void* d_sb, int32_t N, int32_t K, const float* d_gnorm, float eps, void* d_out,
                            int64_t ldo, void* d_ws, size_t ws_bytes, void* stream) {
  if (bits != 8 && bits != 4) return op_fail(Q3_E_ARG, "bits must be 8 or 4");
  if (M < 1 || M > 64) return op_fail(Q3_E_ARG, "M must be 1..64");
  if (epi != EPI_STORE && epi != EPI_RESADD && epi != EPI_SWIGLU) return op_fail(Q3_E_ARG, "epilogue");
  if (d_gnorm && (epi == EPI_RESADD || M > 16)) return op_fail(Q3_E_ARG, "RMSNorm prologue: store/SwiGLU, M <= 16");
  if (!d_x || !d_codes || !d_sb || !d_out) return op_fail(Q3_E_ARG, "NULL pointer");
  float* part = nullptr;
  uint32_t* cnt = nullptr;
  if (epi == EPI_RESADD && d_ws) {
    if (ws_bytes < q3op_qlinear_rows_workspace_bytes(M, N, K)) return op_fail(Q3_E_ARG, "workspace too small");
    part = (float*)d_ws;
    cnt = (uint32_t*)((char*)d_ws + al(std::max<size_t>(16, skinny_split_floats(M, N, K)) * 4));
    OP_TRY(fill_u32(cnt, 0u, N / 16 + 1, (hipStream_t)stream));
  }
  OP_TRY(skinny_q(epi, bits, d_x, M, (const uint8_t*)d_codes, (const uint32_t*)d_sb, N, K, d_gnorm, eps, d_out, ldo,
                  (hipStream_t)stream, part, cnt));
  return Q3_OK;
}

size_t q3op_sample_workspace_bytes(int32_t n_rows) { return sample_workspace_bytes(n_rows); }

q3_status q3op_sample_top_p(const float* d_logits, int32_t n_rows, int32_t vocab, int64_t ld, float temperature,
                            float top_p, const float* d_uniform, int32_t* d_next, uint32_t* d_err, void* d_ws,
                            size_t ws_bytes, void* stream) {
  if (n_rows < 0 || vocab < 1 || ld < vocab) return op_fail(Q3_E_ARG, "bad shape");
  if (temperature != 0.f && n_rows > 0 && (!d_ws || ws_bytes < sample_workspace_bytes(n_rows)))
    return op_fail(Q3_E_ARG, "workspace too small");
  if (n_rows > 0 && (!d_logits || !d_next || !d_err)) return op_fail(Q3_E_ARG, "NULL pointer");
  if (!std::isfinite(temperature) || (temperature != 0.f && temperature < 1e-30f))
    return op_fail(Q3_E_ARG, "temperature must be 0 or a finite value >= 1e-30");
  if (!std::isfinite(top_p)) return op_fail(Q3_E_ARG, "top_p must be finite");
  if (temperature != 0.f && n_rows > 0 && !d_uniform) return op_fail(Q3_E_ARG, "sampling needs d_uniform");
  OP_TRY(sample_top_p(d_logits, ld, n_rows, vocab, temperature, top_p, d_uniform, d_next, d_err, d_ws,
                      (hipStream_t)stream));
  return Q3_OK;
}

size_t q3op_decode_attn_fused_workspace_bytes(int32_t n_seqs, int32_t n_q, int32_t smax, int32_t max_pos) {
  return al(n_seqs * sizeof(SeqState)) + 2 * al((size_t)max_pos * 64 * 4) +
         al((size_t)n_seqs * n_q * (smax > 0 ? smax : 64) * 130 * 4) + al((size_t)n_seqs * n_q * 4);
}

q3_status q3op_decode_attn_fused(const float* d_qkv, int32_t n, const int64_t* h_base, const int32_t* h_cap,
                                 const int32_t* h_len, void* d_kv, int32_t n_q, int32_t n_kv, const float* d_qn,
                                 const float* d_kn, float eps, double theta, int32_t max_pos, int32_t smax,
                                 void* d_out, void* d_ws, size_t ws_bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  SeqBatch sb;
  q3_status st = make_batch(n, nullptr, 1, &sb);
  if (st != Q3_OK) return st;
  if (!d_qkv || !d_kv || !d_qn || !d_kn || !d_out || !h_base || !h_cap || !h_len || max_pos <= 0)
    return op_fail(Q3_E_ARG, "bad argument");
  if (n_kv <= 0 || n_q % n_kv != 0 || n_q / n_kv > 8) return op_fail(Q3_E_UNSUPPORTED, "head grouping");
  int64_t mc = 1;
  int64_t ctx[Q3_MAX_BATCH];
  for (int b = 0; b < n; ++b) {
    if (h_len[b] < 0) return op_fail(Q3_E_ARG, "negative length");
    if (h_len[b] + 1 > h_cap[b] || h_len[b] + 1 > max_pos) return op_fail(Q3_E_CAPACITY, "position beyond capacity");
    mc = std::max<int64_t>(mc, h_cap[b]);
    ctx[b] = h_len[b] + 1;
  }
  AttnPlan plan = fused_attn_plan(n, n_kv, mc, ctx);
  if (smax > 64) return op_fail(Q3_E_ARG, "smax must be <= 64");
  if (smax > 0) plan.smax = smax;
  smax = plan.smax;
  if (!d_ws || ws_bytes < q3op_decode_attn_fused_workspace_bytes(n, n_q, smax, max_pos))
    return op_fail(Q3_E_ARG, "workspace too small");
  char* ws = (char*)d_ws;
  st = upload_states(n, h_base, h_cap, h_len, ws, s);
  if (st != Q3_OK) return st;
  float* cos_t = (float*)(ws + al(n * sizeof(SeqState)));
  float* sin_t = (float*)((char*)cos_t + al((size_t)max_pos * 64 * 4));
  float* part = (float*)((char*)sin_t + al((size_t)max_pos * 64 * 4));
  uint32_t* cnt = (uint32_t*)((char*)part + al((size_t)n * n_q * smax * 130 * 4));
  OP_TRY(fill_u32(cnt, 0u, (int64_t)n * n_kv, s));
  std::vector<float> cs((size_t)max_pos * 64), sn((size_t)max_pos * 64);
  for (int p = 0; p < max_pos; ++p)
    for (int i = 0; i < 64; ++i) {
      const double a = (double)p * std::pow(theta, -(double)i / 64.0);
      cs[(size_t)p * 64 + i] = (float)std::cos(a);
      sn[(size_t)p * 64 + i] = (float)std::sin(a);
    }
  OP_TRY(hipMemcpy(cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
  OP_TRY(hipMemcpy(sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
  OP_TRY(decode_attn_fused(d_qkv, sb, (const SeqState*)ws, (bf16_t*)d_kv, 0, n_q, n_kv, d_qn, d_kn, eps, cos_t,
                           sin_t, plan, part, cnt, (bf16_t*)d_out, s));
  return Q3_OK;
}

q3_status q3op_tune(int32_t key, int32_t value) {
  if (key == Q3OP_TUNE_GEMM_TILES) {
    if (value < -1 || value > 11) return op_fail(Q3_E_ARG, "tile configuration out of range");
    gemm_set_config(value);
    return Q3_OK;
  }
  if (key == Q3OP_TUNE_ROWGEMV) {
    const int rows = value < 0 ? -1 : value & 0xff, waves = value < 0 ? -1 : value >> 8;
    if (value >= 0 && (!(rows == 1 || rows == 2 || rows == 4 || rows == 8) || waves < 1 || waves > 4))
      return op_fail(Q3_E_ARG, "rows per wavefront must be 1, 2, 4 or 8 and wavefronts per block 1..4");
    rowgemv_set_plan(rows, waves);
    return Q3_OK;
  }
  if (key == Q3OP_TUNE_ATTN_SPLITS) {
    if (value == 0 || value < -1 || value > 64) return op_fail(Q3_E_ARG, "split cap must be -1 or 1..64");
    decode_attn_set_split_cap(value);
    return Q3_OK;
  }
  if (key == Q3OP_TUNE_FLASH_TILES) {
    if (value != -1 && value != 1 && value != 2) return op_fail(Q3_E_ARG, "query tiles per block must be -1, 1 or 2");
    flash_set_tiles_per_block(value);
    return Q3_OK;
  }
  if (key == Q3OP_TUNE_QKV_ROPE) {
    if (value != -1 && value != 0) return op_fail(Q3_E_ARG, "fused q/k/v epilogue mode must be -1 or 0");
    gemm_set_qkv_rope(value);
    return Q3_OK;
  }
  if (key == Q3OP_TUNE_FLASH_ROWS) {
    if (value != -1 && value != 1 && value != 2)
      return op_fail(Q3_E_ARG, "rows per wavefront / 16 must be -1, 1 or 2");
    flash_set_rows(value);
    return Q3_OK;
  }
  return op_fail(Q3_E_ARG, "unknown tuning key");
}

}  // extern "C"
