// libq3 host runtime: the C ABI of include/q3.h -- validation, memory layout,
// weight packing, KV arena, the prefill and decode launch sequences and the
// decode-step HIP graphs.
//
// The launch sequence follows "Dentro de un LLM: Inferencia en Python puro
// para Qwen3-0.6B en MLX": Paso 2 (embedding), Paso 7 (pre-norm block with
// two residual adds, repeated per layer), Paso 8 (final norm, tied lm_head,
// greedy pick), Paso 9 (prefill once, then one token per step with the KV
// cache; the position of a new token is the number already cached).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/q3.h"
#include "../../include/q3_ops.h"
#include "checkpoint.h"
#include "kernels.h"

using namespace q3k;

namespace {

thread_local std::string g_err;

q3_status fail(q3_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(Q3_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));         \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct LayerW {
  size_t qkv, o, gu, d;               // packed projection weights (model dtype), or their codes
  size_t qkv_sb = 0, o_sb = 0, gu_sb = 0, d_sb = 0;  // quantized: scale/offset words
  size_t in_norm, post_norm, qn, kn;  // float32
};

struct WeightLayout {
  size_t embed = 0, head = 0, final_norm = 0, cos_t = 0, sin_t = 0, total = 0;  // head == embed when tied
  std::vector<LayerW> layers;
};

struct WsLayout {
  size_t x, h, qkv, q, o, m, logits, amax_val, amax_idx, attn_part, attn_cnt, lin_part, lin_cnt, vstage, sample,
      wdq, state, err, total;
  int64_t rows;        // activation rows (max prefill tokens, at least Q3_MAX_BATCH)
  int64_t vstage_cap;  // keys per kv head of the fp16 value staging
  int amax_blocks;
};

struct HostSlot {
  bool allocated = false;
  int64_t base = 0;  // element offset
  int64_t cap = 0;
  int64_t len = 0;
};

bool valid_config(const q3_config* c, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return false; };
  if (!c) return bad("config is NULL");
  if (c->n_layers < 0) return bad("n_layers < 0");
  if (c->head_dim != 128) return bad("head_dim must be 128");
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads != 0)
    return bad("n_q_heads must be a positive multiple of n_kv_heads");
  if (c->n_q_heads / c->n_kv_heads > 8) return bad("query heads per kv head must be <= 8");
  if (c->hidden <= 0 || c->hidden % 512 != 0) return bad("hidden must be a positive multiple of 512");
  if (c->ffn <= 0 || c->ffn % 512 != 0) return bad("ffn must be a positive multiple of 512");
  if ((c->n_q_heads * 128) % 512 != 0) return bad("n_q_heads*128 must be a multiple of 512");
  if (c->vocab <= 0 || c->vocab % 16 != 0) return bad("vocab must be a positive multiple of 16");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.0)) return bad("rms_eps and rope_theta must be > 0");
  if (c->dtype != Q3_F32 && c->dtype != Q3_BF16) return bad("dtype must be Q3_F32 or Q3_BF16");
  if (c->max_slots <= 0) return bad("max_slots must be > 0");
  if (c->max_positions <= 0 || c->max_positions > (1 << 24)) return bad("max_positions out of range");
  if (c->dtype == Q3_F32 && c->max_positions > 8192) return bad("the float32 model supports at most 8192 positions");
  if (c->max_prefill_tokens <= 0 || c->max_prefill_tokens > (1 << 24)) return bad("max_prefill_tokens out of range");
  if (c->kv_tokens <= 0) return bad("kv_tokens must be > 0");
  if (c->untied_lm_head != 0 && c->untied_lm_head != 1) return bad("untied_lm_head must be 0 or 1");
  if (c->weight_bits != 0 && c->weight_bits != 8 && c->weight_bits != 4) return bad("weight_bits must be 0, 8 or 4");
  if (c->weight_bits != 0 && c->dtype != Q3_BF16) return bad("quantized weights need the bf16 model");
  return true;
}

int esz(const q3_config& c) { return c.dtype == Q3_BF16 ? 2 : 4; }
int qkv_rows(const q3_config& c) { return (c.n_q_heads + 2 * c.n_kv_heads) * 128; }

WeightLayout weight_layout(const q3_config& c) {
  WeightLayout L;
  const size_t e = esz(c), H = c.hidden, Q = (size_t)c.n_q_heads * 128, I = c.ffn;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.embed = take((size_t)c.vocab * H * e);
  const int bits = c.weight_bits;
  // a projection's weights: bf16, or codes then scale/offset words
  auto proj = [&](size_t rows, size_t K, size_t* sb) {
    if (!bits) return take(rows * K * e);
    const size_t o = take(quant_code_bytes((int)rows, (int)K, bits));
    *sb = take(quant_sb_bytes((int)rows, (int)K));
    return o;
  };
  for (int i = 0; i < c.n_layers; ++i) {
    LayerW w;
    w.qkv = proj((size_t)qkv_rows(c), H, &w.qkv_sb);
    w.o = proj(H, Q, &w.o_sb);
    w.gu = proj(2 * I, H, &w.gu_sb);
    w.d = proj(H, I, &w.d_sb);
    w.in_norm = take(H * 4);
    w.post_norm = take(H * 4);
    w.qn = take(128 * 4);
    w.kn = take(128 * 4);
    L.layers.push_back(w);
  }
  L.final_norm = take(H * 4);
  L.head = c.untied_lm_head ? take((size_t)c.vocab * H * e) : L.embed;
  L.cos_t = take((size_t)c.max_positions * 64 * 4);
  L.sin_t = take((size_t)c.max_positions * 64 * 4);
  L.total = off;
  return L;
}

int max_attn_splits_rows(const q3_config& c) {
  int best = 0;
  for (int B = 1; B <= Q3_MAX_BATCH; ++B) {
    best = std::max(best, B * decode_attn_splits(B, c.n_kv_heads, c.max_positions));
    best = std::max(best, B * fused_attn_smax_max(B, c.n_kv_heads, c.max_positions));
  }
  return best;
}

WsLayout ws_layout(const q3_config& c) {
  WsLayout W;
  const size_t e = esz(c), H = c.hidden, Q = (size_t)c.n_q_heads * 128, I = c.ffn;
  const int64_t R = std::max<int64_t>(c.max_prefill_tokens, Q3_MAX_BATCH);
  W.rows = R;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  W.x = take(R * H * 4);
  W.h = take(R * H * e);
  W.qkv = take((size_t)R * qkv_rows(c) * 4);
  W.q = take(R * Q * e);
  W.o = take(R * Q * e);
  W.m = take(R * I * e);
  W.logits = take((size_t)Q3_MAX_BATCH * c.vocab * 4);
  W.amax_blocks = c.vocab / 16;
  W.amax_val = take((size_t)W.amax_blocks * Q3_MAX_BATCH * 4);
  W.amax_idx = take((size_t)W.amax_blocks * Q3_MAX_BATCH * 4);
  W.attn_part = take((size_t)max_attn_splits_rows(c) * c.n_q_heads * 130 * 4);
  W.attn_cnt = take((size_t)Q3_MAX_BATCH * c.n_kv_heads * 4);
  // split-K partials of the residual projections (o, down): batched decode
  // (weight-streaming kernel) and short prefills (tiled GEMM)
  const int mb = std::min(c.max_slots, Q3_MAX_BATCH);
  size_t part = std::max(skinny_split_floats(mb, (int)H, (int)Q), skinny_split_floats(mb, (int)H, (int)I));
  for (int64_t t = 64; t < R + 64; t += 64) {
    const int tt = (int)std::min<int64_t>(t, R);
    part = std::max({part, gemm_split_floats(tt, (int)H, (int)Q), gemm_split_floats(tt, (int)H, (int)I)});
  }
  W.lin_part = take(std::max<size_t>(16, part) * 4);
  W.lin_cnt = take(std::max<size_t>(H / 16 + 1, 256) * 4);
  // fp16 values of a bf16 prefill call for the flash kernel: every call of
  // fresh prompts fits (sum of L rounded up to 64, plus one tile), and so does
  // one continued sequence of up to max_positions
  W.vstage_cap = std::max<int64_t>(R, c.max_positions) + 64 * Q3_MAX_BATCH + 64;
  W.vstage = take(c.dtype == BF16 ? (size_t)W.vstage_cap * c.n_kv_heads * 128 * 2 : 16);
  W.sample = take(sample_workspace_bytes(Q3_MAX_BATCH));  // top-p sampling, 64 rows at a time
  // quantized weights: one layer's projections dequantized to bf16 for the
  // prefill and batched-decode kernels
  W.wdq = take(c.weight_bits ? ((size_t)qkv_rows(c) * H + H * Q + 3 * I * H) * 2 : 16);
  W.state = take((size_t)c.max_slots * sizeof(SeqState));
  W.err = take(16);
  W.total = off;
  return W;
}

// One decode-step graph per (batch, slots, pointers, stream).
struct GraphKey {
  std::vector<int32_t> slots;
  const void *tokens, *logits, *next, *stream;
  bool operator<(const GraphKey& o) const {
    if (slots != o.slots) return slots < o.slots;
    if (tokens != o.tokens) return tokens < o.tokens;
    if (logits != o.logits) return logits < o.logits;
    if (next != o.next) return next < o.next;
    return stream < o.stream;
  }
};

}  // namespace

namespace q3rt {
void set_last_error(const std::string& msg) { g_err = msg; }
}  // namespace q3rt

struct q3_model {
  q3_config cfg;
  WeightLayout wl;
  WsLayout wsl;
  char* w = nullptr;
  char* kv = nullptr;
  char* ws = nullptr;
  size_t kv_bytes = 0;
  bool bound = false, loaded = false;
  std::vector<HostSlot> slots;
  int64_t kv_used = 0;  // elements
  bool use_graph = true;
  std::map<GraphKey, hipGraphExec_t> graphs;

  template <typename T = void>
  T* W(size_t off) const { return reinterpret_cast<T*>(w + off); }
  template <typename T = void>
  T* WS(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  SeqState* state() const { return WS<SeqState>(wsl.state); }
  uint32_t* err() const { return WS<uint32_t>(wsl.err); }

  void drop_graphs() {
    for (auto& kvp : graphs) hipGraphExecDestroy(kvp.second);
    graphs.clear();
  }
};

namespace {

bool ready(const q3_model* m, q3_status* st) {
  if (!m) { *st = fail(Q3_E_ARG, "model is NULL"); return false; }
  if (!m->bound) { *st = fail(Q3_E_STATE, "q3_bind_memory has not been called"); return false; }
  if (!m->loaded) { *st = fail(Q3_E_STATE, "q3_load_weights has not completed"); return false; }
  return true;
}

q3_status upload_state(q3_model* m, int32_t slot, hipStream_t s) {
  const HostSlot& h = m->slots[slot];
  SeqState v{h.base, (int32_t)h.cap, (int32_t)h.len};
  HIP_TRY(hipMemcpyAsync(m->state() + slot, &v, sizeof(v), hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  return Q3_OK;
}

// ------------------------------------------------------------- launch sequences
q3_status check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q3_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return Q3_OK;
}
#define LAUNCH(expr)                                   \
  do {                                                 \
    q3_status st_ = check((expr), #expr);              \
    if (st_ != Q3_OK) return st_;                      \
  } while (0)

// Key splits per (sequence, kv head) of bf16 decode attention and the launch
// order of the sequences, from the contexts at this call (a recorded graph
// keeps the plan it was recorded with, which only matters for speed).
AttnPlan decode_plan(const q3_model* m, const SeqBatch& sb) {
  const q3_config& c = m->cfg;
  int64_t maxcap = 1;
  int64_t ctx[Q3_MAX_BATCH];
  for (int b = 0; b < sb.n; ++b) {
    const auto& hs = m->slots[sb.slot[b]];
    maxcap = std::max<int64_t>(maxcap, std::min<int64_t>(hs.cap, c.max_positions));
    ctx[b] = hs.len + 1;
  }
  return fused_attn_plan(sb.n, c.n_kv_heads, maxcap, ctx);
}

// The transformer blocks of Paso 7 over `T` rows already embedded in x.
q3_status enqueue_layers(q3_model* m, int T, const SeqBatch& sb, bool decode, hipStream_t s) {
  const q3_config& c = m->cfg;
  const WsLayout& L = m->wsl;
  const int H = c.hidden, Q = c.n_q_heads * 128, I = c.ffn, NQKV = qkv_rows(c);
  float* x = m->WS<float>(L.x);
  void* h = m->WS(L.h);
  float* qkv = m->WS<float>(L.qkv);
  void* qb = m->WS(L.q);
  void* ob = m->WS(L.o);
  void* mb = m->WS(L.m);
  const float* cos_t = m->W<float>(m->wl.cos_t);
  const float* sin_t = m->W<float>(m->wl.sin_t);
  RowMap all;
  all.n = -1;
  const bool bf = c.dtype == Q3_BF16;
  AttnPlan plan;
  plan.smax = 1;
  if (decode && bf) plan = decode_plan(m, sb);
  // Batch-1 decode: every projection on the single-row GEMV (RMSNorm fused
  // into q/k/v and gate/up).  Small batches: row GEMV for o and down.
  // Quantized weights: decode reads the codes directly (batch 1: the
  // single-row GEMV; batches: the weight-streaming kernel); prefill
  // dequantizes each layer's projections to bf16 first and runs the GEMMs on
  // that copy.
  const int bits = c.weight_bits;
  const bool qone = bits && decode && T == 1 && qrowgemv_ok(H) && qrowgemv_ok(Q) && qrowgemv_ok(I);
  const bool qsk = bits && decode && !qone;
  const bool one_h = !bits && bf && decode && rowgemv_ok(T, H);
  const bool one_q = !bits && bf && decode && rowgemv_ok(T, Q);
  const bool one_i = !bits && bf && decode && rowgemv_ok(T, I);
  const bool rows_o = !bits && bf && decode && rowdot_ok(T, Q);
  const bool rows_d = !bits && bf && decode && rowdot_ok(T, I);
  // bf16 prefill on the large-tile GEMM: the q/k/v projection's epilogue does
  // the query/key half of Pasos 4-5 (the float32 q/k/v rows never reach HBM)
  const bool qkv_rope = bf && !decode && gemm_qkv_rope_ok(T, NQKV, H);
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& lw = m->wl.layers[l];
    const bf16_t *Wqkv = nullptr, *Wo = nullptr, *Wgu = nullptr, *Wd = nullptr;
    if (bf && !bits) {
      Wqkv = m->W<bf16_t>(lw.qkv);
      Wo = m->W<bf16_t>(lw.o);
      Wgu = m->W<bf16_t>(lw.gu);
      Wd = m->W<bf16_t>(lw.d);
    } else if (bits && !decode) {
      bf16_t* dq = m->WS<bf16_t>(L.wdq);
      Wqkv = dq;
      Wo = Wqkv + (size_t)NQKV * H;
      Wgu = Wo + (size_t)H * Q;
      Wd = Wgu + (size_t)2 * I * H;
      LAUNCH(dequant_rows(m->W<uint8_t>(lw.qkv), m->W<uint32_t>(lw.qkv_sb), NQKV, H, bits, (bf16_t*)Wqkv, s));
      LAUNCH(dequant_rows(m->W<uint8_t>(lw.o), m->W<uint32_t>(lw.o_sb), H, Q, bits, (bf16_t*)Wo, s));
      LAUNCH(dequant_rows(m->W<uint8_t>(lw.gu), m->W<uint32_t>(lw.gu_sb), 2 * I, H, bits, (bf16_t*)Wgu, s));
      LAUNCH(dequant_rows(m->W<uint8_t>(lw.d), m->W<uint32_t>(lw.d_sb), H, I, bits, (bf16_t*)Wd, s));
    }
    // Paso 3 + Paso 5: normalised input, fused q/k/v projection.  Decode with
    // few rows folds the RMSNorm into the projection kernel's prologue.
    const bool fuse_norm = bf && decode && (one_h || qone || skinny_norm_fuse(T));
    if (!fuse_norm) LAUNCH(rmsnorm(c.dtype, x, T, all, m->W<float>(lw.in_norm), H, c.rms_eps, h, s));
    if (!bf) {
      LAUNCH(gemv_f32(EPI_STORE, (const float*)h, T, m->W<float>(lw.qkv), NQKV, H, qkv, NQKV, s));
    } else if (qone) {
      LAUNCH(qrowgemv(EPI_STORE, bits, x, m->W<uint8_t>(lw.qkv), m->W<uint32_t>(lw.qkv_sb), NQKV, H,
                      m->W<float>(lw.in_norm), c.rms_eps, qkv, s));
    } else if (qsk) {
      LAUNCH(skinny_q(EPI_STORE, bits, fuse_norm ? (const void*)x : h, T, m->W<uint8_t>(lw.qkv),
                      m->W<uint32_t>(lw.qkv_sb), NQKV, H, fuse_norm ? m->W<float>(lw.in_norm) : nullptr, c.rms_eps,
                      qkv, NQKV, s));
    } else if (one_h) {
      LAUNCH(rowgemv_bf16(EPI_STORE, x, Wqkv, NQKV, H, m->W<float>(lw.in_norm), c.rms_eps, qkv, nullptr, nullptr, s));
    } else if (decode) {
      LAUNCH(skinny_bf16(EPI_STORE, fuse_norm ? (const void*)x : h, T, Wqkv, NQKV, H,
                         fuse_norm ? m->W<float>(lw.in_norm) : nullptr, c.rms_eps, qkv, NQKV, nullptr, nullptr, s));
    } else if (qkv_rope) {
      // large prefills: QK-Norm, RoPE and the key append in the projection's
      // epilogue, the values out as bf16 rows (in the q/k/v buffer)
      QkvRopeArgs ra;
      std::memset(&ra, 0, sizeof(ra));
      ra.sb = sb;
      ra.st = m->state();
      ra.kv = (bf16_t*)m->kv;
      ra.layer = l;
      ra.n_q = c.n_q_heads;
      ra.n_kv = c.n_kv_heads;
      ra.qn = m->W<float>(lw.qn);
      ra.kn = m->W<float>(lw.kn);
      ra.eps = c.rms_eps;
      ra.cos_t = cos_t;
      ra.sin_t = sin_t;
      ra.q_out = (bf16_t*)qb;
      ra.v_out = (bf16_t*)qkv;
      ra.err = m->err();
      LAUNCH(gemm_qkv_rope((const bf16_t*)h, T, Wqkv, NQKV, H, ra, s));
    } else {
      LAUNCH(gemm_bf16(EPI_STORE, (const bf16_t*)h, T, Wqkv, NQKV, H, qkv, NQKV, s));
    }
    // QK-Norm, RoPE, cache append and attention (Pasos 4-5).  bf16 decode does
    // all of it in one kernel; the other paths append first.
    if (bf && decode) {
      LAUNCH(decode_attn_fused(qkv, sb, m->state(), (bf16_t*)m->kv, l, c.n_q_heads, c.n_kv_heads,
                               m->W<float>(lw.qn), m->W<float>(lw.kn), c.rms_eps, cos_t, sin_t, plan,
                               m->WS<float>(L.attn_part), m->WS<uint32_t>(L.attn_cnt), (bf16_t*)ob, s));
    } else if (qkv_rope) {
      LAUNCH(vt_append_bf16((const bf16_t*)qkv, T, sb, m->state(), (bf16_t*)m->kv, l, c.n_kv_heads,
                            m->WS<uint16_t>(L.vstage), s));
    } else {
      LAUNCH(rope_append(c.dtype, qkv, T, sb, m->state(), m->kv, l, c.n_q_heads, c.n_kv_heads,
                         m->W<float>(lw.qn), m->W<float>(lw.kn), c.rms_eps, cos_t, sin_t, qb, m->err(), s,
                         bf ? m->WS<uint16_t>(L.vstage) : nullptr));
    }
    if (!bf) {
      LAUNCH(attn_f32((const float*)qb, T, sb, m->state(), (const float*)m->kv, l, c.n_q_heads, c.n_kv_heads,
                      (float*)ob, s));
    } else if (decode) {
      // done above
    } else {
      LAUNCH(flash_prefill((const bf16_t*)qb, T, sb, m->state(), (const bf16_t*)m->kv, m->WS<uint16_t>(L.vstage), l,
                           c.n_q_heads, c.n_kv_heads, (bf16_t*)ob, s));
    }
    // Output projection + residual (Paso 5 end, Paso 7).
    if (!bf) {
      LAUNCH(gemv_f32(EPI_RESADD, (const float*)ob, T, m->W<float>(lw.o), H, Q, x, H, s));
    } else if (qone) {
      LAUNCH(qrowgemv(EPI_RESADD, bits, ob, m->W<uint8_t>(lw.o), m->W<uint32_t>(lw.o_sb), H, Q, nullptr, 0.f, x, s));
    } else if (qsk) {
      LAUNCH(skinny_q(EPI_RESADD, bits, ob, T, m->W<uint8_t>(lw.o), m->W<uint32_t>(lw.o_sb), H, Q, nullptr, 0.f, x, H,
                      s, m->WS<float>(L.lin_part), m->WS<uint32_t>(L.lin_cnt)));
    } else if (one_q) {
      LAUNCH(rowgemv_bf16(EPI_RESADD, ob, Wo, H, Q, nullptr, 0.f, x, nullptr, nullptr, s));
    } else if (rows_o) {
      LAUNCH(rowdot_bf16(EPI_RESADD, (const bf16_t*)ob, T, Wo, H, Q, x, H, s));
    } else if (decode) {
      LAUNCH(skinny_bf16(EPI_RESADD, ob, T, Wo, H, Q, nullptr, 0.f, x, H, nullptr, nullptr, s,
                         m->WS<float>(L.lin_part), m->WS<uint32_t>(L.lin_cnt)));
    } else {
      LAUNCH(gemm_bf16(EPI_RESADD, (const bf16_t*)ob, T, Wo, H, Q, x, H, s,
                       m->WS<float>(L.lin_part), m->WS<uint32_t>(L.lin_cnt)));
    }
    // SwiGLU MLP + residual (Paso 6, Paso 7).
    if (!fuse_norm) LAUNCH(rmsnorm(c.dtype, x, T, all, m->W<float>(lw.post_norm), H, c.rms_eps, h, s));
    if (!bf) {
      LAUNCH(gemv_f32(EPI_SWIGLU, (const float*)h, T, m->W<float>(lw.gu), 2 * I, H, mb, I, s));
      LAUNCH(gemv_f32(EPI_RESADD, (const float*)mb, T, m->W<float>(lw.d), H, I, x, H, s));
    } else if (qone) {
      LAUNCH(qrowgemv(EPI_SWIGLU, bits, x, m->W<uint8_t>(lw.gu), m->W<uint32_t>(lw.gu_sb), 2 * I, H,
                      m->W<float>(lw.post_norm), c.rms_eps, mb, s));
      LAUNCH(qrowgemv(EPI_RESADD, bits, mb, m->W<uint8_t>(lw.d), m->W<uint32_t>(lw.d_sb), H, I, nullptr, 0.f, x, s));
    } else if (qsk) {
      LAUNCH(skinny_q(EPI_SWIGLU, bits, fuse_norm ? (const void*)x : h, T, m->W<uint8_t>(lw.gu),
                      m->W<uint32_t>(lw.gu_sb), 2 * I, H, fuse_norm ? m->W<float>(lw.post_norm) : nullptr, c.rms_eps,
                      mb, I, s));
      LAUNCH(skinny_q(EPI_RESADD, bits, mb, T, m->W<uint8_t>(lw.d), m->W<uint32_t>(lw.d_sb), H, I, nullptr, 0.f, x, H,
                      s, m->WS<float>(L.lin_part), m->WS<uint32_t>(L.lin_cnt)));
    } else if (decode) {
      if (one_h)
        LAUNCH(rowgemv_bf16(EPI_SWIGLU, x, Wgu, 2 * I, H, m->W<float>(lw.post_norm), c.rms_eps, mb, nullptr, nullptr,
                            s));
      else
        LAUNCH(skinny_bf16(EPI_SWIGLU, fuse_norm ? (const void*)x : h, T, Wgu, 2 * I, H,
                           fuse_norm ? m->W<float>(lw.post_norm) : nullptr, c.rms_eps, mb, I, nullptr, nullptr, s));
      if (one_i)
        LAUNCH(rowgemv_bf16(EPI_RESADD, mb, Wd, H, I, nullptr, 0.f, x, nullptr, nullptr, s));
      else if (rows_d)
        LAUNCH(rowdot_bf16(EPI_RESADD, (const bf16_t*)mb, T, Wd, H, I, x, H, s));
      else
        LAUNCH(skinny_bf16(EPI_RESADD, mb, T, Wd, H, I, nullptr, 0.f, x, H, nullptr, nullptr, s,
                           m->WS<float>(L.lin_part), m->WS<uint32_t>(L.lin_cnt)));
    } else {
      LAUNCH(gemm_bf16(EPI_SWIGLU, (const bf16_t*)h, T, Wgu, 2 * I, H, mb, I, s));
      LAUNCH(gemm_bf16(EPI_RESADD, (const bf16_t*)mb, T, Wd, H, I, x, H, s,
                       m->WS<float>(L.lin_part), m->WS<uint32_t>(L.lin_cnt)));
    }
  }
  return Q3_OK;
}

// Final norm + tied lm_head + greedy pick on `rows` rows of x (Paso 8), then
// the length update of Paso 9.
q3_status enqueue_head(q3_model* m, const RowMap& rows, int nrows, const SeqBatch& sb, float* d_logits,
                       int32_t* d_next, hipStream_t s) {
  const q3_config& c = m->cfg;
  const WsLayout& L = m->wsl;
  float* x = m->WS<float>(L.x);
  void* h = m->WS(L.h);
  float* logits = d_logits ? d_logits : m->WS<float>(L.logits);
  // The lm_head has ~9500 blocks; a per-block RMSNorm prologue would repeat the
  // norm in each of them, so the final norm stays a separate kernel.
  const bool fuse_norm = false;
  if (!fuse_norm)
    LAUNCH(rmsnorm(c.dtype, x, nrows, rows, m->W<float>(m->wl.final_norm), c.hidden, c.rms_eps, h, s));
  if (c.dtype == Q3_BF16 && rowgemv_ok(nrows, c.hidden)) {
    LAUNCH(rowgemv_bf16(EPI_ARGMAX, h, m->W<bf16_t>(m->wl.head), c.vocab, c.hidden, nullptr, 0.f, logits,
                        m->WS<float>(L.amax_val), m->WS<int32_t>(L.amax_idx), s));
    LAUNCH(argmax_finish(m->WS<float>(L.amax_val), m->WS<int32_t>(L.amax_idx), rowgemv_argmax_blocks(c.vocab, c.hidden),
                         nrows, d_next, sb, m->state(), m->err(), s));
  } else if (c.dtype == Q3_BF16 && nrows > 1 && headstream_ok(nrows, c.vocab, c.hidden)) {
    // several rows: the rows stay on chip and the vocabulary streams past
    // them once (the weight-streaming kernel would read all rows again for
    // every 16 vocabulary rows)
    LAUNCH(headstream_bf16((const bf16_t*)h, nrows, m->W<bf16_t>(m->wl.head), c.vocab, c.hidden, logits, c.vocab,
                           m->WS<float>(L.amax_val), m->WS<int32_t>(L.amax_idx), s));
    LAUNCH(argmax_finish(m->WS<float>(L.amax_val), m->WS<int32_t>(L.amax_idx), headstream_blocks(c.vocab), nrows,
                         d_next, sb, m->state(), m->err(), s));
  } else if (c.dtype == Q3_BF16) {
    LAUNCH(skinny_bf16(EPI_ARGMAX, fuse_norm ? (const void*)x : h, nrows, m->W<bf16_t>(m->wl.head), c.vocab,
                       c.hidden, fuse_norm ? m->W<float>(m->wl.final_norm) : nullptr, c.rms_eps, logits, c.vocab,
                       m->WS<float>(L.amax_val), m->WS<int32_t>(L.amax_idx), s));
    LAUNCH(argmax_finish(m->WS<float>(L.amax_val), m->WS<int32_t>(L.amax_idx), skinny_argmax_blocks(c.vocab),
                         nrows, d_next, sb, m->state(), m->err(), s));
  } else {
    LAUNCH(gemv_f32(EPI_STORE, (const float*)h, nrows, m->W<float>(m->wl.head), c.vocab, c.hidden, logits,
                    c.vocab, s));
    RowMap ident;
    ident.n = nrows;
    for (int i = 0; i < nrows; ++i) ident.row[i] = i;
    LAUNCH(argmax_rows(logits, c.vocab, ident, c.vocab, d_next, m->err(), s));
    LAUNCH(seq_advance(sb, m->state(), s));
  }
  return Q3_OK;
}

q3_status enqueue_decode(q3_model* m, const SeqBatch& sb, const int32_t* d_tokens, float* d_logits,
                         int32_t* d_next, hipStream_t s) {
  const q3_config& c = m->cfg;
  const int B = sb.n;
  LAUNCH(embed(c.dtype, d_tokens, B, m->W(m->wl.embed), c.vocab, c.hidden, m->WS<float>(m->wsl.x), m->err(), s));
  q3_status st = enqueue_layers(m, B, sb, true, s);
  if (st != Q3_OK) return st;
  RowMap all;
  all.n = -1;
  return enqueue_head(m, all, B, sb, d_logits, d_next, s);
}

// ------------------------------------------------------------- weights
// Where a named tensor goes, and its shape (cols < 0: a vector).
struct TensorSlot {
  std::string kind;
  int layer = -1;
  int64_t rows = -1, cols = -1;
};

bool classify_tensor(const q3_config& c, const std::string& name, TensorSlot* ts, std::string* why) {
  const int64_t H = c.hidden, Q = (int64_t)c.n_q_heads * 128, KVW = (int64_t)c.n_kv_heads * 128, I = c.ffn;
  auto set = [&](const char* kind, int64_t r, int64_t k) {
    ts->kind = kind;
    ts->rows = r;
    ts->cols = k;
    return true;
  };
  if (name == "model.embed_tokens.weight") return set("embed", c.vocab, H);
  if (name == "model.norm.weight") return set("final_norm", H, -1);
  if (name == "lm_head.weight") {
    if (!c.untied_lm_head) {
      *why = "lm_head.weight given but the model ties its head to the embedding (untied_lm_head = 0)";
      return false;
    }
    return set("head", c.vocab, H);
  }
  int li = -1;
  char rest[128] = {0};
  if (std::sscanf(name.c_str(), "model.layers.%d.%127s", &li, rest) != 2 || li < 0 || li >= c.n_layers) {
    *why = "unknown tensor " + name;
    return false;
  }
  ts->layer = li;
  const std::string tail = rest;
  if (tail == "self_attn.q_proj.weight") return set("q", Q, H);
  if (tail == "self_attn.k_proj.weight") return set("k", KVW, H);
  if (tail == "self_attn.v_proj.weight") return set("v", KVW, H);
  if (tail == "self_attn.o_proj.weight") return set("o", H, Q);
  if (tail == "self_attn.q_norm.weight") return set("qn", 128, -1);
  if (tail == "self_attn.k_norm.weight") return set("kn", 128, -1);
  if (tail == "input_layernorm.weight") return set("in", H, -1);
  if (tail == "post_attention_layernorm.weight") return set("post", H, -1);
  if (tail == "mlp.gate_proj.weight") return set("gate", I, H);
  if (tail == "mlp.up_proj.weight") return set("up", I, H);
  if (tail == "mlp.down_proj.weight") return set("down", H, I);
  *why = "unknown tensor " + name;
  return false;
}

size_t expected_tensors(const q3_config& c) { return 2 + (size_t)c.n_layers * 11 + (c.untied_lm_head ? 1 : 0); }

// Copies one tensor (device or host memory, the model's dtype, row-major as
// named) into the model's layout: q/k/v stacked, gate/up interleaved in runs
// of 16 rows, norm weights widened to float32.
hipError_t place_tensor(q3_model* m, const TensorSlot& ts, const void* data, hipStream_t s) {
  const q3_config& c = m->cfg;
  const int64_t H = c.hidden, Q = (int64_t)c.n_q_heads * 128, KVW = (int64_t)c.n_kv_heads * 128, I = c.ffn;
  const size_t e = esz(c);
  const char* src = (const char*)data;
  auto copy = [&](size_t dst_off, size_t bytes) { return hipMemcpyAsync(m->W(dst_off), src, bytes, hipMemcpyDefault, s); };
  auto norm = [&](size_t dst_off, int64_t len) {
    if (c.dtype == Q3_BF16) return widen_bf16((const bf16_t*)src, m->W<float>(dst_off), len, s);
    return hipMemcpyAsync(m->W(dst_off), src, len * 4, hipMemcpyDefault, s);
  };
  const std::string& k = ts.kind;
  const int bits = c.weight_bits;
  if (bits && ts.layer >= 0 && ts.cols > 0) {  // a block projection: quantized from the bf16 source
    const LayerW& lw = m->wl.layers[ts.layer];
    const bf16_t* w = (const bf16_t*)data;
    auto q = [&](size_t codes, size_t sb, int rows, int K, int row0, int inter, int up) {
      return quantize_rows(w, rows, K, bits, m->W<uint8_t>(codes), m->W<uint32_t>(sb), row0, inter, up, s);
    };
    if (k == "q") return q(lw.qkv, lw.qkv_sb, (int)Q, (int)H, 0, 0, 0);
    if (k == "k") return q(lw.qkv, lw.qkv_sb, (int)KVW, (int)H, (int)Q, 0, 0);
    if (k == "v") return q(lw.qkv, lw.qkv_sb, (int)KVW, (int)H, (int)(Q + KVW), 0, 0);
    if (k == "o") return q(lw.o, lw.o_sb, (int)H, (int)Q, 0, 0, 0);
    if (k == "down") return q(lw.d, lw.d_sb, (int)H, (int)I, 0, 0, 0);
    if (k == "gate") return q(lw.gu, lw.gu_sb, (int)I, (int)H, 0, 1, 0);
    if (k == "up") return q(lw.gu, lw.gu_sb, (int)I, (int)H, 0, 1, 1);
    return hipErrorInvalidValue;
  }
  if (k == "embed") return copy(m->wl.embed, (size_t)c.vocab * H * e);
  if (k == "head") return copy(m->wl.head, (size_t)c.vocab * H * e);
  if (k == "final_norm") return norm(m->wl.final_norm, H);
  const LayerW& lw = m->wl.layers[ts.layer];
  if (k == "q") return copy(lw.qkv, Q * H * e);
  if (k == "k") return copy(lw.qkv + Q * H * e, KVW * H * e);
  if (k == "v") return copy(lw.qkv + (Q + KVW) * H * e, KVW * H * e);
  if (k == "o") return copy(lw.o, H * Q * e);
  if (k == "down") return copy(lw.d, H * I * e);
  if (k == "gate" || k == "up") {
    // runs of 16 rows: [gate 16 | up 16] [gate 16 | up 16] ...
    const size_t run = 16 * H * e;
    const size_t dst = lw.gu + (k == "up" ? run : 0);
    return hipMemcpy2DAsync(m->W(dst), 2 * run, src, run, run, I / 16, hipMemcpyDefault, s);
  }
  if (k == "qn") return norm(lw.qn, 128);
  if (k == "kn") return norm(lw.kn, 128);
  if (k == "in") return norm(lw.in_norm, H);
  if (k == "post") return norm(lw.post_norm, H);
  return hipErrorInvalidValue;
}

// A tensor of a checkpoint file and where it goes.
struct CkptJob {
  int file, tensor;
  TensorSlot slot;
};

// Reads the headers of the checkpoint files and checks them against the
// model: every expected tensor exactly once across the files, no other
// tensor, shapes as named, stored in the model's dtype (BF16 or F32).
q3_status plan_checkpoint(const q3_config& c, const char* const* paths, int32_t n_paths, std::vector<StFile>* files,
                          std::vector<CkptJob>* jobs) {
  if (!paths || n_paths <= 0) return fail(Q3_E_ARG, "no checkpoint files");
  const std::string want = c.dtype == Q3_BF16 ? "BF16" : "F32";
  std::map<std::string, int> seen;
  files->resize(n_paths);
  for (int fi = 0; fi < n_paths; ++fi) {
    if (!paths[fi]) return fail(Q3_E_ARG, "NULL checkpoint path");
    std::string err;
    if (!st_read_header(paths[fi], &(*files)[fi], &err)) return fail(Q3_E_ARG, err);
    const auto& ts = (*files)[fi].tensors;
    for (int ti = 0; ti < (int)ts.size(); ++ti) {
      const StTensor& t = ts[ti];
      if (seen.count(t.name)) return fail(Q3_E_ARG, "tensor " + t.name + " appears twice");
      seen[t.name] = fi;
      TensorSlot slot;
      std::string why;
      if (!classify_tensor(c, t.name, &slot, &why)) return fail(Q3_E_ARG, why);
      if (t.dtype != want)
        return fail(Q3_E_UNSUPPORTED, t.name + ": stored as " + t.dtype + ", the model needs " + want);
      const bool ok = slot.cols < 0 ? (t.shape.size() == 1 && t.shape[0] == slot.rows)
                                    : (t.shape.size() == 2 && t.shape[0] == slot.rows && t.shape[1] == slot.cols);
      if (!ok) return fail(Q3_E_ARG, t.name + ": wrong shape");
      jobs->push_back({fi, ti, slot});
    }
  }
  if (jobs->size() != expected_tensors(c)) {
    // name the first missing tensor
    std::vector<std::string> names = {"model.embed_tokens.weight", "model.norm.weight"};
    if (c.untied_lm_head) names.push_back("lm_head.weight");
    static const char* tails[] = {"self_attn.q_proj.weight", "self_attn.k_proj.weight", "self_attn.v_proj.weight",
                                  "self_attn.o_proj.weight", "self_attn.q_norm.weight", "self_attn.k_norm.weight",
                                  "input_layernorm.weight", "post_attention_layernorm.weight",
                                  "mlp.gate_proj.weight", "mlp.up_proj.weight", "mlp.down_proj.weight"};
    for (int l = 0; l < c.n_layers; ++l)
      for (const char* t : tails) names.push_back("model.layers." + std::to_string(l) + "." + t);
    for (const auto& nm : names)
      if (!seen.count(nm)) return fail(Q3_E_ARG, "checkpoint lacks " + nm);
    return fail(Q3_E_ARG, "unexpected tensor count");
  }
  return Q3_OK;
}

}  // namespace

// =================================================================== C ABI
extern "C" {

const char* q3_last_error(void) { return g_err.c_str(); }

size_t q3_weights_bytes(const q3_config* cfg) {
  if (!valid_config(cfg, nullptr)) return 0;
  return weight_layout(*cfg).total;
}

size_t q3_kv_bytes(const q3_config* cfg) {
  if (!valid_config(cfg, nullptr)) return 0;
  const int64_t per_tok = (int64_t)cfg->n_layers * 2 * cfg->n_kv_heads * 128 * esz(*cfg);
  return align_up((size_t)cfg->kv_tokens * per_tok);
}

size_t q3_workspace_bytes(const q3_config* cfg) {
  if (!valid_config(cfg, nullptr)) return 0;
  return ws_layout(*cfg).total;
}

q3_status q3_create(const q3_config* cfg, q3_model** out) {
  std::string why;
  if (!out) return fail(Q3_E_ARG, "out is NULL");
  *out = nullptr;
  if (!valid_config(cfg, &why)) return fail(Q3_E_UNSUPPORTED, "config: " + why);
  q3_model* m = new q3_model();
  m->cfg = *cfg;
  m->wl = weight_layout(*cfg);
  m->wsl = ws_layout(*cfg);
  m->slots.resize(cfg->max_slots);
  *out = m;
  g_err.clear();
  return Q3_OK;
}

void q3_destroy(q3_model* m) {
  if (!m) return;
  m->drop_graphs();
  delete m;
}

q3_status q3_bind_memory(q3_model* m, void* d_weights, size_t weights_bytes, void* d_kv, size_t kv_bytes,
                         void* d_workspace, size_t workspace_bytes, void* stream) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (!d_weights || !d_kv || !d_workspace) return fail(Q3_E_ARG, "NULL device region");
  if (((uintptr_t)d_weights | (uintptr_t)d_kv | (uintptr_t)d_workspace) % kAlign)
    return fail(Q3_E_ARG, "device regions must be 256-byte aligned");
  if (weights_bytes < m->wl.total) return fail(Q3_E_ARG, "weights region too small");
  if (kv_bytes < q3_kv_bytes(&m->cfg)) return fail(Q3_E_ARG, "KV region too small");
  if (workspace_bytes < m->wsl.total) return fail(Q3_E_ARG, "workspace region too small");
  hipStream_t s = (hipStream_t)stream;
  m->drop_graphs();
  m->w = (char*)d_weights;
  m->kv = (char*)d_kv;
  m->kv_bytes = kv_bytes;
  m->ws = (char*)d_workspace;
  m->loaded = false;
  m->kv_used = 0;
  for (auto& sl : m->slots) sl = HostSlot();
  // RoPE table: angle(p, i) = p * theta^(-i/64), evaluated in float64 (Paso 4).
  const q3_config& c = m->cfg;
  std::vector<float> cs((size_t)c.max_positions * 64), sn((size_t)c.max_positions * 64);
  for (int64_t p = 0; p < c.max_positions; ++p)
    for (int i = 0; i < 64; ++i) {
      const double a = (double)p * std::pow(c.rope_theta, -(double)i / 64.0);
      cs[p * 64 + i] = (float)std::cos(a);
      sn[p * 64 + i] = (float)std::sin(a);
    }
  HIP_TRY(hipMemcpyAsync(m->W(m->wl.cos_t), cs.data(), cs.size() * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(m->W(m->wl.sin_t), sn.data(), sn.size() * 4, hipMemcpyHostToDevice, s));
  std::vector<SeqState> zero(c.max_slots, SeqState{0, 0, 0});
  HIP_TRY(hipMemcpyAsync(m->state(), zero.data(), zero.size() * sizeof(SeqState), hipMemcpyHostToDevice, s));
  HIP_TRY(fill_u32(m->err(), 0u, 4, s));
  HIP_TRY(fill_u32(m->WS<uint32_t>(m->wsl.attn_cnt), 0u, (int64_t)Q3_MAX_BATCH * c.n_kv_heads, s));
  HIP_TRY(fill_u32(m->WS<uint32_t>(m->wsl.lin_cnt), 0u, std::max<int64_t>((int64_t)c.hidden / 16 + 1, 256), s));
  HIP_TRY(hipStreamSynchronize(s));
  m->bound = true;
  g_err.clear();
  return Q3_OK;
}

q3_status q3_load_weights(q3_model* m, const q3_tensor* t, int32_t n, void* stream) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (!m->bound) return fail(Q3_E_STATE, "q3_bind_memory has not been called");
  if (!t || n <= 0) return fail(Q3_E_ARG, "no tensors");
  const q3_config& c = m->cfg;
  hipStream_t s = (hipStream_t)stream;
  m->loaded = false;
  m->drop_graphs();
  std::map<std::string, int> seen;
  // Validate everything before the first copy.
  std::vector<std::pair<int, TensorSlot>> jobs;
  for (int i = 0; i < n; ++i) {
    if (!t[i].name || !t[i].data) return fail(Q3_E_ARG, "tensor with NULL name or data");
    const std::string name = t[i].name;
    if (seen.count(name)) return fail(Q3_E_ARG, "duplicate tensor " + name);
    seen[name] = i;
    if (t[i].dtype != c.dtype) return fail(Q3_E_ARG, name + ": dtype differs from the model's");
    if (c.weight_bits) {  // the quantizer reads the source on the device
      hipPointerAttribute_t at;
      if (hipPointerGetAttributes(&at, t[i].data) != hipSuccess || at.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return fail(Q3_E_ARG, name + ": a quantized model needs its tensors in device memory");
      }
    }
    TensorSlot ts;
    std::string why;
    if (!classify_tensor(c, name, &ts, &why)) return fail(Q3_E_ARG, why);
    const bool ok = (ts.cols < 0) ? (t[i].ndim == 1 && t[i].shape[0] == ts.rows)
                                  : (t[i].ndim == 2 && t[i].shape[0] == ts.rows && t[i].shape[1] == ts.cols);
    if (!ok) return fail(Q3_E_ARG, name + ": wrong shape");
    jobs.push_back({i, ts});
  }
  if (jobs.size() != expected_tensors(c))
    return fail(Q3_E_ARG, "expected " + std::to_string(expected_tensors(c)) + " tensors");
  for (const auto& j : jobs) {
    const hipError_t err = place_tensor(m, j.second, t[j.first].data, s);
    if (err != hipSuccess) return fail(Q3_E_HIP, std::string("weight copy: ") + hipGetErrorString(err));
  }
  HIP_TRY(hipStreamSynchronize(s));
  m->loaded = true;
  g_err.clear();
  return Q3_OK;
}

size_t q3_checkpoint_staging_bytes(const q3_config* cfg) {
  if (!cfg || !valid_config(cfg, nullptr)) return 0;
  const size_t H = cfg->hidden, Q = (size_t)cfg->n_q_heads * 128, I = cfg->ffn;
  return std::max({(size_t)cfg->vocab * H, I * H, Q * H}) * esz(*cfg);
}

q3_status q3_checkpoint_validate(const q3_config* cfg, const char* const* paths, int32_t n_paths) {
  if (!cfg) return fail(Q3_E_ARG, "config is NULL");
  std::string why;
  if (!valid_config(cfg, &why)) return fail(Q3_E_ARG, why);
  std::vector<CkptJob> jobs;
  std::vector<StFile> files;
  const q3_status st = plan_checkpoint(*cfg, paths, n_paths, &files, &jobs);
  if (st == Q3_OK) g_err.clear();
  return st;
}

q3_status q3_load_safetensors(q3_model* m, const char* const* paths, int32_t n_paths, void* d_staging,
                              size_t staging_bytes, void* stream) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (!m->bound) return fail(Q3_E_STATE, "q3_bind_memory has not been called");
  const q3_config& c = m->cfg;
  if (!d_staging || staging_bytes < q3_checkpoint_staging_bytes(&c)) return fail(Q3_E_ARG, "staging buffer too small");
  std::vector<CkptJob> jobs;
  std::vector<StFile> files;
  q3_status st = plan_checkpoint(c, paths, n_paths, &files, &jobs);
  if (st != Q3_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  m->loaded = false;
  m->drop_graphs();
  // Tensor bytes go file -> pinned host chunks -> device staging, then into
  // place with the same packing as q3_load_weights.  Two pinned chunks
  // alternate: the file read of one overlaps the copy of the other (an event
  // per chunk says when it may be refilled); stream order alone keeps the
  // staging buffer from being refilled before the previous tensor is placed.
  constexpr size_t kChunk = 32u << 20;
  struct Chunks {  // released on every path out
    void* p[2] = {nullptr, nullptr};
    hipEvent_t ev[2] = {nullptr, nullptr};
    ~Chunks() {
      for (int i = 0; i < 2; ++i) {
        if (ev[i]) (void)hipEventDestroy(ev[i]);
        if (p[i]) (void)hipHostFree(p[i]);
      }
    }
  } ck;
  void** pinned = ck.p;
  hipEvent_t* done_ev = ck.ev;
  bool in_use[2] = {false, false};
  for (int i = 0; i < 2; ++i) {
    HIP_TRY(hipHostMalloc(&pinned[i], kChunk, hipHostMallocDefault));
    HIP_TRY(hipEventCreateWithFlags(&done_ev[i], hipEventDisableTiming));
  }
  st = Q3_OK;
  int open_file = -1, turn = 0;
  FILE* f = nullptr;
  for (const CkptJob& j : jobs) {
    const StFile& sf = files[j.file];
    const StTensor& te = sf.tensors[j.tensor];
    if (j.file != open_file) {
      if (f) std::fclose(f);
      f = std::fopen(sf.path.c_str(), "rb");
      open_file = j.file;
      if (!f) { st = fail(Q3_E_ARG, sf.path + ": cannot open"); break; }
    }
    const uint64_t bytes = te.end - te.begin;
    if (std::fseek(f, (long)(sf.data_start + te.begin), SEEK_SET) != 0) {
      st = fail(Q3_E_ARG, sf.path + ": cannot seek to " + te.name);
      break;
    }
    for (uint64_t done = 0; done < bytes && st == Q3_OK;) {
      const size_t part = (size_t)std::min<uint64_t>(kChunk, bytes - done);
      hipError_t e = in_use[turn] ? hipEventSynchronize(done_ev[turn]) : hipSuccess;
      if (e == hipSuccess && std::fread(pinned[turn], 1, part, f) != part) {
        st = fail(Q3_E_ARG, sf.path + ": short read in " + te.name);
        break;
      }
      if (e == hipSuccess) e = hipMemcpyAsync((char*)d_staging + done, pinned[turn], part, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipEventRecord(done_ev[turn], s);
      if (e != hipSuccess) st = fail(Q3_E_HIP, std::string("checkpoint copy: ") + hipGetErrorString(e));
      in_use[turn] = true;
      turn ^= 1;
      done += part;
    }
    if (st != Q3_OK) break;
    const hipError_t e = place_tensor(m, j.slot, d_staging, s);
    if (e != hipSuccess) {
      st = fail(Q3_E_HIP, std::string("weight copy: ") + hipGetErrorString(e));
      break;
    }
  }
  const hipError_t es = hipStreamSynchronize(s);  // before the pinned chunks go
  if (st == Q3_OK && es != hipSuccess) st = fail(Q3_E_HIP, std::string("checkpoint load: ") + hipGetErrorString(es));
  if (f) std::fclose(f);
  if (st != Q3_OK) return st;
  m->loaded = true;
  g_err.clear();
  return Q3_OK;
}

q3_status q3_seq_alloc(q3_model* m, int32_t slot, int64_t capacity, void* stream) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (!m->bound) return fail(Q3_E_STATE, "q3_bind_memory has not been called");
  if (slot < 0 || slot >= m->cfg.max_slots) return fail(Q3_E_ARG, "slot out of range");
  if (m->slots[slot].allocated) return fail(Q3_E_STATE, "slot already allocated");
  if (capacity <= 0) return fail(Q3_E_ARG, "capacity must be > 0");
  const int64_t cap = (capacity + 63) / 64 * 64;
  if (cap > (int64_t)1 << 30) return fail(Q3_E_UNSUPPORTED, "capacity too large");
  const int64_t per_tok = (int64_t)m->cfg.n_layers * 2 * m->cfg.n_kv_heads * 128;
  const int64_t need = cap * per_tok;
  const int64_t total = (int64_t)(m->kv_bytes / esz(m->cfg));
  if (m->kv_used + need > total) return fail(Q3_E_CAPACITY, "KV arena full");
  HostSlot& h = m->slots[slot];
  h.allocated = true;
  h.base = m->kv_used;
  h.cap = cap;
  h.len = 0;
  m->kv_used += need;
  m->drop_graphs();
  q3_status st = upload_state(m, slot, (hipStream_t)stream);
  if (st != Q3_OK) return st;
  g_err.clear();
  return Q3_OK;
}

q3_status q3_seq_reset(q3_model* m, int32_t n, const int32_t* slots, void* stream) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (!m->bound) return fail(Q3_E_STATE, "q3_bind_memory has not been called");
  if (n < 0 || (n > 0 && !slots)) return fail(Q3_E_ARG, "bad slot list");
  for (int i = 0; i < n; ++i)
    if (slots[i] < 0 || slots[i] >= m->cfg.max_slots) return fail(Q3_E_ARG, "slot out of range");
  // Queued on the stream (no host synchronisation), in batches of Q3_MAX_BATCH.
  for (int i0 = 0; i0 < n; i0 += Q3_MAX_BATCH) {
    SeqBatch sb;
    std::memset(&sb, 0, sizeof(sb));
    sb.n = std::min(n - i0, Q3_MAX_BATCH);
    for (int b = 0; b < sb.n; ++b) sb.slot[b] = slots[i0 + b];
    HIP_TRY(seq_set_len(sb, m->state(), 0, (hipStream_t)stream));
  }
  for (int i = 0; i < n; ++i) m->slots[slots[i]].len = 0;
  g_err.clear();
  return Q3_OK;
}

q3_status q3_kv_reset(q3_model* m, void* stream) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (!m->bound) return fail(Q3_E_STATE, "q3_bind_memory has not been called");
  m->drop_graphs();
  m->kv_used = 0;
  for (int i = 0; i < m->cfg.max_slots; ++i) {
    m->slots[i] = HostSlot();
  }
  std::vector<SeqState> zero(m->cfg.max_slots, SeqState{0, 0, 0});
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipMemcpyAsync(m->state(), zero.data(), zero.size() * sizeof(SeqState), hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  g_err.clear();
  return Q3_OK;
}

q3_status q3_seq_length(const q3_model* m, int32_t slot, int64_t* out) {
  if (!m || !out) return fail(Q3_E_ARG, "NULL argument");
  if (slot < 0 || slot >= m->cfg.max_slots) return fail(Q3_E_ARG, "slot out of range");
  *out = m->slots[slot].len;
  return Q3_OK;
}

q3_status q3_set_option(q3_model* m, int32_t option, int64_t value) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (option == Q3_OPT_DECODE_GRAPH) {
    m->use_graph = value != 0;
    if (!m->use_graph) m->drop_graphs();
    return Q3_OK;
  }
  return fail(Q3_E_ARG, "unknown option");
}

q3_status q3_error_flags(q3_model* m, uint32_t* out, void* stream) {
  if (!m || !out) return fail(Q3_E_ARG, "NULL argument");
  if (!m->bound) return fail(Q3_E_STATE, "q3_bind_memory has not been called");
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipStreamSynchronize(s));
  HIP_TRY(hipMemcpy(out, m->err(), 4, hipMemcpyDeviceToHost));
  HIP_TRY(fill_u32(m->err(), 0u, 1, s));
  HIP_TRY(hipStreamSynchronize(s));
  return Q3_OK;
}

static q3_status check_slots(q3_model* m, int32_t n, const int32_t* slots) {
  if (n < 1 || n > Q3_MAX_BATCH) return fail(Q3_E_ARG, "n_seqs must be in [1, 64]");
  if (!slots) return fail(Q3_E_ARG, "slots is NULL");
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= m->cfg.max_slots) return fail(Q3_E_ARG, "slot out of range");
    if (!m->slots[slots[i]].allocated) return fail(Q3_E_STATE, "slot not allocated");
    for (int j = 0; j < i; ++j)
      if (slots[j] == slots[i]) return fail(Q3_E_ARG, "a slot appears twice");
  }
  return Q3_OK;
}

q3_status q3_prefill(q3_model* m, int32_t n, const int32_t* h_slots, const int32_t* h_cu,
                     const int32_t* d_tokens, float* d_logits, int32_t* d_next, uint32_t flags,
                     void* stream) {
  q3_status st;
  if (!ready(m, &st)) return st;
  if ((st = check_slots(m, n, h_slots)) != Q3_OK) return st;
  if (!h_cu || !d_tokens || !d_next) return fail(Q3_E_ARG, "NULL cu_seqlens, tokens or next");
  const bool all = (flags & Q3_PREFILL_ALL_LOGITS) != 0;
  if (flags & ~Q3_PREFILL_ALL_LOGITS) return fail(Q3_E_ARG, "unknown flag");
  if (all && !d_logits) return fail(Q3_E_ARG, "Q3_PREFILL_ALL_LOGITS needs d_logits");
  if (h_cu[0] != 0) return fail(Q3_E_ARG, "cu_seqlens[0] must be 0");
  for (int b = 0; b < n; ++b) {
    const int64_t L = (int64_t)h_cu[b + 1] - h_cu[b];
    if (L < 1) return fail(Q3_E_ARG, "every sequence needs at least one token");
    const HostSlot& hs = m->slots[h_slots[b]];
    if (hs.len + L > hs.cap) return fail(Q3_E_CAPACITY, "KV cache full: prompt longer than the slot");
    if (hs.len + L > m->cfg.max_positions) return fail(Q3_E_CAPACITY, "sequence longer than max_positions");
  }
  const int64_t T = h_cu[n];
  if (T > m->cfg.max_prefill_tokens) return fail(Q3_E_CAPACITY, "more tokens than max_prefill_tokens");
  const q3_config& c = m->cfg;
  hipStream_t s = (hipStream_t)stream;
  SeqBatch sb;
  std::memset(&sb, 0, sizeof(sb));
  sb.n = n;
  sb.decode = 0;
  for (int b = 0; b < n; ++b) sb.slot[b] = h_slots[b];
  for (int b = 0; b <= n; ++b) sb.cu[b] = h_cu[b];
  for (int b = 0; b < n; ++b) sb.prior[b] = (int32_t)m->slots[h_slots[b]].len;
  if (c.dtype == Q3_BF16 && vstage_keys(sb) > m->wsl.vstage_cap)
    return fail(Q3_E_CAPACITY, "continued sequences too long for one call: split it");

  LAUNCH(embed(c.dtype, d_tokens, (int)T, m->W(m->wl.embed), c.vocab, c.hidden, m->WS<float>(m->wsl.x), m->err(), s));
  st = enqueue_layers(m, (int)T, sb, false, s);
  if (st != Q3_OK) return st;
  RowMap last;
  last.n = n;
  for (int b = 0; b < n; ++b) last.row[b] = h_cu[b + 1] - 1;
  if (!all) {
    st = enqueue_head(m, last, n, sb, d_logits, d_next, s);
    if (st != Q3_OK) return st;
  } else {
    // Every position's logits (Paso 8 as printed computes all rows).
    RowMap every;
    every.n = -1;
    void* h = m->WS(m->wsl.h);
    LAUNCH(rmsnorm(c.dtype, m->WS<float>(m->wsl.x), (int)T, every, m->W<float>(m->wl.final_norm), c.hidden,
                   c.rms_eps, h, s));
    if (c.dtype == Q3_BF16)
      LAUNCH(gemm_bf16(EPI_STORE, (const bf16_t*)h, (int)T, m->W<bf16_t>(m->wl.head), c.vocab, c.hidden, d_logits,
                       c.vocab, s));
    else
      LAUNCH(gemv_f32(EPI_STORE, (const float*)h, (int)T, m->W<float>(m->wl.head), c.vocab, c.hidden, d_logits,
                      c.vocab, s));
    LAUNCH(argmax_rows(d_logits, c.vocab, last, c.vocab, d_next, m->err(), s));
    LAUNCH(seq_advance(sb, m->state(), s));
  }
  for (int b = 0; b < n; ++b) m->slots[h_slots[b]].len += h_cu[b + 1] - h_cu[b];
  g_err.clear();
  return Q3_OK;
}

q3_status q3_decode_step(q3_model* m, int32_t n, const int32_t* h_slots, const int32_t* d_tokens,
                         float* d_logits, int32_t* d_next, void* stream) {
  q3_status st;
  if (!ready(m, &st)) return st;
  if ((st = check_slots(m, n, h_slots)) != Q3_OK) return st;
  if (!d_tokens || !d_next) return fail(Q3_E_ARG, "NULL tokens or next");
  for (int b = 0; b < n; ++b) {
    const HostSlot& hs = m->slots[h_slots[b]];
    if (hs.len + 1 > hs.cap) return fail(Q3_E_CAPACITY, "KV cache full");
    if (hs.len + 1 > m->cfg.max_positions) return fail(Q3_E_CAPACITY, "sequence reached max_positions");
  }
  hipStream_t s = (hipStream_t)stream;
  SeqBatch sb;
  std::memset(&sb, 0, sizeof(sb));
  sb.n = n;
  sb.decode = 1;
  for (int b = 0; b < n; ++b) {
    sb.slot[b] = h_slots[b];
    sb.cu[b] = b;
  }
  sb.cu[n] = n;

  if (m->use_graph && s != nullptr) {
    GraphKey key{std::vector<int32_t>(h_slots, h_slots + n), d_tokens, d_logits, d_next, stream};
    auto it = m->graphs.find(key);
    if (it == m->graphs.end()) {
      if (m->graphs.size() >= 64) m->drop_graphs();  // bound the cache of recorded steps
      HIP_TRY(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
      st = enqueue_decode(m, sb, d_tokens, d_logits, d_next, s);
      hipGraph_t g = nullptr;
      hipError_t ec = hipStreamEndCapture(s, &g);
      if (st != Q3_OK) {
        if (g) hipGraphDestroy(g);
        return st;
      }
      if (ec != hipSuccess) return fail(Q3_E_HIP, std::string("graph capture: ") + hipGetErrorString(ec));
      hipGraphExec_t ge = nullptr;
      hipError_t ei = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
      hipGraphDestroy(g);
      if (ei != hipSuccess) return fail(Q3_E_HIP, std::string("graph instantiate: ") + hipGetErrorString(ei));
      it = m->graphs.emplace(key, ge).first;
    }
    HIP_TRY(hipGraphLaunch(it->second, s));
  } else {
    st = enqueue_decode(m, sb, d_tokens, d_logits, d_next, s);
    if (st != Q3_OK) return st;
  }
  for (int b = 0; b < n; ++b) m->slots[h_slots[b]].len += 1;
  g_err.clear();
  return Q3_OK;
}

q3_status q3_check_tokens(const q3_model* m, const int32_t* h_tokens, int64_t n) {
  if (!m) return fail(Q3_E_ARG, "model is NULL");
  if (n < 0 || (n > 0 && !h_tokens)) return fail(Q3_E_ARG, "bad token array");
  for (int64_t i = 0; i < n; ++i)
    if (h_tokens[i] < 0 || h_tokens[i] >= m->cfg.vocab)
      return fail(Q3_E_ARG, "token " + std::to_string(i) + " has ID " + std::to_string(h_tokens[i]) +
                                " outside [0, " + std::to_string(m->cfg.vocab) + ")");
  g_err.clear();
  return Q3_OK;
}

q3_status q3_sample(q3_model* m, int32_t n_rows, const float* d_logits, int64_t ld, float temperature,
                    float top_p, const float* d_uniform, int32_t* d_next, void* stream) {
  q3_status st;
  if (!ready(m, &st)) return st;
  const int V = (int)m->cfg.vocab;
  if (n_rows < 0 || (n_rows > 0 && (!d_logits || !d_next))) return fail(Q3_E_ARG, "bad rows or NULL pointer");
  if (ld < V) return fail(Q3_E_ARG, "ld smaller than the vocabulary");
  if (!std::isfinite(temperature) || (temperature != 0.f && temperature < 1e-30f))
    return fail(Q3_E_ARG, "temperature must be 0 or a finite value >= 1e-30");
  if (!std::isfinite(top_p)) return fail(Q3_E_ARG, "top_p must be finite");
  if (temperature != 0.f && n_rows > 0 && !d_uniform) return fail(Q3_E_ARG, "sampling needs d_uniform");
  HIP_TRY(sample_top_p(d_logits, ld, n_rows, V, temperature, top_p, d_uniform, d_next, m->err(),
                       m->WS(m->wsl.sample), (hipStream_t)stream));
  g_err.clear();
  return Q3_OK;
}

}  // extern "C"

// Single-kernel entry on a live model (include/q3_ops.h): the fused decode
// attention of one layer for the given slots, as q3_decode_step runs it.
q3_status q3op_model_decode_attention(q3_model* m, int32_t layer, int32_t n, const int32_t* h_slots, void* stream) {
  q3_status st;
  if (!ready(m, &st)) return st;
  if ((st = check_slots(m, n, h_slots)) != Q3_OK) return st;
  const q3_config& c = m->cfg;
  if (c.dtype != Q3_BF16) return fail(Q3_E_UNSUPPORTED, "the fused decode attention is the bf16 model's kernel");
  if (layer < 0 || layer >= c.n_layers) return fail(Q3_E_ARG, "layer out of range");
  SeqBatch sb;
  std::memset(&sb, 0, sizeof(sb));
  sb.n = n;
  sb.decode = 1;
  for (int b = 0; b < n; ++b) {
    const HostSlot& hs = m->slots[h_slots[b]];
    if (hs.len < 1) return fail(Q3_E_STATE, "slot is empty");
    if (hs.len + 1 > hs.cap || hs.len + 1 > c.max_positions) return fail(Q3_E_CAPACITY, "KV cache full");
    sb.slot[b] = h_slots[b];
    sb.cu[b] = b;
  }
  sb.cu[n] = n;
  const WsLayout& L = m->wsl;
  const LayerW& lw = m->wl.layers[layer];
  LAUNCH(decode_attn_fused(m->WS<float>(L.qkv), sb, m->state(), (bf16_t*)m->kv, layer, c.n_q_heads, c.n_kv_heads,
                           m->W<float>(lw.qn), m->W<float>(lw.kn), c.rms_eps, m->W<float>(m->wl.cos_t),
                           m->W<float>(m->wl.sin_t), decode_plan(m, sb), m->WS<float>(L.attn_part),
                           m->WS<uint32_t>(L.attn_cnt), (bf16_t*)m->WS(L.o), (hipStream_t)stream));
  g_err.clear();
  return Q3_OK;
}
