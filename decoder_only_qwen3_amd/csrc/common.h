// Device-side helpers shared by the gfx950 kernels of libq3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 held as its bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define Q3_HEAD_DIM 128
#define Q3_MAX_BATCH 64

#define Q3_DEV static __device__ __forceinline__

Q3_DEV float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest, ties to even (NaN kept quiet).
Q3_DEV bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

Q3_DEV uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Storage conversion helpers for the two activation/KV element types.
template <typename T> Q3_DEV float ld_f(const T* p);
template <> Q3_DEV float ld_f<float>(const float* p) { return *p; }
template <> Q3_DEV float ld_f<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <typename T> Q3_DEV void st_f(T* p, float v);
template <> Q3_DEV void st_f<float>(float* p, float v) { *p = v; }
template <> Q3_DEV void st_f<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }

// Sum across the 64 lanes of a wavefront; every lane gets the total.
Q3_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
Q3_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

Q3_DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

Q3_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
Q3_DEV f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

Q3_DEV f32x4 mfma16_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two floats -> packed fp16, round to nearest even.
Q3_DEV uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 h = __builtin_convertvector((f32x2){lo, hi}, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Eight bf16 values -> eight fp16 values.  Every bf16 value inside fp16's
// normal range is exact in fp16; conversion rounds toward zero, so a magnitude
// beyond fp16's range saturates at 65504 instead of becoming infinite.
Q3_DEV u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16);
    const float hi = __uint_as_float(v[i] & 0xffff0000u);
    r[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return r;
}

Q3_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming 16-byte load (nontemporal hint): for data read once per launch,
// such as the KV cache in decode.  On MI355X a read stream of such loads
// reaches ~7.0 TB/s against ~6.2 TB/s with ordinary loads.
Q3_DEV u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
Q3_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier without the fence of __syncthreads(), whose wait for every
// outstanding vector-memory operation would drain a load pipeline; the memory
// clobber keeps the compiler from moving LDS accesses across it.
Q3_DEV void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Sixteen-byte accesses with the agent-scope cache policy (sc1: written through
// to, and read back from, memory that every XCD's L2 sees), for partial results
// that another block merges.  The four-byte agent-scope atomics carry the same
// policy, but four times the transactions.
constexpr int kCpolSc1 = 16;  // cache-policy operand of the buffer builtins: sc1
Q3_DEV __amdgpu_buffer_rsrc_t agent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
Q3_DEV void st4_agent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kCpolSc1);
}
Q3_DEV f32x4 ld4_agent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCpolSc1));
}

// Sequences of one call.  Prefill: token t of the call belongs to sequence b
// with cu[b] <= t < cu[b+1] and sits at position prior[b] + t - cu[b], where
// prior[b] tokens of that sequence are already cached (0 for a fresh prompt;
// a continuation attends to them too).  Decode: token b is the single new
// token of sequence b, at position = that slot's length.
struct SeqBatch {
  int32_t n;
  int32_t decode;
  int32_t slot[Q3_MAX_BATCH];
  int32_t cu[Q3_MAX_BATCH + 1];
  int32_t prior[Q3_MAX_BATCH];
};

// Per-slot KV placement and length, resident on the device.
struct SeqState {
  int64_t base;   // element offset of the slot's region in the KV arena
  int32_t cap;    // token capacity (multiple of 64)
  int32_t len;    // tokens currently cached
};

// KV arena addressing.  A slot's region holds, for each layer, the keys of
// each kv head (cap * 128 elements per head, laid out by kk_off) followed by
// the values as [kv_head][cap/32][128][32] (transposed within blocks of 32
// keys).
struct KvGeom {
  int32_t n_kv;
  int32_t layer;
};
template <typename T>
Q3_DEV T* kv_k(T* arena, const SeqState& s, KvGeom g, int head) {
  return arena + s.base + ((int64_t)(g.layer * 2) * g.n_kv + head) * (int64_t)s.cap * Q3_HEAD_DIM;
}
// Element of (key, dim) from a head's key base.  float32 caches: rows
// [cap][128].  bf16 caches: blocks of 32 keys (8 KiB), each stored in the
// order the attention kernels take its keys as MFMA operands: 16-byte chunk
// c = (sbk * 4 + ks) * 64 + fq * 16 + fr of a block holds dims
// ks * 32 + fq * 8 .. +7 of its key 8 * (fr / 4) + 4 * sbk + fr % 4.  A
// wavefront's operand load (one chunk per lane, lane = fq * 16 + fr) is then
// 1 KiB of consecutive bytes; with rows, each load took 64 bytes from each of
// 16 rows, and streamed about 8 % slower on MI355X.
template <typename T>
Q3_DEV int64_t kk_off(int key, int dim);
template <>
Q3_DEV int64_t kk_off<float>(int key, int dim) { return (int64_t)key * Q3_HEAD_DIM + dim; }
template <>
Q3_DEV int64_t kk_off<bf16_t>(int key, int dim) {
  const int k = key & 31;
  const int sbk = (k >> 2) & 1, fr = ((k >> 3) << 2) | (k & 3);
  const int ks = dim >> 5, fq = (dim >> 3) & 3;
  return ((int64_t)(key >> 5) << 12) + ((((sbk * 4 + ks) * 4 + fq) * 16 + fr) << 3) + (dim & 7);
}
// Values are stored in blocks of 32 keys, each block [128 dims][32 keys]: a
// 32-key run of every dim is one contiguous 8 KiB read, and a dim's 8-key
// run is 16 contiguous bytes (the MFMA operand).  vt_off gives the element
// of (key, dim) from the head's value base.
Q3_DEV int64_t vt_off(int key, int dim) { return ((int64_t)(key >> 5) * Q3_HEAD_DIM + dim) * 32 + (key & 31); }
template <typename T>
Q3_DEV T* kv_vt(T* arena, const SeqState& s, KvGeom g, int head) {
  return arena + s.base + ((int64_t)(g.layer * 2 + 1) * g.n_kv + head) * (int64_t)s.cap * Q3_HEAD_DIM;
}

// fp16 staging of a prefill call's values (the P.V operand of the flash
// kernel): per kv head, all keys 0 .. prior + L - 1 of sequence b from key
// vstage_start(sb, b) on (whole 64-key tiles, the tail zero), in the value
// layout above; vstage_keys(sb) keys per head.  Host side: the kernels get
// the starts in their tile tables.
inline int vstage_start(const SeqBatch& sb, int b) {
  int s = 0;
  for (int i = 0; i < b; ++i) s += ((sb.prior[i] + sb.cu[i + 1] - sb.cu[i] + 63) >> 6) << 6;
  return s;
}
inline int64_t vstage_keys(const SeqBatch& sb) { return (int64_t)vstage_start(sb, sb.n) + 64; }

Q3_DEV int seq_of_token(const SeqBatch& sb, int t) {
  if (sb.decode) return t;
  int lo = 0, hi = sb.n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (sb.cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Four consecutive outputs as one store (16 bytes float32, 8 bytes bf16).
template <typename T>
Q3_DEV void store4(T* p, float a, float b, float c, float d);
template <>
Q3_DEV void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = float4{a, b, c, d};
}
template <>
Q3_DEV void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  u32x2 w;
  w[0] = pack_bf2(a, b);
  w[1] = pack_bf2(c, d);
  *reinterpret_cast<u32x2*>(p) = w;
}

// QK-Norm + rotate-half RoPE of one 128-wide query or key head, spread over
// 16 lanes (lane j holds dims 4j..4j+3 in x and 64+4j..64+4j+3 in y, i.e.
// four whole RoPE pairs): RMSNorm over the head with weight w, then the pair
// rotation by the position's angles (cos_t/sin_t rows of 64); dims 4j..4j+3
// are stored at lo, dims 64+4j..64+4j+3 at hi.  Every kernel that does this
// step calls these functions, so the paths round identically.
struct RopeIn {
  float4 wa, wc, cs, sn;
};
Q3_DEV RopeIn rope_inputs(const float* __restrict__ w, const float* __restrict__ cos_t,
                          const float* __restrict__ sin_t, int pos, int j) {
  RopeIn in;
  in.wa = *reinterpret_cast<const float4*>(w + 4 * j);
  in.wc = *reinterpret_cast<const float4*>(w + 64 + 4 * j);
  in.cs = *reinterpret_cast<const float4*>(cos_t + (int64_t)pos * 64 + 4 * j);
  in.sn = *reinterpret_cast<const float4*>(sin_t + (int64_t)pos * 64 + 4 * j);
  return in;
}
template <typename T>
Q3_DEV void qk_norm_rope_apply(float4 x, float4 y, const RopeIn& in, float eps, T* __restrict__ lo,
                               T* __restrict__ hi) {
  float ss = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w + y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 16);
  const float inv = rsqrtf(ss * (1.f / Q3_HEAD_DIM) + eps);
  const float4 wa = in.wa, wc = in.wc, cs = in.cs, sn = in.sn;
  x = float4{x.x * inv * wa.x, x.y * inv * wa.y, x.z * inv * wa.z, x.w * inv * wa.w};
  y = float4{y.x * inv * wc.x, y.y * inv * wc.y, y.z * inv * wc.z, y.w * inv * wc.w};
  store4<T>(lo, x.x * cs.x - y.x * sn.x, x.y * cs.y - y.y * sn.y, x.z * cs.z - y.z * sn.z,
            x.w * cs.w - y.w * sn.w);
  store4<T>(hi, x.x * sn.x + y.x * cs.x, x.y * sn.y + y.y * cs.y, x.z * sn.z + y.z * cs.z,
            x.w * sn.w + y.w * cs.w);
}
template <typename T>
Q3_DEV void qk_norm_rope_store(float4 x, float4 y, const float* __restrict__ w, float eps,
                               const float* __restrict__ cos_t, const float* __restrict__ sin_t, int pos, int j,
                               T* __restrict__ lo, T* __restrict__ hi) {
  qk_norm_rope_apply<T>(x, y, rope_inputs(w, cos_t, sin_t, pos, j), eps, lo, hi);
}

// Error bits raised by kernels (read back by q3_error_flags).
#define Q3_ERRBIT_TOKEN 1u
#define Q3_ERRBIT_NONFINITE 2u
