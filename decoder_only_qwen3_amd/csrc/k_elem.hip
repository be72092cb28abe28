// Memory-bound element/row kernels: embedding gather, RMSNorm, QK-Norm + RoPE
// + KV append, argmax and sequence bookkeeping.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" (reactapp.top) -- Paso 2 (embedding lookup), Paso 3 (RMSNorm),
// Paso 4 (RoPE), Paso 5 (QK-Norm and the KV cache), Paso 8 (greedy pick),
// Paso 9 (the generation loop's position bookkeeping).
#include "kernels.h"

namespace q3k {

// ---------------------------------------------------------------- Paso 2
// x[r][:] = E[ids[r]][:] widened to float32.  An out-of-range ID writes a zero
// row and raises Q3_ERRBIT_TOKEN.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids, const T* __restrict__ E,
                                                    int V, int H, float* __restrict__ x,
                                                    uint32_t* err) {
  const int r = blockIdx.x;
  int id = ids[r];
  const bool bad = id < 0 || id >= V;
  if (bad) {
    if (threadIdx.x == 0) atomicOr(err, Q3_ERRBIT_TOKEN);
    id = 0;
  }
  const T* src = E + (int64_t)id * H;
  float* dst = x + (int64_t)r * H;
  for (int c = threadIdx.x; c < H; c += blockDim.x) dst[c] = bad ? 0.f : ld_f<T>(src + c);
}

hipError_t embed(int dtype, const int32_t* ids, int n, const void* E, int V, int H, float* x,
                 uint32_t* err, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == BF16)
    embed_kernel<bf16_t><<<n, 256, 0, s>>>(ids, (const bf16_t*)E, V, H, x, err);
  else
    embed_kernel<float><<<n, 256, 0, s>>>(ids, (const float*)E, V, H, x, err);
  return hipGetLastError();
}


// ---------------------------------------------------------------- Paso 3
// One wavefront per row: out = x * rsqrt(mean(x^2) + eps) * w.  H % 256 == 0.
template <typename Tout>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int rows, RowMap map,
                                                      const float* __restrict__ w, int H, float eps,
                                                      Tout* __restrict__ out) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int src = map.n >= 0 ? map.row[r] : r;
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)src * H);
  float ss = 0.f;
  for (int c = lane; c < H / 4; c += 64) {
    float4 v = xr[c];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)H + eps);
  const float4* wr = reinterpret_cast<const float4*>(w);
  Tout* o = out + (int64_t)r * H;
  for (int c = lane; c < H / 4; c += 64) {
    float4 v = xr[c], g = wr[c];
    st_f<Tout>(o + 4 * c + 0, v.x * inv * g.x);
    st_f<Tout>(o + 4 * c + 1, v.y * inv * g.y);
    st_f<Tout>(o + 4 * c + 2, v.z * inv * g.z);
    st_f<Tout>(o + 4 * c + 3, v.w * inv * g.w);
  }
}

// The same with the row held in registers (NV float4 per lane, H = 256 NV):
// x and w are loaded once, all loads issued before the reduction, and each
// lane writes its four outputs with one store.  On MI355X a launch over 32-64
// decode rows is one memory round trip plus the launch itself, which is what
// this form keeps it to.
template <typename Tout, int NV>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(const float* __restrict__ x, int rows, RowMap map,
                                                          const float* __restrict__ w, float eps,
                                                          Tout* __restrict__ out) {
  constexpr int H = 256 * NV;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int src = map.n >= 0 ? map.row[r] : r;
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)src * H);
  const float4* wr = reinterpret_cast<const float4*>(w);
  float4 v[NV], g[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = xr[lane + 64 * i];
    g[i] = wr[lane + 64 * i];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)H + eps);
  Tout* o = out + (int64_t)r * H;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    store4<Tout>(o + 4 * (lane + 64 * i), v[i].x * inv * g[i].x, v[i].y * inv * g[i].y, v[i].z * inv * g[i].z,
                 v[i].w * inv * g[i].w);
}

hipError_t rmsnorm(int out_dtype, const float* x, int rows, const RowMap& map, const float* w,
                   int H, float eps, void* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((rows + 3) / 4);
#define Q3_RMS_REG(NV)                                                                                   \
  do {                                                                                                   \
    if (out_dtype == BF16)                                                                               \
      rmsnorm_reg_kernel<bf16_t, NV><<<grid, 256, 0, s>>>(x, rows, map, w, eps, (bf16_t*)out);           \
    else                                                                                                 \
      rmsnorm_reg_kernel<float, NV><<<grid, 256, 0, s>>>(x, rows, map, w, eps, (float*)out);             \
    return hipGetLastError();                                                                            \
  } while (0)
  if (H == 1024) Q3_RMS_REG(4);
  if (H == 512) Q3_RMS_REG(2);
  if (H == 2048) Q3_RMS_REG(8);
#undef Q3_RMS_REG
  if (out_dtype == BF16)
    rmsnorm_kernel<bf16_t><<<grid, 256, 0, s>>>(x, rows, map, w, H, eps, (bf16_t*)out);
  else
    rmsnorm_kernel<float><<<grid, 256, 0, s>>>(x, rows, map, w, H, eps, (float*)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- Pasos 4-5
// Sixteen lanes per (token, head unit); units are the n_q query heads, then
// the n_kv key heads, then (decode only) the n_kv value heads of the fused
// projection row.  Lane j of a unit owns dims 4j..4j+3 and 64+4j..64+4j+3,
// i.e. four whole RoPE pairs, read and written as 16-byte runs.
//   query/key: per-head RMSNorm (weights q_norm / k_norm, same eps), then the
//              pair rotation by pos * theta^(-i/64) read from the cos/sin table;
//              queries go to q_out [T][n_q][128], keys to the cache row `pos`.
//   value:     (decode) stored unchanged into the cache's value block.

// Prefill values: block (64-position tile of one sequence, kv head g).  Tiles
// are aligned to positions (tile i covers positions 64i .. 64i + 63), so a
// continuation's first and last tiles may be partial.  The tile's values are
// read as rows, transposed through LDS and written as 16-byte runs of
// consecutive positions into the cache's value blocks ([128 dims][32 keys]
// per 32 positions), so both sides move whole cache lines.
constexpr int VT_TILE = 64;

struct VtTiles {
  int32_t tile_cu[Q3_MAX_BATCH + 1];  // prefix sums of tiles per sequence
  int32_t first[Q3_MAX_BATCH];        // position tile index of each sequence's first tile
  int32_t vstart[Q3_MAX_BATCH];       // vstage_start of each sequence
};

Q3_DEV int vt_seq(const VtTiles& tt, int n, int tix) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tt.tile_cu[mid] <= tix) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Four values of a value row as float32 (bf16 sources widen exactly).
Q3_DEV float4 load4v(const float* p) { return *reinterpret_cast<const float4*>(p); }
Q3_DEV float4 load4v(const bf16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return float4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                __uint_as_float(w[1] & 0xffff0000u)};
}

// Value rows of the call's tokens: token t's value head g at
// vsrc + t * vstride + g * 128 (float32 projection rows, or the bf16 values
// the fused projection epilogue writes).
template <typename T, typename S>
Q3_DEV void vt_append_tile(const S* __restrict__ vsrc, int64_t vstride, const SeqBatch& sb, const VtTiles& tt,
                           const SeqState* __restrict__ st, T* __restrict__ kv, int layer, int n_kv,
                           uint16_t* __restrict__ vh, int64_t vh_keys, int tix, int g) {
  __shared__ T tile[Q3_HEAD_DIM][VT_TILE + 16 / sizeof(T)];
  const int b = vt_seq(tt, sb.n, tix);
  const int P = sb.prior[b], L = sb.cu[b + 1] - sb.cu[b];
  const int p0 = (tt.first[b] + tix - tt.tile_cu[b]) * VT_TILE;  // first position of the tile
  // new positions in the tile: p0 + lo .. p0 + n - 1
  const int lo = max(P - p0, 0), n = min(VT_TILE, P + L - p0);
  const S* src = vsrc + (int64_t)(sb.cu[b] + p0 - P) * vstride + (int64_t)g * Q3_HEAD_DIM;
  // read: thread -> (token r0 + 8i, 4 dims); 256 threads cover 8 tokens per
  // pass, and all eight passes' loads are issued before the first LDS store
  const int c4 = (threadIdx.x & 31) * 4, r0 = threadIdx.x >> 5;
  float4 v[VT_TILE / 8];
#pragma unroll
  for (int i = 0; i < VT_TILE / 8; ++i) {
    const int r = r0 + 8 * i;
    if (r >= lo && r < n) v[i] = load4v(src + (int64_t)r * vstride + c4);
  }
#pragma unroll
  for (int i = 0; i < VT_TILE / 8; ++i) {
    const int r = r0 + 8 * i;
    if (r >= lo && r < n) {
      st_f<T>(&tile[c4 + 0][r], v[i].x);
      st_f<T>(&tile[c4 + 1][r], v[i].y);
      st_f<T>(&tile[c4 + 2][r], v[i].z);
      st_f<T>(&tile[c4 + 3][r], v[i].w);
    }
  }
  __syncthreads();
  const SeqState s = st[sb.slot[b]];
  T* vt = kv_vt(kv, s, KvGeom{n_kv, layer}, g);
  // write: thread -> (dim, 16-byte run of positions)
  constexpr int RUN = 16 / sizeof(T), RUNS = VT_TILE / RUN;
  for (int e = threadIdx.x; e < Q3_HEAD_DIM * RUNS; e += 256) {
    const int d = e / RUNS, k0 = (e % RUNS) * RUN;
    if (k0 >= lo && k0 + RUN <= n) {  // a run never crosses a 32-key block (p0 is a multiple of 64)
      *reinterpret_cast<u32x4*>(vt + vt_off(p0 + k0, d)) = *reinterpret_cast<const u32x4*>(&tile[d][k0]);
    } else {
      for (int k = max(k0, lo); k < min(k0 + RUN, n); ++k) vt[vt_off(p0 + k, d)] = tile[d][k];
    }
  }
  if constexpr (sizeof(T) == 2) {
    // fp16 staging copy of the stored bf16 values for the flash kernel, the
    // tile's keys past the sequence end zero (only for calls without cached
    // tokens: then the tile holds every key of its positions)
    if (vh) {
      uint16_t* dst = vh + ((int64_t)g * vh_keys + tt.vstart[b]) * Q3_HEAD_DIM;
      for (int e = threadIdx.x; e < Q3_HEAD_DIM * (VT_TILE / 8); e += 256) {
        const int d = e >> 3, k0 = (e & 7) * 8;
        u32x4 v;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = k0 + 2 * w < n ? tile[d][k0 + 2 * w] : 0u;
          const uint32_t hi = k0 + 2 * w + 1 < n ? tile[d][k0 + 2 * w + 1] : 0u;
          v[w] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(dst + vt_off(p0 + k0, d)) = bf16x8_to_f16x8(v);
      }
    }
  }
}

constexpr int ROPE_UPG = 2;                         // heads per 16-lane group
constexpr int ROPE_UNITS_PER_BLOCK = 16 * ROPE_UPG;  // 256 threads = 16 groups

template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(
    const float* __restrict__ qkv, int T_, SeqBatch sb, SeqState* __restrict__ st, T* __restrict__ kv,
    int layer, int n_q, int n_kv, const float* __restrict__ qn, const float* __restrict__ kn, float eps,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, T* __restrict__ q_out,
    uint32_t* err, int rope_blocks, VtTiles tt, uint16_t* __restrict__ vh, int64_t vh_keys) {
  // Prefill: blocks from rope_blocks on transpose the value heads (one
  // 64-position tile of one KV head each); the others normalise, rotate and
  // store query and key heads (in decode also the value heads), 32 heads per
  // block.
  if ((int)blockIdx.x >= rope_blocks) {
    const int i = (int)blockIdx.x - rope_blocks;
    vt_append_tile<T, float>(qkv + (int64_t)(n_q + n_kv) * Q3_HEAD_DIM, (int64_t)(n_q + 2 * n_kv) * Q3_HEAD_DIM, sb,
                             tt, st, kv, layer, n_kv, vh, vh_keys, i / n_kv, i % n_kv);
    return;
  }
  // Each 16-lane group takes ROPE_UPG heads (16 apart), loading all of them
  // before any arithmetic so that more of the stream is in flight.
  const int units = sb.decode ? n_q + 2 * n_kv : n_q + n_kv;
  const int stride_units = n_q + 2 * n_kv;
  const int j = threadIdx.x & 15;
  const int64_t n_units = (int64_t)T_ * units;
  int64_t gu[ROPE_UPG];
  float4 a[ROPE_UPG], c[ROPE_UPG];
#pragma unroll
  for (int k = 0; k < ROPE_UPG; ++k) {
    gu[k] = (int64_t)blockIdx.x * ROPE_UNITS_PER_BLOCK + 16 * k + (threadIdx.x >> 4);  // uniform per 16 lanes
    if (gu[k] < n_units) {
      const int t = (int)(gu[k] / units), u = (int)(gu[k] - (int64_t)t * units);
      const float* src = qkv + (int64_t)t * stride_units * Q3_HEAD_DIM + u * Q3_HEAD_DIM;
      a[k] = *reinterpret_cast<const float4*>(src + 4 * j);
      c[k] = *reinterpret_cast<const float4*>(src + 64 + 4 * j);
    }
  }
  const KvGeom g{n_kv, layer};
#pragma unroll
  for (int k = 0; k < ROPE_UPG; ++k) {
    if (gu[k] >= n_units) continue;
    const int t = (int)(gu[k] / units), u = (int)(gu[k] - (int64_t)t * units);
    const int b = seq_of_token(sb, t);
    const SeqState s = st[sb.slot[b]];
    const int pos = sb.decode ? s.len : sb.prior[b] + t - sb.cu[b];
    if (pos < 0 || pos >= s.cap) {  // host validation makes this unreachable
      if (j == 0) atomicOr(err, 4u);
      continue;
    }
    const float4 x = a[k], y = c[k];
    if (u < n_q + n_kv) {
      T *lo, *hi;
      if (u < n_q) {
        T* row = q_out + ((int64_t)t * n_q + u) * Q3_HEAD_DIM;
        lo = row + 4 * j;
        hi = row + 64 + 4 * j;
      } else {
        T* kh = kv_k(kv, s, g, u - n_q);
        lo = kh + kk_off<T>(pos, 4 * j);
        hi = kh + kk_off<T>(pos, 64 + 4 * j);
      }
      qk_norm_rope_store<T>(x, y, u < n_q ? qn : kn, eps, cos_t, sin_t, pos, j, lo, hi);
    } else {
      T* dst = kv_vt(kv, s, g, u - n_q - n_kv);
      const float av[4] = {x.x, x.y, x.z, x.w}, cv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st_f<T>(dst + vt_off(pos, 4 * j + e), av[e]);
        st_f<T>(dst + vt_off(pos, 64 + 4 * j + e), cv[e]);
      }
    }
  }
}

// fp16 staging of values already in the cache (the standalone flash entry
// point): block (64-key tile of one sequence, kv head g).
__global__ __launch_bounds__(256) void vstage_kernel(SeqBatch sb, VtTiles tt, const SeqState* __restrict__ st,
                                                     const bf16_t* __restrict__ kv, int layer, int n_kv,
                                                     uint16_t* __restrict__ vh, int64_t vh_keys) {
  const int tix = blockIdx.x, g = blockIdx.y;
  const int b = vt_seq(tt, sb.n, tix);
  const int L = sb.prior[b] + sb.cu[b + 1] - sb.cu[b];  // every key of the sequence after the call
  const int p0 = (tt.first[b] + tix - tt.tile_cu[b]) * VT_TILE;
  const bf16_t* vt = kv_vt(kv, st[sb.slot[b]], KvGeom{n_kv, layer}, g);
  uint16_t* dst = vh + ((int64_t)g * vh_keys + tt.vstart[b]) * Q3_HEAD_DIM;
  for (int e = threadIdx.x; e < Q3_HEAD_DIM * (VT_TILE / 8); e += 256) {
    const int d = e >> 3, k0 = p0 + (e & 7) * 8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (k0 + 8 <= L) {
      v = ld16(vt + vt_off(k0, d));
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = k0 + 2 * w < L ? vt[vt_off(k0 + 2 * w, d)] : 0u;
        const uint32_t hi = k0 + 2 * w + 1 < L ? vt[vt_off(k0 + 2 * w + 1, d)] : 0u;
        v[w] = lo | (hi << 16);
      }
    }
    *reinterpret_cast<u32x4*>(dst + vt_off(k0, d)) = bf16x8_to_f16x8(v);
  }
}

// Tiles of each sequence's new positions (all = false) or of all its
// positions 0 .. prior + L - 1 (all = true).
VtTiles vt_tiles(const SeqBatch& sb, bool all) {
  VtTiles tt;
  tt.tile_cu[0] = 0;
  for (int b = 0; b < sb.n; ++b) {
    const int P = sb.prior[b], end = P + sb.cu[b + 1] - sb.cu[b];
    tt.first[b] = all ? 0 : P / VT_TILE;
    tt.vstart[b] = vstage_start(sb, b);
    tt.tile_cu[b + 1] = tt.tile_cu[b] + (end + VT_TILE - 1) / VT_TILE - tt.first[b];
  }
  return tt;
}

bool has_prior(const SeqBatch& sb) {
  if (sb.decode) return false;
  for (int b = 0; b < sb.n; ++b)
    if (sb.prior[b] != 0) return true;
  return false;
}

hipError_t rope_append(int dtype, const float* qkv, int T, const SeqBatch& sb, SeqState* st,
                       void* kv, int layer, int n_q, int n_kv, const float* qn, const float* kn,
                       float eps, const float* cos_t, const float* sin_t, void* q_out,
                       uint32_t* err, hipStream_t s, uint16_t* vstage) {
  if (T <= 0) return hipSuccess;
  const int64_t units = (int64_t)T * (sb.decode ? n_q + 2 * n_kv : n_q + n_kv);
  const int64_t rope_blocks = (units + ROPE_UNITS_PER_BLOCK - 1) / ROPE_UNITS_PER_BLOCK;
  // Prefill: the value tiles ride in the same launch (blocks past rope_blocks).
  // A continuation stages all of its sequences' values from the cache once
  // the new ones are in; a fresh prompt stages them here, as they pass.
  VtTiles tt{};
  int64_t vt_blocks = 0;
  const bool cont = has_prior(sb);
  const int64_t vh_keys = sb.decode ? 0 : vstage_keys(sb);
  if (!sb.decode) {
    tt = vt_tiles(sb, false);
    vt_blocks = (int64_t)tt.tile_cu[sb.n] * n_kv;
  }
  if (rope_blocks + vt_blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)(rope_blocks + vt_blocks));
  if (dtype == BF16)
    rope_append_kernel<bf16_t><<<grid, 256, 0, s>>>(qkv, T, sb, st, (bf16_t*)kv, layer, n_q, n_kv, qn, kn,
                                                    eps, cos_t, sin_t, (bf16_t*)q_out, err, (int)rope_blocks, tt,
                                                    cont ? nullptr : vstage, vh_keys);
  else
    rope_append_kernel<float><<<grid, 256, 0, s>>>(qkv, T, sb, st, (float*)kv, layer, n_q, n_kv, qn, kn,
                                                   eps, cos_t, sin_t, (float*)q_out, err, (int)rope_blocks, tt,
                                                   nullptr, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sb.decode || !cont || !vstage || dtype != BF16) return e;
  return vstage_from_cache(T, sb, st, (const bf16_t*)kv, layer, n_kv, vstage, s);
}

hipError_t vstage_from_cache(int T, const SeqBatch& sb, const SeqState* st, const bf16_t* kv, int layer, int n_kv,
                             uint16_t* vstage, hipStream_t s) {
  if (T <= 0 || sb.decode) return hipSuccess;
  const VtTiles tt = vt_tiles(sb, true);
  dim3 grid((unsigned)tt.tile_cu[sb.n], n_kv);
  vstage_kernel<<<grid, 256, 0, s>>>(sb, tt, st, kv, layer, n_kv, vstage, vstage_keys(sb));
  return hipGetLastError();
}

// The value half of Pasos 4-5 for a prefill whose projection epilogue has
// already normalised, rotated and stored the queries and keys: the bf16 value
// rows v [T][n_kv][128] go into the cache's transposed value blocks (and the
// fp16 staging of the flash kernel), as the trailing blocks of
// rope_append_kernel do from the float32 rows.
__global__ __launch_bounds__(256) void vt_append_kernel(const bf16_t* __restrict__ v, SeqBatch sb, VtTiles tt,
                                                        const SeqState* __restrict__ st, bf16_t* __restrict__ kv,
                                                        int layer, int n_kv, uint16_t* __restrict__ vh,
                                                        int64_t vh_keys) {
  const int i = blockIdx.x;
  vt_append_tile<bf16_t, bf16_t>(v, (int64_t)n_kv * Q3_HEAD_DIM, sb, tt, st, kv, layer, n_kv, vh, vh_keys, i / n_kv,
                                 i % n_kv);
}

hipError_t vt_append_bf16(const bf16_t* v, int T, const SeqBatch& sb, SeqState* st, bf16_t* kv, int layer, int n_kv,
                          uint16_t* vstage, hipStream_t s) {
  if (T <= 0 || sb.decode) return hipSuccess;
  const VtTiles tt = vt_tiles(sb, false);
  const bool cont = has_prior(sb);
  const int64_t blocks = (int64_t)tt.tile_cu[sb.n] * n_kv;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (blocks > 0) {
    vt_append_kernel<<<(unsigned)blocks, 256, 0, s>>>(v, sb, tt, st, kv, layer, n_kv, cont ? nullptr : vstage,
                                                      vstage_keys(sb));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!cont || !vstage) return hipSuccess;
  return vstage_from_cache(T, sb, st, kv, layer, n_kv, vstage, s);
}

// ---------------------------------------------------------------- Paso 8
// Greedy pick: largest value, lowest index among equal maxima.
Q3_DEV void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

// Block-wide (max, lowest index) over up to 1024 threads; result valid in thread 0.
Q3_DEV void block_argmax(float& bv, int& bi) {
  __shared__ float sv[16];
  __shared__ int si[16];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float ov = __shfl_xor(bv, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    better(bv, bi, ov, oi);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < (int)(blockDim.x >> 6); ++k) better(bv, bi, sv[k], si[k]);
  }
}

__global__ __launch_bounds__(256) void argmax_rows_kernel(const float* __restrict__ logits, int64_t ld,
                                                          RowMap rows, int V, int32_t* next,
                                                          uint32_t* err) {
  const int r = blockIdx.x;
  const int src = rows.n >= 0 ? rows.row[r] : r;
  const float* p = logits + (int64_t)src * ld;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool finite = true;
  for (int i = threadIdx.x; i < V; i += blockDim.x) {
    float v = p[i];
    finite &= __builtin_isfinite(v);
    better(bv, bi, v, i);
  }
  if (!finite) atomicOr(err, Q3_ERRBIT_NONFINITE);
  block_argmax(bv, bi);
  if (threadIdx.x == 0) next[r] = bi == 0x7fffffff ? 0 : bi;
}

hipError_t argmax_rows(const float* logits, int64_t ld, const RowMap& rows, int V, int32_t* next,
                       uint32_t* err, hipStream_t s) {
  const int n = rows.n;
  if (n <= 0) return hipSuccess;
  argmax_rows_kernel<<<n, 256, 0, s>>>(logits, ld, rows, V, next, err);
  return hipGetLastError();
}

// Pasos 8-9: reduce the lm_head kernel's per-block partials, then move the
// sequences forward (decode: one more cached token; prefill: the prompt).
__global__ __launch_bounds__(1024) void argmax_finish_kernel(const float* __restrict__ pval,
                                                             const int32_t* __restrict__ pidx,
                                                             int nblocks, int M, int32_t* next,
                                                             SeqBatch sb, SeqState* st, uint32_t* err) {
  const int m = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool finite = true;
  int j = threadIdx.x;
  // four independent loads in flight per thread
  for (; j + 3 * (int)blockDim.x < nblocks; j += 4 * blockDim.x) {
    float v[4];
    int ix[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = pval[(int64_t)m * nblocks + j + u * blockDim.x];
      ix[u] = pidx[(int64_t)m * nblocks + j + u * blockDim.x];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      finite &= __builtin_isfinite(v[u]) || ix[u] < 0;
      if (ix[u] >= 0) better(bv, bi, v[u], ix[u]);
    }
  }
  for (; j < nblocks; j += blockDim.x) {
    const float v = pval[(int64_t)m * nblocks + j];
    const int i = pidx[(int64_t)m * nblocks + j];
    finite &= __builtin_isfinite(v) || i < 0;
    if (i >= 0) better(bv, bi, v, i);
  }
  if (!finite) atomicOr(err, Q3_ERRBIT_NONFINITE);
  block_argmax(bv, bi);
  if (threadIdx.x == 0) {
    next[m] = bi == 0x7fffffff ? 0 : bi;
    if (m < sb.n) {
      SeqState* s = st + sb.slot[m];
      s->len = sb.decode ? s->len + 1 : sb.prior[m] + sb.cu[m + 1] - sb.cu[m];
    }
  }
}

hipError_t argmax_finish(const float* pval, const int32_t* pidx, int nblocks, int M, int32_t* next,
                         const SeqBatch& sb, SeqState* st, uint32_t* err, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  argmax_finish_kernel<<<M, 1024, 0, s>>>(pval, pidx, nblocks, M, next, sb, st, err);
  return hipGetLastError();
}

__global__ void seq_advance_kernel(SeqBatch sb, SeqState* st) {
  const int b = threadIdx.x;
  if (b < sb.n) {
    SeqState* s = st + sb.slot[b];
    s->len = sb.decode ? s->len + 1 : sb.prior[b] + sb.cu[b + 1] - sb.cu[b];
  }
}

hipError_t seq_advance(const SeqBatch& sb, SeqState* st, hipStream_t s) {
  seq_advance_kernel<<<1, 64, 0, s>>>(sb, st);
  return hipGetLastError();
}

__global__ void seq_set_len_kernel(SeqBatch sb, SeqState* st, int32_t len) {
  const int b = threadIdx.x;
  if (b < sb.n) st[sb.slot[b]].len = len;
}

hipError_t seq_set_len(const SeqBatch& sb, SeqState* st, int32_t len, hipStream_t s) {
  seq_set_len_kernel<<<1, 64, 0, s>>>(sb, st, len);
  return hipGetLastError();
}

__global__ void widen_kernel(const bf16_t* __restrict__ src, float* __restrict__ dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf2f(src[i]);
}

hipError_t widen_bf16(const bf16_t* src, float* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  widen_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_u32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

}  // namespace q3k
