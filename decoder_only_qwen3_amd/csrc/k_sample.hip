// Temperature + top-p (nucleus) sampling of logit rows.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" (reactapp.top) -- Paso 8 (sampling): scale the logits by
// 1/temperature, softmax, order the probabilities from largest to smallest,
// keep the shortest leading run whose running sum reaches top_p (the count of
// running sums below top_p, plus one), renormalise, draw one.  Equal
// probabilities are ordered by increasing token ID; the draw is an inverse
// transform with a caller-supplied uniform u in [0, 1).
//
// No sort.  With d_i = (max - l_i) * log2(e) / T >= 0, the weight of token i
// is w_i = 2^-d_i in (0, 1], and the float32 bit pattern of d_i (the key)
// orders the tokens from the most to the least probable.  Each weight's mass
// is held as a 2^-40 fixed-point integer, so every sum below is exact and
// independent of summation order: the choice is deterministic.  The running
// mass of the ordered tokens reaches a target t at the token found by a radix
// descent over the key: a histogram of mass per key digit, scanned from the
// smallest key up, picks the digit whose bucket holds the crossing, and the
// next digit refines inside that bucket (13 + 9 + 9 bits).  Tokens with one
// exact key share one mass, so the crossing inside such a group is an index
// count.  The nucleus cut is one search (t = ceil(top_p * S)), the draw
// another (t = floor(u * kept mass) + 1).
//
// Five launches per batch of up to 64 rows; the three passes over the logits
// split each row over up to 64 blocks:
//   1. per-block maxima (a non-finite logit makes the block's maximum NaN);
//   2. weights, total mass S and the first-digit mass histogram (per-block
//      LDS histograms merged by 64-bit integer atomics);
//   3. one block per row: the first-digit buckets that can hold the nucleus
//      cut and the draw (the draw's bucket is bracketed by the smallest and
//      largest kept mass the cut's bucket allows);
//   4. the tokens of those buckets gathered into a per-row list;
//   5. one block per row: both refinements and the index count over the list,
//      or, when the list overflowed (a very flat row), over the whole row.
#include "kernels.h"

namespace q3k {
namespace {

constexpr int kB1 = 8192;      // first digit: key bits 30..18
constexpr int kB2 = 512;       // second and third digits: bits 17..9, 8..0
constexpr int kCap = 65536;    // gathered tokens per row
constexpr int kEqMax = 1024;   // equal-key tokens ranked in LDS
constexpr int kMaxW = 4;       // gathered first-digit buckets besides the cut's
constexpr int kMaxNB = 64;     // blocks per row in the row passes
constexpr int kPassThreads = 256;
constexpr int kRowThreads = 1024;
constexpr int kRows = 64;      // rows per batch of launches
constexpr float kMassScale = 1099511627776.f;  // 2^40
constexpr float kLog2e = 1.4426950408889634f;

typedef unsigned long long u64;

// Per-row workspace.
struct RowMeta {
  u64 S;             // total mass
  uint32_t n_cand;   // gathered tokens (may exceed kCap: overflow)
  int32_t c1, dlo, dhi;
  int32_t few;       // dhi - dlo < kMaxW: the gather ran
  u64 c1_above;      // mass of the buckets below c1
  u64 dlo_above;     // mass of the buckets below dlo
  u64 hw[kMaxW];     // masses of buckets dlo .. dhi (when few)
};
struct Cand {
  uint32_t key, idx;
};
constexpr size_t kOffMax = 256;
constexpr size_t kOffH1 = kOffMax + kMaxNB * 4;
constexpr size_t kOffCand = kOffH1 + (size_t)kB1 * 8;
constexpr size_t kRowBytes = (kOffCand + (size_t)kCap * 8 + 255) / 256 * 256;

struct RowWs {
  RowMeta* meta;
  float* maxpart;
  u64* h1;
  Cand* cand;
};
Q3_DEV RowWs row_ws(void* ws, int row) {
  char* b = (char*)ws + (size_t)row * kRowBytes;
  return RowWs{(RowMeta*)b, (float*)(b + kOffMax), (u64*)(b + kOffH1), (Cand*)(b + kOffCand)};
}

struct Row {
  const float* p;
  int V;
  bool vec;       // 16-byte aligned row start: float4 loads
  float lmax, k;  // d = (lmax - l) * k, k = log2(e) / T
};

Q3_DEV uint32_t key_of(const Row& r, float l) { return __float_as_uint((r.lmax - l) * r.k); }

// floor(2^-d * 2^40) from the float32 weight's bits (weights below 2^-40 have
// no mass; the weight of d = 0 is 1, mass 2^40).
Q3_DEV u64 mass_of_key(uint32_t key) {
  const uint32_t b = __float_as_uint(__builtin_amdgcn_exp2f(-__uint_as_float(key)));
  const int e = (int)(b >> 23);  // biased exponent (sign 0, weight <= 1)
  const u64 m = (u64)((b & 0x7fffffu) | 0x800000u);
  const int sh = e - 110;        // weight = m * 2^(e - 150); mass = m * 2^(e - 110)
  if (e == 0 || sh <= -24) return 0;
  return sh >= 0 ? m << sh : m >> -sh;
}

// f(index, logit) over elements [i0, i1) of the row, every thread a strided
// share; float4 loads in batches of four so that many loads are in flight.
template <class F>
Q3_DEV void for_range(const Row& r, int i0, int i1, F&& f) {
  const int nt = blockDim.x;
  int done = i0;
  if (r.vec && (i0 & 3) == 0) {
    const float4* p4 = reinterpret_cast<const float4*>(r.p + i0);
    const int n4 = (i1 - i0) >> 2;
    int i = threadIdx.x;
    for (; i + 3 * nt < n4; i += 4 * nt) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = p4[i + u * nt];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = i0 + 4 * (i + u * nt);
        f(b, v[u].x);
        f(b + 1, v[u].y);
        f(b + 2, v[u].z);
        f(b + 3, v[u].w);
      }
    }
    for (; i < n4; i += nt) {
      const float4 v = p4[i];
      const int b = i0 + 4 * i;
      f(b, v.x);
      f(b + 1, v.y);
      f(b + 2, v.z);
      f(b + 3, v.w);
    }
    done = i0 + (n4 << 2);
  }
  for (int i = done + (int)threadIdx.x; i < i1; i += nt) f(i, r.p[i]);
}

Q3_DEV u64 shfl_up_u64(u64 v, int o) {
  const uint32_t lo = __shfl_up((uint32_t)v, o, 64), hi = __shfl_up((uint32_t)(v >> 32), o, 64);
  return ((u64)hi << 32) | lo;
}
Q3_DEV u64 shfl_xor_u64(u64 v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
  return ((u64)hi << 32) | lo;
}

// Exclusive prefix sum over the block's threads in thread order (red: one
// slot per wavefront).
Q3_DEV u64 block_exclusive_scan(u64 v, u64* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u64 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 t = shfl_up_u64(inc, o);
    if (lane >= o) inc += t;
  }
  __syncthreads();  // red may still be read by a previous call
  if (lane == 63) red[w] = inc;
  __syncthreads();
  u64 before = 0;
  for (int k = 0; k < w; ++k) before += red[k];
  return before + inc - v;
}

Q3_DEV u64 block_sum(u64 v, u64* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_u64(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  u64 all = 0;
  for (int k = 0; k < (int)(blockDim.x >> 6); ++k) all += red[k];
  return all;
}

// Adds `q` to bucket d, committing a run of equal buckets at once (a row whose
// tokens share a bucket costs few LDS atomics).
struct RunAdd {
  int cur = -1;
  u64 run = 0;
  __device__ __forceinline__ void add(u64* h, int d, u64 q) {
    if (d != cur) {
      if (run) atomicAdd(&h[cur], run);
      cur = d;
      run = 0;
    }
    run += q;
  }
  __device__ __forceinline__ void flush(u64* h) {
    if (run) atomicAdd(&h[cur], run);
  }
};

Q3_DEV void clear(u64* h, int n) {
  for (int b = threadIdx.x; b < n; b += blockDim.x) h[b] = 0;
}

struct Crossing {
  int digit;
  u64 above;  // base + mass of the smaller-key buckets
};

// The bucket, scanning from bucket 0 up, that takes the running mass
// (starting at `base`) to at least t.  Requires base < t <= base + sum(h).
// 1024 threads; n is a multiple of 1024 or at most 1024.
Q3_DEV Crossing find_crossing(const u64* h, int n, u64 base, u64 t, u64* red, Crossing* out) {
  const int per = n > kRowThreads ? n / kRowThreads : 1;
  const int b0 = (int)threadIdx.x * per;
  u64 mine = 0;
  if (b0 < n)
    for (int k = 0; k < per; ++k) mine += h[b0 + k];
  u64 run = base + block_exclusive_scan(mine, red);
  if (b0 < n && run < t && run + mine >= t) {
    for (int k = 0; k < per; ++k) {
      if (run + h[b0 + k] >= t) {
        *out = Crossing{b0 + k, run};
        break;
      }
      run += h[b0 + k];
    }
  }
  __syncthreads();
  const Crossing c = *out;
  __syncthreads();
  return c;
}

struct Found {
  uint32_t key;
  u64 above, q, j;  // mass of smaller keys; mass per token of `key`; 1-based rank among equal keys
};

Q3_DEV Found finish(uint32_t key, u64 above, u64 t) {
  Found f;
  f.key = key;
  f.above = above;
  f.q = mass_of_key(key);  // > 0: the crossing bucket has mass
  f.j = (t - above + f.q - 1) / f.q;
  return f;
}

// Refine a first-digit crossing c1 over a gathered token list.
Q3_DEV Found search_list(const Cand* cand, int nc, Crossing c1, u64 t, u64* h2, u64* red, Crossing* cx) {
  clear(h2, kB2);
  __syncthreads();
  for (int i = threadIdx.x; i < nc; i += blockDim.x) {
    const Cand c = cand[i];
    if ((int)(c.key >> 18) == c1.digit) atomicAdd(&h2[(c.key >> 9) & 511u], mass_of_key(c.key));
  }
  __syncthreads();
  const Crossing c2 = find_crossing(h2, kB2, c1.above, t, red, cx);
  const uint32_t pre = ((uint32_t)c1.digit << 9) | (uint32_t)c2.digit;
  clear(h2, kB2);
  __syncthreads();
  for (int i = threadIdx.x; i < nc; i += blockDim.x) {
    const Cand c = cand[i];
    if ((c.key >> 9) == pre) atomicAdd(&h2[c.key & 511u], mass_of_key(c.key));
  }
  __syncthreads();
  const Crossing c3 = find_crossing(h2, kB2, c2.above, t, red, cx);
  return finish((pre << 9) | (uint32_t)c3.digit, c3.above, t);
}

// The same over the whole row.
Q3_DEV Found search_row(const Row& r, Crossing c1, u64 t, u64* h2, u64* red, Crossing* cx) {
  clear(h2, kB2);
  __syncthreads();
  {
    RunAdd ra;
    for_range(r, 0, r.V, [&](int, float l) {
      const uint32_t key = key_of(r, l);
      if ((int)(key >> 18) == c1.digit) ra.add(h2, (int)((key >> 9) & 511u), mass_of_key(key));
    });
    ra.flush(h2);
  }
  __syncthreads();
  const Crossing c2 = find_crossing(h2, kB2, c1.above, t, red, cx);
  const uint32_t pre = ((uint32_t)c1.digit << 9) | (uint32_t)c2.digit;
  clear(h2, kB2);
  __syncthreads();
  {
    RunAdd ra;
    for_range(r, 0, r.V, [&](int, float l) {
      const uint32_t key = key_of(r, l);
      if ((key >> 9) == pre) ra.add(h2, (int)(key & 511u), mass_of_key(key));
    });
    ra.flush(h2);
  }
  __syncthreads();
  const Crossing c3 = find_crossing(h2, kB2, c2.above, t, red, cx);
  return finish((pre << 9) | (uint32_t)c3.digit, c3.above, t);
}

struct Params {
  const float* logits;
  int64_t ld;
  int V, per_block, nb;  // row split: nb blocks of per_block tokens
  float k, top_p;        // k = log2(e) / T
  const float* uniform;
  int32_t* next;
  uint32_t* err;
  void* ws;
};

Q3_DEV Row make_row(const Params& P, int row) {
  const float* p = P.logits + (int64_t)row * P.ld;
  return Row{p, P.V, (reinterpret_cast<uintptr_t>(p) & 15) == 0, 0.f, P.k};
}

// What every per-row step reads first: the row maximum (from the per-block
// maxima; ok = false if one of them is NaN), the row's workspace record and
// its uniform number, fetched in one round trip and shared through LDS.
struct Head {
  float lmax, u;
  int ok;
  RowMeta meta;
};
Q3_DEV void load_head(const Params& P, const RowWs& w, int row, Head* h) {
  constexpr int kWords = sizeof(RowMeta) / 4;
  const int t = threadIdx.x;
  if (t < 64) {
    const float v = t < P.nb ? w.maxpart[t] : -INFINITY;
    const bool nan = __builtin_isnan(v);
    const float m = wave_max(nan ? -INFINITY : v);
    const bool any_nan = __ballot(nan) != 0;
    if (t == 0) {
      h->lmax = m;
      h->ok = !any_nan;
    }
  } else if (t < 64 + kWords) {
    reinterpret_cast<uint32_t*>(&h->meta)[t - 64] = reinterpret_cast<const uint32_t*>(w.meta)[t - 64];
  } else if (t == 64 + kWords) {
    h->u = fminf(fmaxf(P.uniform[row], 0.f), 0x1.fffffep-1f);
  }
  __syncthreads();
}

Q3_DEV u64 cut_target(const Params& P, u64 S) {
  const double tp = (double)P.top_p * (double)S;
  return tp <= 1.0 ? 1 : (tp >= (double)S ? S : (u64)ceil(tp));
}
Q3_DEV u64 draw_target(float u, u64 kept) {
  u64 m = (u64)floor((double)u * (double)kept);
  if (m >= kept) m = kept - 1;
  return m + 1;
}

// 1: per-block maxima; blocks also clear the row's histogram and counters.
__global__ __launch_bounds__(kPassThreads) void topp_max_kernel(Params P) {
  __shared__ float red[kPassThreads / 64];
  const int row = blockIdx.y, b = blockIdx.x;
  const RowWs w = row_ws(P.ws, row);
  const Row r = make_row(P, row);
  const int stripe = (kB1 + P.nb - 1) / P.nb;
  for (int i = b * stripe + threadIdx.x; i < min(kB1, (b + 1) * stripe); i += blockDim.x) w.h1[i] = 0;
  if (b == 0 && threadIdx.x == 0) {
    w.meta->S = 0;
    w.meta->n_cand = 0;
  }
  float mx = -INFINITY;
  bool finite = true;
  for_range(r, b * P.per_block, min(P.V, (b + 1) * P.per_block), [&](int, float l) {
    finite &= __builtin_isfinite(l);
    mx = fmaxf(mx, l);
  });
  mx = wave_max(mx);
  const bool all = __syncthreads_and(finite);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int k = 1; k < kPassThreads / 64; ++k) m = fmaxf(m, red[k]);
    w.maxpart[b] = all ? m : __builtin_nanf("");
  }
}

// 2: total mass and first-digit histogram.
__global__ __launch_bounds__(kPassThreads) void topp_hist_kernel(Params P) {
  __shared__ u64 h[kB1];
  __shared__ u64 red[kPassThreads / 64];
  __shared__ Head hd;
  const int row = blockIdx.y, b = blockIdx.x;
  const RowWs w = row_ws(P.ws, row);
  Row r = make_row(P, row);
  load_head(P, w, row, &hd);
  if (!hd.ok) return;
  r.lmax = hd.lmax;
  clear(h, kB1);
  __syncthreads();
  u64 part = 0;
  {
    RunAdd ra;
    for_range(r, b * P.per_block, min(P.V, (b + 1) * P.per_block), [&](int, float l) {
      const uint32_t key = key_of(r, l);
      const u64 q = mass_of_key(key);
      part += q;
      ra.add(h, (int)(key >> 18), q);
    });
    ra.flush(h);
  }
  const u64 S = block_sum(part, red);  // (its barriers also publish h)
  for (int i = threadIdx.x; i < kB1; i += blockDim.x)
    if (h[i]) atomicAdd(&w.h1[i], h[i]);
  if (threadIdx.x == 0) atomicAdd(&w.meta->S, S);
}

// 3: the first-digit buckets of the cut and of the draw's possible range
// (one prefix scan of the histogram serves the three crossings).
__global__ __launch_bounds__(kRowThreads) void topp_plan_kernel(Params P) {
  constexpr int per = kB1 / kRowThreads;
  __shared__ u64 red[kRowThreads / 64];
  __shared__ Crossing cx[3];
  __shared__ Head hd;
  const int row = blockIdx.x;
  const RowWs w = row_ws(P.ws, row);
  load_head(P, w, row, &hd);
  if (!hd.ok) return;
  const int b0 = (int)threadIdx.x * per;
  u64 h[per], mine = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    h[k] = w.h1[b0 + k];
    mine += h[k];
  }
  const u64 before = block_exclusive_scan(mine, red);
  // the thread whose buckets hold the running mass t writes its crossing
  auto locate = [&](u64 t, Crossing* out) {
    if (before < t && before + mine >= t) {
      u64 run = before;
#pragma unroll
      for (int k = 0; k < per; ++k) {
        if (run < t && run + h[k] >= t) *out = Crossing{b0 + k, run};
        run += h[k];
      }
    }
    __syncthreads();
    return *out;
  };
  const u64 S = hd.meta.S;
  const float u = hd.u;
  const Crossing c1 = locate(cut_target(P, S), &cx[0]);
  const Crossing dlo = locate(draw_target(u, cut_target(P, S)), &cx[1]);
#pragma unroll
  for (int k = 0; k < per; ++k)  // mass through c1 (static indices keep h in registers)
    if (b0 + k == c1.digit) cx[0].above += h[k];
  __syncthreads();
  const u64 kmax = cx[0].above;
  const Crossing dhi = locate(draw_target(u, kmax), &cx[2]);
  const bool few = dhi.digit - dlo.digit < kMaxW;
  if (threadIdx.x == 0) {
    w.meta->c1 = c1.digit;
    w.meta->dlo = dlo.digit;
    w.meta->dhi = dhi.digit;
    w.meta->few = few;
    w.meta->c1_above = c1.above;
    w.meta->dlo_above = dlo.above;
  }
  if (few && (int)threadIdx.x <= dhi.digit - dlo.digit) w.meta->hw[threadIdx.x] = w.h1[dlo.digit + threadIdx.x];
}

// 4: gather the tokens of the planned buckets.  Each thread counts its
// matches; a block scan gives every thread its slots, one atomic reserves the
// block's range in the row's list, and a second read of the slice (from
// cache, in the same order) places them.
__global__ __launch_bounds__(kPassThreads) void topp_gather_kernel(Params P) {
  __shared__ u64 red[kPassThreads / 64];
  __shared__ uint32_t base;
  __shared__ Head hd;
  const int row = blockIdx.y, b = blockIdx.x;
  const RowWs w = row_ws(P.ws, row);
  Row r = make_row(P, row);
  load_head(P, w, row, &hd);
  if (!hd.ok || !hd.meta.few) return;
  r.lmax = hd.lmax;
  const int c1 = hd.meta.c1, dlo = hd.meta.dlo, dhi = hd.meta.dhi;
  const int i0 = b * P.per_block, i1 = min(P.V, (b + 1) * P.per_block);
  auto hit_of = [&](uint32_t key) {
    const int d = (int)(key >> 18);
    return d == c1 || (d >= dlo && d <= dhi);
  };
  uint32_t mine = 0;
  for_range(r, i0, i1, [&](int, float l) { mine += hit_of(key_of(r, l)); });
  const uint32_t before = (uint32_t)block_exclusive_scan(mine, red);
  if (threadIdx.x == blockDim.x - 1) base = before + mine ? atomicAdd(&w.meta->n_cand, before + mine) : 0u;
  __syncthreads();
  if (!mine) return;
  uint32_t slot = base + before;
  for_range(r, i0, i1, [&](int i, float l) {
    const uint32_t key = key_of(r, l);
    if (hit_of(key)) {
      if (slot < (uint32_t)kCap) w.cand[slot] = Cand{key, (uint32_t)i};
      ++slot;
    }
  });
}

// 5: both searches and the index count; writes next[row].
__global__ __launch_bounds__(kRowThreads) void topp_pick_kernel(Params P) {
  constexpr int kLdsCand = kB1;  // list entries that fit in the histogram's space
  __shared__ union {
    u64 h1[kB1];
    Cand cand[kLdsCand];
  } lds;
  u64* h1 = lds.h1;
  __shared__ u64 h2[kB2];
  __shared__ uint32_t eq[kEqMax];
  __shared__ u64 red[kRowThreads / 64];
  __shared__ Crossing cx;
  __shared__ uint32_t n_eq, pick, n_sub;
  __shared__ Head hd;
  const int row = blockIdx.x;
  const RowWs w = row_ws(P.ws, row);
  Row r = make_row(P, row);
  load_head(P, w, row, &hd);
  if (!hd.ok) {
    if (threadIdx.x == 0) {
      atomicOr(P.err, Q3_ERRBIT_NONFINITE);
      P.next[row] = 0;
    }
    return;
  }
  r.lmax = hd.lmax;
  const RowMeta& meta = hd.meta;
  const bool few = meta.few;
  if (!few)  // the draw's first-digit bucket may be anywhere: the full histogram
    for (int i = threadIdx.x; i < kB1; i += blockDim.x) h1[i] = w.h1[i];
  if (threadIdx.x == 0) {
    n_eq = 0;
    pick = 0;
  }
  __syncthreads();
  const u64 S = meta.S;
  const float u = hd.u;
  const int nc = (int)meta.n_cand;
  const bool listed = few && nc <= kCap;
  // Each search works on the list's tokens of its first-digit bucket, moved
  // to LDS (the histogram's space is free when few) unless they are too many.
  auto bucket_list = [&](int digit, int* count) -> const Cand* {
    if (threadIdx.x == 0) n_sub = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nc; i += blockDim.x) {
      const Cand c = w.cand[i];
      if ((int)(c.key >> 18) == digit) {
        const uint32_t slot = atomicAdd(&n_sub, 1u);
        if (slot < (uint32_t)kLdsCand) lds.cand[slot] = c;
      }
    }
    __syncthreads();
    const int m = (int)n_sub;
    __syncthreads();
    if (m <= kLdsCand) {
      *count = m;
      return lds.cand;
    }
    *count = nc;
    return w.cand;
  };

  const u64 t1 = cut_target(P, S);
  const Crossing c1{meta.c1, meta.c1_above};
  Found cut;
  if (listed) {
    int n1;
    const Cand* l1 = bucket_list(c1.digit, &n1);
    cut = search_list(l1, n1, c1, t1, h2, red, &cx);
  } else {
    cut = search_row(r, c1, t1, h2, red, &cx);
  }
  const u64 t2 = draw_target(u, cut.above + cut.j * cut.q);
  Crossing c1d;
  if (few) {  // within the planned buckets dlo .. dhi
    c1d = Crossing{meta.dlo, meta.dlo_above};
    for (int k = 0; k < meta.dhi - meta.dlo; ++k) {
      if (c1d.above + meta.hw[k] >= t2) break;
      c1d.above += meta.hw[k];
      c1d.digit += 1;
    }
  } else {
    c1d = find_crossing(h1, kB1, 0, t2, red, &cx);
  }
  Found d;
  const Cand* list = nullptr;
  int nl = 0;
  if (listed) {
    list = bucket_list(c1d.digit, &nl);
    d = search_list(list, nl, c1d, t2, h2, red, &cx);
  } else {
    d = search_row(r, c1d, t2, h2, red, &cx);
  }

  // The d.j-th token, in token order, among those whose key is d.key: ranked
  // in LDS when the list holds them and they are few, else by an ordered pass.
  if (listed) {
    for (int i = threadIdx.x; i < nl; i += blockDim.x)
      if (list[i].key == d.key) {
        const uint32_t slot = atomicAdd(&n_eq, 1u);
        if (slot < (uint32_t)kEqMax) eq[slot] = list[i].idx;
      }
  }
  __syncthreads();
  const u64 c_eq = n_eq;
  if (listed && c_eq <= (u64)kEqMax) {
    if (threadIdx.x < c_eq) {
      const uint32_t mine = eq[threadIdx.x];
      uint32_t rank = 0;
      for (int k = 0; k < (int)c_eq; ++k) rank += eq[k] < mine;
      if (rank + 1 == d.j) pick = mine;
    }
  } else {
    // ordered pass: thread t scans indices [t * chunk, (t + 1) * chunk)
    const int chunk = (r.V + kRowThreads - 1) / kRowThreads;
    const int i0 = min(r.V, (int)threadIdx.x * chunk), i1 = min(r.V, i0 + chunk);
    uint32_t cnt = 0;
    for (int i = i0; i < i1; ++i) cnt += key_of(r, r.p[i]) == d.key;
    const u64 before = block_exclusive_scan(cnt, red);
    if (before < d.j && d.j <= before + cnt) {
      u64 seen = before;
      for (int i = i0; i < i1; ++i)
        if (key_of(r, r.p[i]) == d.key && ++seen == d.j) {
          pick = (uint32_t)i;
          break;
        }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) P.next[row] = (int32_t)pick;
}

}  // namespace

size_t sample_workspace_bytes(int n_rows) { return (size_t)std::min(std::max(n_rows, 1), kRows) * kRowBytes; }

hipError_t sample_top_p(const float* logits, int64_t ld, int n, int V, float temperature, float top_p,
                        const float* uniform, int32_t* next, uint32_t* err, void* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (temperature == 0.f) {  // greedy, Q3_MAX_BATCH rows per launch
    for (int r0 = 0; r0 < n; r0 += Q3_MAX_BATCH) {
      RowMap rows;
      rows.n = min(Q3_MAX_BATCH, n - r0);
      for (int i = 0; i < rows.n; ++i) rows.row[i] = r0 + i;
      const hipError_t e = argmax_rows(logits, ld, rows, V, next + r0, err, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // Row split for the passes over the logits: about 512 blocks over the
  // batch's rows (at most 64 per row), each a multiple of 4 tokens (aligned
  // float4 runs); fewer blocks per row amortise the per-block histogram.
  const int rows_max = std::min(kRows, n);
  const int want = std::max(1, std::min(kMaxNB, (512 + rows_max - 1) / rows_max));
  const int per = std::max(4, ((V + want - 1) / want + 3) / 4 * 4);
  const int nb = (V + per - 1) / per;
  for (int r0 = 0; r0 < n; r0 += kRows) {
    const int rows = std::min(kRows, n - r0);
    Params P{logits + (int64_t)r0 * ld, ld, V, per, nb, kLog2e / temperature, top_p, uniform + r0,
             next + r0, err, ws};
    topp_max_kernel<<<dim3(nb, rows), kPassThreads, 0, s>>>(P);
    topp_hist_kernel<<<dim3(nb, rows), kPassThreads, 0, s>>>(P);
    topp_plan_kernel<<<rows, kRowThreads, 0, s>>>(P);
    topp_gather_kernel<<<dim3(nb, rows), kPassThreads, 0, s>>>(P);
    topp_pick_kernel<<<rows, kRowThreads, 0, s>>>(P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace q3k
