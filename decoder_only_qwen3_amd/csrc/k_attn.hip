// Causal grouped-query attention over the KV cache.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" -- Paso 5: scores q.k / sqrt(128); a query sees only keys at or
// before its own position (the page masks the upper triangle; excluding those
// keys is the same softmax); softmax over the visible keys weights the values;
// query head h reads key/value head h / (n_q / n_kv).
//
// Cache layout (per slot and layer, bf16): keys in blocks of 32, each block
// stored in the order its keys are taken as MFMA operands (kk_off), values
// [kv_head][cap/32][128][32] (transposed within 32-key blocks).  With that
// layout both MFMA products read 16-byte runs, every operand load of a
// wavefront is 1 KiB of consecutive bytes, and a 32-key run of keys or of
// values is one contiguous 8 KiB stretch (strided value rows read about 30 %
// slower on MI355X):
//   S^T[key][row] = K[key][:] . Q[row][:]   A = K rows,    B = Q rows
//   O^T[dim][row] = V^T[dim][keys] . P^T     A = V^T rows,  B = P from registers
// The key order inside each 32-key chunk is permuted for the S^T product so
// that lane group q (= lane/16) ends up holding the scores of keys 8q..8q+7,
// which is exactly the eight-key run it must supply as the B operand of the
// P.V product.  No shuffles or LDS round trips are needed for P.
//
// Precision: S = Q.K^T takes the bf16 queries and keys as they are.  The P.V
// product runs on fp16 MFMA operands: the bf16 values convert to fp16 exactly,
// and each softmax weight enters as two fp16 terms (fp16(p) and the fp16 of
// the remainder), about 22 significant bits.  A single fp16 weight (11 bits)
// moved the attention output by ~2^-12 of its size, enough to flip many of
// its bf16 roundings; downstream of those flips the logits of a two-layer
// random-init model moved by up to 3e-2 of their RMS.
#include <algorithm>
#include <cstring>
#include <vector>

#include "kernels.h"

namespace q3k {

namespace {
constexpr float kLog2e = 1.4426950408889634f;

Q3_DEV float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight softmax weights as two fp16 MFMA operands, hi = fp16(p) and
// lo = fp16(p - hi): hi + lo carries about 22 significant bits, so the P.V
// product keeps near-fp32 weights while running on fp16 MFMA.  The weights
// (unrounded) are added to `sum`.
struct PSplit {
  f16x8 hi, lo;
};
// p - (float)half (the half being the low or high fp16 of `h`), in one
// mixed-precision FMA: -half * 1 + p.
Q3_DEV float minus_half_lo(uint32_t h, float p) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(p));
  return r;
}
Q3_DEV float minus_half_hi(uint32_t h, float p) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(p));
  return r;
}
Q3_DEV PSplit split_p(const f32x4& a, const f32x4& b, float& sum) {
  const float p[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_f16x2(p[2 * i], p[2 * i + 1]);
    const uint32_t hi = h[i];
    l[i] = pack_f16x2(minus_half_lo(hi, p[2 * i]), minus_half_hi(hi, p[2 * i + 1]));
    sum += p[2 * i] + p[2 * i + 1];
  }
  return PSplit{as_f16x8(h), as_f16x8(l)};
}

// Zero the bf16 elements of an 8-key run whose key index is >= limit.
Q3_DEV u32x4 mask_keys(u32x4 v, int key0, int limit) {
  if (key0 + 8 <= limit) return v;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t x = v[w];
    if (key0 + 2 * w >= limit) x &= 0xffff0000u;
    if (key0 + 2 * w + 1 >= limit) x &= 0x0000ffffu;
    v[w] = x;
  }
  return v;
}

// ---------------------------------------------------------------- prefill
constexpr int KT = 64;          // keys per tile
constexpr float kLazyLog2 = 8.f;  // headroom of the stale reference maximum (log2 units)
// LDS tiles are stored unpadded.  A key tile is the cache's two 32-key
// blocks copied as they are (the MFMA operand order of kk_off), so a key
// fragment read is 1 KiB of consecutive LDS per wavefront.  Value^T tiles
// have the 16-byte chunk index of each row XOR-swizzled by the row (8 chunks
// per row), so the fragment reads (16 rows, one chunk) do not collide in LDS
// banks (checked with the bank-conflict counter on gfx950: zero conflict
// cycles).
Q3_DEV int vswz(int dim) { return dim & 7; }
Q3_DEV int voff(int dim, int key) { return dim * KT + ((((key >> 3) ^ vswz(dim)) << 3) | (key & 7)); }

struct TileTable {
  int32_t tile_cu[Q3_MAX_BATCH + 1];  // prefix sums of query tiles per sequence
  int32_t item_cu[Q3_MAX_BATCH + 1];  // prefix sums of work items (groups of TPB tiles) per sequence and head
  int32_t vstart[Q3_MAX_BATCH];       // vstage_start of each sequence
  int32_t xbnd[9];                    // work items of XCD x: xbnd[x] .. xbnd[x+1] - 1
};

// Block: one kv head and one query tile of `qt` tokens of one sequence; its
// 64*CB query rows are the group's query heads x qt tokens (row r -> head
// r / qt, token r % qt).  Token i of the sequence's call sits at position
// prior + i and sees keys 0 .. prior + i (the prior ones already cached).  4 wavefronts x 16*CB rows.  K tiles (bf16) and V^T
// tiles (fp16 staging) of 64 keys are double-buffered in LDS, filled by
// direct global-to-LDS loads (each lane fetches the global chunk that belongs
// at its fixed LDS position under the swizzle) and shared by the 4 wavefronts.
//
// The loop is rotated so each iteration holds independent MFMA and VALU work:
// iteration j runs P(j-1).V(j-1) while taking the row maxima of S(j), then
// S(j+1) = K(j+1).Q^T while exponentiating S(j).  LDS: K(t) in sK[t & 1],
// V(t) in sV[t & 1]; iteration j reads V(j-1) and K(j+1) and loads V(j) and
// K(j+2) over the buffers of V(j-2) and K(j), used up in iteration j-1.
//
// TPB = 2: a block of 8 wavefronts takes two consecutive query tiles of one
// (sequence, head) -- wavefronts 0-3 the later tile, 4-7 the one before it --
// and both halves share every K/V tile it loads; the loop runs over the later
// tile's keys (the earlier tile's rows mask the extra ones).  Half the
// blocks, each with twice the work, halve the per-block start and finish.
template <int CB, int TPB>
__global__ __launch_bounds__(256 * TPB, 2 / TPB) void flash_prefill_kernel(
    const bf16_t* __restrict__ q, SeqBatch sb, TileTable tt, const SeqState* __restrict__ st,
    const bf16_t* __restrict__ kv, const uint16_t* __restrict__ vstage, int64_t vh_keys, int layer, int n_q,
    int n_kv, int qt, bf16_t* __restrict__ o, float scale_log2) {
  // One LDS array for both double buffers: [0], [1] = K tiles (bf16), [2],
  // [3] = V^T tiles (fp16 bits).  With the key and value tiles in two arrays,
  // the compiler could not tell which one a direct-to-LDS load writes and put
  // a wait for every outstanding load (vmcnt(0)) before each LDS read -- right
  // after the next tiles' loads were issued, which drained the pipeline; with
  // one array it leaves the waits to the loop (wait_vm + barrier at the top
  // of each iteration), checked in the compiled code.
  __shared__ __attribute__((aligned(16))) uint16_t sKV[4][KT * 128];
  uint16_t (*sK)[KT * 128] = sKV;
  uint16_t (*sV)[KT * 128] = sKV + 2;

  // Work item = (sequence b, kv head g, query tile), ordered by b, then g,
  // then tile from the last (longest) down.  Blocks are dealt to the eight
  // XCDs round robin (block i runs on XCD i % 8), each with an L2 of its own;
  // XCD x takes the contiguous run of items xbnd[x] .. xbnd[x+1]-1 (balanced
  // by key tiles on the host), so the query tiles of one (sequence, head)
  // read its keys and values through one L2 instead of all eight.
  constexpr int NWV = 4 * TPB;   // wavefronts per block
  constexpr int LPW = 4 / TPB;   // 1 KiB loads per wavefront per K or V tile
  const int xcd = blockIdx.x & 7;
  const int item = tt.xbnd[xcd] + (int)(blockIdx.x >> 3);
  if (item >= tt.xbnd[xcd + 1]) return;  // the grid covers the longest run
  int b = 0;
  {
    int lo = 0, hi = sb.n - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (tt.item_cu[mid] * n_kv <= item) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  const int ntb = tt.tile_cu[b + 1] - tt.tile_cu[b];
  const int nib = tt.item_cu[b + 1] - tt.item_cu[b];  // items per head: ceil(ntb / TPB)
  const int rr = item - tt.item_cu[b] * n_kv;
  const int g = rr / nib;
  const int k = rr - g * nib;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wq = wid & 3, tsel = wid >> 2;  // wavefront within its tile, tile of the item
  const int tlocA = ntb - 1 - TPB * k;      // the item's last (longest) tile
  const int tloc = tlocA - tsel;            // this wavefront's tile (< 0: none, it only helps load)
  const int L = sb.cu[b + 1] - sb.cu[b], P = sb.prior[b];
  const int q0 = tloc * qt;
  const SeqState s = st[sb.slot[b]];
  const KvGeom geo{n_kv, layer};
  const bf16_t* Kc = kv_k(kv, s, geo, g);
  const uint16_t* Vh = vstage + ((int64_t)g * vh_keys + tt.vstart[b]) * Q3_HEAD_DIM;  // fp16, zero-padded
  const int group = n_q / n_kv;
  const int fr = lane & 15, fq = lane >> 4;

  // V(-1) is all zeros (the first iteration's P.V adds nothing).
  for (int i = tid; i < 128 * KT / 8; i += 64 * NWV) reinterpret_cast<u32x4*>(sV[1])[i] = u32x4{0u, 0u, 0u, 0u};

  // Query fragments (B operand of S^T) for this wavefront's 16-row blocks.
  bf16x8 qf[CB][4];
  int qpos[CB], qhead[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int r = wq * 16 * CB + cb * 16 + fr;
    const int hh = r / qt, tq = r - hh * qt;
    qpos[cb] = tloc >= 0 ? q0 + tq : L;  // no tile: rows past the end (never stored)
    qhead[cb] = g * group + hh;
    const bool ok = qpos[cb] < L;
    const bf16_t* qp = q + ((int64_t)(sb.cu[b] + (ok ? qpos[cb] : 0)) * n_q + qhead[cb]) * 128 + fq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = ld16(qp + ks * 32);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      qf[cb][ks] = as_bf16x8(v);
    }
  }

  const int kend = P + min(L, tlocA * qt + qt);  // keys of the item's last row, + 1
  const int ntiles = (kend + KT - 1) / KT;

  // Load i of wavefront w fills LDS chunks (NWV*i + w)*64 + lane of a tile:
  // the K chunk p is chunk p of the tile's two cache blocks; the V^T chunk
  // (dim, j) holds keys 8 (j ^ vswz(dim)) .. +7 of that dim.
  int ksrc[LPW], vsrc[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int p = (NWV * i + wid) * 64 + lane;
    const int dim = p >> 3;
    ksrc[i] = p * 8;
    vsrc[i] = (int)vt_off(((p & 7) ^ vswz(dim)) << 3, dim);
  }
  auto issue_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPW; ++i)  // (non-const pointers: with a const source the host pass drops the kernel stub)
      __builtin_amdgcn_global_load_lds((void*)(Kc + (int64_t)t * KT * 128 + ksrc[i]),
                                       (void*)(&sK[t & 1][(NWV * i + wid) * 512]), 16, 0, 0);
  };
  auto issue_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPW; ++i)  // a 64-key tile is two 32-key value blocks: 64 * 128 elements
      __builtin_amdgcn_global_load_lds((void*)(Vh + (int64_t)t * KT * 128 + vsrc[i]),
                                       (void*)(&sV[t & 1][(NWV * i + wid) * 512]), 16, 0, 0);
  };

  // S^T of tile t: sacc[c][sb][cb], keys t*64 + c*32 + 8*fq + 4*sb + r.
  auto scores = [&](int t, f32x4 (&sacc)[2][2][CB]) {
    const bf16_t* kb = sK[t & 1];  // bf16 bits
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) sacc[c][sbk][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 kf[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int sbk = 0; sbk < 2; ++sbk)  // keys c*32 + 8*(fr/4) + 4*sbk + fr%4, dims ks*32 + fq*8 ..
          kf[c][sbk] = *reinterpret_cast<const bf16x8*>(&kb[((c * 8 + sbk * 4 + ks) * 64 + lane) * 8]);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) sacc[c][sbk][cb] = mfma16(kf[c][sbk], qf[cb][ks], sacc[c][sbk][cb]);
    }
  };

  f32x4 oacc[8][CB];
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[d][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // O^T += V^T(t) . P^T (fp16 operands) over the keys of half c of the tile,
  // four dim blocks at a time: hi products then lo, so no MFMA waits on the
  // one before it.
  auto accumulate = [&](int t, const PSplit (&pf)[2][CB], int c) {
    const uint16_t* vb = sV[t & 1];
#pragma unroll
    for (int dh = 0; dh < 8; dh += 4) {
      f16x8 vf[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        vf[d] = *reinterpret_cast<const f16x8*>(&vb[voff((dh + d) * 16 + fr, c * 32 + fq * 8)]);
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[dh + d][cb] = mfma16_f16(vf[d], pf[c][cb].hi, oacc[dh + d][cb]);
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[dh + d][cb] = mfma16_f16(vf[d], pf[c][cb].lo, oacc[dh + d][cb]);
    }
  };

  float mref[CB], lrun[CB];  // reference maximum (scaled, log2 units) and weight sum per row
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    mref[cb] = -INFINITY;
    lrun[cb] = 0.f;
  }
  PSplit pf[2][CB];  // weights of the previous tile (zero before the first)
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      pf[c][cb].hi = as_f16x8(u32x4{0u, 0u, 0u, 0u});
      pf[c][cb].lo = pf[c][cb].hi;
    }

  // Prologue: K(0) then K(1); S(0) once K(0) has landed (K(1) may still fly).
  issue_k(0);
  if (ntiles > 1) {
    issue_k(1);
    wait_vm<LPW>();
  } else {
    wait_vm<0>();
  }
  __syncthreads();  // also orders the zeroing of sV[1]
  // Iteration j: sacc holds S(j) on entry; S(j+1) goes to snext.
  auto step = [&](int j, f32x4 (&sacc)[2][2][CB], f32x4 (&snext)[2][2][CB]) {
    // K(j+1) and V(j-1) (loaded during the previous iteration) have landed.
    wait_vm<0>();
    bare_barrier();
    issue_v(j);
    if (j + 2 < ntiles) issue_k(j + 2);

    if (j * KT + KT - 1 > P + q0 || j * KT + KT > P + L) {
      // keys after a row's position (the diagonal tile) or past the sequence end
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = j * KT + c * 32 + 8 * fq + 4 * sbk + r;
              if (key > P + qpos[cb] || key >= P + L) sacc[c][sbk][cb][r] = -INFINITY;
            }
    }
    // P(j-1).V(j-1) (buffer (j - 1) & 1), the row maxima of S(j) beside it.
    // Raised wave priority for this MFMA-heavy stretch: when the SIMD's other
    // wavefront is in its VALU-heavy softmax, both pipes stay fed (10 % faster
    // at 32K keys on MI355X than equal priorities).
    __builtin_amdgcn_s_setprio(1);
    accumulate(j + 1, pf, 0);
    accumulate(j + 1, pf, 1);
    __builtin_amdgcn_s_setprio(0);
    // Row maxima of the raw scores (the scale is positive, so it commutes with max).
    float mx[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      mx[cb] = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx[cb] = fmaxf(mx[cb], sacc[c][sbk][cb][r]);
      mx[cb] = fmaxf(mx[cb], __shfl_xor(mx[cb], 16, 64));
      mx[cb] = fmaxf(mx[cb], __shfl_xor(mx[cb], 32, 64));
      mx[cb] *= scale_log2;
    }
    // The reference maximum of a row moves only when the tile's maximum passes
    // it by more than kLazyLog2 (then for every row of the wavefront, a uniform
    // branch): weights stay <= 2^kLazyLog2, well inside fp16, and most tiles of
    // a long row skip the rescale of its accumulators.
    bool grow = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) grow |= mx[cb] > mref[cb] + kLazyLog2;
    if (__ballot(grow)) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float mnew = fmaxf(mref[cb], mx[cb]);
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2_f(mref[cb] - mnew);
        mref[cb] = mnew;
        lrun[cb] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[d][cb] *= alpha;
      }
    }

    // S(j+1) on the MFMA pipe while the VALU turns S(j) into split weights.
    // (Past the last tile the product reads a stale buffer and is discarded.)
    scores(j + 1, snext);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float mu = (mref[cb] == -INFINITY) ? 0.f : mref[cb];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[c][sbk][cb][r] = exp2_f(fmaf(sacc[c][sbk][cb][r], scale_log2, -mu));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) pf[c][cb] = split_p(sacc[c][0][cb], sacc[c][1][cb], lrun[cb]);
  };
  // Unrolled by two so the score buffers swap roles instead of being copied.
  f32x4 sA[2][2][CB], sB[2][2][CB];
  scores(0, sA);
  for (int j = 0;;) {
    step(j, sA, sB);
    if (++j >= ntiles) break;
    step(j, sB, sA);
    if (++j >= ntiles) break;
  }

  // The last tile's P.V.
  wait_vm<0>();
  bare_barrier();
  accumulate(ntiles - 1, pf, 0);
  accumulate(ntiles - 1, pf, 1);

  // Normalise and store: lane holds dims d*16 + fq*4 + r of row (cb, fr).
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    float l = lrun[cb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (qpos[cb] >= L) continue;
    const float inv = 1.f / l;
    bf16_t* op = o + ((int64_t)(sb.cu[b] + qpos[cb]) * n_q + qhead[cb]) * 128 + fq * 4;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      u32x2 w;
      w[0] = pack_bf2(oacc[d][cb][0] * inv, oacc[d][cb][1] * inv);
      w[1] = pack_bf2(oacc[d][cb][2] * inv, oacc[d][cb][3] * inv);
      *reinterpret_cast<u32x2*>(op + d * 16) = w;
    }
  }
}

// ---------------------------------------------------------------- decode
// Block (split j, kv head g, sequence b), one wavefront: the keys of split j
// against the group's query heads (MFMA columns 0..group-1; other columns
// zero).  Writes (max, sum, unnormalised output) partials; the combine kernel
// merges splits in index order.  The number of splits is fixed per launch and
// the split length follows the sequence's current length on the device, so a
// captured graph stays valid as the cache grows.
constexpr int PSTRIDE = 128 + 2;

// Split length used for a context of `ctx` keys over `splits` splits.
Q3_DEV int split_chunk_len(int ctx, int splits) {
  const int chunk = (ctx + splits - 1) / splits;
  return (chunk + 31) & ~31;
}

__global__ __launch_bounds__(64) void decode_attn_kernel(const bf16_t* __restrict__ q, SeqBatch sb,
                                                         const SeqState* __restrict__ st,
                                                         const bf16_t* __restrict__ kv, int layer,
                                                         int n_q, int n_kv, int splits,
                                                         float* __restrict__ part, float scale_log2) {
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, fr = lane & 15, fq = lane >> 4;
  const SeqState s = st[sb.slot[b]];
  const int ctx = s.len + 1;
  const int chunk = split_chunk_len(ctx, splits);
  const int k_begin = j * chunk;
  const int k_end = min(ctx, k_begin + chunk);
  const int group = n_q / n_kv;
  if (k_begin >= k_end) {
    if (fq == 0 && fr < group) {
      float* pp = part + (((int64_t)b * n_q + g * group + fr) * splits + j) * PSTRIDE;
      pp[0] = -INFINITY;
      pp[1] = 0.f;
    }
    return;
  }
  const KvGeom geo{n_kv, layer};
  const bf16_t* Kc = kv_k(kv, s, geo, g);
  const bf16_t* Vt = kv_vt(kv, s, geo, g);

  bf16x8 qf[4];
  {
    const bool ok = fr < group;
    const bf16_t* qp = q + ((int64_t)b * n_q + g * group + (ok ? fr : 0)) * 128 + fq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 v = ld16(qp + ks * 32);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = as_bf16x8(v);
    }
  }
  f32x4 oacc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  for (int c0 = k_begin; c0 < k_end; c0 += 32) {
    f32x4 sacc[2];
#pragma unroll
    for (int sbk = 0; sbk < 2; ++sbk) {
      // keys c0 + 8*(fr/4) + 4*sbk + fr%4 of the 32-key block (the ones at or
      // past k_end are read but masked below)
      sacc[sbk] = f32x4{0.f, 0.f, 0.f, 0.f};
      const bf16_t* kp = Kc + (int64_t)(c0 >> 5) * 4096 + lane * 8;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc[sbk] = mfma16(as_bf16x8(ld16_nt(kp + (sbk * 4 + ks) * 512)), qf[ks], sacc[sbk]);
    }
    u32x4 vraw[8];
    const int vkey0 = c0 + fq * 8;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      vraw[d] = mask_keys(ld16_nt(Vt + vt_off(vkey0, d * 16 + fr)), vkey0, k_end);

    float mx = -INFINITY;
#pragma unroll
    for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = c0 + 8 * fq + 4 * sbk + r;
        float v = sacc[sbk][r] * scale_log2;
        if (key >= k_end) v = -INFINITY;
        sacc[sbk][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrun, mx);
    const float alpha = exp2_f(mrun - mnew);
    mrun = mnew;
#pragma unroll
    for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[sbk][r] = exp2_f(sacc[sbk][r] - mnew);
    float ls = 0.f;
    const PSplit pf = split_p(sacc[0], sacc[1], ls);
    lrun = lrun * alpha + ls;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const f16x8 vf = as_f16x8(bf16x8_to_f16x8(vraw[d]));
      oacc[d] = mfma16_f16(vf, pf.lo, mfma16_f16(vf, pf.hi, oacc[d] * alpha));
    }
  }
  lrun += __shfl_xor(lrun, 16, 64);
  lrun += __shfl_xor(lrun, 32, 64);
  if (fr < group) {
    float* pp = part + (((int64_t)b * n_q + g * group + fr) * splits + j) * PSTRIDE;
    if (fq == 0) {
      pp[0] = mrun;
      pp[1] = lrun;
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) pp[2 + d * 16 + fq * 4 + r] = oacc[d][r];
  }
}

// One block of 128 threads per (sequence, query head): merge the non-empty
// splits in index order (max-shifted weights 2^(m_j - M)), normalise, store.
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ part, SeqBatch sb,
                                                             const SeqState* __restrict__ st, int n_q,
                                                             int splits, bf16_t* __restrict__ o) {
  __shared__ float wgt[1024];
  __shared__ float red[2];
  const int bh = blockIdx.x, d = threadIdx.x;
  const int b = bh / n_q;
  const int ctx = st[sb.slot[b]].len + 1;
  const int chunk = split_chunk_len(ctx, splits);
  const int nact = min(min(splits, (ctx + chunk - 1) / chunk), 1024);
  const float* p = part + (int64_t)bh * splits * PSTRIDE;
  // Split maxima loaded in parallel, then the global max and the weights.
  float mx = -INFINITY;
  for (int j = d; j < nact; j += 128) {
    const float m = p[(int64_t)j * PSTRIDE];
    wgt[j] = m;
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if ((d & 63) == 0) red[d >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  for (int j = d; j < nact; j += 128) wgt[j] = exp2_f(wgt[j] - M);
  __syncthreads();
  float L = 0.f, acc = 0.f;
  for (int j = 0; j < nact; ++j) {
    const float w = wgt[j];
    L += p[(int64_t)j * PSTRIDE + 1] * w;
    acc += p[(int64_t)j * PSTRIDE + 2 + d] * w;
  }
  o[(int64_t)bh * 128 + d] = f2bf(acc / L);
}

// ---------------------------------------------------------------- fused decode
// Decode attention with the QK-Norm + RoPE + cache append of Pasos 4-5 folded
// in.  Block (split j, kv head g, sequence b), FW wavefronts:
//   0. read the sequence's length; every wavefront issues the loads of its
//      first two 32-key runs of cached keys and values at once, so the cache
//      stream starts before any of the steps below;
//   A. normalise and rotate the group's query heads from the fused projection
//      row (into LDS, bf16).  The block whose key range holds the new
//      position also normalises/rotates the new key, stores it and the new
//      value into the cache for later steps, and keeps both in LDS: this
//      step takes the new key from LDS, never from the cache, so nothing
//      waits on those stores;
//   B. attend over the wavefront's cached keys (MFMA; two register buffers,
//      each refilled with the run two ahead as soon as its keys, then its
//      values, are used), then the wavefront that holds the new position
//      adds the new key as one more online-softmax term;
//   C. merge the block's wavefronts in order.  One split: write the output.
//      Several splits: publish a (max, sum, output) partial with agent-scope
//      stores, count the finished splits of this (b, g) on an agent-scope
//      counter, and let the last block merge the partials in split order
//      (deterministic) and re-arm the counter.
// Agent-scope atomic loads/stores keep the partials coherent across the
// GPU's L2 slices without device-wide fences (which on gfx950 write back and
// invalidate whole L2 caches).  The launch fixes `smax`; the number of
// splits used and the keys per split follow the sequence's current length
// on the device, so a captured graph stays valid as the cache grows.
struct RopeArgs {
  const float* qn;
  const float* kn;
  const float* cos_t;
  const float* sin_t;
  float eps;
};

struct FusedGeom {
  int nact;   // non-empty splits
  int cb;     // keys per split (multiple of 32)
};

template <int FW>
Q3_DEV FusedGeom fused_geom(int ctx, int smax) {
  constexpr int unit = 32 * FW;  // whole 32-key runs for each of the FW wavefronts
  int cb = (ctx + smax - 1) / smax;
  cb = max(unit, (cb + unit - 1) / unit * unit);
  return FusedGeom{(ctx + cb - 1) / cb, cb};
}

Q3_DEV float ld_agent(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
Q3_DEV void st_agent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Per-head RMSNorm + rotate-half RoPE of one 128-wide head held as lanes
// (l, l+64); the rotated pair replaces (a, c).
Q3_DEV void norm_rope_pair(float& a, float& c, const float* w, float eps, float cs, float sn) {
  const float ss = wave_sum(a * a + c * c);
  const float inv = rsqrtf(ss * (1.f / 128.f) + eps);
  const int lane = threadIdx.x & 63;
  a = a * inv * w[lane];
  c = c * inv * w[lane + 64];
  const float ra = a * cs - c * sn, rc = a * sn + c * cs;
  a = ra;
  c = rc;
}


// One 32-key run of the cache in registers, in the MFMA operand layouts:
// k[sbk][ks] = K[key(sbk)][ks*32 + fq*8 ..], key(sbk) = c0 + 8*(fr/4) + 4*sbk + fr%4;
// v[d] = V^T[d*16 + fr][c0 + fq*8 ..].  Keys at or beyond the caller's end
// are read too (the caller masks their scores and zeroes their values).  c0
// is a multiple of 32.
struct KvRun {
  u32x4 k[2][4];
  u32x4 v[8];
};

// A head's key or value blocks (8 KiB per 32 keys) as a buffer resource
// whose range ends with the last block a wavefront attends: a run past it
// loads zeros and moves no bytes, so runs can be requested ahead without a
// bounds test (which would make the loads conditional).  gfx9 raw buffer:
// stride 0, the range in bytes, untyped 32-bit data.  Loads are
// nontemporal (the cache is read once per layer).
Q3_DEV __amdgpu_buffer_rsrc_t kv_rsrc(const bf16_t* base, int nblocks) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane(nblocks * 8192), 0x00020000);
}
Q3_DEV u32x4 ld16_rs(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 2));
}
// Byte offsets within a head's blocks of the run at key c0 (a multiple of
// 32): key chunk (sbk * 4 + ks) * 64 + lane at kro + (sbk * 4 + ks) * 1024
// (kk_off); value dim d * 16 + fr of keys c0 + fq * 8 .. +7 at
// vro + d * 1024 (vt_off).
Q3_DEV int run_koff(int c0, int lane) { return (c0 >> 5) * 8192 + lane * 16; }
Q3_DEV int run_voff(int c0, int lane) { return ((c0 >> 5) * 128 + (lane & 15)) * 64 + (lane >> 4) * 16; }

// Loads of one half of a run at the given byte offset.  Every address is
// formed before the first load is issued: when the address arithmetic sat
// between the loads, the register allocator reused the destination registers
// of loads still in flight for it, which forced waits for those loads (and
// for the previous run's) in the middle of the issue.
Q3_DEV void load_k(KvRun& r, __amdgpu_buffer_rsrc_t krs, int ko) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) r.k[sbk][ks] = ld16_rs(krs, ko + (sbk * 4 + ks) * 1024);
  __builtin_amdgcn_sched_barrier(0);
}
Q3_DEV void load_v(KvRun& r, __amdgpu_buffer_rsrc_t vrs, int vo) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < 8; ++d) r.v[d] = ld16_rs(vrs, vo + d * 1024);
  __builtin_amdgcn_sched_barrier(0);
}

// Sequence of each z-index of the grid: blocks are dispatched in z order.
struct SeqOrder {
  uint8_t v[Q3_MAX_BATCH];
};

template <int FW>
__global__ __launch_bounds__(64 * FW, 8 / FW) void decode_attn_fused_kernel(
    const float* __restrict__ qkv, SeqBatch sb, const SeqState* __restrict__ st, bf16_t* __restrict__ kv,
    int layer, int n_q, int n_kv, RopeArgs ra, int smax, float* __restrict__ part, uint32_t* __restrict__ cnt,
    bf16_t* __restrict__ o, float scale_log2, SeqOrder ord) {
  __shared__ __attribute__((aligned(16))) uint16_t qs[8 * 128];
  __shared__ __attribute__((aligned(16))) uint16_t knew[128], vnew[128];
  __shared__ float wred[FW][8][PSTRIDE];
  __shared__ int last;
  const int j = blockIdx.x, g = blockIdx.y, b = ord.v[blockIdx.z];
  const int tid = threadIdx.x, lane = tid & 63, fr = lane & 15, fq = lane >> 4;
  // the wavefront index is uniform: held in a scalar register, the key-run
  // loop below is scalar control flow (no lane masks around its loads)
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = n_q / n_kv;
  const SeqState s = st[sb.slot[b]];
  const int pos = s.len, ctx = pos + 1;
  const FusedGeom fg = fused_geom<FW>(ctx, smax);
  if (j >= fg.nact) return;
  const int k_begin = j * fg.cb, k_end = min(ctx, k_begin + fg.cb);
  const KvGeom geo{n_kv, layer};
  bf16_t* Kc = kv_k(kv, s, geo, g);
  bf16_t* Vt = kv_vt(kv, s, geo, g);

  // 0: this wavefront's keys are [w0, w1); those before `pos` come from the
  // cache ([w0, cend)), the key at `pos` (if in range) from LDS.
  const int cw = fg.cb / FW;
  const int w0 = k_begin + wid * cw, w1 = min(k_end, w0 + cw);
  const int cend = min(w1, pos);
  const bool has_new = pos >= w0 && pos < w1;
  KvRun run[2];
  // the blocks up to this wavefront's last cached key
  const int nblk = (cend + 31) >> 5;
  const __amdgpu_buffer_rsrc_t krs = kv_rsrc(Kc, nblk), vrs = kv_rsrc(Vt, nblk);
  // The first two runs go out before the query work, whose loads are all
  // waited for before the loop (so a condition here costs no later wait).
  if (w0 < cend) {
    load_k(run[0], krs, run_koff(w0, lane));
    load_v(run[0], vrs, run_voff(w0, lane));
    if (w0 + 32 < cend) {
      load_k(run[1], krs, run_koff(w0 + 32, lane));
      load_v(run[1], vrs, run_voff(w0 + 32, lane));
    }
  }

  // A: wavefront u handles unit u, u+FW, ...: the group's query heads, then
  // (in the block holding the new position) the new key and value.
  const int units = n_q + 2 * n_kv;
  const float* row = qkv + (int64_t)b * units * 128;
  const float cs = ra.cos_t[(int64_t)pos * 64 + lane], sn = ra.sin_t[(int64_t)pos * 64 + lane];
  const bool owns = pos >= k_begin && pos < k_end;
  for (int u = wid; u < group + (owns ? 1 : 0); u += FW) {
    if (u < group) {
      const int h = g * group + u;
      float a = row[h * 128 + lane], c = row[h * 128 + lane + 64];
      norm_rope_pair(a, c, ra.qn, ra.eps, cs, sn);
      qs[u * 128 + lane] = f2bf(a);
      qs[u * 128 + lane + 64] = f2bf(c);
    } else {
      float a = row[(n_q + g) * 128 + lane], c = row[(n_q + g) * 128 + lane + 64];
      norm_rope_pair(a, c, ra.kn, ra.eps, cs, sn);
      const bf16_t ka = f2bf(a), kc = f2bf(c);
      const bf16_t va = f2bf(row[(n_q + n_kv + g) * 128 + lane]);
      const bf16_t vc = f2bf(row[(n_q + n_kv + g) * 128 + lane + 64]);
      Kc[kk_off<bf16_t>(pos, lane)] = ka;
      Kc[kk_off<bf16_t>(pos, lane + 64)] = kc;
      Vt[vt_off(pos, lane)] = va;
      Vt[vt_off(pos, lane + 64)] = vc;
      knew[lane] = ka;
      knew[lane + 64] = kc;
      vnew[lane] = va;
      vnew[lane + 64] = vc;
    }
  }
  __syncthreads();

  // B: cached keys, 32 at a time.
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (fr < group) v = *reinterpret_cast<const u32x4*>(&qs[fr * 128 + ks * 32 + fq * 8]);
    qf[ks] = as_bf16x8(v);
  }
  f32x4 oacc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;
  // Attend to the run in r (keys c0 ..), then refill r with the run at nc0:
  // its keys as soon as the score products have used r's, its values after
  // the P.V products.
  auto attend = [&](KvRun& r, int c0, int kro, int vro) {
    f32x4 sacc[2];
#pragma unroll
    for (int sbk = 0; sbk < 2; ++sbk) {
      sacc[sbk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[sbk] = mfma16(as_bf16x8(r.k[sbk][ks]), qf[ks], sacc[sbk]);
    }
    load_k(r, krs, kro);
    float mx = -INFINITY;
#pragma unroll
    for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float v = sacc[sbk][rr] * scale_log2;
        if (c0 + 8 * fq + 4 * sbk + rr >= cend) v = -INFINITY;
        sacc[sbk][rr] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrun, mx);
    const float alpha = exp2_f(mrun - mnew);
    mrun = mnew;
#pragma unroll
    for (int sbk = 0; sbk < 2; ++sbk)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sacc[sbk][rr] = exp2_f(sacc[sbk][rr] - mnew);
    float ls = 0.f;
    const PSplit pf = split_p(sacc[0], sacc[1], ls);
    lrun = lrun * alpha + ls;
    const int vkey0 = c0 + fq * 8;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const f16x8 vf = as_f16x8(bf16x8_to_f16x8(mask_keys(r.v[d], vkey0, cend)));
      oacc[d] = mfma16_f16(vf, pf.lo, mfma16_f16(vf, pf.hi, oacc[d] * alpha));
    }
    load_v(r, vrs, vro);
  };
  // Two register buffers, used in turn, each refilled with the run two ahead
  // (past the wavefront's last run: zeros, no bytes moved).  Every path loads
  // the same runs: with a conditional load the compiler counts outstanding
  // loads by the path without it and waits for the just-issued run before
  // using the current one.
  if (w0 < cend) {
    // byte offsets of the runs two ahead, advanced by two blocks per step
    int ko0 = run_koff(w0 + 64, lane), vo0 = run_voff(w0 + 64, lane);
    for (int c0 = w0;; c0 += 64) {
      attend(run[0], c0, ko0, vo0);
      if (c0 + 32 >= cend) break;
      attend(run[1], c0 + 32, ko0 + 8192, vo0 + 8192);
      if (c0 + 64 >= cend) break;
      ko0 += 16384;
      vo0 += 16384;
    }
  }
  if (has_new) {
    // The new key: score q.k over 128 dims (bf16 operands, fp32 sums), then
    // one more term of the online softmax with its fp16-rounded weight.
    const float k0 = bf2f(knew[lane]), k1 = bf2f(knew[lane + 64]);
    float snew = -INFINITY;
    for (int hh = 0; hh < group; ++hh) {
      const float d = wave_sum(bf2f(qs[hh * 128 + lane]) * k0 + bf2f(qs[hh * 128 + lane + 64]) * k1);
      if (fr == hh) snew = d * scale_log2;
    }
    if (fr < group) {
      const float mnew = fmaxf(mrun, snew);
      const float alpha = exp2_f(mrun - mnew);
      const float p = (float)(_Float16)exp2_f(snew - mnew);
      mrun = mnew;
      lrun = lrun * alpha + (fq == 0 ? p : 0.f);
#pragma unroll
      for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) oacc[d][rr] = oacc[d][rr] * alpha + p * bf2f(vnew[d * 16 + fq * 4 + rr]);
    }
  }
  lrun += __shfl_xor(lrun, 16, 64);
  lrun += __shfl_xor(lrun, 32, 64);
  if (fr < group) {
    float* wp = wred[wid][fr];
    if (fq == 0) {
      wp[0] = mrun;
      wp[1] = lrun;
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) wp[2 + d * 16 + fq * 4 + rr] = oacc[d][rr];
  }
  __syncthreads();

  // C: merge the block's wavefronts in order; then output or publish.
  for (int e = tid; e < group * 128; e += 64 * FW) {
    const int hh = e >> 7, d = e & 127;
    float M = -INFINITY;
    for (int w = 0; w < FW; ++w) M = fmaxf(M, wred[w][hh][0]);
    float L = 0.f, A = 0.f;
    for (int w = 0; w < FW; ++w) {
      if (wred[w][hh][0] == -INFINITY) continue;
      const float wt = exp2_f(wred[w][hh][0] - M);
      L += wred[w][hh][1] * wt;
      A += wred[w][hh][2 + d] * wt;
    }
    const int h = g * group + hh;
    if (fg.nact == 1) {
      o[((int64_t)b * n_q + h) * 128 + d] = f2bf(A / L);
    } else {
      float* pp = part + (((int64_t)b * n_q + h) * smax + j) * PSTRIDE;
      if (d == 0) {
        st_agent(pp, M);
        st_agent(pp + 1, L);
      }
      st_agent(pp + 2 + d, A);
    }
  }
  if (fg.nact == 1) return;
  __builtin_amdgcn_s_waitcnt(0);  // partial stores complete before the count below
  __syncthreads();
  uint32_t* c = cnt + (int64_t)b * n_kv + g;
  if (tid == 0) last = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(fg.nact - 1);
  __syncthreads();
  if (!last) return;
  // Last block of (b, g): merge the splits of each head in split order.
  for (int e = tid; e < group * 128; e += 64 * FW) {
    const int hh = e >> 7, d = e & 127;
    const float* pp = part + ((int64_t)b * n_q + g * group + hh) * smax * PSTRIDE;
    // up to MCH splits' partials in flight at once (one round trip for up to
    // 16 splits), then a running merge in split order
    constexpr int MCH = 16;
    float mj[MCH], lj[MCH], aj[MCH];
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int j0 = 0; j0 < fg.nact; j0 += MCH) {
#pragma unroll
      for (int u = 0; u < MCH; ++u) {
        const int jj = min(j0 + u, fg.nact - 1);
        const float* q = pp + (int64_t)jj * PSTRIDE;
        mj[u] = ld_agent(q);
        lj[u] = ld_agent(q + 1);
        aj[u] = ld_agent(q + 2 + d);
      }
#pragma unroll
      for (int u = 0; u < MCH; ++u) {
        if (j0 + u >= fg.nact) break;
        const float mn = fmaxf(M, mj[u]);
        const float so = exp2_f(M - mn), sj = exp2_f(mj[u] - mn);
        L = L * so + lj[u] * sj;
        A = A * so + aj[u] * sj;
        M = mn;
      }
    }
    o[((int64_t)b * n_q + g * group + hh) * 128 + d] = f2bf(A / L);
  }
  if (tid == 0) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- float32
constexpr int F32_MAX_CTX = 8192;

// Block (token t, query head h), 128 threads: plain softmax over the visible
// keys, all in fp32.  Used for the float32 model.
__global__ __launch_bounds__(128) void attn_f32_kernel(const float* __restrict__ q, SeqBatch sb,
                                                       const SeqState* __restrict__ st,
                                                       const float* __restrict__ kv, int layer, int n_q,
                                                       int n_kv, float* __restrict__ o, float scale) {
  __shared__ float qs[128];
  __shared__ float sc[F32_MAX_CTX];
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int b = seq_of_token(sb, t);
  const SeqState s = st[sb.slot[b]];
  const int pos = sb.decode ? s.len : sb.prior[b] + t - sb.cu[b];
  const int ctx = min(pos + 1, F32_MAX_CTX);
  const int g = h / (n_q / n_kv);
  const KvGeom geo{n_kv, layer};
  const float* Kc = kv_k(kv, s, geo, g);
  const float* Vt = kv_vt(kv, s, geo, g);
  qs[tid] = q[((int64_t)t * n_q + h) * 128 + tid];
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < ctx; j += 128) {
    const float* kr = Kc + (int64_t)j * 128;
    float dot = 0.f;
    for (int d = 0; d < 128; ++d) dot = fmaf(qs[d], kr[d], dot);
    sc[j] = dot * scale;
    mx = fmaxf(mx, sc[j]);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < ctx; j += 128) {
    const float p = __expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if ((tid & 63) == 0) red[2 + (tid >> 6)] = sum;
  __syncthreads();
  sum = red[2] + red[3];
  float acc = 0.f;
  for (int j = 0; j < ctx; ++j) acc = fmaf(sc[j], Vt[vt_off(j, tid)], acc);
  o[((int64_t)t * n_q + h) * 128 + tid] = acc / sum;
}
}  // namespace

namespace {
int g_flash_cb = -1;   // rows-per-wavefront override (q3op_tune); -1 = automatic
int g_flash_tpb = -1;  // query tiles per block override (q3op_tune); -1 = automatic
}
void flash_set_rows(int cb) { g_flash_cb = cb; }
void flash_set_tiles_per_block(int tpb) { g_flash_tpb = tpb; }

hipError_t flash_prefill(const bf16_t* q, int T, const SeqBatch& sb, const SeqState* st,
                         const bf16_t* kv, const uint16_t* vstage, int layer, int n_q, int n_kv, bf16_t* o,
                         hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int group = n_q / n_kv;
  if (group < 1 || group > 8 || 128 % group != 0) return hipErrorInvalidValue;
  // Rows per wavefront (16*CB).  CB = 2 halves the LDS reads per MFMA and still
  // fits two blocks per CU (248 registers per lane); 64 rows per wavefront (one
  // block per CU, with register spills) measured slower on gfx950 and is not
  // built.  Short prefills keep CB = 1 for more blocks.
  int CB = g_flash_cb;
  if (CB < 0) {
    // 32 rows per wavefront when that still gives every CU two blocks, else 16
    int64_t tiles2 = 0;
    for (int b = 0; b < sb.n; ++b) tiles2 += (sb.cu[b + 1] - sb.cu[b] + 128 / group - 1) / (128 / group);
    CB = tiles2 * n_kv >= 512 ? 2 : 1;
  }
  const int qt = 64 * CB / group;
  // Two query tiles per block when the call's tiles read 64 key tiles or
  // more on average (MI355X: 32K keys 5.32 -> 5.12 ms, 8K 1.43 -> 1.41 ms;
  // shorter prompts lose: 512 keys 263 -> 299 us, 2K 989 -> 1002 us).
  int TPB = g_flash_tpb;
  if (TPB < 0) {
    int64_t kt = 0, nt = 0;
    for (int b = 0; b < sb.n; ++b) {
      const int L = sb.cu[b + 1] - sb.cu[b], P = sb.prior[b];
      for (int t = 0; t * qt < L; ++t, ++nt) kt += (P + std::min(L, (t + 1) * qt) + 63) / 64;
    }
    TPB = (nt > 0 && kt >= 64 * nt) ? 2 : 1;
  }
  TileTable tt;
  tt.tile_cu[0] = 0;
  tt.item_cu[0] = 0;
  for (int b = 0; b < sb.n; ++b) {
    const int L = sb.cu[b + 1] - sb.cu[b];
    const int ntb = (L + qt - 1) / qt;
    tt.tile_cu[b + 1] = tt.tile_cu[b] + ntb;
    tt.item_cu[b + 1] = tt.item_cu[b] + (ntb + TPB - 1) / TPB;
    tt.vstart[b] = vstage_start(sb, b);
  }
  const int total = tt.tile_cu[sb.n];
  if (total <= 0) return hipSuccess;
  const int items = tt.item_cu[sb.n] * n_kv;
  // XCD runs of work items, balanced by the key tiles each item's loop reads
  // (items in the kernel's order: sequence, head, last query tile descending)
  {
    auto item_work = [&](int L, int P, int tA) { return (int64_t)(P + std::min(L, (tA + 1) * qt) + 63) / 64; };
    int64_t wsum = 0;
    for (int b = 0; b < sb.n; ++b) {
      const int L = sb.cu[b + 1] - sb.cu[b], P = sb.prior[b];
      const int ntb = (L + qt - 1) / qt;
      for (int tA = ntb - 1; tA >= 0; tA -= TPB) wsum += item_work(L, P, tA) * n_kv;
    }
    // walk the items in order, cutting at each eighth of the work
    int x = 1;
    int64_t acc = 0;
    int idx = 0;
    tt.xbnd[0] = 0;
    for (int b = 0; b < sb.n && x < 8; ++b) {
      const int L = sb.cu[b + 1] - sb.cu[b], P = sb.prior[b];
      const int ntb = (L + qt - 1) / qt;
      for (int g = 0; g < n_kv && x < 8; ++g)
        for (int tA = ntb - 1; tA >= 0 && x < 8; tA -= TPB, ++idx) {
          while (x < 8 && acc * 8 >= wsum * x) tt.xbnd[x++] = idx;
          acc += item_work(L, P, tA);
        }
    }
    while (x < 8) tt.xbnd[x++] = items;
    tt.xbnd[8] = items;
  }
  int longest = 0;
  for (int x = 0; x < 8; ++x) longest = std::max(longest, tt.xbnd[x + 1] - tt.xbnd[x]);
  if ((int64_t)longest * 8 > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)longest * 8);
  const float scale_log2 = kLog2e / sqrtf(128.f);
  const int64_t vh_keys = vstage_keys(sb);
#define Q3_FLASH(CBV, TPBV)                                                                                \
  flash_prefill_kernel<CBV, TPBV><<<grid, 256 * TPBV, 0, s>>>(q, sb, tt, st, kv, vstage, vh_keys, layer, n_q, \
                                                              n_kv, qt, o, scale_log2)
  if (CB == 2 && TPB == 1) Q3_FLASH(2, 1);
  else if (CB == 2 && TPB == 2) Q3_FLASH(2, 2);
  else if (CB == 1 && TPB == 1) Q3_FLASH(1, 1);
  else if (CB == 1 && TPB == 2) Q3_FLASH(1, 2);
  else return hipErrorInvalidValue;
#undef Q3_FLASH
  return hipGetLastError();
}

int decode_attn_splits(int B, int n_kv, int64_t max_ctx) {
  const int64_t by_len = (max_ctx + 63) / 64;
  int64_t want = (2048 + (int64_t)B * n_kv - 1) / ((int64_t)B * n_kv);
  if (want < 1) want = 1;
  int64_t sp = by_len < want ? by_len : want;
  return sp < 1 ? 1 : (int)sp;
}

hipError_t decode_attn(const bf16_t* q, const SeqBatch& sb, const SeqState* st, const bf16_t* kv,
                       int layer, int n_q, int n_kv, int splits, float* part, bf16_t* o,
                       hipStream_t s) {
  if (sb.n <= 0) return hipSuccess;
  const float scale_log2 = kLog2e / sqrtf(128.f);
  dim3 grid(splits, n_kv, sb.n);
  decode_attn_kernel<<<grid, 64, 0, s>>>(q, sb, st, kv, layer, n_q, n_kv, splits, part, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<<<sb.n * n_q, 128, 0, s>>>(part, sb, st, n_q, splits, o);
  return hipGetLastError();
}

namespace {
int g_attn_smax_cap = -1;  // upper bound on splits (q3op_tune); -1 = none
}
void decode_attn_set_split_cap(int cap) { g_attn_smax_cap = cap; }

constexpr int kRaggedSplits = 8;

int fused_attn_smax_max(int B, int n_kv, int64_t max_ctx) {
  // about one block per CU (256), at least 128 keys each, at most 64 splits;
  // measured on MI355X, more splits only add merge work once the CUs are busy
  // -- unless the batch is ragged (below)
  int64_t by_len = (max_ctx + 127) / 128;
  int64_t want = (256 + (int64_t)B * n_kv - 1) / ((int64_t)B * n_kv);
  int64_t sm = by_len < want ? by_len : want;
  if ((int64_t)B * n_kv >= 256) sm = std::max<int64_t>(sm, std::min<int64_t>(kRaggedSplits, by_len));
  if (sm > 64) sm = 64;
  return sm < 1 ? 1 : (int)sm;
}

AttnPlan fused_attn_plan(int B, int n_kv, int64_t max_cap, const int64_t* ctx) {
  AttnPlan p;
  std::memset(&p, 0, sizeof(p));
  // About three blocks for every four CUs: one 32,800-key sequence (8 KV
  // heads) measured 28.4-28.6 us per layer at 24 splits against 29.5 at 32,
  // 29.0 at 28, 29.7 at 20, 32.7-33.0 at 16 and 30.8 at 64 (MI355X, cold
  // cache; the merge of fewer partials and longer runs per block).
  int64_t by_len = (max_cap + 127) / 128;
  int64_t want = (192 + (int64_t)B * n_kv - 1) / ((int64_t)B * n_kv);
  int64_t sm = by_len < want ? by_len : want;
  int64_t maxctx = 1, sumctx = 0;
  for (int b = 0; b < B; ++b) {
    maxctx = std::max<int64_t>(maxctx, ctx[b]);
    sumctx += std::max<int64_t>(1, ctx[b]);
  }
  // A batch that fills the CUs with one block per (sequence, head) but has
  // sequences of different lengths ends on a tail of its longest blocks.
  // Its blocks go longest first, and each sequence is split
  // ceil(2 max/mean - 1) ways: equal lengths stay at one split, where more
  // splits only add merge work (32 x 2,112 keys on MI355X: 48.6 us per layer
  // at one split, 52.9 at two); 64 sequences of 128-8192 keys (max/mean
  // 1.9) take three (196 us at two splits, 192 at three, 206 at one).
  if ((int64_t)B * n_kv >= 256 && B > 0) {
    const int64_t r = (2 * maxctx * B - 1) / sumctx;  // ceil(2 max/mean - 1)
    sm = std::min<int64_t>(by_len, std::min<int64_t>(kRaggedSplits, std::max<int64_t>(1, r)));
  }
  if (sm > 64) sm = 64;
  if (sm < 1) sm = 1;
  if (g_attn_smax_cap > 0 && sm > g_attn_smax_cap) sm = g_attn_smax_cap;
  p.smax = (int)sm;
  int idx[Q3_MAX_BATCH];
  for (int b = 0; b < B; ++b) idx[b] = b;
  std::stable_sort(idx, idx + B, [&](int x, int y) { return ctx[x] > ctx[y]; });
  for (int b = 0; b < B; ++b) p.order[b] = (uint8_t)idx[b];
  return p;
}

hipError_t decode_attn_fused(const float* qkv, const SeqBatch& sb, const SeqState* st, bf16_t* kv, int layer,
                             int n_q, int n_kv, const float* qn, const float* kn, float eps, const float* cos_t,
                             const float* sin_t, const AttnPlan& plan, float* part, uint32_t* counters,
                             bf16_t* o, hipStream_t s) {
  if (sb.n <= 0) return hipSuccess;
  if (sb.n > Q3_MAX_BATCH || plan.smax < 1 || plan.smax > 64) return hipErrorInvalidValue;
  const int group = n_q / n_kv;
  if (group < 1 || group > 8) return hipErrorInvalidValue;
  const float scale_log2 = kLog2e / sqrtf(128.f);
  RopeArgs ra{qn, kn, cos_t, sin_t, eps};
  // the order must be a permutation: every output row written exactly once
  static_assert(Q3_MAX_BATCH <= 64, "one bit per sequence below");
  SeqOrder ord;
  uint64_t seen = 0;
  for (int b = 0; b < sb.n; ++b) {
    if (plan.order[b] >= sb.n || (seen >> plan.order[b] & 1)) return hipErrorInvalidValue;
    seen |= uint64_t(1) << plan.order[b];
    ord.v[b] = plan.order[b];
  }
  dim3 grid(plan.smax, n_kv, sb.n);
  // Four wavefronts per block: eight measured slower at every batch and
  // context tried (one CU's stream does not grow with more wavefronts).
  decode_attn_fused_kernel<4><<<grid, 256, 0, s>>>(qkv, sb, st, kv, layer, n_q, n_kv, ra, plan.smax, part, counters,
                                                   o, scale_log2, ord);
  return hipGetLastError();
}

hipError_t attn_f32(const float* q, int T, const SeqBatch& sb, const SeqState* st, const float* kv,
                    int layer, int n_q, int n_kv, float* o, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid(T, n_q);
  attn_f32_kernel<<<grid, 128, 0, s>>>(q, sb, st, kv, layer, n_q, n_kv, o, 1.f / sqrtf(128.f));
  return hipGetLastError();
}

}  // namespace q3k
