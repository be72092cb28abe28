// Streaming lm_head for decode batches: M <= 64 activation rows against the
// tied embedding matrix W[N,K] (N = 151,936 vocabulary rows), logits out and
// the per-row greedy pick folded in.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" -- Paso 8 (the final norm's output times the embedding matrix gives
// the logits; greedy decoding takes the highest).
//
// The weight-streaming kernel of k_skinny.hip gives each block one 16-row
// group of W, so every block reads all M activation rows again (for 64 rows
// as many bytes from L2 as the whole matrix from HBM, four times over) and
// lives for a single load/multiply/reduce round.  Here a grid of one block per
// CU keeps the activations in LDS for its whole life and each wavefront
// streams whole 16-row groups of W (all of K) through a register double
// buffer: the next 256-column chunk is in flight while the MFMAs use the
// current one, across group boundaries.  No cross-wavefront reduction is
// needed per group (a wavefront owns every K of its groups); the argmax runs
// per wavefront over its groups, then once per block.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_bf16), as in k_skinny.hip:
//   A = activations: lane l supplies X[mt*16 + l%16][k .. k+7]
//   B = W^T:         lane l supplies W[g*16 + l%16][k .. k+7]
//   k = ks*32 + (l/16)*8; lane l holds C[m = mt*16 + (l/16)*4 + r][n = g*16 + l%16].
// LDS holds X row m's 16-byte chunk c at chunk c ^ (m % 16) of the row, so the
// 16 rows of one fragment read fall in 16 different 16-byte bank groups.
#include "kernels.h"

namespace q3k {

namespace {

constexpr int kHeadWaves = 8;   // wavefronts per block
constexpr int kHeadChunk = 8;   // 32-wide K steps per weight chunk (256 columns)

Q3_DEV int xs_off(int m, int K, int k) { return m * K + ((((k >> 3) ^ (m & 15)) << 3) | (k & 7)); }

// (v, i) beats the current best (bv, bi), without branches: any entry beats
// an empty best (bi = INT_MAX); a non-finite value beats finite ones (it is
// reported, and the reduction then flags the row), the lower index among
// non-finite ones; otherwise the larger value, and the lower index among
// equal values.
Q3_DEV bool beats(float v, int i, float bv, int bi) {
  const bool fv = __builtin_isfinite(v), fb = __builtin_isfinite(bv);
  const bool normal = (v > bv) | ((v == bv) & (i < bi));
  const bool nonfin = (fv != fb) ? !fv : (!fv & (i < bi));
  return (bi == 0x7fffffff) | ((fv & fb) ? normal : nonfin);
}

// CPG = K / 256 chunks per 16-row group (even, so each group starts on the
// same register buffer and the loop body is free of run-time branches, whose
// merged wait counts made the compiler drain the load pipeline).
template <int MT, int CPG>
__global__ __launch_bounds__(64 * kHeadWaves) void headstream_kernel(const bf16_t* __restrict__ X, int M,
                                                                    const bf16_t* __restrict__ W, int N,
                                                                    float* __restrict__ out, int64_t ldo,
                                                                    float* __restrict__ amax_val,
                                                                    int32_t* __restrict__ amax_idx) {
  static_assert(CPG % 2 == 0, "chunks per group must be even");
  constexpr int K = CPG * 32 * kHeadChunk;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_h[];
  uint16_t* xs = smem_h;                                                      // [MT*16][K] bf16, swizzled
  float* rv = reinterpret_cast<float*>(smem_h + (size_t)MT * 16 * K);         // [waves][64] best values
  int* ri = reinterpret_cast<int*>(rv + kHeadWaves * 64);                     // [waves][64] their indices
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int fr = lane & 15, fq = lane >> 4;

  // Stage X (rows >= M are zero).
  constexpr int kc8 = K >> 3;
  for (int c = threadIdx.x; c < MT * 16 * kc8; c += blockDim.x) {
    const int m = c / kc8, kc = c - m * kc8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (m < M) v = ld16(X + (int64_t)m * K + kc * 8);
    *reinterpret_cast<u32x4*>(&xs[xs_off(m, K, kc * 8)]) = v;
  }

  // This wavefront's groups: w0, w0 + TW, ... over the whole grid's wavefronts.
  const int groups = N / 16;
  const int TW = gridDim.x * kHeadWaves;
  const int w0 = blockIdx.x * kHeadWaves + wid;
  const int ng = w0 < groups ? (groups - 1 - w0) / TW + 1 : 0;

  float best_v[MT][4];
  int best_i[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      best_v[mt][r] = -INFINITY;
      best_i[mt][r] = 0x7fffffff;
    }

  // Chunk c of the wavefront's j-th group (clamped to its last group: past
  // the end it re-reads that one, always issued).
  auto load_chunk = [&](u32x4 (&buf)[kHeadChunk], int j, int c) {
    const int g = w0 + min(j, ng - 1) * TW;
    const bf16_t* wp = W + (int64_t)(g * 16 + fr) * K + c * (32 * kHeadChunk) + fq * 8;
#pragma unroll
    for (int s = 0; s < kHeadChunk; ++s)
      buf[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + s * 32));
  };
  // The lane's fragment of row mt*16 + fr at K step s of chunk c is the
  // row's 16-byte chunk c*32 + s*4 + fq, stored at chunk
  // c*32 + (s/4)*16 + ((s%4)*4 + fq) ^ (row % 16): a per-lane base for each
  // (mt, s % 4) plus a compile-time offset (the read's immediate), rather
  // than one address register per (mt, c, s).
  const uint16_t* xb[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = mt * 16 + fr;
      xb[mt][q] = xs + row * K + ((((q * 4 + fq) ^ (row & 15))) << 3);
    }
  auto consume = [&](const u32x4 (&buf)[kHeadChunk], int c, f32x4 (&acc)[MT]) {
#pragma unroll
    for (int s = 0; s < kHeadChunk; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xb[mt][s & 3] + c * 256 + (s >> 2) * 128);
        acc[mt] = mfma16(as_bf16x8(xv), as_bf16x8(buf[s]), acc[mt]);
      }
    }
  };

  __syncthreads();  // X staged
  if (ng > 0) {
    u32x4 b0[kHeadChunk], b1[kHeadChunk];
    load_chunk(b0, 0, 0);
    for (int j = 0; j < ng; ++j) {
      f32x4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < CPG; c += 2) {
        // chunk c sits in b0, c + 1 goes to b1; then c + 2 (or the next
        // group's first chunk) to b0 while b1 is used
        // (scheduling barriers keep the compiler from hoisting later chunks'
        // loads ahead of their turn)
        load_chunk(b1, j, c + 1);
        __builtin_amdgcn_sched_barrier(0);
        consume(b0, c, acc);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 2 < CPG) load_chunk(b0, j, c + 2);
        else load_chunk(b0, j + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        consume(b1, c + 1, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
      // group done: logits out, then each row's best of the group's 16
      const int n = (w0 + j * TW) * 16 + fr;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mt * 16 + fq * 4 + r;
          float v = acc[mt][r];
          if (m < M) out[(int64_t)m * ldo + n] = v;
          int i = n;
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            const float ov = __shfl_xor(v, o, 64);
            const int oi = __shfl_xor(i, o, 64);
            const bool t = beats(ov, oi, v, i);
            v = t ? ov : v;
            i = t ? oi : i;
          }
          const bool t = beats(v, i, best_v[mt][r], best_i[mt][r]);
          best_v[mt][r] = t ? v : best_v[mt][r];
          best_i[mt][r] = t ? i : best_i[mt][r];
        }
    }
  }

  // Block result per row: the wavefronts' bests, combined in wavefront order.
  if (fr == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rv[wid * 64 + mt * 16 + fq * 4 + r] = best_v[mt][r];
        ri[wid * 64 + mt * 16 + fq * 4 + r] = best_i[mt][r];
      }
  }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    const int m = threadIdx.x;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int w = 0; w < kHeadWaves; ++w) {
      const float v = rv[w * 64 + m];
      const int i = ri[w * 64 + m];
      if (i != 0x7fffffff && beats(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
    amax_val[(int64_t)m * gridDim.x + blockIdx.x] = bv;
    amax_idx[(int64_t)m * gridDim.x + blockIdx.x] = bi == 0x7fffffff ? -1 : bi;
  }
}

template <int MT>
hipError_t headstream_mt(const bf16_t* X, int M, const bf16_t* W, int N, int K, float* out, int64_t ldo,
                         float* av, int32_t* ai, dim3 grid, size_t lds, hipStream_t s) {
  const dim3 block(64 * kHeadWaves);
  switch (K / (32 * kHeadChunk)) {
    case 2: headstream_kernel<MT, 2><<<grid, block, lds, s>>>(X, M, W, N, out, ldo, av, ai); break;
    case 4: headstream_kernel<MT, 4><<<grid, block, lds, s>>>(X, M, W, N, out, ldo, av, ai); break;
    case 6: headstream_kernel<MT, 6><<<grid, block, lds, s>>>(X, M, W, N, out, ldo, av, ai); break;
    case 8: headstream_kernel<MT, 8><<<grid, block, lds, s>>>(X, M, W, N, out, ldo, av, ai); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int headstream_blocks(int N) {
  const int groups = N / 16;
  const int per_block = kHeadWaves;
  int g = (groups + per_block - 1) / per_block;
  return g < 256 ? g : 256;
}

bool headstream_ok(int M, int N, int K) {
  const int cpg = K / (32 * kHeadChunk);
  return M >= 1 && M <= 64 && N % 16 == 0 && K % (32 * kHeadChunk) == 0 &&
         (cpg == 2 || cpg == 4 || cpg == 6 || cpg == 8) &&
         (size_t)((M + 15) / 16) * 16 * K * 2 + kHeadWaves * 64 * 8 <= 160 * 1024;
}

hipError_t headstream_bf16(const bf16_t* X, int M, const bf16_t* W, int N, int K, float* out, int64_t ldo,
                           float* amax_val, int32_t* amax_idx, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!headstream_ok(M, N, K)) return hipErrorInvalidValue;
  const int MT = (M + 15) / 16;
  const size_t lds = (size_t)MT * 16 * K * 2 + kHeadWaves * 64 * 8;
  const dim3 grid(headstream_blocks(N));
  switch (MT) {
    case 1: return headstream_mt<1>(X, M, W, N, K, out, ldo, amax_val, amax_idx, grid, lds, s);
    case 2: return headstream_mt<2>(X, M, W, N, K, out, ldo, amax_val, amax_idx, grid, lds, s);
    case 3: return headstream_mt<3>(X, M, W, N, K, out, ldo, amax_val, amax_idx, grid, lds, s);
    default: return headstream_mt<4>(X, M, W, N, K, out, ldo, amax_val, amax_idx, grid, lds, s);
  }
}

}  // namespace q3k
