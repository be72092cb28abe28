// Weight-streaming projections for decode (and the lm_head of every call):
// M <= 64 activation rows against a bf16 weight matrix W[N,K].  The work is
// bound by reading W once from HBM, so each weight byte is loaded exactly once
// with 16-byte loads and fed to MFMA straight from registers (no conversion,
// no LDS staging); the few activation rows come from L2.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" -- Paso 5 (projections), Paso 6 (SwiGLU), Paso 7 (residuals),
// Paso 8 (lm_head and the greedy pick).
//
// Decomposition: a block of 4 wavefronts owns RG groups of 16 weight rows and
// a K range of 4*NST*32 columns; wavefront w takes NST consecutive 32-wide K
// steps of that range.  MFMA operand mapping (v_mfma_f32_16x16x32_bf16):
//   A = activations: lane l supplies X[mt*16 + l%16][k .. k+7]
//   B = W^T:         lane l supplies W[row0 + l%16][k .. k+7]
//   with k = kstep*32 + (l/16)*8, so each weight row is read as 64 contiguous
//   bytes per load instruction.  The four wavefronts' partial sums are added
//   in LDS in a fixed order.  When K needs several blocks (ksplit > 1) each
//   block writes its partial to a workspace and the last block to finish a row
//   range adds all partials in split order, so results are deterministic.
#include "kernels.h"

namespace q3k {

namespace {
Q3_DEV float silu_f(float g) { return g / (1.f + __expf(-g)); }

template <int EPI, int MT, int NST>
__global__ __launch_bounds__(256) void skinny_kernel(const bf16_t* __restrict__ X, int M,
                                                     const bf16_t* __restrict__ W, int N, int K,
                                                     void* __restrict__ out, int64_t ldo,
                                                     float* __restrict__ partials,
                                                     uint32_t* __restrict__ counters,
                                                     float* __restrict__ amax_val,
                                                     int32_t* __restrict__ amax_idx, int ksplit) {
  constexpr int RG = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int KW = NST * 32;  // K columns per wavefront
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int kidx = blockIdx.y;
  const int k0 = kidx * (4 * KW) + wid * KW + (lane >> 4) * 8;
  const int row0 = blockIdx.x * RG * 16;

  // Weight fragments first: they are the HBM stream.
  u32x4 wf[RG][NST];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const bf16_t* wp = W + (int64_t)(row0 + g * 16 + (lane & 15)) * K + k0;
#pragma unroll
    for (int s = 0; s < NST; ++s) wf[g][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + s * 32));
  }
  f32x4 acc[RG][MT];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[g][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    const bf16_t* xp = X + (int64_t)(m < M ? m : 0) * K + k0;
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      u32x4 xv = ld16(xp + s * 32);
      if (m >= M) xv = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int g = 0; g < RG; ++g) acc[g][mt] = mfma16(as_bf16x8(xv), as_bf16x8(wf[g][s]), acc[g][mt]);
    }
  }

  // Cross-wavefront reduction.  red[w][g][mt][lane*4 + r].
  __shared__ __attribute__((aligned(16))) float red[4][RG][MT][256];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(&red[wid][g][mt][lane * 4]) = acc[g][mt];
  __syncthreads();

  // Entry e = (mt, lane', r) of the C fragment: m = mt*16 + (lane'/16)*4 + r,
  // n = row0 + g*16 + lane'%16.
  constexpr int NE = MT * 256;
  __shared__ float vals[RG][MT * 256];
  for (int e = threadIdx.x; e < NE; e += 256) {
    const int mt = e >> 8, le = e & 255;
#pragma unroll
    for (int g = 0; g < RG; ++g)
      vals[g][e] = red[0][g][mt][le] + red[1][g][mt][le] + red[2][g][mt][le] + red[3][g][mt][le];
  }

  if (ksplit > 1) {
    // Publish this split's partial, then let the last block of the row range finish.
    for (int e = threadIdx.x; e < NE; e += 256) {
      const int mt = e >> 8, le = e & 255;
      const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
      const int nl = (le >> 2) & 15;
      if (m < M) {
#pragma unroll
        for (int g = 0; g < RG; ++g)
          partials[((int64_t)kidx * M + m) * N + row0 + g * 16 + nl] = vals[g][e];
      }
    }
    __threadfence();
    __syncthreads();
    __shared__ uint32_t ticket;
    if (threadIdx.x == 0) ticket = atomicAdd(&counters[blockIdx.x], 1u);
    __syncthreads();
    if (ticket != (uint32_t)(ksplit - 1)) return;
    __threadfence();
    for (int e = threadIdx.x; e < NE; e += 256) {
      const int mt = e >> 8, le = e & 255;
      const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
      const int nl = (le >> 2) & 15;
      if (m < M) {
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          float sum = 0.f;
          for (int k = 0; k < ksplit; ++k)
            sum += __builtin_nontemporal_load(&partials[((int64_t)k * M + m) * N + row0 + g * 16 + nl]);
          vals[g][e] = sum;
        }
      }
    }
    if (threadIdx.x == 0) counters[blockIdx.x] = 0u;
    __syncthreads();
  }

  // Epilogue.
  if constexpr (EPI == EPI_ARGMAX) {
    // logits out, then per-row (max, lowest index) over this block's 16 rows
    __syncthreads();
    float* o = reinterpret_cast<float*>(out);
    for (int e = threadIdx.x; e < NE; e += 256) {
      const int mt = e >> 8, le = e & 255;
      const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
      const int nl = (le >> 2) & 15;
      if (m < M) o[(int64_t)m * ldo + row0 + nl] = vals[0][e];
    }
    if (threadIdx.x < M) {
      const int m = threadIdx.x, mt = m >> 4, mr = m & 15;
      float bv = -INFINITY;
      int bi = -1;
      for (int nl = 0; nl < 16; ++nl) {
        const int le = ((((mr >> 2) << 4) + nl) << 2) + (mr & 3);
        const float v = vals[0][mt * 256 + le];
        if (bi < 0 || v > bv) { bv = v; bi = row0 + nl; }
        if (!__builtin_isfinite(v)) { bv = v; bi = row0 + nl; break; }
      }
      amax_val[(int64_t)blockIdx.x * M + m] = bv;
      amax_idx[(int64_t)blockIdx.x * M + m] = bi;
    }
  } else {
    for (int e = threadIdx.x; e < NE; e += 256) {
      const int mt = e >> 8, le = e & 255;
      const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
      const int nl = (le >> 2) & 15;
      if (m >= M) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        bf16_t* o = reinterpret_cast<bf16_t*>(out);
        o[(int64_t)m * ldo + (row0 >> 1) + nl] = f2bf(silu_f(vals[0][e]) * vals[1][e]);
      } else if constexpr (EPI == EPI_RESADD) {
        float* o = reinterpret_cast<float*>(out);
        o[(int64_t)m * ldo + row0 + nl] += vals[0][e];
      } else {
        float* o = reinterpret_cast<float*>(out);
        o[(int64_t)m * ldo + row0 + nl] = vals[0][e];
      }
    }
  }
}

template <int EPI, int NST>
hipError_t launch_mt(int MT, dim3 grid, const bf16_t* X, int M, const bf16_t* W, int N, int K, void* out,
                     int64_t ldo, float* partials, uint32_t* counters, float* av, int32_t* ai,
                     int ksplit, hipStream_t s) {
  switch (MT) {
    case 1: skinny_kernel<EPI, 1, NST><<<grid, 256, 0, s>>>(X, M, W, N, K, out, ldo, partials, counters, av, ai, ksplit); break;
    case 2: skinny_kernel<EPI, 2, NST><<<grid, 256, 0, s>>>(X, M, W, N, K, out, ldo, partials, counters, av, ai, ksplit); break;
    case 3: skinny_kernel<EPI, 3, NST><<<grid, 256, 0, s>>>(X, M, W, N, K, out, ldo, partials, counters, av, ai, ksplit); break;
    default: skinny_kernel<EPI, 4, NST><<<grid, 256, 0, s>>>(X, M, W, N, K, out, ldo, partials, counters, av, ai, ksplit); break;
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_nst(int nst, int MT, dim3 grid, const bf16_t* X, int M, const bf16_t* W, int N, int K,
                      void* out, int64_t ldo, float* partials, uint32_t* counters, float* av,
                      int32_t* ai, int ksplit, hipStream_t s) {
  if (nst == 8)
    return launch_mt<EPI, 8>(MT, grid, X, M, W, N, K, out, ldo, partials, counters, av, ai, ksplit, s);
  return launch_mt<EPI, 4>(MT, grid, X, M, W, N, K, out, ldo, partials, counters, av, ai, ksplit, s);
}
}  // namespace

// Choose how many 32-wide K steps each wavefront takes: 8 when the matrix has
// enough 16-row groups to fill the GPU with one block per group, else 4 so
// that more blocks share the rows.
SkinnyPlan skinny_plan(int epi, int M, int N, int K) {
  (void)M;
  const int rg = (epi == EPI_SWIGLU) ? 2 : 1;
  const int groups = N / (16 * rg);
  SkinnyPlan p;
  p.nst = (K % 1024 == 0 && groups >= 512) ? 8 : 4;
  p.ksplit = K / (4 * 32 * p.nst);
  return p;
}

size_t skinny_partials_floats(int M, int N, int ksplit) {
  return ksplit > 1 ? (size_t)ksplit * M * N : 0;
}

int skinny_argmax_blocks(int N, SkinnyPlan plan) {
  (void)plan;
  return N / 16;
}

hipError_t skinny_bf16(int epi, const bf16_t* X, int M, const bf16_t* W, int N, int K, void* out,
                       int64_t ldo, float* partials, uint32_t* counters, float* amax_val,
                       int32_t* amax_idx, SkinnyPlan plan, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (M > 64) return hipErrorInvalidValue;
  const int nst = plan.nst;
  const int rg = (epi == EPI_SWIGLU) ? 2 : 1;
  if (N % (16 * rg) != 0 || K % (4 * 32 * nst) != 0 || plan.ksplit * 4 * 32 * nst != K)
    return hipErrorInvalidValue;
  const int MT = (M + 15) / 16;
  dim3 grid(N / (16 * rg), plan.ksplit);
  switch (epi) {
    case EPI_STORE: return launch_nst<EPI_STORE>(nst, MT, grid, X, M, W, N, K, out, ldo, partials, counters, amax_val, amax_idx, plan.ksplit, s);
    case EPI_RESADD: return launch_nst<EPI_RESADD>(nst, MT, grid, X, M, W, N, K, out, ldo, partials, counters, amax_val, amax_idx, plan.ksplit, s);
    case EPI_SWIGLU: return launch_nst<EPI_SWIGLU>(nst, MT, grid, X, M, W, N, K, out, ldo, partials, counters, amax_val, amax_idx, plan.ksplit, s);
    case EPI_ARGMAX: return launch_nst<EPI_ARGMAX>(nst, MT, grid, X, M, W, N, K, out, ldo, partials, counters, amax_val, amax_idx, plan.ksplit, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- float32 model
// One wavefront per output column (SwiGLU: per output j, both its gate row and
// its up row), rows of X in chunks of 8.  Plain fp32 FMA; used for the
// float32 model only.
template <int EPI>
__global__ __launch_bounds__(256) void gemv_f32_kernel(const float* __restrict__ X, int M,
                                                       const float* __restrict__ W, int N, int K,
                                                       void* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x & 63;
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ncols = (EPI == EPI_SWIGLU) ? N / 2 : N;
  if (col >= ncols) return;
  int r0 = col, r1 = col;
  if (EPI == EPI_SWIGLU) {
    r0 = (col / 16) * 32 + (col % 16);
    r1 = r0 + 16;
  }
  const float* w0 = W + (int64_t)r0 * K;
  const float* w1 = W + (int64_t)r1 * K;
  for (int m0 = 0; m0 < M; m0 += 8) {
    float a0[8], a1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { a0[j] = 0.f; a1[j] = 0.f; }
    for (int k = lane; k < K; k += 64) {
      const float x0 = w0[k], x1 = w1[k];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (m0 + j < M) {
          const float xv = X[(int64_t)(m0 + j) * K + k];
          a0[j] = fmaf(x0, xv, a0[j]);
          a1[j] = fmaf(x1, xv, a1[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float s0 = wave_sum(a0[j]);
      const float s1 = (EPI == EPI_SWIGLU) ? wave_sum(a1[j]) : 0.f;
      if (lane == 0 && m0 + j < M) {
        float* o = reinterpret_cast<float*>(out) + (int64_t)(m0 + j) * ldo + col;
        if (EPI == EPI_SWIGLU)
          *o = silu_f(s0) * s1;
        else if (EPI == EPI_RESADD)
          *o += s0;
        else
          *o = s0;
      }
    }
  }
}

hipError_t gemv_f32(int epi, const float* X, int M, const float* W, int N, int K, void* out,
                    int64_t ldo, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int ncols = (epi == EPI_SWIGLU) ? N / 2 : N;
  dim3 grid((ncols + 3) / 4);
  switch (epi) {
    case EPI_STORE:
    case EPI_ARGMAX: gemv_f32_kernel<EPI_STORE><<<grid, 256, 0, s>>>(X, M, W, N, K, out, ldo); break;
    case EPI_RESADD: gemv_f32_kernel<EPI_RESADD><<<grid, 256, 0, s>>>(X, M, W, N, K, out, ldo); break;
    case EPI_SWIGLU:
      if (N % 32 != 0) return hipErrorInvalidValue;
      gemv_f32_kernel<EPI_SWIGLU><<<grid, 256, 0, s>>>(X, M, W, N, K, out, ldo);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q3k
