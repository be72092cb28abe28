// Single-row decode projections: one activation row against a bf16 weight
// matrix W[N,K], wavefronts working on whole rows with no LDS staging and no
// block barrier on the projection path.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" -- Paso 3 (RMSNorm, here a prologue), Paso 5 (q/k/v and o
// projections), Paso 6 (SwiGLU: gate, up, silu(gate) * up, down), Paso 7
// (residual adds), Paso 8 (tied lm_head and the greedy pick).
//
// Wavefront layout: a wavefront owns RW weight rows.  Lane l covers the
// elements k = 8*l + 512*i (i < KS, K = 512*KS) of every row, so each row is
// read as 64 lanes x 16 contiguous bytes per load instruction and all RW*KS
// loads of a lane are in flight together.  Products are bf16 pairs summed in
// fp32 by v_dot2_f32_bf16; a butterfly over the 64 lanes finishes each row.
//
// NORM: the activation is the float32 residual row x; every wavefront
// computes the row's sum of squares itself (x is L2-resident, 4 KiB for the
// 1024-wide model) and forms bf16(x * rsqrt(mean(x^2) + eps) * g), the same
// rounding point as the standalone RMSNorm kernel.  The activation and norm
// loads are issued before the weight loads, so the norm arithmetic runs while
// the weight stream is still arriving.
#include "kernels.h"

namespace q3k {

namespace {
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

Q3_DEV float silu_f(float g) { return g / (1.f + __expf(-g)); }

Q3_DEV void take_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

template <int EPI, int KS, int RW, bool NORM>
__global__ __launch_bounds__(256) void rowgemv_kernel(const void* __restrict__ Xin, const bf16_t* __restrict__ W,
                                                      int N, int K, const float* __restrict__ gnorm, float eps,
                                                      void* __restrict__ out, float* __restrict__ amax_val,
                                                      int32_t* __restrict__ amax_idx) {
  static_assert(EPI != EPI_SWIGLU || RW % 2 == 0, "SwiGLU pairs a gate row with its up row");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wg = blockIdx.x * (blockDim.x >> 6) + wid;  // global wavefront index
  const int koff = lane * 8;

  // Rows of this wavefront.  SwiGLU: output column c uses gate row
  // (c/16)*32 + c%16 and up row 16 further (runs of 16 rows, interleaved).
  int rows[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int c = wg * (RW / 2) + (r >> 1);
      rows[r] = (c >> 4) * 32 + (c & 15) + (r & 1) * 16;
    } else {
      rows[r] = wg * RW + r;
    }
  }

  // Activations first (and the norm weights), then the weight stream.
  u32x4 xv[KS];
  float4 xf[NORM ? KS : 1][2], gf[NORM ? KS : 1][2];
  if constexpr (NORM) {
    const float* x = reinterpret_cast<const float*>(Xin);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      xf[i][0] = *reinterpret_cast<const float4*>(x + koff + 512 * i);
      xf[i][1] = *reinterpret_cast<const float4*>(x + koff + 512 * i + 4);
      gf[i][0] = *reinterpret_cast<const float4*>(gnorm + koff + 512 * i);
      gf[i][1] = *reinterpret_cast<const float4*>(gnorm + koff + 512 * i + 4);
    }
  } else {
    const bf16_t* x = reinterpret_cast<const bf16_t*>(Xin);
#pragma unroll
    for (int i = 0; i < KS; ++i) xv[i] = ld16(x + koff + 512 * i);
  }
  // RESADD: lane r < RW fetches the residual of row r now, so that the
  // read-modify-write at the end costs no extra round trip.
  float resv = 0.f;
  if constexpr (EPI == EPI_RESADD) {
    int rr = N;
#pragma unroll
    for (int r = 0; r < RW; ++r)
      if (lane == r) rr = rows[r];
    if (rr < N) resv = reinterpret_cast<const float*>(out)[rr];
  }
  u32x4 wv[RW][KS];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const bf16_t* wr = W + (int64_t)(rows[r] < N ? rows[r] : 0) * K + koff;
#pragma unroll
    for (int i = 0; i < KS; ++i) wv[r][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + 512 * i));
  }
  // Keep every load above issued before any arithmetic below: the compiler
  // would otherwise start the norm reduction first and hold the weight
  // stream back behind the activation loads' latency.
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const float4 a = xf[i][0], b = xf[i][1];
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
    }
    ss = wave_sum(ss);
    const float inv = rsqrtf(ss / (float)K + eps);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const float4 a = xf[i][0], b = xf[i][1], ga = gf[i][0], gb = gf[i][1];
      xv[i][0] = pack_bf2(a.x * inv * ga.x, a.y * inv * ga.y);
      xv[i][1] = pack_bf2(a.z * inv * ga.z, a.w * inv * ga.w);
      xv[i][2] = pack_bf2(b.x * inv * gb.x, b.y * inv * gb.y);
      xv[i][3] = pack_bf2(b.z * inv * gb.z, b.w * inv * gb.w);
    }
  }

  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // element copies first: bit-casting a vector element in place picked
        // the wrong element in this compiler
        const uint32_t wu = wv[r][i][c], xu = xv[i][c];
        acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wu), __builtin_bit_cast(bf16x2_t, xu),
                                                 acc[r], false);
      }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = wave_sum(acc[r]);

  if constexpr (EPI == EPI_SWIGLU) {
    bf16_t* o = reinterpret_cast<bf16_t*>(out);
#pragma unroll
    for (int j = 0; j < RW / 2; ++j) {
      const int c = wg * (RW / 2) + j;
      if (lane == j && 2 * c < N) o[c] = f2bf(silu_f(acc[2 * j]) * acc[2 * j + 1]);
    }
  } else {
    float* o = reinterpret_cast<float*>(out);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (lane == r && rows[r] < N) {
        if constexpr (EPI == EPI_RESADD)
          o[rows[r]] = resv + acc[r];
        else
          o[rows[r]] = acc[r];
      }
    }
  }

  if constexpr (EPI == EPI_ARGMAX) {
    // (max, lowest index) over the block's rows; a non-finite logit is passed
    // on as the partial so that the finishing pass flags it.
    float bv = -INFINITY, bad = 0.f;
    int bi = 0x7fffffff, badi = -1;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (rows[r] >= N) continue;
      if (!__builtin_isfinite(acc[r]) && badi < 0) {
        bad = acc[r];
        badi = rows[r];
      }
      take_better(bv, bi, acc[r], rows[r]);
    }
    __shared__ float sv[4], sb[4];
    __shared__ int si[4], sbi[4];
    if (lane == 0) {
      sv[wid] = bv;
      si[wid] = bi;
      sb[wid] = bad;
      sbi[wid] = badi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const int nw = blockDim.x >> 6;
      float v = -INFINITY;
      int ix = 0x7fffffff;
      float bv2 = 0.f;
      int bi2 = -1;
      for (int w = 0; w < nw; ++w) {
        take_better(v, ix, sv[w], si[w]);
        if (bi2 < 0 && sbi[w] >= 0) {
          bv2 = sb[w];
          bi2 = sbi[w];
        }
      }
      if (bi2 >= 0) {
        v = bv2;
        ix = bi2;
      }
      amax_val[blockIdx.x] = v;
      amax_idx[blockIdx.x] = ix == 0x7fffffff ? -1 : ix;
    }
  }
}

int g_rows_override = -1;   // rows per wavefront (q3op_tune); -1 = automatic
int g_waves_override = -1;  // wavefronts per block (q3op_tune); -1 = automatic

struct RowPlan {
  int rw;     // rows per wavefront
  int waves;  // wavefronts per block
};

// About eight 16-byte weight loads in flight per lane (RW * K/512), and four
// wavefronts per block unless that leaves fewer blocks than the 256 CUs.
// Measured on MI355X with the weights cold in HBM: q/k/v 3.4 us, gate/up
// 5.0 us, o 3.4-3.9 us, down 3.3-3.4 us, lm_head 53 us.
RowPlan row_plan(int epi, int N, int K) {
  const int ks = K / 512;
  int rw = ks >= 8 ? 1 : (ks >= 6 ? 1 : (ks >= 4 ? 2 : (ks >= 2 ? 4 : 8)));
  if (epi == EPI_SWIGLU && rw < 2) rw = 2;
  const int64_t nwaves = ((int64_t)N + rw - 1) / rw;
  int waves = 4;
  while (waves > 1 && (nwaves + waves - 1) / waves < 256) waves >>= 1;
  RowPlan p{rw, waves};
  if (g_rows_override > 0) p.rw = g_rows_override;
  if (g_waves_override > 0) p.waves = g_waves_override;
  return p;
}

template <int EPI, int KS, bool NORM>
hipError_t launch_rw(int rw, dim3 grid, dim3 block, const void* X, const bf16_t* W, int N, int K, const float* g,
                     float eps, void* out, float* av, int32_t* ai, hipStream_t s) {
  switch (rw) {
    case 1:
      if constexpr (EPI == EPI_SWIGLU) return hipErrorInvalidValue;  // gate and up rows come in pairs
      else rowgemv_kernel<EPI, KS, 1, NORM><<<grid, block, 0, s>>>(X, W, N, K, g, eps, out, av, ai);
      break;
    case 2: rowgemv_kernel<EPI, KS, 2, NORM><<<grid, block, 0, s>>>(X, W, N, K, g, eps, out, av, ai); break;
    case 4: rowgemv_kernel<EPI, KS, 4, NORM><<<grid, block, 0, s>>>(X, W, N, K, g, eps, out, av, ai); break;
    case 8: rowgemv_kernel<EPI, KS, 8, NORM><<<grid, block, 0, s>>>(X, W, N, K, g, eps, out, av, ai); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI, bool NORM>
hipError_t launch_ks(int KS, int rw, dim3 grid, dim3 block, const void* X, const bf16_t* W, int N, int K,
                     const float* g, float eps, void* out, float* av, int32_t* ai, hipStream_t s) {
  switch (KS) {
    case 1: return launch_rw<EPI, 1, NORM>(rw, grid, block, X, W, N, K, g, eps, out, av, ai, s);
    case 2: return launch_rw<EPI, 2, NORM>(rw, grid, block, X, W, N, K, g, eps, out, av, ai, s);
    case 4: return launch_rw<EPI, 4, NORM>(rw, grid, block, X, W, N, K, g, eps, out, av, ai, s);
    case 6: return launch_rw<EPI, 6, NORM>(rw, grid, block, X, W, N, K, g, eps, out, av, ai, s);
    case 8: return launch_rw<EPI, 8, NORM>(rw, grid, block, X, W, N, K, g, eps, out, av, ai, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

void rowgemv_set_plan(int rows, int waves) {
  g_rows_override = rows;
  g_waves_override = waves;
}

bool rowgemv_ok(int M, int K) {
  if (M != 1 || K % 512 != 0) return false;
  const int ks = K / 512;
  return ks == 1 || ks == 2 || ks == 4 || ks == 6 || ks == 8;
}

int rowgemv_argmax_blocks(int N, int K) {
  const RowPlan p = row_plan(EPI_ARGMAX, N, K);
  const int per_block = p.rw * p.waves;
  return (N + per_block - 1) / per_block;
}

hipError_t rowgemv_bf16(int epi, const void* X, const bf16_t* W, int N, int K, const float* gnorm, float eps,
                        void* out, float* amax_val, int32_t* amax_idx, hipStream_t s) {
  if (!rowgemv_ok(1, K) || N <= 0) return hipErrorInvalidValue;
  const bool norm = gnorm != nullptr;
  if (norm && (epi == EPI_RESADD || epi == EPI_ARGMAX)) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && N % 32 != 0) return hipErrorInvalidValue;
  if (epi == EPI_ARGMAX && (amax_val == nullptr || amax_idx == nullptr)) return hipErrorInvalidValue;
  const RowPlan p = row_plan(epi, N, K);
  if (p.waves < 1 || p.waves > 4) return hipErrorInvalidValue;
  // RW rows per wavefront (SwiGLU: RW/2 outputs, each a gate and an up row).
  const int64_t nwaves = ((int64_t)N + p.rw - 1) / p.rw;
  dim3 grid((unsigned)((nwaves + p.waves - 1) / p.waves));
  dim3 block(64 * p.waves);
  const int KS = K / 512;
  switch (epi) {
    case EPI_STORE:
      return norm ? launch_ks<EPI_STORE, true>(KS, p.rw, grid, block, X, W, N, K, gnorm, eps, out, nullptr, nullptr, s)
                  : launch_ks<EPI_STORE, false>(KS, p.rw, grid, block, X, W, N, K, nullptr, eps, out, nullptr, nullptr, s);
    case EPI_SWIGLU:
      return norm ? launch_ks<EPI_SWIGLU, true>(KS, p.rw, grid, block, X, W, N, K, gnorm, eps, out, nullptr, nullptr, s)
                  : launch_ks<EPI_SWIGLU, false>(KS, p.rw, grid, block, X, W, N, K, nullptr, eps, out, nullptr, nullptr, s);
    case EPI_RESADD:
      return launch_ks<EPI_RESADD, false>(KS, p.rw, grid, block, X, W, N, K, nullptr, eps, out, nullptr, nullptr, s);
    case EPI_ARGMAX:
      return launch_ks<EPI_ARGMAX, false>(KS, p.rw, grid, block, X, W, N, K, nullptr, eps, out, amax_val, amax_idx, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace q3k
