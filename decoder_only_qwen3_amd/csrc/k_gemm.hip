// bf16 MFMA GEMM for the prefill projections and the SwiGLU MLP.
//
//   C[M,N] = A[M,K] . W[N,K]^T,  A = activations (row-major, K contiguous),
//   W = a weight matrix stored (out_features, in_features) as the page's
//   listings apply it (x @ W^T).  fp32 accumulation on v_mfma_f32_16x16x32_bf16.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" -- Paso 5 (q/k/v and o projections), Paso 6 (SwiGLU: gate, up,
// silu(gate) * up, down), Paso 7 (residual adds).
//
// Tiling: block tile (16*WM*GM) x (16*WN*GN), K step 64; GM x GN wavefronts,
// each owning a (16*WM) x (16*WN) sub-tile as 16x16 MFMA tiles.  Large
// problems use 256x256 tiles on 16 wavefronts, small ones 64x64 on 4.
// Global -> register prefetch of the next K step overlaps the MFMAs of the
// current one; tiles are staged through LDS with 16-byte row padding.
#include "kernels.h"

namespace q3k {

namespace {
constexpr int BK = 64, LDK = BK + 8;

Q3_DEV float silu_f(float g) { return g / (1.f + __expf(-g)); }

// Block tile (16*WM*GM) x (16*WN*GN): GM x GN wavefronts, each owning a
// (16*WM) x (16*WN) sub-tile of 16x16 MFMA tiles.
template <int EPI, int WM, int WN, int GM, int GN>
__global__ __launch_bounds__(64 * GM * GN) void gemm_bf16_kernel(const bf16_t* __restrict__ A, int M,
                                                                const bf16_t* __restrict__ W, int N, int K,
                                                                void* __restrict__ out, int64_t ldo) {
  constexpr int NT = 64 * GM * GN;
  constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN;
  constexpr int RSTEP = NT / 8;                      // rows covered by one pass of 16-byte loads
  constexpr int LA = BM / RSTEP, LW = BN / RSTEP;    // 16-byte chunks per thread per K step
  static_assert(BM % RSTEP == 0 && BN % RSTEP == 0, "tile rows must be a multiple of the load pass");
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sW[2][BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / GN, wn = wid % GN;
  const int bn0 = blockIdx.x * BN, bm0 = blockIdx.y * BM;
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;

  u32x4 ra[LA], rw[LW];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = lrow + RSTEP * i;
      const u32x4 z = {0u, 0u, 0u, 0u};
      ra[i] = (bm0 + r < M) ? ld16(A + (int64_t)(bm0 + r) * K + k0 + lcol) : z;
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int r = lrow + RSTEP * i;
      const u32x4 z = {0u, 0u, 0u, 0u};
      rw[i] = (bn0 + r < N) ? ld16(W + (int64_t)(bn0 + r) * K + k0 + lcol) : z;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(&sA[buf][(lrow + RSTEP * i) * LDK + lcol]) = ra[i];
#pragma unroll
    for (int i = 0; i < LW; ++i) *reinterpret_cast<u32x4*>(&sW[buf][(lrow + RSTEP * i) * LDK + lcol]) = rw[i];
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[WM], bw[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][(wm * 16 * WM + i * 16 + fr) * LDK + ks * 32 + fk]);
#pragma unroll
      for (int j = 0; j < WN; ++j)
        bw[j] = *reinterpret_cast<const bf16x8*>(&sW[buf][(wn * 16 * WN + j * 16 + fr) * LDK + ks * 32 + fk]);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma16(af[i], bw[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // C layout of a 16x16 MFMA tile: lane l holds rows (l/16)*4 + r, column l%16.
  const int rbase = bm0 + wm * 16 * WM + (lane >> 4) * 4;
  const int cbase = bn0 + wn * 16 * WN + (lane & 15);
  if constexpr (EPI == EPI_SWIGLU) {
    // Packed rows: every 32 rows of W are 16 gate rows then the matching 16 up
    // rows, so tile j=2p is gate and j=2p+1 is up for the same output column.
    bf16_t* o = reinterpret_cast<bf16_t*>(out);
    const int ocol0 = (bn0 + wn * 16 * WN) / 2 + (lane & 15);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int p = 0; p < WN / 2; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          const int col = ocol0 + p * 16;
          if (row < M && 2 * col < N) {
            const float g = acc[i][2 * p][r], u = acc[i][2 * p + 1][r];
            o[(int64_t)row * ldo + col] = f2bf(silu_f(g) * u);
          }
        }
  } else {
    float* o = reinterpret_cast<float*>(out);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rbase + i * 16 + r;
          const int col = cbase + j * 16;
          if (row < M && col < N) {
            float* p = o + (int64_t)row * ldo + col;
            if constexpr (EPI == EPI_RESADD)
              *p += acc[i][j][r];
            else
              *p = acc[i][j][r];
          }
        }
  }
}

template <int WM, int WN, int GM, int GN>
hipError_t gemm_launch(int epi, const bf16_t* A, int M, const bf16_t* W, int N, int K, void* out, int64_t ldo,
                       hipStream_t s) {
  constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN, NT = 64 * GM * GN;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  switch (epi) {
    case EPI_STORE:
    case EPI_ARGMAX:
      gemm_bf16_kernel<EPI_STORE, WM, WN, GM, GN><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo);
      break;
    case EPI_RESADD:
      gemm_bf16_kernel<EPI_RESADD, WM, WN, GM, GN><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo);
      break;
    case EPI_SWIGLU:
      gemm_bf16_kernel<EPI_SWIGLU, WM, WN, GM, GN><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int g_gemm_cfg = -1;  // tile configuration override (q3op_tune); -1 = automatic
}  // namespace

void gemm_set_config(int cfg) { g_gemm_cfg = cfg; }

hipError_t gemm_bf16(int epi, const bf16_t* A, int M, const bf16_t* W, int N, int K, void* out,
                     int64_t ldo, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (K % BK != 0 || N % 16 != 0) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && N % 64 != 0) return hipErrorInvalidValue;
  int cfg = g_gemm_cfg;
  if (cfg < 0) {
    // The largest tile whose grid still gives each of the 256 CUs a block:
    // 256 x 256 (16 wavefronts), else 128 x 128, else 64 x 64.
    const int64_t g256 = (int64_t)((N + 255) / 256) * ((M + 255) / 256);
    const int64_t g128 = (int64_t)((N + 127) / 128) * ((M + 127) / 128);
    cfg = g256 >= 256 ? 6 : (g128 >= 256 ? 1 : 0);
  }
  switch (cfg) {
    case 0: return gemm_launch<2, 2, 2, 2>(epi, A, M, W, N, K, out, ldo, s);   //  64 x  64, 4 waves
    case 1: return gemm_launch<4, 4, 2, 2>(epi, A, M, W, N, K, out, ldo, s);   // 128 x 128, 4 waves
    case 2: return gemm_launch<4, 4, 4, 2>(epi, A, M, W, N, K, out, ldo, s);   // 256 x 128, 8 waves
    case 3: return gemm_launch<4, 4, 2, 4>(epi, A, M, W, N, K, out, ldo, s);   // 128 x 256, 8 waves
    case 4: return gemm_launch<4, 8, 2, 2>(epi, A, M, W, N, K, out, ldo, s);   // 128 x 256, 4 waves
    case 5: return gemm_launch<8, 4, 2, 2>(epi, A, M, W, N, K, out, ldo, s);   // 256 x 128, 4 waves
    case 6: return gemm_launch<4, 4, 4, 4>(epi, A, M, W, N, K, out, ldo, s);   // 256 x 256, 16 waves
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q3k
