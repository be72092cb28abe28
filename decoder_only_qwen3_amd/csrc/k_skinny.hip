// Weight-streaming projections for decode (and the lm_head of every call):
// M <= 64 activation rows against a bf16 weight matrix W[N,K].  The work is
// bound by reading W once from HBM, so each weight byte is loaded exactly once
// with 16-byte loads and fed to MFMA straight from registers (no conversion,
// no LDS staging); the few activation rows come from L2.
//
// Method source: "Dentro de un LLM: Inferencia en Python puro para Qwen3-0.6B
// en MLX" -- Paso 3 (RMSNorm, fused here as a prologue), Paso 5 (projections),
// Paso 6 (SwiGLU), Paso 7 (residuals), Paso 8 (lm_head and the greedy pick).
//
// Decomposition: a block owns RG groups of 16 weight rows (RG = 2 for SwiGLU:
// a gate group and its up group) over the whole K range; its W wavefronts each
// take NST consecutive 32-wide K steps (K = W * NST * 32).  Blocks never talk
// to each other, so no device-scope fence is needed.  MFMA operand mapping
// (v_mfma_f32_16x16x32_bf16):
//   A = activations: lane l supplies X[mt*16 + l%16][k .. k+7]
//   B = W^T:         lane l supplies W[row0 + l%16][k .. k+7]
//   with k = kstep*32 + (l/16)*8, so each weight row is read as 64 contiguous
//   bytes per load instruction.  The wavefronts' partial sums are added in
//   LDS in wavefront order, so results do not depend on scheduling.
//
// NORM = true: X is not given; the prologue computes it from the float32
// residual rows x and the norm weight g as bf16(x * rsqrt(mean(x^2)+eps) * g),
// the same rounding point as the standalone RMSNorm kernel (decode, M <= 64).
#include "kernels.h"

namespace q3k {

namespace {
Q3_DEV float silu_f(float g) { return g / (1.f + __expf(-g)); }

typedef __bf16 bf16x2_k __attribute__((ext_vector_type(2)));
// Two floats -> packed bf16 by v_cvt_pk_bf16_f32 (round to nearest even), as
// the dequantizer and the single-row GEMV on codes round.
Q3_DEV uint32_t pack_bf2_hw(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2_k));
}

constexpr int kMaxWaves = 16;
constexpr int kNormMaxM = 64;
constexpr int kMaxSplit = 4;  // K slices of a split residual projection

// BITS = 8 or 4: W holds affine group codes of the weights (groups of 64
// along K, a 32-bit fp16 scale/offset word per group in sbw); each lane
// loads its 8 codes and the group's word and forms bf16(q * s + b), the same
// bf16 values the dequantizer writes, before the MFMA loop.
template <int EPI, int MT, int NST, bool NORM, int BITS = 0>
__global__ __launch_bounds__(1024) void skinny_kernel(const void* __restrict__ Xin, int M,
                                                      const void* __restrict__ Wv, int N, int K,
                                                      const float* __restrict__ gnorm, float eps,
                                                      void* __restrict__ out, int64_t ldo,
                                                      float* __restrict__ amax_val,
                                                      int32_t* __restrict__ amax_idx,
                                                      const uint32_t* __restrict__ sbw) {
  constexpr int RG = (EPI == EPI_SWIGLU) ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int nw = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // Split K (RESADD only): block (x, y) covers K slice y of gridDim.y.
  const int nsplit = gridDim.y, sk = blockIdx.y;
  const int k0 = sk * (K / nsplit) + wid * (NST * 32) + (lane >> 4) * 8;
  const int row0 = blockIdx.x * RG * 16;

  // Weight fragments first: they are the HBM stream.
  u32x4 wf[RG][NST];
  uint32_t wq[BITS ? RG : 1][BITS ? NST : 1][BITS == 8 ? 2 : 1], wsb[BITS ? RG : 1][BITS ? NST : 1];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int64_t row = row0 + g * 16 + (lane & 15);
    if constexpr (BITS == 0) {
      const bf16_t* wp = reinterpret_cast<const bf16_t*>(Wv) + row * K + k0;
#pragma unroll
      for (int s = 0; s < NST; ++s)
        wf[g][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + s * 32));
    } else {
      const uint8_t* cp = reinterpret_cast<const uint8_t*>(Wv) + row * (K * BITS / 8);
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        const int kk = k0 + s * 32;
        if constexpr (BITS == 8) {
          const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cp + kk));
          wq[g][s][0] = c[0];
          wq[g][s][1] = c[1];
        } else {
          wq[g][s][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(cp + kk / 2));
        }
        wsb[g][s] = sbw[row * (K / 64) + kk / 64];
      }
    }
  }
  // Keep the weight loads ahead of everything else (the compiler would
  // otherwise issue the activation loads first and wait on one of them
  // before the weight stream starts).
  __builtin_amdgcn_sched_barrier(0);

  float* red = smem;                                  // [nw][RG][MT][256]
  float* inv = smem + nw * RG * MT * 256;             // [kNormMaxM] (NORM only)
  // NORM: the row sums of squares are reduced from the wavefronts' slices of
  // the float32 residual rows.  One 16-row tile (M <= 16): the slice stays in
  // registers; more rows: it is read again (from L2) when the bf16 operand is
  // formed, rather than held in registers across the reduction.
  constexpr bool XREG = NORM && MT == 1;
  float4 xs[XREG ? NST : 1][2];
  if constexpr (NORM) {
    const float* x = reinterpret_cast<const float*>(Xin);
    float ss[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + (lane & 15);
      ss[mt] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NST; ++s2) {
        float4 a = float4{0.f, 0.f, 0.f, 0.f}, b = a;
        if (m < M) {
          const float* xp = x + (int64_t)m * K + k0 + s2 * 32;
          a = *reinterpret_cast<const float4*>(xp);
          b = *reinterpret_cast<const float4*>(xp + 4);
        }
        if constexpr (XREG) {
          xs[s2][0] = a;
          xs[s2][1] = b;
        }
        ss[mt] += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
      }
      // lanes m, m+16, m+32, m+48 hold row m's four K groups
      ss[mt] += __shfl_xor(ss[mt], 16, 64);
      ss[mt] += __shfl_xor(ss[mt], 32, 64);
    }
    if (lane < 16) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[wid * kNormMaxM + mt * 16 + lane] = ss[mt];
    }
    __syncthreads();
    if (threadIdx.x < M) {
      float t = 0.f;
      for (int w = 0; w < nw; ++w) t += red[w * kNormMaxM + threadIdx.x];
      inv[threadIdx.x] = rsqrtf(t / (float)K + eps);
    }
    __syncthreads();
  }

  if constexpr (BITS != 0) {  // codes -> bf16(q * s + b) fragments
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(wsb[g][s] & 0xffffu));
        const float of = (float)__builtin_bit_cast(_Float16, (uint16_t)(wsb[g][s] >> 16));
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t q;
          if constexpr (BITS == 8) q = (wq[g][s][i >> 2] >> (8 * (i & 3))) & 0xffu;
          else q = (wq[g][s][0] >> (4 * i)) & 0xfu;
          v[i] = fmaf((float)q, sc, of);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) wf[g][s][i] = pack_bf2_hw(v[2 * i], v[2 * i + 1]);
      }
  }

  f32x4 acc[RG][MT];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[g][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // bf16 activations: every fragment of the wavefront's slice is loaded (from
  // L2) before the first product, so they take one round trip; rows past M
  // read row 0 (their results are never stored).
  u32x4 xf[NORM ? 1 : MT][NORM ? 1 : NST];
  if constexpr (!NORM) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + (lane & 15);
      const bf16_t* xp = reinterpret_cast<const bf16_t*>(Xin) + (int64_t)(m < M ? m : 0) * K + k0;
#pragma unroll
      for (int s = 0; s < NST; ++s) xf[mt][s] = ld16(xp + s * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    const bool live = m < M;
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      u32x4 xv = {0u, 0u, 0u, 0u};
      if constexpr (NORM) {
        if (live) {
          float4 a, b;
          if constexpr (XREG) {
            a = xs[s][0];
            b = xs[s][1];
          } else {
            const float* xp = reinterpret_cast<const float*>(Xin) + (int64_t)m * K + k0 + s * 32;
            a = *reinterpret_cast<const float4*>(xp);
            b = *reinterpret_cast<const float4*>(xp + 4);
          }
          const float4 ga = *reinterpret_cast<const float4*>(gnorm + k0 + s * 32);
          const float4 gb = *reinterpret_cast<const float4*>(gnorm + k0 + s * 32 + 4);
          const float r = inv[m];
          xv[0] = pack_bf2(a.x * r * ga.x, a.y * r * ga.y);
          xv[1] = pack_bf2(a.z * r * ga.z, a.w * r * ga.w);
          xv[2] = pack_bf2(b.x * r * gb.x, b.y * r * gb.y);
          xv[3] = pack_bf2(b.z * r * gb.z, b.w * r * gb.w);
        }
      } else {
        xv = xf[mt][s];
      }
#pragma unroll
      for (int g = 0; g < RG; ++g) acc[g][mt] = mfma16(as_bf16x8(xv), as_bf16x8(wf[g][s]), acc[g][mt]);
    }
  }
  if constexpr (NORM) __syncthreads();  // red[] doubled as the norm scratch

  // Cross-wavefront reduction: red[w][g][mt][lane*4 + r].
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(&red[((wid * RG + g) * MT + mt) * 256 + lane * 4]) = acc[g][mt];
  __syncthreads();

  // Entry e = (mt, lane', r) of the C fragment: m = mt*16 + (lane'/16)*4 + r,
  // n = row0 + g*16 + lane'%16.  Summed over wavefronts in order into red[0].
  constexpr int NE = MT * 256;
  for (int e = threadIdx.x; e < NE; e += blockDim.x) {
    const int mt = e >> 8, le = e & 255;
    if (mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3) >= M) continue;  // padding rows of the MFMA tile
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      float sum = 0.f;
      for (int w = 0; w < nw; ++w) sum += red[((w * RG + g) * MT + mt) * 256 + le];
      red[(g * MT + mt) * 256 + le] = sum;  // slot of wavefront 0, already read by this thread
    }
  }
  __syncthreads();

  if constexpr (EPI == EPI_ARGMAX) {
    // logits out, then per-row (max, lowest index) over this block's 16 rows
    float* o = reinterpret_cast<float*>(out);
    for (int e = threadIdx.x; e < NE; e += blockDim.x) {
      const int mt = e >> 8, le = e & 255;
      const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
      const int nl = (le >> 2) & 15;
      if (m < M) o[(int64_t)m * ldo + row0 + nl] = red[mt * 256 + le];
    }
    if (threadIdx.x < M) {
      const int m = threadIdx.x, mt = m >> 4, mr = m & 15;
      float bv = -INFINITY;
      int bi = -1;
      for (int nl = 0; nl < 16; ++nl) {
        const int le = ((((mr >> 2) << 4) + nl) << 2) + (mr & 3);
        const float v = red[mt * 256 + le];
        if (bi < 0 || v > bv) { bv = v; bi = row0 + nl; }
        if (!__builtin_isfinite(v)) { bv = v; bi = row0 + nl; break; }
      }
      amax_val[(int64_t)m * gridDim.x + blockIdx.x] = bv;  // [M][blocks]: each row's partials contiguous
      amax_idx[(int64_t)m * gridDim.x + blockIdx.x] = bi;
    }
  } else {
    for (int e = threadIdx.x; e < NE; e += blockDim.x) {
      const int mt = e >> 8, le = e & 255;
      const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
      const int nl = (le >> 2) & 15;
      if (m >= M) continue;
      const float v0 = red[mt * 256 + le];
      if constexpr (EPI == EPI_SWIGLU) {
        const float v1 = red[(MT + mt) * 256 + le];
        bf16_t* o = reinterpret_cast<bf16_t*>(out);
        o[(int64_t)m * ldo + (row0 >> 1) + nl] = f2bf(silu_f(v0) * v1);
      } else if constexpr (EPI == EPI_RESADD) {
        if (nsplit == 1) {
          float* o = reinterpret_cast<float*>(out);
          o[(int64_t)m * ldo + row0 + nl] += v0;
        }
      } else {
        float* o = reinterpret_cast<float*>(out);
        o[(int64_t)m * ldo + row0 + nl] = v0;
      }
    }
    if constexpr (EPI == EPI_RESADD) {
      if (nsplit > 1) {
        // Publish this slice's sums (agent scope: coherent across the L2
        // slices), count the slices of this row group, and let the last one
        // add them in slice order (deterministic) into the residual rows.
        float* part = amax_val;                                  // [N/16][nsplit][MT*256]
        uint32_t* cnt = reinterpret_cast<uint32_t*>(amax_idx);  // [N/16], zero between calls
        float* mine = part + ((int64_t)blockIdx.x * nsplit + sk) * NE;
        for (int e = threadIdx.x; e < NE; e += blockDim.x)
          __hip_atomic_store(mine + e, red[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        __shared__ int last;
        if (threadIdx.x == 0)
          last = __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(nsplit - 1);
        __syncthreads();
        if (last) {
          // Every load of the merge (up to kMaxSplit partials and the
          // residual for each of this thread's entries) is issued before the
          // first add; the sums still run in slice order.  Entries of rows
          // past M read row 0 and are not stored.  blockDim >= 256, so a
          // thread has at most MT entries.
          const float* grp = part + (int64_t)blockIdx.x * nsplit * NE;
          float* o = reinterpret_cast<float*>(out);
          float pv[MT][kMaxSplit], rv[MT];
          int64_t oi[MT];
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const int e = min((int)threadIdx.x + i * (int)blockDim.x, NE - 1);
            const int mt = e >> 8, le = e & 255;
            const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
            oi[i] = (int64_t)(m < M ? m : 0) * ldo + row0 + ((le >> 2) & 15);
#pragma unroll
            for (int j = 0; j < kMaxSplit; ++j)
              pv[i][j] = __hip_atomic_load(grp + (int64_t)min(j, nsplit - 1) * NE + e, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            rv[i] = o[oi[i]];
          }
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const int e = (int)threadIdx.x + i * (int)blockDim.x;
            const int mt = e >> 8, le = e & 255;
            const int m = mt * 16 + ((le >> 2) >> 4) * 4 + (le & 3);
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxSplit; ++j)
              if (j < nsplit) v += pv[i][j];
            if (e < NE && m < M) o[oi[i]] = rv[i] + v;
          }
          if (threadIdx.x == 0) __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

template <int EPI, int NST, bool NORM, int BITS>
hipError_t launch_mt(int MT, dim3 grid, dim3 block, size_t lds, const void* X, int M, const void* W, int N,
                     int K, const float* g, float eps, void* out, int64_t ldo, float* av, int32_t* ai,
                     hipStream_t s, const uint32_t* sb) {
#define Q3_SK(mt) \
  skinny_kernel<EPI, mt, NST, NORM, BITS><<<grid, block, lds, s>>>(X, M, W, N, K, g, eps, out, ldo, av, ai, sb)
  switch (MT) {
    case 1: Q3_SK(1); break;
    case 2: Q3_SK(2); break;
    case 3: Q3_SK(3); break;
    default: Q3_SK(4); break;
  }
#undef Q3_SK
  return hipGetLastError();
}

template <int EPI, bool NORM, int BITS>
hipError_t launch_nst(const SkinnyPlan& p, int MT, dim3 grid, const void* X, int M, const void* W, int N,
                      int K, const float* g, float eps, void* out, int64_t ldo, float* av, int32_t* ai,
                      hipStream_t s, const uint32_t* sb) {
  const int rg = (EPI == EPI_SWIGLU) ? 2 : 1;
  const size_t lds = (size_t)p.waves * rg * MT * 256 * 4 + kNormMaxM * 4;
  dim3 block(64 * p.waves);
  if (p.nst == 8)
    return launch_mt<EPI, 8, NORM, BITS>(MT, grid, block, lds, X, M, W, N, K, g, eps, out, ldo, av, ai, s, sb);
  return launch_mt<EPI, 4, NORM, BITS>(MT, grid, block, lds, X, M, W, N, K, g, eps, out, ldo, av, ai, s, sb);
}

template <int EPI, int BITS = 0>
hipError_t launch_norm(bool norm, const SkinnyPlan& p, int MT, dim3 grid, const void* X, int M, const void* W,
                       int N, int K, const float* g, float eps, void* out, int64_t ldo, float* av, int32_t* ai,
                       hipStream_t s, const uint32_t* sb = nullptr) {
  if (norm) return launch_nst<EPI, true, BITS>(p, MT, grid, X, M, W, N, K, g, eps, out, ldo, av, ai, s, sb);
  return launch_nst<EPI, false, BITS>(p, MT, grid, X, M, W, N, K, g, eps, out, ldo, av, ai, s, sb);
}
}  // namespace

// Wavefronts per block and K steps per wavefront: 32-wide K steps in runs of
// 4 (more wavefronts, more loads in flight per CU) unless that needs more than
// 16 wavefronts or more than 96 KiB of LDS for the reduction (gfx950 gives a
// block up to 160 KiB).
SkinnyPlan skinny_plan(int epi, int M, int N, int K) {
  (void)N;
  const int rg = (epi == EPI_SWIGLU) ? 2 : 1;
  const int MT = (M + 15) / 16;
  SkinnyPlan p{4, K / 128};
  if (p.waves > kMaxWaves || p.waves * rg * MT > 96) p = SkinnyPlan{8, K / 256};
  return p;
}

bool skinny_norm_ok(int M) { return M <= kNormMaxM; }

// Whether a decode step should fold the RMSNorm into the projection: for one
// 16-row tile the residual slice is read once into registers; beyond that
// every block reads all rows of x twice, which on MI355X cost more (13 us at
// 32 rows) than a separate RMSNorm kernel plus bf16 operands (5.5 + 6 us).
bool skinny_norm_fuse(int M) { return M <= 16; }

// Residual projections with few row groups (N/16 < 128, e.g. the 1024-wide o
// and down projections: 64 blocks) split K over up to 4 block slices so that
// the weight and activation streams spread over more CUs; slices of at least
// 512 so each block keeps 4+ wavefronts.
int skinny_splits(int epi, int M, int N, int K) {
  (void)M;
  if (epi != EPI_RESADD || N / 16 >= 128) return 1;
  for (int sp = kMaxSplit; sp >= 2; sp >>= 1)
    if (K % (sp * 128) == 0 && K / sp >= 512) return sp;
  return 1;
}

size_t skinny_split_floats(int M, int N, int K) {
  const int sp = skinny_splits(EPI_RESADD, M, N, K);
  if (sp <= 1) return 0;
  return (size_t)(N / 16) * sp * ((M + 15) / 16) * 256;
}

int skinny_argmax_blocks(int N) { return N / 16; }

hipError_t skinny_bf16(int epi, const void* X, int M, const bf16_t* W, int N, int K, const float* gnorm,
                       float eps, void* out, int64_t ldo, float* amax_val, int32_t* amax_idx, hipStream_t s,
                       float* split_part, uint32_t* split_cnt) {
  if (M <= 0) return hipSuccess;
  if (M > 64) return hipErrorInvalidValue;
  const bool norm = gnorm != nullptr;
  if (norm && M > kNormMaxM) return hipErrorInvalidValue;
  const int sp = (!norm && split_part && split_cnt) ? skinny_splits(epi, M, N, K) : 1;
  if (sp > 1) {
    // K slices: the kernel sees the slice length through its plan
    const SkinnyPlan p = skinny_plan(epi, M, N, K / sp);
    const int MT = (M + 15) / 16;
    if (N % 16 != 0 || p.waves * p.nst * 32 * sp != K || p.waves > kMaxWaves || p.waves * MT > 96)
      return hipErrorInvalidValue;
    dim3 grid(N / 16, sp);
    return launch_norm<EPI_RESADD>(false, p, MT, grid, X, M, W, N, K, nullptr, eps, out, ldo, split_part,
                                   reinterpret_cast<int32_t*>(split_cnt), s);
  }
  const SkinnyPlan p = skinny_plan(epi, M, N, K);
  const int rg = (epi == EPI_SWIGLU) ? 2 : 1;
  const int MT = (M + 15) / 16;
  if (N % (16 * rg) != 0 || p.waves * p.nst * 32 != K || p.waves > kMaxWaves || p.waves * rg * MT > 96 ||
      (norm && K % 4 != 0))
    return hipErrorInvalidValue;
  dim3 grid(N / (16 * rg));
  switch (epi) {
    case EPI_STORE: return launch_norm<EPI_STORE>(norm, p, MT, grid, X, M, W, N, K, gnorm, eps, out, ldo, amax_val, amax_idx, s);
    case EPI_RESADD: return launch_norm<EPI_RESADD>(norm, p, MT, grid, X, M, W, N, K, gnorm, eps, out, ldo, amax_val, amax_idx, s);
    case EPI_SWIGLU: return launch_norm<EPI_SWIGLU>(norm, p, MT, grid, X, M, W, N, K, gnorm, eps, out, ldo, amax_val, amax_idx, s);
    case EPI_ARGMAX: return launch_norm<EPI_ARGMAX>(norm, p, MT, grid, X, M, W, N, K, gnorm, eps, out, ldo, amax_val, amax_idx, s);
  }
  return hipErrorInvalidValue;
}

hipError_t skinny_q(int epi, int bits, const void* X, int M, const uint8_t* codes, const uint32_t* sb, int N, int K,
                    const float* gnorm, float eps, void* out, int64_t ldo, hipStream_t s, float* split_part,
                    uint32_t* split_cnt) {
  if (M <= 0) return hipSuccess;
  if (M > 64 || (bits != 8 && bits != 4) || K % 64 != 0) return hipErrorInvalidValue;
  if (epi != EPI_STORE && epi != EPI_RESADD && epi != EPI_SWIGLU) return hipErrorInvalidValue;
  const bool norm = gnorm != nullptr;
  if (norm && M > kNormMaxM) return hipErrorInvalidValue;
  auto go = [&](auto bits_c, const SkinnyPlan& p, int MT, dim3 grid, float* av, int32_t* ai) -> hipError_t {
    constexpr int B = decltype(bits_c)::value;
    switch (epi) {
      case EPI_STORE: return launch_norm<EPI_STORE, B>(norm, p, MT, grid, X, M, codes, N, K, gnorm, eps, out, ldo, av, ai, s, sb);
      case EPI_RESADD: return launch_norm<EPI_RESADD, B>(norm, p, MT, grid, X, M, codes, N, K, gnorm, eps, out, ldo, av, ai, s, sb);
      default: return launch_norm<EPI_SWIGLU, B>(norm, p, MT, grid, X, M, codes, N, K, gnorm, eps, out, ldo, av, ai, s, sb);
    }
  };
  const int sp = (!norm && split_part && split_cnt) ? skinny_splits(epi, M, N, K) : 1;
  const int MT = (M + 15) / 16;
  if (sp > 1) {
    const SkinnyPlan p = skinny_plan(epi, M, N, K / sp);
    if (N % 16 != 0 || p.waves * p.nst * 32 * sp != K || p.waves > kMaxWaves || p.waves * MT > 96)
      return hipErrorInvalidValue;
    dim3 grid(N / 16, sp);
    float* av = split_part;
    int32_t* ai = reinterpret_cast<int32_t*>(split_cnt);
    return bits == 8 ? go(std::integral_constant<int, 8>{}, p, MT, grid, av, ai)
                     : go(std::integral_constant<int, 4>{}, p, MT, grid, av, ai);
  }
  const SkinnyPlan p = skinny_plan(epi, M, N, K);
  const int rg = (epi == EPI_SWIGLU) ? 2 : 1;
  if (N % (16 * rg) != 0 || p.waves * p.nst * 32 != K || p.waves > kMaxWaves || p.waves * rg * MT > 96 ||
      (norm && K % 4 != 0))
    return hipErrorInvalidValue;
  dim3 grid(N / (16 * rg));
  return bits == 8 ? go(std::integral_constant<int, 8>{}, p, MT, grid, nullptr, nullptr)
                   : go(std::integral_constant<int, 4>{}, p, MT, grid, nullptr, nullptr);
}

// ---------------------------------------------------------------- row-parallel decode GEMV
// One wavefront per output row for M <= 4 activation rows: lane l reads
// 16-byte runs W[n][k .. k+8) at k = 8*l + 512*i (the whole row in flight at
// once), multiplies them with the matching bf16 activations by packed bf16
// dot products (fp32 accumulate) and the wavefront sums its lanes.  No
// cross-wavefront or cross-block reduction, so matrices with few rows (the
// 1024-row o and down projections) still spread over every CU.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int EPI, int MR, int KS>
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16_t* __restrict__ X, const bf16_t* __restrict__ W,
                                                     int N, int K, float* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const bf16_t* wr = W + (int64_t)n * K + lane * 8;
  u32x4 wv[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i) wv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + i * 512));
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    acc[m] = 0.f;
    const bf16_t* xr = X + (int64_t)m * K + lane * 8;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const u32x4 xv = ld16(xr + i * 512);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // element copies first: bit-casting a vector element in place picked
        // the wrong element in this compiler
        const uint32_t wu = wv[i][c], xu = xv[c];
        acc[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wu), __builtin_bit_cast(bf16x2_t, xu),
                                                 acc[m], false);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const float v = wave_sum(acc[m]);
    if (lane == 0) {
      float* o = out + (int64_t)m * ldo + n;
      if constexpr (EPI == EPI_RESADD) *o += v; else *o = v;
    }
  }
}

bool rowdot_ok(int M, int K) { return M >= 1 && M <= 4 && K % 512 == 0 && K / 512 <= 8; }

template <int EPI, int MR>
hipError_t rowdot_ks(int KS, dim3 grid, const bf16_t* X, const bf16_t* W, int N, int K, float* out, int64_t ldo,
                     hipStream_t s) {
  switch (KS) {
    case 1: rowdot_kernel<EPI, MR, 1><<<grid, 256, 0, s>>>(X, W, N, K, out, ldo); break;
    case 2: rowdot_kernel<EPI, MR, 2><<<grid, 256, 0, s>>>(X, W, N, K, out, ldo); break;
    case 4: rowdot_kernel<EPI, MR, 4><<<grid, 256, 0, s>>>(X, W, N, K, out, ldo); break;
    case 6: rowdot_kernel<EPI, MR, 6><<<grid, 256, 0, s>>>(X, W, N, K, out, ldo); break;
    case 8: rowdot_kernel<EPI, MR, 8><<<grid, 256, 0, s>>>(X, W, N, K, out, ldo); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t rowdot_m(int M, int KS, dim3 grid, const bf16_t* X, const bf16_t* W, int N, int K, float* out,
                    int64_t ldo, hipStream_t s) {
  switch (M) {
    case 1: return rowdot_ks<EPI, 1>(KS, grid, X, W, N, K, out, ldo, s);
    case 2: return rowdot_ks<EPI, 2>(KS, grid, X, W, N, K, out, ldo, s);
    case 3: return rowdot_ks<EPI, 3>(KS, grid, X, W, N, K, out, ldo, s);
    default: return rowdot_ks<EPI, 4>(KS, grid, X, W, N, K, out, ldo, s);
  }
}

hipError_t rowdot_bf16(int epi, const bf16_t* X, int M, const bf16_t* W, int N, int K, float* out, int64_t ldo,
                       hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!rowdot_ok(M, K) || (epi != EPI_STORE && epi != EPI_RESADD)) return hipErrorInvalidValue;
  const int KS = K / 512;
  if (KS != 1 && KS != 2 && KS != 4 && KS != 6 && KS != 8) return hipErrorInvalidValue;
  dim3 grid((N + 3) / 4);
  if (epi == EPI_RESADD) return rowdot_m<EPI_RESADD>(M, KS, grid, X, W, N, K, out, ldo, s);
  return rowdot_m<EPI_STORE>(M, KS, grid, X, W, N, K, out, ldo, s);
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
