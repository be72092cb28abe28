// Weight-only affine group quantization of the block projections: codes of 8
// or 4 bits with a float16 scale and offset per group of 64 consecutive
// weights of a row (w ~ q * s + b), the quantizer, the dequantizer and the
// single-row decode GEMV that reads the codes directly.
//
// Method source: "Investigación de rendimiento de Laya MLX", its
// quantization section (affine, grouped by 64, 8 or 4 bits, fp16 scales and
// offsets, weight-only matrix products); "Dentro de un LLM: Inferencia en
// Python puro para Qwen3-0.6B en MLX", Pasos 3, 5, 6, 7 for the projections
// themselves.
//
// Layout of a quantized [N, K] matrix: codes [N][K * bits / 8] bytes (4-bit:
// byte j holds k = 2j in its low nibble, 2j + 1 in its high nibble); scales
// and offsets [N][K / 64] as 32-bit words, the scale's float16 bits low, the
// offset's high.
#include "kernels.h"

namespace q3k {

namespace {

constexpr int kGroup = 64;

typedef __bf16 bf16x2_q __attribute__((ext_vector_type(2)));

Q3_DEV float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
// Two floats -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32;
// the dequantizer and the GEMV on codes both round this way).
Q3_DEV uint32_t pack_bf2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2_q));
}
Q3_DEV float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// One thread per (row, group).  Destination row: dst_row0 + r, or for the
// gate/up interleave (runs of 16 rows, [gate 16 | up 16]) (r/16)*32 + r%16 +
// 16*up.  Codes and the float16 scale and offset follow one fixed sequence of
// float32 steps: b = fp16(min), s = fp16((max - min) / (2^bits - 1)), q =
// clamp(floor((w - b) / s + 0.5)), q = 0 when s is 0.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const bf16_t* __restrict__ src, int rows, int K,
                                                       uint8_t* __restrict__ codes, uint32_t* __restrict__ sb,
                                                       int dst_row0, int interleave, int up) {
  const int groups = K / kGroup;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rows * groups) return;
  const int r = (int)(t / groups), g = (int)(t - (int64_t)r * groups);
  const bf16_t* w = src + (int64_t)r * K + g * kGroup;
  float v[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup / 8; ++i) {
    const u32x4 u = ld16(w + 8 * i);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[8 * i + 2 * c] = __uint_as_float(u[c] << 16);
      v[8 * i + 2 * c + 1] = __uint_as_float(u[c] & 0xffff0000u);
    }
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < kGroup; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  constexpr float levels = (float)((1 << BITS) - 1);
  const _Float16 s16 = (_Float16)((mx - mn) / levels);
  const _Float16 b16 = (_Float16)mn;
  const float s = (float)s16, b = (float)b16;
  const int dr = interleave ? (r >> 4) * 32 + (r & 15) + 16 * up : dst_row0 + r;
  uint8_t q[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    float f = s == 0.f ? 0.f : floorf((v[i] - b) / s + 0.5f);
    f = fminf(fmaxf(f, 0.f), levels);
    q[i] = (uint8_t)f;
  }
  uint8_t* dst = codes + (int64_t)dr * (K * BITS / 8) + g * (kGroup * BITS / 8);
  if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < kGroup / 16; ++i) {
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        o[c] = (uint32_t)q[16 * i + 4 * c] | ((uint32_t)q[16 * i + 4 * c + 1] << 8) |
               ((uint32_t)q[16 * i + 4 * c + 2] << 16) | ((uint32_t)q[16 * i + 4 * c + 3] << 24);
      reinterpret_cast<u32x4*>(dst)[i] = o;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kGroup / 32; ++i) {
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t word = 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) word |= (uint32_t)q[32 * i + 8 * c + n] << (4 * n);
        o[c] = word;
      }
      reinterpret_cast<u32x4*>(dst)[i] = o;
    }
  }
  sb[(int64_t)dr * groups + g] = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
                                 ((uint32_t)__builtin_bit_cast(uint16_t, b16) << 16);
}

// bf16(q * s + b): thread per 8 consecutive weights.
template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint32_t* __restrict__ sb, int N, int K,
                                                      bf16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = K / 8;
  if (t >= (int64_t)N * per_row) return;
  const int r = (int)(t / per_row), k0 = (int)(t - (int64_t)r * per_row) * 8;
  const uint32_t w = sb[(int64_t)r * (K / kGroup) + k0 / kGroup];
  const float s = half_lo(w), b = half_hi(w);
  uint32_t q[8];
  if constexpr (BITS == 8) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(codes + (int64_t)r * K + k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (c[i >> 2] >> (8 * (i & 3))) & 0xffu;
  } else {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + (int64_t)r * (K / 2) + k0 / 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (c >> (4 * i)) & 0xfu;
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf2_rne(fmaf((float)q[2 * i], s, b), fmaf((float)q[2 * i + 1], s, b));
  *reinterpret_cast<u32x4*>(out + (int64_t)r * K + k0) = o;
}

Q3_DEV float silu_q(float g) { return g / (1.f + __expf(-g)); }

// One activation row against a quantized W[N,K].  A wavefront owns RW rows;
// lane l covers k = 16 l + 1024 i (i < KS, K = 1024 KS): 16 codes per load (16
// bytes at 8 bits, 8 bytes at 4 bits) and the scale/offset word of their
// group.  Each weight enters the product as the bf16 value bf16(q * s + b),
// the same value the dequantizer writes, so this kernel and the bf16 kernels
// run on the dequantized copy compute with identical weights; pairs of
// weights and activations go through v_dot2_f32_bf16 with fp32 sums, and a
// butterfly over the lanes finishes the row.
// NORM: the activation is bf16(rmsnorm(x) * g) from the float32 residual x,
// rounded where the standalone RMSNorm rounds.
template <int EPI, int BITS, int KS, int RW, bool NORM>
__global__ __launch_bounds__(256) void qrowgemv_kernel(const void* __restrict__ Xin,
                                                       const uint8_t* __restrict__ codes,
                                                       const uint32_t* __restrict__ sbw, int N, int K,
                                                       const float* __restrict__ gnorm, float eps,
                                                       void* __restrict__ out) {
  static_assert(EPI != EPI_SWIGLU || RW % 2 == 0, "SwiGLU pairs a gate row with its up row");
  constexpr int CB = 16 * BITS / 8;  // code bytes per lane and load
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wg = blockIdx.x * (blockDim.x >> 6) + wid;
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
  // activations first (as bf16 pairs), then the code and scale stream
  uint32_t ap[KS][8];
  float4 xf[NORM ? KS : 1][4], gf[NORM ? KS : 1][4];
#pragma unroll
  for (int i = 0; i < KS; ++i) {
    const int k0 = 16 * lane + 1024 * i;
    if constexpr (NORM) {
      const float* x = reinterpret_cast<const float*>(Xin);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        xf[i][c] = *reinterpret_cast<const float4*>(x + k0 + 4 * c);
        gf[i][c] = *reinterpret_cast<const float4*>(gnorm + k0 + 4 * c);
      }
    } else {
      const bf16_t* x = reinterpret_cast<const bf16_t*>(Xin);
      const u32x4 lo = ld16(x + k0), hi = ld16(x + k0 + 8);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ap[i][c] = lo[c];
        ap[i][4 + c] = hi[c];
      }
    }
  }
  uint32_t cw[RW][KS][CB / 4];
  uint32_t sw[RW][KS];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = rows[r] < N ? rows[r] : 0;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int k0 = 16 * lane + 1024 * i;
      const uint8_t* p = codes + (int64_t)row * (K * BITS / 8) + k0 * BITS / 8;
      if constexpr (BITS == 8) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
        for (int c = 0; c < 4; ++c) cw[r][i][c] = v[c];
      } else {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        cw[r][i][0] = v[0];
        cw[r][i][1] = v[1];
      }
      sw[r][i] = sbw[(int64_t)row * (K / kGroup) + k0 / kGroup];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = xf[i][c];
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    ss = wave_sum(ss);
    const float inv = rsqrtf(ss / (float)K + eps);
#pragma unroll
    for (int i = 0; i < KS; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = xf[i][c], g = gf[i][c];
        ap[i][2 * c] = pack_bf2(v.x * inv * g.x, v.y * inv * g.y);
        ap[i][2 * c + 1] = pack_bf2(v.z * inv * g.z, v.w * inv * g.w);
      }
  }

  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const uint32_t sbr = sw[r][i];
      const float s = half_lo(sbr), b = half_hi(sbr);
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        uint32_t q0, q1;
        if constexpr (BITS == 8) {
          q0 = (cw[r][i][j >> 2] >> (8 * (j & 3))) & 0xffu;
          q1 = (cw[r][i][j >> 2] >> (8 * ((j + 1) & 3))) & 0xffu;
        } else {
          q0 = (cw[r][i][j >> 3] >> (4 * (j & 7))) & 0xfu;
          q1 = (cw[r][i][j >> 3] >> (4 * ((j + 1) & 7))) & 0xfu;
        }
        const uint32_t wpair = pack_bf2_rne(fmaf((float)q0, s, b), fmaf((float)q1, s, b));
        const uint32_t apair = ap[i][j >> 1];
        acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_q, wpair),
                                                 __builtin_bit_cast(bf16x2_q, apair), acc[r], false);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = wave_sum(acc[r]);

  if constexpr (EPI == EPI_SWIGLU) {
    bf16_t* o = reinterpret_cast<bf16_t*>(out);
#pragma unroll
    for (int j = 0; j < RW / 2; ++j) {
      const int c = wg * (RW / 2) + j;
      if (lane == j && 2 * c < N) o[c] = f2bf(silu_q(acc[2 * j]) * acc[2 * j + 1]);
    }
  } else {
    float* o = reinterpret_cast<float*>(out);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (lane == r && rows[r] < N) {
        if constexpr (EPI == EPI_RESADD)
          o[rows[r]] += acc[r];
        else
          o[rows[r]] = acc[r];
      }
    }
  }
}

template <int EPI, int BITS, int KS, bool NORM>
hipError_t launch_q(int rw, dim3 grid, dim3 block, const void* X, const uint8_t* C, const uint32_t* S, int N, int K,
                    const float* g, float eps, void* out, hipStream_t s) {
  switch (rw) {
    case 1:
      if constexpr (EPI == EPI_SWIGLU) return hipErrorInvalidValue;  // gate and up rows come in pairs
      else qrowgemv_kernel<EPI, BITS, KS, 1, NORM><<<grid, block, 0, s>>>(X, C, S, N, K, g, eps, out);
      break;
    case 2: qrowgemv_kernel<EPI, BITS, KS, 2, NORM><<<grid, block, 0, s>>>(X, C, S, N, K, g, eps, out); break;
    case 4: qrowgemv_kernel<EPI, BITS, KS, 4, NORM><<<grid, block, 0, s>>>(X, C, S, N, K, g, eps, out); break;
    case 8: qrowgemv_kernel<EPI, BITS, KS, 8, NORM><<<grid, block, 0, s>>>(X, C, S, N, K, g, eps, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI, int BITS, bool NORM>
hipError_t launch_qks(int KS, int rw, dim3 grid, dim3 block, const void* X, const uint8_t* C, const uint32_t* S,
                      int N, int K, const float* g, float eps, void* out, hipStream_t s) {
  switch (KS) {
    case 1: return launch_q<EPI, BITS, 1, NORM>(rw, grid, block, X, C, S, N, K, g, eps, out, s);
    case 2: return launch_q<EPI, BITS, 2, NORM>(rw, grid, block, X, C, S, N, K, g, eps, out, s);
    case 3: return launch_q<EPI, BITS, 3, NORM>(rw, grid, block, X, C, S, N, K, g, eps, out, s);
    case 4: return launch_q<EPI, BITS, 4, NORM>(rw, grid, block, X, C, S, N, K, g, eps, out, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t qrowgemv_bits(int epi, const void* X, const uint8_t* C, const uint32_t* S, int N, int K,
                         const float* gnorm, float eps, void* out, hipStream_t s) {
  const int KS = K / 1024;
  // Dequantizing costs about three VALU operations per weight, so the rows
  // are spread thin for many wavefronts and SIMDs; with the RMSNorm prologue
  // every wavefront also reads the whole activation and norm rows (8 KiB at
  // K = 1024), so there four rows share that read.
  const bool norm_in = gnorm != nullptr;
  const int rw = norm_in ? 4 : 2;
  const int64_t nwaves = ((int64_t)N + rw - 1) / rw;
  int waves = 4;
  while (waves > 1 && (nwaves + waves - 1) / waves < 256) waves >>= 1;
  dim3 grid((unsigned)((nwaves + waves - 1) / waves)), block(64 * waves);
  const bool norm = norm_in;
  switch (epi) {
    case EPI_STORE:
      return norm ? launch_qks<EPI_STORE, BITS, true>(KS, rw, grid, block, X, C, S, N, K, gnorm, eps, out, s)
                  : launch_qks<EPI_STORE, BITS, false>(KS, rw, grid, block, X, C, S, N, K, nullptr, eps, out, s);
    case EPI_SWIGLU:
      return norm ? launch_qks<EPI_SWIGLU, BITS, true>(KS, rw, grid, block, X, C, S, N, K, gnorm, eps, out, s)
                  : launch_qks<EPI_SWIGLU, BITS, false>(KS, rw, grid, block, X, C, S, N, K, nullptr, eps, out, s);
    case EPI_RESADD:
      if (norm) return hipErrorInvalidValue;
      return launch_qks<EPI_RESADD, BITS, false>(KS, rw, grid, block, X, C, S, N, K, nullptr, eps, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t quant_code_bytes(int rows, int K, int bits) { return (size_t)rows * K * bits / 8; }
size_t quant_sb_bytes(int rows, int K) { return (size_t)rows * (K / kGroup) * 4; }

hipError_t quantize_rows(const bf16_t* src, int rows, int K, int bits, uint8_t* codes, uint32_t* sb, int dst_row0,
                         int interleave, int up, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K % kGroup != 0 || (bits != 8 && bits != 4)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * (K / kGroup);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bits == 8)
    quantize_kernel<8><<<grid, 256, 0, s>>>(src, rows, K, codes, sb, dst_row0, interleave, up);
  else
    quantize_kernel<4><<<grid, 256, 0, s>>>(src, rows, K, codes, sb, dst_row0, interleave, up);
  return hipGetLastError();
}

hipError_t dequant_rows(const uint8_t* codes, const uint32_t* sb, int N, int K, int bits, bf16_t* out, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (K % kGroup != 0 || (bits != 8 && bits != 4)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)N * (K / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bits == 8)
    dequant_kernel<8><<<grid, 256, 0, s>>>(codes, sb, N, K, out);
  else
    dequant_kernel<4><<<grid, 256, 0, s>>>(codes, sb, N, K, out);
  return hipGetLastError();
}

bool qrowgemv_ok(int K) {
  if (K % 1024 != 0) return false;
  const int ks = K / 1024;
  return ks >= 1 && ks <= 4;
}

hipError_t qrowgemv(int epi, int bits, const void* X, const uint8_t* codes, const uint32_t* sb, int N, int K,
                    const float* gnorm, float eps, void* out, hipStream_t s) {
  if (!qrowgemv_ok(K) || N <= 0) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && N % 32 != 0) return hipErrorInvalidValue;
  if (bits == 8) return qrowgemv_bits<8>(epi, X, codes, sb, N, K, gnorm, eps, out, s);
  if (bits == 4) return qrowgemv_bits<4>(epi, X, codes, sb, N, K, gnorm, eps, out, s);
  return hipErrorInvalidValue;
}

}  // namespace q3k
