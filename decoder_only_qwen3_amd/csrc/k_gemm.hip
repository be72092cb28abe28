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
// Tiling: block tile (16*WM*GM) x (16*WN*GN); GM x GN wavefronts, each owning
// a (16*WM) x (16*WN) sub-tile as 16x16 MFMA tiles.  Two K loops:
//  - register-prefetched (K step 64): the next step's global loads go to
//    registers while the MFMAs use the LDS copy of the current one;
//  - LDS pipeline (32-wide K slices, 4 slices in LDS, loaded directly from
//    global memory into LDS): three slices in flight behind the one in use.
// Large problems use 256x256 tiles on 16 wavefronts with the pipeline,
// small ones 64x64 tiles on 4 wavefronts.  The products run as C^T = W . A^T
// so that each lane writes four consecutive outputs (one 16-byte store).
#include <cstring>

#include "kernels.h"

namespace q3k {

namespace {
constexpr int BK = 64;

// LDS row layout of a 64-wide K slice: SW = 0 pads each row by 16 bytes;
// SW = 1 / 2 store it unpadded with the 16-byte chunk index XORed with
// (row & 7) / ((row >> 1) & 7).  Counters on MI355X: the padded layout has
// about 0.6 bank conflicts per LDS access in this kernel, both XOR layouts
// none (the kernels use SW = 1).
template <int SW>
Q3_DEV int lds_off(int row, int col) {
  if constexpr (SW == 0) return row * (BK + 8) + col;
  const int x = SW == 1 ? (row & 7) : ((row >> 1) & 7);
  return row * BK + ((((col >> 3) ^ x) << 3) | (col & 7));
}

Q3_DEV float silu_f(float g) { return g / (1.f + __expf(-g)); }

// The products run as C^T = W . A^T (the W fragment is the MFMA's A operand),
// so in a 16x16 tile lane l holds output row l%16 and the four consecutive
// output columns (l/16)*4 + r: one 16-byte store per lane and tile (8 bytes
// for the bf16 SwiGLU output).  acc[i][j] covers A rows i*16.. and W rows j*16..
// of the wavefront's tile; (r0, c0) = its first output row and column.
template <int EPI, int WM, int WN>
Q3_DEV void gemm_epilogue(const f32x4 (&acc)[WM][WN], int r0, int c0, int M, int N, void* __restrict__ out,
                          int64_t ldo) {
  const int lane = threadIdx.x & 63;
  const int row0 = r0 + (lane & 15);
  const int cq = (lane >> 4) * 4;
  if constexpr (EPI == EPI_SWIGLU) {
    // Packed rows: every 32 rows of W are 16 gate rows then the matching 16 up
    // rows, so tile j=2p is gate and j=2p+1 is up for the same output columns.
    bf16_t* o = reinterpret_cast<bf16_t*>(out);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int row = row0 + i * 16;
      if (row >= M) continue;
#pragma unroll
      for (int p = 0; p < WN / 2; ++p) {
        const int col = c0 / 2 + p * 16 + cq;
        if (2 * col >= N) continue;
        const f32x4 g = acc[i][2 * p], u = acc[i][2 * p + 1];
        u32x2 w;
        w[0] = pack_bf2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
        w[1] = pack_bf2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
        *reinterpret_cast<u32x2*>(o + (int64_t)row * ldo + col) = w;
      }
    }
  } else {
    float* o = reinterpret_cast<float*>(out);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int row = row0 + i * 16;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int col = c0 + j * 16 + cq;
        if (col >= N) continue;
        f32x4* p = reinterpret_cast<f32x4*>(o + (int64_t)row * ldo + col);
        if constexpr (EPI == EPI_RESADD)
          *p = *p + acc[i][j];
        else
          *p = acc[i][j];
      }
    }
  }
}

// Block tile (16*WM*GM) x (16*WN*GN): GM x GN wavefronts, each owning a
// (16*WM) x (16*WN) sub-tile of 16x16 MFMA tiles.
//
// Split K (EPI_RESADD, gridDim.z > 1): block z accumulates the K slice z, publishes
// its partial tile with agent-scope stores (coherent across the L2 slices),
// and the last slice to finish a tile adds the partials in slice order
// (deterministic) into the residual.  Small grids (M = 512 prefill) get four
// times the blocks and a quarter of the dependent K steps.
constexpr int kGemmMaxSplit = 4;

template <int EPI, int WM, int WN, int GM, int GN, int SW>
__global__ __launch_bounds__(64 * GM * GN) void gemm_bf16_kernel(const bf16_t* __restrict__ A, int M,
                                                                const bf16_t* __restrict__ W, int N, int K,
                                                                void* __restrict__ out, int64_t ldo,
                                                                float* __restrict__ part,
                                                                uint32_t* __restrict__ cnt) {
  constexpr int NT = 64 * GM * GN;
  constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN;
  constexpr int RSTEP = NT / 8;                      // rows covered by one pass of 16-byte loads
  constexpr int LA = BM / RSTEP, LW = BN / RSTEP;    // 16-byte chunks per thread per K step
  static_assert(BM % RSTEP == 0 && BN % RSTEP == 0, "tile rows must be a multiple of the load pass");
  constexpr int LDK = SW == 0 ? BK + 8 : BK;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sW[2][BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / GN, wn = wid % GN;
  const int bn0 = blockIdx.x * BN, bm0 = blockIdx.y * BM;
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;
  const int nsplit = gridDim.z, ksl = K / nsplit;
  A += (int64_t)blockIdx.z * ksl;  // this block's K slice (rows keep stride K)
  W += (int64_t)blockIdx.z * ksl;

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
    for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(&sA[buf][lds_off<SW>(lrow + RSTEP * i, lcol)]) = ra[i];
#pragma unroll
    for (int i = 0; i < LW; ++i) *reinterpret_cast<u32x4*>(&sW[buf][lds_off<SW>(lrow + RSTEP * i, lcol)]) = rw[i];
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = ksl / BK;
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
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][lds_off<SW>(wm * 16 * WM + i * 16 + fr, ks * 32 + fk)]);
#pragma unroll
      for (int j = 0; j < WN; ++j)
        bw[j] = *reinterpret_cast<const bf16x8*>(&sW[buf][lds_off<SW>(wn * 16 * WN + j * 16 + fr, ks * 32 + fk)]);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma16(bw[j], af[i], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  if constexpr (EPI == EPI_RESADD) {
    if (nsplit > 1) {
      // partial tile of slice z: float4 v of thread t at ((tile*nsplit + z)*NA + v)*NT + t,
      // so one store instruction covers a contiguous kilobyte
      constexpr int NA = WM * WN;
      const int tile = blockIdx.y * gridDim.x + blockIdx.x;
      const auto rs = agent_rsrc(part, (uint32_t)gridDim.x * gridDim.y * nsplit * NA * NT * 16);
      const uint32_t tbase = ((uint32_t)tile * nsplit * NA * NT + tid) * 16;
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          st4_agent(rs, tbase + ((blockIdx.z * NA + i * WN + j) * NT) * 16, acc[i][j]);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      __shared__ int last;
      if (tid == 0)
        last = __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)(nsplit - 1);
      __syncthreads();
      if (!last) return;
      // all slices' partials (this block's own reads back what it stored), loaded
      // together and summed in slice order; slices past nsplit re-read the last
      // one and add nothing
      f32x4 pz[kGemmMaxSplit][WM][WN];
#pragma unroll
      for (int z = 0; z < kGemmMaxSplit; ++z)
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            pz[z][i][j] = ld4_agent(rs, tbase + ((min(z, nsplit - 1) * NA + i * WN + j) * NT) * 16);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int z = 0; z < kGemmMaxSplit; ++z) t += z < nsplit ? pz[z][i][j] : f32x4{0.f, 0.f, 0.f, 0.f};
          acc[i][j] = t;
        }
      if (tid == 0) __hip_atomic_store(cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  gemm_epilogue<EPI, WM, WN>(acc, bm0 + wm * 16 * WM, bn0 + wn * 16 * WN, M, N, out, ldo);
}

template <int WM, int WN, int GM, int GN, int SW>
hipError_t gemm_launch(int epi, const bf16_t* A, int M, const bf16_t* W, int N, int K, void* out, int64_t ldo,
                       hipStream_t s, float* part = nullptr, uint32_t* cnt = nullptr, int nsplit = 1) {
  constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN, NT = 64 * GM * GN;
  if (nsplit > 1 && (epi != EPI_RESADD || !part || !cnt || nsplit > kGemmMaxSplit || K % (nsplit * BK) != 0))
    return hipErrorInvalidValue;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, nsplit);
  switch (epi) {
    case EPI_STORE:
    case EPI_ARGMAX:
      gemm_bf16_kernel<EPI_STORE, WM, WN, GM, GN, SW><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo, part, cnt);
      break;
    case EPI_RESADD:
      gemm_bf16_kernel<EPI_RESADD, WM, WN, GM, GN, SW><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo, part, cnt);
      break;
    case EPI_SWIGLU:
      gemm_bf16_kernel<EPI_SWIGLU, WM, WN, GM, GN, SW><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo, part, cnt);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- pipelined variant
// Same tiling, but the K loop is an NS-stage pipeline of 32-wide K slices
// loaded straight from global memory into LDS (global_load_lds_dwordx4, no
// register staging): while the MFMAs work on slice kt, slices kt+1 ..
// kt+NS-1 are in flight, which covers the L2/MALL latency that a single
// register-prefetched step does not.  One block barrier per slice.
//
// LDS: each load instruction of a wavefront fills 1 KiB = 16 rows x 64 bytes
// (lane i -> row i/4, 16-byte chunk i%4).  Chunks are stored XOR-swizzled by
// (row >> 1) & 3, so the MFMA fragment reads (16 rows, one chunk) spread
// over the LDS banks; the lane loads the global chunk that belongs at its
// fixed LDS position.
constexpr int DBK = 32;

Q3_DEV int dswz(int row) { return (row >> 1) & 3; }

// Blocks are dealt to the eight XCDs round robin (block b runs on XCD b % 8),
// each XCD with an L2 of its own.  Tile t of the TM x TN output grid goes to
// the block that makes every XCD work through one contiguous run of tiles,
// taken in groups of kGroupM tile rows with the tile columns outer, so the
// blocks an XCD runs together share A and W tiles in its L2 instead of every
// XCD fetching every A tile.
constexpr int kGroupM = 4;
Q3_DEV void xcd_tile(int TM, int TN, int& tm, int& tn) {
  const int T = TM * TN, b = blockIdx.x;
  const int x = b & 7, slot = b >> 3;
  const int per = T >> 3, extra = T & 7;  // XCD x runs per + (x < extra) tiles
  const int t = x * per + min(x, extra) + slot;
  const int g = t / (kGroupM * TN), r = t - g * (kGroupM * TN);
  const int rows = min(kGroupM, TM - g * kGroupM);
  tm = g * kGroupM + r % rows;
  tn = r / rows;
}

// Epilogue of the fused prefill q/k/v projection (gemm_qkv_rope), beside the
// public EPI_* values.
constexpr int EPI_QKROPE = 16;
constexpr int kRopeStageStride = 256 + 4;  // floats per staged row (padded against LDS bank conflicts)

template <int EPI, int WM, int WN, int GM, int GN, int NS, bool DB>
__global__ __launch_bounds__(64 * GM * GN) void gemm_dma_kernel(const bf16_t* __restrict__ A, int M,
                                                               const bf16_t* __restrict__ W, int N, int K,
                                                               void* __restrict__ out, int64_t ldo,
                                                               QkvRopeArgs ra) {
  constexpr int NW = GM * GN;
  constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN;
  constexpr int GA = BM / 16, GB = BN / 16;  // 1 KiB load groups per slice
  static_assert((GA + GB) % NW == 0, "load groups must split evenly over the wavefronts");
  constexpr int LPW = (GA + GB) / NW;        // load instructions per wavefront per slice
  constexpr int STAGE = (BM + BN) * DBK;     // bf16 elements per slice
  // the fused epilogue stages 128 rows of float32 outputs in the same LDS
  constexpr int LDS_N = (EPI == EPI_QKROPE && 128 * kRopeStageStride * 2 > NS * STAGE) ? 128 * kRopeStageStride * 2
                                                                                       : NS * STAGE;
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_N];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / GN, wn = wid % GN;
  int tm, tn;
  xcd_tile((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int bn0 = tn * BN, bm0 = tm * BM;

  // This lane's source pointer and its wavefront's LDS offset per load group.
  const bf16_t* src[LPW];
  int dst[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int g = wid * LPW + u;
    const int rr = lane >> 2, sc = lane & 3;
    if (g < GA) {
      const int row = g * 16 + rr;
      src[u] = A + (int64_t)min(bm0 + row, M - 1) * K + ((sc ^ dswz(row)) << 3);
      dst[u] = g * 16 * DBK;
    } else {
      const int row = (g - GA) * 16 + rr;
      src[u] = W + (int64_t)min(bn0 + row, N - 1) * K + ((sc ^ dswz(row)) << 3);
      dst[u] = BM * DBK + (g - GA) * 16 * DBK;
    }
  }
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int u = 0; u < LPW; ++u)  // (non-const pointers: with a const source the host pass drops the kernel stub)
      __builtin_amdgcn_global_load_lds((void*)(src[u] + kt * DBK), (void*)(lds + buf * STAGE + dst[u]), 16, 0, 0);
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / DBK;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st, st);
  const int fr = lane & 15, fq = lane >> 4;
  auto read_frags = [&](int kt, bf16x8 (&af)[WM], bf16x8 (&bw)[WN]) {
    const bf16_t* sa = lds + (kt % NS) * STAGE;
    const bf16_t* sb = sa + BM * DBK;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int row = wm * 16 * WM + i * 16 + fr;
      af[i] = *reinterpret_cast<const bf16x8*>(sa + row * DBK + ((fq ^ dswz(row)) << 3));
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int row = wn * 16 * WN + j * 16 + fr;
      bw[j] = *reinterpret_cast<const bf16x8*>(sb + row * DBK + ((fq ^ dswz(row)) << 3));
    }
  };
  if constexpr (!DB) {
    for (int kt = 0; kt < nk; ++kt) {
      // slice kt is complete once at most the later slices' loads are pending
      if (kt + NS - 2 < nk) wait_vm<(NS - 2) * LPW>();
      else wait_vm<0>();
      bare_barrier();
      if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
      bf16x8 af[WM], bw[WN];
      read_frags(kt, af, bw);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma16(bw[j], af[i], acc[i][j]);
    }
  } else {
    // Slice 0 complete once at most slices 1 .. NS-2 are pending.
    if (NS - 2 < nk) wait_vm<(NS - 2) * LPW>();
    else wait_vm<0>();
    bare_barrier();
    // Step kt: the MFMAs of slice kt run on fragments read during step kt-1,
    // while the fragments of slice kt+1 are read.  Before the reads, slice kt+1
    // must be complete (at most slices kt+2 .. kt+NS-2 pending) and every
    // wavefront past step kt-1, so the load of slice kt+NS-1 may reuse the
    // buffer of slice kt-1.  (A bare barrier: __syncthreads() would also wait
    // for every load in flight, emptying the pipeline.)
    auto step = [&](int kt, const bf16x8 (&af)[WM], const bf16x8 (&bw)[WN], bf16x8 (&an)[WM], bf16x8 (&bn)[WN]) {
      if (kt + 1 < nk) {
        if (kt + NS - 2 < nk) wait_vm<(NS - 3) * LPW>();
        else wait_vm<0>();
        bare_barrier();
        if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
        read_frags(kt + 1, an, bn);
      }
  #pragma unroll
      for (int i = 0; i < WM; ++i)
  #pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma16(bw[j], af[i], acc[i][j]);
    };
    bf16x8 a0[WM], b0[WN], a1[WM], b1[WN];
    read_frags(0, a0, b0);
    for (int kt = 0;;) {  // unrolled by two so the fragment buffers swap roles
      step(kt, a0, b0, a1, b1);
      if (++kt >= nk) break;
      step(kt, a1, b1, a0, b0);
      if (++kt >= nk) break;
    }
  }
  if constexpr (EPI == EPI_QKROPE) {
    // Pasos 4-5 per token on the tile's two heads (columns bn0 .. bn0 + 255),
    // 128 rows at a time: the float32 outputs are staged in LDS (padded rows),
    // then 16 lanes take one (token, head): a query or key head is normalised,
    // rotated and stored by the same function as rope_append, a value head is
    // rounded to bf16 for the value pass.
    static_assert(BM == 256 && BN == 256 && WM == 4 && WN == 4 && !DB, "written for the 256 x 256 tiles");
    wait_vm<0>();
    __syncthreads();  // every wavefront is done with the pipeline's LDS
    float* stg = reinterpret_cast<float*>(lds);
    constexpr int SP = kRopeStageStride;
    const int units = ra.n_q + 2 * ra.n_kv;
    const int unit0 = bn0 / Q3_HEAD_DIM;
    const KvGeom geo{ra.n_kv, ra.layer};
    const int j16 = threadIdx.x & 15;
    // Thread: head hl of the tile's two, tokens tl0 + 32 p (p = 0..3) of each
    // 128-token half.  The sequence of each token is found by walking the
    // sequence starts inside the half from the sequence of the tile's first
    // token; every load of that walk has a wave-uniform address (scalar
    // loads), so a pass waits on two memory round trips (slot state, then the
    // rope rows) instead of a per-lane binary search before them.
    const int hl = (threadIdx.x >> 4) & 1, tl0 = threadIdx.x >> 5;
    const int u = unit0 + hl;
    const int b0 = seq_of_token(ra.sb, min(bm0, M - 1));
    for (int half = 0; half < 2; ++half) {
      if ((wm >> 1) == half) {
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const int tl = (wm & 1) * 64 + i * 16 + (lane & 15);
            const int col = wn * 64 + j * 16 + (lane >> 4) * 4;
            *reinterpret_cast<f32x4*>(&stg[tl * SP + col]) = acc[i][j];
          }
      }
      __syncthreads();
      const int h0 = bm0 + half * 128;  // the half's first token
      if (h0 >= M) break;
      static_assert(64 * NW == 1024, "32 token rows per pass");
      for (int p = 0; p < 4; ++p) {
        const int tl = tl0 + 32 * p;
        const int t = h0 + tl;
        if (t >= M || u >= units) continue;  // uniform over the 16 lanes
        const float4 x = *reinterpret_cast<const float4*>(&stg[tl * SP + hl * Q3_HEAD_DIM + 4 * j16]);
        const float4 y = *reinterpret_cast<const float4*>(&stg[tl * SP + hl * Q3_HEAD_DIM + 64 + 4 * j16]);
        if (u >= ra.n_q + ra.n_kv) {
          bf16_t* dst = ra.v_out + ((int64_t)t * ra.n_kv + (u - ra.n_q - ra.n_kv)) * Q3_HEAD_DIM;
          store4<bf16_t>(dst + 4 * j16, x.x, x.y, x.z, x.w);
          store4<bf16_t>(dst + 64 + 4 * j16, y.x, y.y, y.z, y.w);
          continue;
        }
        int slot = ra.sb.slot[b0], cub = ra.sb.cu[b0], prb = ra.sb.prior[b0];
        for (int nb = b0 + 1; nb < ra.sb.n; ++nb) {
          const int c = ra.sb.cu[nb];
          if (c > h0 + 127) break;  // starts after the half
          if (t >= c) {
            slot = ra.sb.slot[nb];
            cub = c;
            prb = ra.sb.prior[nb];
          }
        }
        const SeqState sst = ra.st[slot];
        const int pos = prb + t - cub;
        if (pos < 0 || pos >= sst.cap) {  // host validation makes this unreachable
          if (j16 == 0) atomicOr(ra.err, 4u);
          continue;
        }
        bf16_t *lo, *hi;
        if (u < ra.n_q) {
          bf16_t* row = ra.q_out + ((int64_t)t * ra.n_q + u) * Q3_HEAD_DIM;
          lo = row + 4 * j16;
          hi = row + 64 + 4 * j16;
        } else {
          bf16_t* kh = kv_k(ra.kv, sst, geo, u - ra.n_q);
          lo = kh + kk_off<bf16_t>(pos, 4 * j16);
          hi = kh + kk_off<bf16_t>(pos, 64 + 4 * j16);
        }
        qk_norm_rope_store<bf16_t>(x, y, u < ra.n_q ? ra.qn : ra.kn, ra.eps, ra.cos_t, ra.sin_t, pos, j16, lo, hi);
      }
      __syncthreads();  // the staging is rewritten by the next half
    }
  } else {
    gemm_epilogue<EPI, WM, WN>(acc, bm0 + wm * 16 * WM, bn0 + wn * 16 * WN, M, N, out, ldo);
  }
}

template <int WM, int WN, int GM, int GN, int NS, bool DB>
hipError_t gemm_dma_launch(int epi, const bf16_t* A, int M, const bf16_t* W, int N, int K, void* out, int64_t ldo,
                           hipStream_t s) {
  constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN, NT = 64 * GM * GN;
  if (K % DBK != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)(((N + BN - 1) / BN) * ((M + BM - 1) / BM)));
  QkvRopeArgs none;
  std::memset(&none, 0, sizeof(none));
  switch (epi) {
    case EPI_STORE:
    case EPI_ARGMAX:
      gemm_dma_kernel<EPI_STORE, WM, WN, GM, GN, NS, DB><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo, none);
      break;
    case EPI_RESADD:
      gemm_dma_kernel<EPI_RESADD, WM, WN, GM, GN, NS, DB><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo, none);
      break;
    case EPI_SWIGLU:
      gemm_dma_kernel<EPI_SWIGLU, WM, WN, GM, GN, NS, DB><<<grid, NT, 0, s>>>(A, M, W, N, K, out, ldo, none);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int g_gemm_cfg = -1;  // tile configuration override (q3op_tune); -1 = automatic
int g_qkv_rope = -1;  // fused q/k/v epilogue: -1 automatic, 0 never

// The automatic tile configuration (see gemm_bf16).
int auto_config(int M, int N) {
  const int64_t g256 = (int64_t)((N + 255) / 256) * ((M + 255) / 256);
  const int64_t g128 = (int64_t)((N + 127) / 128) * ((M + 127) / 128);
  return g256 >= 256 ? 7 : (g128 >= 256 ? 8 : 0);
}
}  // namespace

void gemm_set_config(int cfg) { g_gemm_cfg = cfg; }
void gemm_set_qkv_rope(int mode) { g_qkv_rope = mode; }

// Fused only where the unfused call would run the 256 x 256 pipeline (large
// prefills), so both paths multiply in the same order.
bool gemm_qkv_rope_ok(int M, int N, int K) {
  if (g_qkv_rope == 0 || M <= 0 || N % 256 != 0 || K % BK != 0) return false;
  const int cfg = g_gemm_cfg >= 0 ? g_gemm_cfg : auto_config(M, N);
  return cfg == 7;
}

hipError_t gemm_qkv_rope(const bf16_t* A, int M, const bf16_t* W, int N, int K, const QkvRopeArgs& ra,
                         hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!gemm_qkv_rope_ok(M, N, K) || N != (ra.n_q + 2 * ra.n_kv) * Q3_HEAD_DIM || !ra.q_out || !ra.v_out ||
      !ra.kv || !ra.st || ra.sb.decode)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((N + 255) / 256) * ((M + 255) / 256)));
  gemm_dma_kernel<EPI_QKROPE, 4, 4, 4, 4, 4, false><<<grid, 1024, 0, s>>>(A, M, W, N, K, nullptr, 0, ra);
  return hipGetLastError();
}

int gemm_splits(int epi, int M, int N, int K) {
  // residual GEMMs whose 64 x 64 grid leaves CUs idle: up to 4 K slices of at
  // least 512 (8 K steps), at most 1024 blocks
  if (epi != EPI_RESADD) return 1;
  const int64_t tiles = (int64_t)((N + 63) / 64) * ((M + 63) / 64);
  if (tiles >= 256) return 1;
  for (int sp = kGemmMaxSplit; sp >= 2; sp >>= 1)
    if (K % (sp * BK) == 0 && K / sp >= 512 && tiles * sp <= 1024) return sp;
  return 1;
}

size_t gemm_split_floats(int M, int N, int K) {
  const int sp = gemm_splits(EPI_RESADD, M, N, K);
  if (sp <= 1) return 0;
  return (size_t)((N + 63) / 64) * ((M + 63) / 64) * sp * 64 * 64;
}

hipError_t gemm_bf16(int epi, const bf16_t* A, int M, const bf16_t* W, int N, int K, void* out,
                     int64_t ldo, hipStream_t s, float* split_part, uint32_t* split_cnt) {
  if (M <= 0) return hipSuccess;
  if (K % BK != 0 || N % 16 != 0) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && N % 64 != 0) return hipErrorInvalidValue;
  // the epilogue writes four consecutive outputs per lane (16 / 8 bytes)
  if (ldo % 4 != 0 || reinterpret_cast<uintptr_t>(out) % (epi == EPI_SWIGLU ? 8 : 16) != 0) return hipErrorInvalidValue;
  if (g_gemm_cfg < 0 && split_part && split_cnt) {
    const int sp = gemm_splits(epi, M, N, K);
    if (sp > 1) return gemm_launch<2, 2, 2, 2, 1>(epi, A, M, W, N, K, out, ldo, s, split_part, split_cnt, sp);
  }
  int cfg = g_gemm_cfg;
  if (cfg < 0) {
    // The largest tile whose grid still gives each of the 256 CUs a block:
    // 256 x 256 (4-slice LDS pipeline, 16 wavefronts), else 128 x 128 (the
    // same pipeline, 4 wavefronts), else 64 x 64.  Measured on MI355X at
    // M = 32768: 790, 970 and 950 TFLOP/s for the q/k/v, gate/up and down
    // shapes with the 256 x 256 pipeline; the other configurations
    // (8-wavefront tiles, two blocks per CU, two LDS slices, fragment
    // double-buffering) measured 5-25 % below it.  At M = 4096 the 128 x 128
    // pipeline runs the o and down shapes (256 tiles) at 445 and 516 TFLOP/s,
    // 15 % above the 128 x 128 tile without it.
    cfg = auto_config(M, N);
  }
  switch (cfg) {
    case 0: return gemm_launch<2, 2, 2, 2, 1>(epi, A, M, W, N, K, out, ldo, s);   //  64 x  64, 4 waves
    case 1: return gemm_launch<4, 4, 2, 2, 1>(epi, A, M, W, N, K, out, ldo, s);   // 128 x 128, 4 waves
    case 2: return gemm_launch<4, 4, 4, 2, 1>(epi, A, M, W, N, K, out, ldo, s);   // 256 x 128, 8 waves
    case 3: return gemm_launch<4, 4, 2, 4, 1>(epi, A, M, W, N, K, out, ldo, s);   // 128 x 256, 8 waves
    case 4: return gemm_launch<4, 8, 2, 2, 1>(epi, A, M, W, N, K, out, ldo, s);   // 128 x 256, 4 waves
    case 5: return gemm_launch<8, 4, 2, 2, 1>(epi, A, M, W, N, K, out, ldo, s);   // 256 x 128, 4 waves
    case 6: return gemm_launch<4, 4, 4, 4, 1>(epi, A, M, W, N, K, out, ldo, s);   // 256 x 256, 16 waves
    case 7: return gemm_dma_launch<4, 4, 4, 4, 4, false>(epi, A, M, W, N, K, out, ldo, s);  // 256 x 256, 4-slice pipeline
    case 8: return gemm_dma_launch<4, 4, 2, 2, 4, true>(epi, A, M, W, N, K, out, ldo, s);  // 128 x 128, 4-slice pipeline
    case 9: return gemm_dma_launch<4, 4, 4, 2, 3, false>(epi, A, M, W, N, K, out, ldo, s); // 256 x 128, 3 slices, 2 blocks/CU
    case 10: return gemm_dma_launch<4, 4, 2, 4, 3, false>(epi, A, M, W, N, K, out, ldo, s); // 128 x 256, 3 slices, 2 blocks/CU
    case 11: return gemm_dma_launch<4, 4, 4, 4, 2, false>(epi, A, M, W, N, K, out, ldo, s); // 256 x 256, 2 slices
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q3k
