// Grouped output projection (Evidence Ledger Section 2.3.1: n_h heads -> g
// groups -> d_g intermediates -> d; shuhuayu page section 03: the outputs are
// rotated back by -q before it -- that rotation is the attention epilogue's).
//
//   u[r, j*d_g + e] = sum_k o[r, j*K1 + k] * W_a[j, e, k]     K1 = nh/g * c
//   y[r, n]         = sum_k u[r, k] * W_b[n, k]                 (k < g*d_g)
//
// Two products of the same shape class C[M, N] = A[M, K] . W[N, K]^T with
// linear-layer weights [out, in], so both MFMA operands run along K in memory.
// u is kept in bf16 between them (an activation like any other).
//
//  * few rows (decode: M = query rows <= 64): the weights are the traffic
//    (128 MiB for g*d_g = 8192, d = 4096) and the product is HBM-bound.
//    oproj_skinny_kernel: a block owns 128 output columns (8 waves x 16) over
//    one K-slice; the slice of A's M rows is staged once in LDS and serves all
//    8 waves as the B operand of v_mfma_f32_16x16x32_bf16, while each wave
//    streams its 16 weight rows straight from HBM into the A operand (16 B per
//    lane, two batches of k-steps in flight).  Re-reading A through L2 per
//    16-column tile would move twice the weights' bytes; per 128-column tile
//    it moves an eighth of them.  The K-slices' fp32 partial sums are added in
//    slice order by oproj_reduce_kernel: deterministic.
//  * many rows (prefill): oproj_tiled_kernel, 256 x 128 output tiles through a
//    double-buffered LDS stage, 128 x 64 per wave on v_mfma_f32_32x32x16_bf16
//    (24 B of LDS reads per MFMA cycle per wave, against 32 for 64 x 64), row
//    panels kept on one XCD.
//  * fp32 operands: oproj_generic_kernel, one thread per output (small cases).
#include "common.hpp"
#include "internal.hpp"

namespace csa {

constexpr int OS_WAVES = 8;     // waves of a skinny block, 16 output columns each
constexpr int OS_COLS = OS_WAVES * 16;
constexpr int OS_UNROLL = 4;    // k-steps of 32 per batch of loads

// K-slice length of the skinny kernel for M rows (LDS holds 16 T rows x KS)
__host__ __device__ constexpr int os_kslice(int T) { return T <= 2 ? 1024 : 512; }

// P[ks, m, c_off + n] (row stride ldp) = sum over the block's K-slice ks of
// A[m, a_off + k] W[n, k], for the block's 128 columns n and m < M.
template <int T>  // m-tiles of 16 rows (M <= 16 T)
__global__ __launch_bounds__(OS_WAVES * 64, 2) void oproj_skinny_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t a_goff, const uint16_t* __restrict__ W,
    int64_t w_gstride, float* __restrict__ P, int64_t ldp, int64_t p_goff, int64_t p_split,
    int M, int K) {
  constexpr int KS = os_kslice(T);
  constexpr int LDX = KS + 8;   // LDS row stride (bf16): 16 rows at one k hit distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * T][LDX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = blockIdx.z, ks = blockIdx.y;
  const int n0 = blockIdx.x * OS_COLS + 16 * wave;
  const int k0 = ks * KS;
  // ---- A[:, k0 .. k0 + KS) into registers first (rows past M are zero): these
  // loads are issued before the weight prefetch, so they return first
  constexpr int XCH = 16 * T * (KS / 8) / (OS_WAVES * 64);  // 16-byte chunks per thread
  u32x4 xv[XCH];
#pragma unroll
  for (int j = 0; j < XCH; ++j) {
    const int i = threadIdx.x + j * OS_WAVES * 64;
    const int m = i / (KS / 8), kc = 8 * (i % (KS / 8));
    xv[j] = m < M ? *reinterpret_cast<const u32x4*>(A + (int64_t)m * lda + grp * a_goff + k0 + kc)
                  : u32x4{0u, 0u, 0u, 0u};
  }
  const int kq = 8 * (lane >> 4);  // k offset of the lane's 8 values in a 32-step
  const uint16_t* wrow = W + grp * w_gstride + (int64_t)(n0 + (lane & 15)) * K + k0 + kq;
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 w0[OS_UNROLL], w1[OS_UNROLL];
  constexpr int KB = 32 * OS_UNROLL;
#define OS_LOAD(WW, K_)                                                                   \
  _Pragma("unroll") for (int u = 0; u < OS_UNROLL; ++u)                                   \
    WW[u] = *reinterpret_cast<const u32x4*>(wrow + (K_) + 32 * u);
#define OS_MMA(WW, K_)                                                                    \
  _Pragma("unroll") for (int u = 0; u < OS_UNROLL; ++u)                                   \
    _Pragma("unroll") for (int t = 0; t < T; ++t) {                                        \
      const u32x4 xb = *reinterpret_cast<const u32x4*>(&xs[16 * t + (lane & 15)][(K_) + 32 * u + kq]); \
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, WW[u]),  \
                                                      __builtin_bit_cast(bf16x8, xb), acc[t], 0, 0, 0); \
    }
  OS_LOAD(w0, 0);
  OS_LOAD(w1, KB);
#pragma unroll
  for (int j = 0; j < XCH; ++j) {
    const int i = threadIdx.x + j * OS_WAVES * 64;
    *reinterpret_cast<u32x4*>(&xs[i / (KS / 8)][8 * (i % (KS / 8))]) = xv[j];
  }
  __syncthreads();  // A slice staged
  for (int k = 0; k < KS; k += 2 * KB) {
    OS_MMA(w0, k);
    if (k + 2 * KB < KS) { OS_LOAD(w0, k + 2 * KB); }
    OS_MMA(w1, k + KB);
    if (k + 3 * KB < KS) { OS_LOAD(w1, k + 3 * KB); }
  }
#undef OS_LOAD
#undef OS_MMA
  // lane holds P^T[n = 4(l/16) + r][m = 16t + l%16]: four consecutive columns
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int m = 16 * t + (lane & 15);
    if (m < M)
      *reinterpret_cast<f32x4*>(P + ks * p_split + (int64_t)m * ldp + grp * p_goff + n0 +
                                4 * (lane >> 4)) = acc[t];
  }
}

// C[m, n] = sum over the `splits` (<= OS_MAX_SPLITS) K-slices of P[s, m, n], in
// slice order; every slice's load is issued before the first add
constexpr int OS_MAX_SPLITS = 16;

__global__ __launch_bounds__(256) void oproj_reduce_kernel(const float* __restrict__ P,
                                                           int64_t p_split, int splits,
                                                           void* __restrict__ C, int c_bf16,
                                                           int64_t count) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  f32x4 v[OS_MAX_SPLITS];
#pragma unroll
  for (int k = 0; k < OS_MAX_SPLITS; ++k)
    if (k < splits) v[k] = *reinterpret_cast<const f32x4*>(P + k * p_split + i);
  f32x4 s = v[0];
#pragma unroll
  for (int k = 1; k < OS_MAX_SPLITS; ++k)
    if (k < splits) s += v[k];
  if (c_bf16)
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(C) + i) =
        make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
  else
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(C) + i) = s;
}

// =============================================================== many rows
constexpr int OT_M = 256, OT_N = 128, OT_K = 32, OT_LD = OT_K + 8;

// C tile 256 x 128 per 256-thread block; wave w owns rows 128 (w / 2) .. +127
// and columns 64 (w % 2) .. +63 as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.
// K advances by 32 through a double-buffered LDS stage: the next slice is read
// from global memory into registers while the current one is multiplied, then
// written to the other buffer; one barrier per step.  Blocks are ordered for
// the XCDs: every column tile of row panel mt runs on XCD mt % 8, so the panel
// of A is fetched into one L2.
__global__ __launch_bounds__(256, 2) void oproj_tiled_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t a_goff, const uint16_t* __restrict__ W,
    int64_t w_gstride, void* __restrict__ C, int64_t ldc, int64_t c_goff, int c_bf16, int M, int N,
    int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][OT_M][OT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][OT_N][OT_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nN = (N + OT_N - 1) / OT_N, nM = (M + OT_M - 1) / OT_M;
  const int per_grp = (nM + 7) / 8 * 8 * nN;
  const int grp = blockIdx.x / per_grp, L = blockIdx.x % per_grp;
  const int mt = (L / 8 / nN) * 8 + (L & 7), nt = (L / 8) % nN;
  if (mt >= nM) return;
  const int m0 = mt * OT_M, n0 = nt * OT_N;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 64;
  const uint16_t* Ag = A + grp * a_goff;
  const uint16_t* Wg = W + grp * w_gstride;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  // per K-step: A 256 x 32 = 1024 chunks of 8 (4 per thread), W 128 x 32 = 512 (2 per thread)
  u32x4 ra[4], rw[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = tid + 256 * p, r = idx >> 2, kc = (idx & 3) * 8;
      ra[p] = m0 + r < M ? *reinterpret_cast<const u32x4*>(Ag + (int64_t)(m0 + r) * lda + k0 + kc)
                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = tid + 256 * p, r = idx >> 2, kc = (idx & 3) * 8;
      rw[p] = n0 + r < N ? *reinterpret_cast<const u32x4*>(Wg + (int64_t)(n0 + r) * K + k0 + kc)
                         : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = tid + 256 * p;
      *reinterpret_cast<u32x4*>(&As[b][idx >> 2][(idx & 3) * 8]) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = tid + 256 * p;
      *reinterpret_cast<u32x4*>(&Ws[b][idx >> 2][(idx & 3) * 8]) = rw[p];
    }
  };
  const int nk = K / OT_K;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * OT_K);
#pragma unroll
    for (int ks = 0; ks < OT_K / 16; ++ks) {
      const int kof = 16 * ks + 8 * (lane >> 5);
      bf16x8 af[4], wf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&As[cur][wm + 32 * i + (lane & 31)][kof]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Ws[cur][wn + 32 * j + (lane & 31)][kof]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
  // D: lane holds column l%32, rows 8(r/4) + 4(l/32) + r%4 of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn + 32 * j + (lane & 31);
      if (gn >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (gm >= M) continue;
        const int64_t o = (int64_t)gm * ldc + grp * c_goff + gn;
        if (c_bf16)
          reinterpret_cast<uint16_t*>(C)[o] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        else
          reinterpret_cast<float*>(C)[o] = acc[i][j][r];
      }
    }
}


// C tile 256 x 256 per 256-thread block, one block per CU and one wave per
// SIMD: wave w owns rows 128 (w / 2) .. +127 and columns 128 (w % 2) .. +127 as
// 4 x 4 tiles of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane (in
// the accumulation registers: one wave per SIMD may use 512 registers).  Every
// 16-byte operand read from LDS feeds four matrix-core instructions: 16 B of
// LDS per lane per 32x32x16 instruction, half the 256 x 128 kernel's, and half
// its global traffic per flop.  Same K-step, staging and XCD order otherwise.
constexpr int OB_M = 256, OB_N = 256, OB_K = 64, OB_LD = OB_K + 8;

__global__ __launch_bounds__(256, 1) void oproj_big_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t a_goff, const uint16_t* __restrict__ W,
    int64_t w_gstride, void* __restrict__ C, int64_t ldc, int64_t c_goff, int c_bf16, int M, int N,
    int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][OB_M][OB_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][OB_N][OB_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nN = (N + OB_N - 1) / OB_N, nM = (M + OB_M - 1) / OB_M;
  const int per_grp = (nM + 7) / 8 * 8 * nN;
  const int grp = blockIdx.x / per_grp, L = blockIdx.x % per_grp;
  const int mt = (L / 8 / nN) * 8 + (L & 7), nt = (L / 8) % nN;
  if (mt >= nM) return;
  const int m0 = mt * OB_M, n0 = nt * OB_N;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const uint16_t* Ag = A + grp * a_goff;
  const uint16_t* Wg = W + grp * w_gstride;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  // per K-step: A and W 256 x 64 each = 2048 chunks of 8 (8 per thread each)
  u32x4 ra[8], rw[8];
  auto load = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int idx = tid + 256 * p, r = idx >> 3, kc = (idx & 7) * 8;
      ra[p] = m0 + r < M ? *reinterpret_cast<const u32x4*>(Ag + (int64_t)(m0 + r) * lda + k0 + kc)
                         : u32x4{0u, 0u, 0u, 0u};
      rw[p] = n0 + r < N ? *reinterpret_cast<const u32x4*>(Wg + (int64_t)(n0 + r) * K + k0 + kc)
                         : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int idx = tid + 256 * p;
      *reinterpret_cast<u32x4*>(&As[b][idx >> 3][(idx & 7) * 8]) = ra[p];
      *reinterpret_cast<u32x4*>(&Ws[b][idx >> 3][(idx & 7) * 8]) = rw[p];
    }
  };
  const int nk = K / OB_K;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * OB_K);
    // operand fragments of sub-step ks + 1 are read while ks multiplies
    bf16x8 af[2][4], wf[2][4];
    auto frags = [&](int ks, int fb) {
      const int kof = 16 * ks + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[fb][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&As[cur][wm + 32 * i + (lane & 31)][kof]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wf[fb][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Ws[cur][wn + 32 * j + (lane & 31)][kof]));
    };
    frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < OB_K / 16; ++ks) {
      if (ks + 1 < OB_K / 16) frags(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], wf[ks & 1][j], acc[i][j], 0, 0, 0);
      if (ks + 1 < OB_K / 16) {
        // the next fragments' 8 reads spread over this sub-step's 16 products
        _Pragma("unroll") for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
      }
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
  // D: lane holds column l%32, rows 8(r/4) + 4(l/32) + r%4 of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + wn + 32 * j + (lane & 31);
      if (gn >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (gm >= M) continue;
        const int64_t o = (int64_t)gm * ldc + grp * c_goff + gn;
        if (c_bf16)
          reinterpret_cast<uint16_t*>(C)[o] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        else
          reinterpret_cast<float*>(C)[o] = acc[i][j][r];
      }
    }
}

// =============================================================== fp32 operands
__global__ __launch_bounds__(256) void oproj_generic_kernel(
    const float* __restrict__ A, int64_t lda, int64_t a_goff, const float* __restrict__ W,
    int64_t w_gstride, void* __restrict__ C, int64_t ldc, int64_t c_goff, int c_bf16, int M, int N,
    int K) {
  const int grp = blockIdx.z;
  const int n = blockIdx.x * 256 + threadIdx.x, m = blockIdx.y;
  if (n >= N) return;
  const float* a = A + (int64_t)m * lda + grp * a_goff;
  const float* w = W + grp * w_gstride + (int64_t)n * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], w[k], s);
  const int64_t o = (int64_t)m * ldc + grp * c_goff + n;
  if (c_bf16)
    reinterpret_cast<uint16_t*>(C)[o] = (uint16_t)f32_to_bf16(s);
  else
    reinterpret_cast<float*>(C)[o] = s;
}

static bool skinny_fits(int M, int N, int K) {
  const int ks = os_kslice((M + 15) / 16 > 2 ? 4 : 2);
  return M <= 64 && N % OS_COLS == 0 && K % ks == 0 && K / ks <= OS_MAX_SPLITS;
}

// C_g[M, N] (fp32, row stride ldc, groups c_goff apart) = A[M, K] . W_g[N, K]^T
// with W_g = W + g * w_gstride, for g < groups, on the 256 x 256-tile kernel
// (the compressor's projections: M = tokens, K = d).  K % 64 == 0 and 16-byte
// aligned rows are the caller's to check.
hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t w_gstride,
                          float* C, int64_t ldc, int64_t c_goff, int M, int N, int K, int groups,
                          hipStream_t s) {
  const int64_t nN = (N + OB_N - 1) / OB_N, nM = (M + OB_M - 1) / OB_M;
  dim3 grid((unsigned)((nM + 7) / 8 * 8 * nN * groups));
  hipLaunchKernelGGL(oproj_big_kernel, grid, dim3(256), 0, s, A, lda, (int64_t)0, W, w_gstride,
                     (void*)C, ldc, c_goff, 0, M, N, K);
  return hipGetLastError();
}

// one product C[M, groups * N] = A . W^T over `groups` column groups (C row
// stride ldc = groups * N); `part` is fp32 workspace for the skinny path
static hipError_t launch_oproj_gemm(const void* A, int64_t lda, int64_t a_goff, const void* W,
                                    int64_t w_gstride, void* C, int c_bf16, int M, int N, int K,
                                    int groups, bool bf16, float* part, hipStream_t s) {
  const int64_t ldc = (int64_t)groups * N;
  if (!bf16) {
    dim3 grid((N + 255) / 256, M, groups);
    hipLaunchKernelGGL(oproj_generic_kernel, grid, dim3(256), 0, s, (const float*)A, lda, a_goff,
                       (const float*)W, w_gstride, C, ldc, (int64_t)N, c_bf16, M, N, K);
  } else if (skinny_fits(M, N, K)) {
    const int T = (M + 15) / 16 <= 1 ? 1 : ((M + 15) / 16 <= 2 ? 2 : 4);
    const int splits = K / os_kslice(T);
    const int64_t p_split = (int64_t)M * ldc;
    dim3 grid(N / OS_COLS, splits, groups);
    if (T == 1)
      hipLaunchKernelGGL(oproj_skinny_kernel<1>, grid, dim3(OS_WAVES * 64), 0, s, (const uint16_t*)A,
                         lda, a_goff, (const uint16_t*)W, w_gstride, part, ldc, (int64_t)N, p_split,
                         M, K);
    else if (T == 2)
      hipLaunchKernelGGL(oproj_skinny_kernel<2>, grid, dim3(OS_WAVES * 64), 0, s, (const uint16_t*)A,
                         lda, a_goff, (const uint16_t*)W, w_gstride, part, ldc, (int64_t)N, p_split,
                         M, K);
    else
      hipLaunchKernelGGL(oproj_skinny_kernel<4>, grid, dim3(OS_WAVES * 64), 0, s, (const uint16_t*)A,
                         lda, a_goff, (const uint16_t*)W, w_gstride, part, ldc, (int64_t)N, p_split,
                         M, K);
    const int64_t count = p_split;  // M * ldc, a multiple of 4
    hipLaunchKernelGGL(oproj_reduce_kernel, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0,
                       s, (const float*)part, p_split, splits, C, c_bf16, count);
  } else if (M >= OB_M && N >= OB_N && K % OB_K == 0) {
    const int64_t nN = (N + OB_N - 1) / OB_N, nM = (M + OB_M - 1) / OB_M;
    dim3 grid((unsigned)((nM + 7) / 8 * 8 * nN * groups));
    hipLaunchKernelGGL(oproj_big_kernel, grid, dim3(256), 0, s, (const uint16_t*)A, lda, a_goff,
                       (const uint16_t*)W, w_gstride, C, ldc, (int64_t)N, c_bf16, M, N, K);
  } else {
    const int64_t nN = (N + OT_N - 1) / OT_N, nM = (M + OT_M - 1) / OT_M;
    dim3 grid((unsigned)((nM + 7) / 8 * 8 * nN * groups));
    hipLaunchKernelGGL(oproj_tiled_kernel, grid, dim3(256), 0, s, (const uint16_t*)A, lda, a_goff,
                       (const uint16_t*)W, w_gstride, C, ldc, (int64_t)N, c_bf16, M, N, K);
  }
  return hipGetLastError();
}

// workspace: u (R x g*d_g in the operand type), then for the skinny path the
// fp32 K-slice partials of the larger of the two products
static size_t part_floats(int R, int N, int K, int groups) {
  if (!skinny_fits(R, N, K)) return 0;
  const int T = (R + 15) / 16 > 2 ? 4 : 2;
  return (size_t)(K / os_kslice(T)) * R * N * groups;
}

size_t oproj_workspace(int R, int nh, int c, int g, int d_g, int d, csa_dtype t) {
  const size_t u = (size_t)R * g * d_g * (t == CSA_BF16 ? sizeof(uint16_t) : sizeof(float));
  if (t != CSA_BF16) return u;
  const size_t ua = (u + 255) / 256 * 256;
  const size_t p1 = part_floats(R, d_g, nh / g * c, g), p2 = part_floats(R, d, g * d_g, 1);
  return ua + (p1 > p2 ? p1 : p2) * sizeof(float);
}

hipError_t launch_oproj(const void* o, csa_dtype t, int R, int nh, int c, int g, int d_g,
                        const void* W_a, const void* W_b, int d, void* y, csa_dtype y_t, void* ws,
                        hipStream_t s) {
  if (R == 0) return hipSuccess;
  const bool bf = t == CSA_BF16;
  const int K1 = nh / g * c, Ku = g * d_g;
  const size_t ub = (size_t)R * Ku * (bf ? sizeof(uint16_t) : sizeof(float));
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + (ub + 255) / 256 * 256);
  // u = per-group o . W_a[j]^T  (bf16 for bf16 operands, else fp32)
  hipError_t e = launch_oproj_gemm(o, (int64_t)nh * c, K1, W_a, (int64_t)d_g * K1, ws, bf ? 1 : 0,
                                   R, d_g, K1, g, bf, part, s);
  if (e != hipSuccess) return e;
  // y = u . W_b^T
  return launch_oproj_gemm(ws, Ku, 0, W_b, 0, y, y_t == CSA_BF16 ? 1 : 0, R, d, Ku, 1, bf, part, s);
}

}  // namespace csa
