// Token compression (Evidence Ledger Eqs 9-12 for CSA, 20-26 for HCA) and the
// row finisher (Section 2.3.3 RMSNorm + partial RoPE, Section 2.3.4 storage).
//
//   projections  C = H W  (fp32 accumulate): an MFMA bf16 GEMM (gfx950
//                v_mfma_f32_32x32x16_bf16, LDS-staged 128x128 tiles) or a
//                fp32 VALU GEMM for fp32 inputs;
//   pooling      per entry and channel, a softmax over the 2m candidates
//                (own block via the a-series, preceding block via the b-series)
//                and the weighted sum, then RMSNorm, RoPE and the store, all in
//                one block per entry.
#include "common.hpp"
#include "internal.hpp"
#include "rowops.hpp"

namespace csa {

// =============================================================== row prep
__global__ __launch_bounds__(256) void prep_rows_kernel(
    const uint8_t* __restrict__ x, csa_dtype x_t, int c, const float* __restrict__ norm_w,
    float eps, int d_r, Rope rt, const int32_t* __restrict__ pos, int rows_per_seq,
    int pos_stride, int pos_offset, uint8_t* __restrict__ out, uint8_t* __restrict__ out_scale,
    csa_dtype out_t) {
  extern __shared__ float smem[];
  float* row = smem;
  float* red = smem + c;
  const int64_t r = blockIdx.x;
  const uint8_t* src = x + r * row_bytes(x_t, c, 0);
  for (int j = threadIdx.x; j < c; j += blockDim.x) row[j] = load_elem(src, x_t, j);
  __syncthreads();
  const double p = pos != nullptr ? (double)pos[r]
                                  : (double)pos_offset + (double)pos_stride * (double)(r % rows_per_seq);
  const int64_t ob = row_bytes(out_t, c, d_r);
  finish_row(row, c, norm_w, eps, d_r, rt, p, out + r * ob,
             out_t == CSA_MXFP4 ? out_scale + r * (c / 32) : nullptr, out_t, red);
}

hipError_t launch_prep_rows(const void* x, csa_dtype x_t, int64_t rows, int c,
                            const float* norm_w, float eps, int rope_dims, float rope_theta,
                            const int32_t* pos, int rows_per_seq, int pos_stride, int pos_offset,
                            void* out, uint8_t* out_scale, csa_dtype out_t, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // one 256-thread block per row; rows <= 2^24 keeps the grid within 2^32 lanes
  const size_t shm = (size_t)(c + 16) * sizeof(float);
  hipLaunchKernelGGL(prep_rows_kernel, dim3((unsigned)rows), dim3(256), shm, s,
                     (const uint8_t*)x, x_t, c, norm_w, eps, rope_dims,
                     make_rope(rope_dims, rope_theta), pos, rows_per_seq, pos_stride,
                     pos_offset, (uint8_t*)out, out_scale, out_t);
  return hipGetLastError();
}

// =============================================================== fp32 / bf16 VALU GEMM
// C[M,N] = A[M,K] B[K,N]; 64x64 tile, 16-deep K slices, 4x4 outputs per thread.
template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__global__ __launch_bounds__(256) void gemm_valu_kernel(const T* __restrict__ A,
                                                        const T* __restrict__ Bm,
                                                        float* __restrict__ C, int M, int N, int K) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      const int r = i >> 4, kk = i & 15;  // A tile element (row r, k kk)
      const int gm = m0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? ld<T>(A, (int64_t)gm * K + gk) : 0.f;
      const int bk = i >> 6, bn = i & 63;  // B tile element (k bk, col bn)
      const int gk2 = k0 + bk, gn = n0 + bn;
      Bs[bk][bn] = (gk2 < K && gn < N) ? ld<T>(Bm, (int64_t)gk2 * N + gn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + ty + 16 * i, gn = n0 + tx + 16 * j;
      if (gm < M && gn < N) C[(int64_t)gm * N + gn] = acc[i][j];
    }
}

// =============================================================== bf16 MFMA GEMM
// 128x128 output tile per 256-thread block, K sliced by 32.  Each wave owns a
// 64x64 quadrant = 2x2 MFMA 32x32 tiles.  LDS holds the A slice row-major
// [m][k] and the B slice transposed [n][k], so both MFMA operands are 16-byte
// contiguous reads (lane: row l%32, k = 8*(l/32) + 0..7 of each 16-deep step).
constexpr int GB_M = 128, GB_N = 128, GB_K = 32, GB_LD = GB_K + 8;

__global__ __launch_bounds__(256) void gemm_bf16_mfma_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ Bm,
                                                             float* __restrict__ C, int M, int N,
                                                             int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GB_M][GB_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[GB_N][GB_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * GB_M, n0 = blockIdx.x * GB_N;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  for (int k0 = 0; k0 < K; k0 += GB_K) {
    // A slice: 128 rows x 32 k = 512 chunks of 8 bf16
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = tid + 256 * p;
      const int r = idx >> 2, kc = (idx & 3) * 8;
      const int gm = m0 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gm < M) v = *reinterpret_cast<const u32x4*>(A + (int64_t)gm * K + k0 + kc);
      *reinterpret_cast<u32x4*>(&As[r][kc]) = v;
    }
    // B slice: 32 k x 128 n = 512 chunks of 8 n-consecutive values, stored transposed
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = tid + 256 * p;
      const int kk = idx >> 4, nc = (idx & 15) * 8;
      const int gn = n0 + nc;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gn + 7 < N) {
        v = *reinterpret_cast<const u32x4*>(Bm + (int64_t)(k0 + kk) * N + gn);
      } else {
        uint16_t t[8];
        for (int i = 0; i < 8; ++i) t[i] = (gn + i < N) ? Bm[(int64_t)(k0 + kk) * N + gn + i] : 0;
        v = {t[0] | (uint32_t)t[1] << 16, t[2] | (uint32_t)t[3] << 16, t[4] | (uint32_t)t[5] << 16,
             t[6] | (uint32_t)t[7] << 16};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Bt[nc + 2 * i][kk] = (uint16_t)(v[i] & 0xFFFFu);
        Bt[nc + 2 * i + 1][kk] = (uint16_t)(v[i] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < GB_K / 16; ++ks) {
      const int kof = 16 * ks + 8 * (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               &As[wm + 32 * i + (lane & 31)][kof]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                &Bt[wn + 32 * j + (lane & 31)][kof]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // D layout: lane holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (gm < M && gn < N) C[(int64_t)gm * N + gn] = acc[i][j][r];
      }
    }
}

// dst[c][r] = src[r][c] for a [R, Cc] bf16 matrix (weights [d, c] -> [c, d]),
// through a 32 x 33 shared tile
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst, int R,
                                                             int Cc) {
  __shared__ uint16_t t[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int j = ty; j < 32; j += 8) {
    const int r = r0 + j, c = c0 + tx;
    t[j][tx] = (r < R && c < Cc) ? src[(int64_t)r * Cc + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int j = ty; j < 32; j += 8) {
    const int c = c0 + j, r = r0 + tx;
    if (c < Cc && r < R) dst[(int64_t)c * R + r] = t[tx][j];
  }
}

hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int R, int Cc, hipStream_t s) {
  dim3 grid((Cc + 31) / 32, (R + 31) / 32);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, src, dst, R, Cc);
  return hipGetLastError();
}

hipError_t launch_gemm(const void* A, const void* Bm, csa_dtype t, float* C, int M, int N, int K,
                       hipStream_t s) {
  if (t == CSA_BF16 && K % GB_K == 0 && N % 8 == 0) {
    dim3 grid((N + GB_N - 1) / GB_N, (M + GB_M - 1) / GB_M);
    hipLaunchKernelGGL(gemm_bf16_mfma_kernel, grid, dim3(256), 0, s, (const uint16_t*)A,
                       (const uint16_t*)Bm, C, M, N, K);
  } else {
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    if (t == CSA_BF16)
      hipLaunchKernelGGL(gemm_valu_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)A,
                         (const uint16_t*)Bm, C, M, N, K);
    else
      hipLaunchKernelGGL(gemm_valu_kernel<float>, grid, dim3(256), 0, s, (const float*)A,
                         (const float*)Bm, C, M, N, K);
  }
  return hipGetLastError();
}

// =============================================================== pooling + finish
// Evidence Ledger Eqs 11-12: entry i, channel j pools the candidates
//   own block       Z^a[m i + u, j] + bias_a[u, j]  ->  C^a[m i + u, j]
//   preceding block Z^b[m(i-1) + u, j] + bias_b[u, j] -> C^b[m(i-1) + u, j]  (overlap, i > 0)
// by a max-subtracted softmax over the candidates; Za == NULL means m == 1
// with a single candidate (the entry is C^a's row).
// Append mode (entry != NULL): each sequence's T rows are only the tail -- the
// preceding block (overlap) then the block just completed -- and its one new
// entry is entry[b], written to row entry[b] of that sequence's Nmax cache
// rows.  The candidates and the order of every operation are those of the
// full pass, so the appended row equals the full pass's row bit for bit.
__global__ __launch_bounds__(256) void pool_kernel(
    const float* __restrict__ Ca, const float* __restrict__ Za, const float* __restrict__ Cb,
    const float* __restrict__ Zb, const float* __restrict__ bias_a,
    const float* __restrict__ bias_b, int T, int m, int c, const float* __restrict__ norm_w,
    float eps, int d_r, Rope rt, int pos_stride, int pos_offset, uint8_t* __restrict__ out,
    uint8_t* __restrict__ out_scale, csa_dtype out_t, const int32_t* __restrict__ entry,
    int Nmax, PageMap pg) {
  extern __shared__ float smem[];
  float* row = smem;
  float* red = smem + c;
  const int b = blockIdx.y;
  const int i = entry != nullptr ? entry[b] : blockIdx.x;  // entry index in the sequence
  if (entry != nullptr && (i < 0 || i >= Nmax)) return;
  const int own0 = entry != nullptr ? T - m : m * i;        // first row of the own block
  const int prv0 = entry != nullptr ? 0 : m * (i - 1);      // first row of the preceding block
  const int64_t base = (int64_t)b * T * c;
  const bool prev = (Cb != nullptr) && i > 0;
  for (int j = threadIdx.x; j < c; j += blockDim.x) {
    if (Za == nullptr) {
      row[j] = Ca[base + (int64_t)i * c + j];
      continue;
    }
    float mx = -INFINITY;
    for (int u = 0; u < m; ++u)
      mx = fmaxf(mx, Za[base + (int64_t)(own0 + u) * c + j] + bias_a[u * c + j]);
    if (prev)
      for (int u = 0; u < m; ++u)
        mx = fmaxf(mx, Zb[base + (int64_t)(prv0 + u) * c + j] + bias_b[u * c + j]);
    float den = 0.f, num = 0.f;
    for (int u = 0; u < m; ++u) {
      const int64_t t = base + (int64_t)(own0 + u) * c + j;
      const float e = expf(Za[t] + bias_a[u * c + j] - mx);
      den += e;
      num = fmaf(e, Ca[t], num);
    }
    if (prev)
      for (int u = 0; u < m; ++u) {
        const int64_t t = base + (int64_t)(prv0 + u) * c + j;
        const float e = expf(Zb[t] + bias_b[u * c + j] - mx);
        den += e;
        num = fmaf(e, Cb[t], num);
      }
    row[j] = num / den;
  }
  __syncthreads();
  // the row (and the MXFP4 scales, a series of c/32-byte rows sharing the
  // pages) of entry i of sequence b
  const int nrows = entry != nullptr ? Nmax : T / m;
  const int64_t ob = row_bytes(out_t, c, d_r);
  finish_row(row, c, norm_w, eps, d_r, rt, (double)pos_stride * i + pos_offset,
             out + pg.off(b, i, nrows, ob),
             out_t == CSA_MXFP4 ? out_scale + pg.off(b, i, nrows, c / 32) : nullptr, out_t, red);
}

hipError_t launch_pool(const float* Ca, const float* Za, const float* Cb, const float* Zb,
                       const float* bias_a, const float* bias_b, int B, int T, int m, int c,
                       const float* norm_w, float eps, int rope_dims, float rope_theta,
                       int pos_stride, int pos_offset, void* out, uint8_t* out_scale,
                       csa_dtype out_t, hipStream_t s, const int32_t* entry, int Nmax,
                       const PageMap& pg) {
  const int n_out = entry != nullptr ? 1 : T / m;
  if (n_out == 0 || B == 0) return hipSuccess;
  const size_t shm = (size_t)(c + 16) * sizeof(float);
  hipLaunchKernelGGL(pool_kernel, dim3(n_out, B), dim3(256), shm, s, Ca, Za, Cb, Zb, bias_a,
                     bias_b, T, m, c, norm_w, eps, rope_dims,
                     make_rope(rope_dims, rope_theta), pos_stride, pos_offset,
                     (uint8_t*)out, out_scale, out_t, entry, Nmax, pg);
  return hipGetLastError();
}

}  // namespace csa
