// Host-side launch wrappers of the gfx950 kernels.  The entry points in api.hip
// validate every argument before calling these; the launchers only size grids.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

// Where entry s of sequence b of one cache series lives.  Dense (table ==
// nullptr): row b * nrows + s of a [B, nrows] array.  Paged (shuhuayu section
// 06 / Evidence Ledger Section 3.5.1: blocks of lcm(m, m') tokens, each holding
// 2^shift entries of the series): slot s & (2^shift - 1) of page
// table[b * max_blocks + (s >> shift)], pages page_bytes apart.
struct PageMap {
  const int32_t* table;
  int64_t page_bytes;
  int max_blocks;
  int shift;
  __host__ __device__ bool paged() const { return table != nullptr; }
  // page id of the block holding entry s (paged only)
  __device__ __forceinline__ int page(int b, int s) const {
    return table[(int64_t)b * max_blocks + (s >> shift)];
  }
  // byte offset of entry s of sequence b from the series base, rows rb bytes
  __device__ __forceinline__ int64_t off(int b, int s, int nrows, int64_t rb) const {
    if (table == nullptr) return ((int64_t)b * nrows + s) * rb;
    return (int64_t)page(b, s) * page_bytes + (int64_t)(s & ((1 << shift) - 1)) * rb;
  }
};
constexpr PageMap kDense = {nullptr, 0, 0, 0};

// prep.hip / compress.hip -------------------------------------------------
hipError_t launch_prep_rows(const void* x, csa_dtype x_t, int64_t rows, int c,
                            const float* norm_w, float eps, int rope_dims, float rope_theta,
                            const int32_t* pos, int rows_per_seq, int pos_stride, int pos_offset,
                            void* out, uint8_t* out_scale, csa_dtype out_t, hipStream_t s);

// C[M, N] (fp32) = A[M, K] * B[K, N]; A and B both f32 or both bf16, row-major
hipError_t launch_gemm(const void* A, const void* Bm, csa_dtype t, float* C, int M, int N, int K,
                       hipStream_t s);
// dst[c][r] = src[r][c], bf16 [R, Cc] -> [Cc, R]
hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int R, int Cc, hipStream_t s);
// oproj.hip: C_g[M, N] (fp32, row stride ldc, groups c_goff apart) = A[M, K] . W_g[N, K]^T,
// W_g = W + g * w_gstride (bf16, K % 64 == 0, 16-byte aligned rows)
hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t w_gstride,
                          float* C, int64_t ldc, int64_t c_goff, int M, int N, int K, int groups,
                          hipStream_t s);

hipError_t launch_pool(const float* Ca, const float* Za, const float* Cb, const float* Zb,
                       const float* bias_a, const float* bias_b, int B, int T, int m, int c,
                       const float* norm_w, float eps, int rope_dims, float rope_theta,
                       int pos_stride, int pos_offset, void* out, uint8_t* out_scale,
                       csa_dtype out_t, hipStream_t s, const int32_t* entry = nullptr,
                       int Nmax = 0, const PageMap& pg = kDense);

// indexer.hip ---------------------------------------------------------------
hipError_t launch_indexer(const void* qI, const uint8_t* qI_scale, csa_dtype in_t, const float* w,
                          const void* kI, const uint8_t* kI_scale, const int32_t* q_pos,
                          const int32_t* n_entries, int B, int Tq, int nI, int cI, int Nmax,
                          int m, void* scores, csa_dtype score_t, hipStream_t s,
                          const PageMap& pg = kDense);

// topk.hip --------------------------------------------------------------------
// workspace bytes top-k needs (0 for rows of up to 16384 entries)
size_t topk_workspace(int B, int Tq, int Nmax);
hipError_t launch_topk(const void* scores, csa_dtype score_t, const int32_t* q_pos,
                       const int32_t* n_entries, int B, int Tq, int Nmax, int m, int k,
                       int32_t* idx, void* ws, hipStream_t s);

// oproj.hip --------------------------------------------------------------------
size_t oproj_workspace(int R, int nh, int c, int g, int d_g, int d, csa_dtype t);
hipError_t launch_oproj(const void* o, csa_dtype t, int R, int nh, int c, int g, int d_g,
                        const void* W_a, const void* W_b, int d, void* y, csa_dtype y_t, void* ws,
                        hipStream_t s);

// attend.hip -------------------------------------------------------------------
struct AttendArgs {
  const void* q;
  csa_dtype q_t;
  const float* q_norm_w;
  float eps;
  int rope_dims;
  float rope_theta;
  const int32_t* q_pos;
  const void* kv;
  csa_dtype kv_t;
  int Nmax;
  const int32_t* idx;        // sparse: [B, Tq, k]; NULL for dense (HCA)
  int k;
  const int32_t* n_entries;  // dense only
  int m_prime;               // dense only
  const void* win;
  int win_len;
  int n_win;
  const float* sink;
  float scale;
  int B, Tq, nh, c;
  void* out;
  csa_dtype out_t;
  PageMap pages;             // kv rows: dense [B, Nmax] or paged
};

// workspace bytes the attention call needs for these host sizes
// host checks of every attention argument (api.hip)
csa_status check_attend(const AttendArgs& a);
size_t attend_workspace(const AttendArgs& a);
hipError_t launch_attend(const AttendArgs& a, void* ws, hipStream_t s);

}  // namespace csa
